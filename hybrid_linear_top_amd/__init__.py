"""MI355X-native LISA (Linear-Indexed Sparse Attention) layer forward pass.

The compute path lives in the HIP library built from ``csrc/`` and is reached
through :mod:`hybrid_linear_top_amd.lisa`; :mod:`hybrid_linear_top_amd.inputs`
holds the seeded synthetic workloads.  Importing this package loads nothing.
"""
