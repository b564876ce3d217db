"""lisa_decode_step_noalloc (static scratch, no workspace argument) against
lisa_decode_step with a caller workspace, through the C ABI: the same
kernels on the same inputs must give the same outputs, sets and states bit
for bit.  Two calls in a row, the second with a smaller batch, shorter
contexts and another shape, so the second reads scratch the first left
behind."""
import ctypes
import sys

import numpy as np
import pytest

from hybrid_linear_top_amd import inputs as gen
from hybrid_linear_top_amd.inputs import LayerConfig

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _run_both(cfg, lengths):
    import torch
    from hybrid_linear_top_amd import lisa
    inp = gen.make_decode_inputs(cfg, lengths=lengths)
    dims = lisa.dims_from_config(cfg)
    dv = lisa.to_device
    B, max_ctx = inp["B"], inp["max_ctx"]
    args = [dv(inp[k]) for k in ("q", "k_cache", "v_cache", "q_idx", "k_idx_cache", "w_idx", "gate")]
    cu = dv(inp["cu_ctx"])
    st_ref = dv(inp["state"])
    out_ref, idx_ref = lisa.decode_step(dims, cu, max_ctx, *args, st_ref)
    st = dv(inp["state"])
    out = torch.empty_like(args[0])
    idx = torch.full((B, cfg.Hkv, cfg.M), -7, dtype=torch.int32, device=args[0].device)
    p = lisa._ptr
    status = lisa.lisa_decode_step_noalloc(dims, B, p(cu), int(max_ctx), *[p(a) for a in args], p(st), p(out),
                                           p(idx), 0)
    assert status == lisa.LISA_OK, lisa.lisa_last_error()
    torch.cuda.synchronize()
    for name, x, y in (("out", out, out_ref), ("topm", idx, idx_ref), ("state", st, st_ref)):
        assert torch.equal(x, y), f"{name} differs from lisa_decode_step"
    # without topm_out the sets stay in scratch; the output is unchanged
    st2 = dv(inp["state"])
    out2 = torch.empty_like(args[0])
    status = lisa.lisa_decode_step_noalloc(dims, B, p(cu), int(max_ctx), *[p(a) for a in args], p(st2),
                                           p(out2), None, 0)
    assert status == lisa.LISA_OK, lisa.lisa_last_error()
    torch.cuda.synchronize()
    assert torch.equal(out2, out_ref) and torch.equal(st2, st_ref)


def test_noalloc_decode_matches_workspace_decode():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = LayerConfig("noalloc_big", "decode", "bf16", B=8, Hq=12, Hkv=2, d=128, HI=4, dI=64, M=256, seed=91)
    L1 = np.array([16385, 900, 20000, 257, 5000, 33000, 1, 12000])
    _say("decode noalloc", big.name, "lengths", L1.tolist())
    _run_both(big, L1)
    small = LayerConfig("noalloc_small", "decode", "bf16", B=3, Hq=8, Hkv=4, d=64, HI=2, dI=32, M=64, seed=92)
    L2 = np.array([70, 3000, 64])
    _say("decode noalloc", small.name, "lengths", L2.tolist())
    _run_both(small, L2)


def test_noalloc_decode_rejects_oversized_scratch():
    """A step whose scratch exceeds the static 32 MiB is refused before any
    launch (B x G x max_ctx fp32 scores above it)."""
    from hybrid_linear_top_amd import lisa
    dims = lisa.make_dims(28, 4, 128, 4, 64, 512, "bf16")
    fake = 1 << 20
    st = lisa.lisa_decode_step_noalloc(dims, 64, fake, 65536, *([fake] * 7), fake, fake, 0, 0)
    assert st == lisa.LISA_ERR_UNSUPPORTED
    assert "scratch" in lisa.lisa_last_error()
