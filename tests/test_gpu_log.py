"""LISA_LOG=1: every call prints its entry point and shapes to stderr (once
the arguments pass their checks).  Runs in a child process, since the
library reads the variable once per process."""
import os
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import torch
from hybrid_linear_top_amd import inputs as gen, lisa
from hybrid_linear_top_amd.inputs import LayerConfig
cfg = LayerConfig("log_probe", "prefill", "bf16", B=1, n=70, Hq=4, Hkv=2, d=64, HI=4, dI=32, M=16, chunk=64, seed=3)
inp = gen.make_prefill_inputs(cfg)
dims = lisa.dims_from_config(cfg)
dv = lisa.to_device
lisa.prefill(dims, *[dv(inp[k]) for k in ("q", "k", "v", "q_idx", "k_idx", "w_idx", "gate")])
torch.cuda.synchronize()
print("child done", flush=True)
"""


@pytest.mark.gpu
def test_lisa_log_prints_the_call():
    env = dict(os.environ, LISA_LOG="1", PYTHONPATH=REPO)
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=REPO, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "child done" in r.stdout
    lines = [l for l in r.stderr.splitlines() if l.startswith("lisa: ")]
    assert lines == ["lisa: prefill B=1 past=0 n=70 heads=4/2 d=64 indexer=4x32 top_m=16 chunk=64 bf16"], lines
