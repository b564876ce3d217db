"""The backward oracle against its pins, and planted mistakes in copies of it
(CPU only): every mutant must be caught by at least one pin."""
import os
import types

import pytest

from oracle import backward as bwd
from tests.backward_pins import ALL_BWD_PINS


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    pin(bwd.prefill_backward)


MUTANTS = {
    "gate_derivative_dropped": ("ga * (1.0 - ga) * float(", "ga * float("),
    "gate_sign": ("(osp[b, t, h] - olin[b, t, h])", "(olin[b, t, h] - osp[b, t, h])"),
    "softmax_mean_term_dropped": ("dlogit = p * (dp - float(p @ dp))", "dlogit = p * dp"),
    "dq_unscaled": ("dq[b, t, h] += scale * (dlogit @ K)", "dq[b, t, h] += dlogit @ K"),
    "dk_unscaled": ("dk[b, sel, g] += scale * np.outer(dlogit, q[b, t, h])",
                    "dk[b, sel, g] += np.outer(dlogit, q[b, t, h])"),
    "dv_uses_output_grad_ungated": ("dv[b, sel, g] += np.outer(p, d_sp)",
                                    "dv[b, sel, g] += np.outer(p, dO)"),
    "linear_dq_transposed": ("dq[b, t, h] += states[t] @ d_lin", "dq[b, t, h] += states[t].T @ d_lin"),
    "suffix_excludes_self": ("                H = H + np.outer(q[b, t, h], d_lin)\n                dk[b, t, g] += H @ v[b, t, g]\n                dv[b, t, g] += H.T @ k[b, t, g]",
                             "                dk[b, t, g] += H @ v[b, t, g]\n                dv[b, t, g] += H.T @ k[b, t, g]\n                H = H + np.outer(q[b, t, h], d_lin)"),
    "state_out_grad_ignored": ("H = np.zeros((d, d)) if d_state_out is None else np.array(d_state_out[b, h], dtype=np.float64)",
                               "H = np.zeros((d, d))"),
    "dv_transposed_state": ("dv[b, t, g] += H.T @ k[b, t, g]", "dv[b, t, g] += H @ k[b, t, g]"),
    "gqa_grad_to_group_zero": ("g = (h * G) // Hq", "g = 0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(name):
    orig, repl = MUTANTS[name]
    with open(bwd.__file__) as f:
        src = f.read()
    assert src.count(orig) >= 1, f"mutation site vanished: {orig}"
    mod = types.ModuleType(f"bwd_{name}")
    exec(compile(src.replace(orig, repl), f"<mutant {name}>", "exec"), mod.__dict__)
    caught = []
    for pin in ALL_BWD_PINS:
        try:
            pin(mod.prefill_backward)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"


def test_backward_rows_equal_full():
    """The per-row form (used at lengths the full oracle cannot reach) gives
    the full oracle's values at every query row and key row, with and
    without states, on inputs with ragged sets (M < n) and full ones."""
    import numpy as np
    from oracle import oracle as orc
    from tests.backward_pins import _cfg, _forward, _setup
    for n, M, states in ((40, 7, True), (23, 32, False), (33, 5, True)):
        cfg = _cfg(n=n, Hq=6, Hkv=2, d=8, M=M, seed=n)
        inp, x, extra = _setup(cfg)
        S0 = extra["state_in"] if states else None
        dS = extra["d_state_out"] if states else None
        fwd = _forward(cfg, inp, x, S0, orc.load())
        full = bwd.prefill_backward(x["q"], x["k"], x["v"], x["gate"], fwd["idx"], extra["d_out"],
                                    state_in=S0, d_state_out=dS)
        every = list(range(n))
        part = bwd.prefill_backward_rows(x["q"], x["k"], x["v"], x["gate"], fwd["idx"], extra["d_out"],
                                         every, every[::-1], state_in=S0, d_state_out=dS)
        for name in ("dq", "dz"):
            np.testing.assert_allclose(part[name], full[name], rtol=1e-12, atol=1e-13)
        for name in ("dk", "dv"):
            np.testing.assert_allclose(part[name], full[name][:, ::-1], rtol=1e-12, atol=1e-13)
