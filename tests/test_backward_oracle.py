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
