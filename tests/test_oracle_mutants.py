"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
at least one pin catches each.  This shows the pins constrain every step of
the oracle: indexer score, selection and its tie-break, causal range, softmax,
linear state update and readout, GQA mapping and the gate."""
import os

import pytest

from oracle import oracle as orc
from tests.oracle_pins import ALL_PINS

MUTANTS = {
    "relu_dropped": ("double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;"),
    "head_weight_ignored": ("total += w[j] * relu;", "total += relu;"),
    "head_weight_first_only": ("total += w[j] * relu;", "total += w[0] * relu;"),
    "indexer_dim_short": ("for (int c = 0; c < dI; ++c) dot += qI[j * dI + c] * ks[c];",
                          "for (int c = 0; c < dI - 1; ++c) dot += qI[j * dI + c] * ks[c];"),
    "indexer_head_stride": ("dot += qI[j * dI + c] * ks[c];", "dot += qI[c] * ks[c];"),
    "tie_highest_index": ("return (x->index > y->index) - (x->index < y->index);",
                          "return (x->index < y->index) - (x->index > y->index);"),
    "select_lowest_scores": ("for (int i = 0; i < m; ++i) idx_out[i] = c[i].index;",
                             "for (int i = 0; i < m; ++i) idx_out[i] = c[T - 1 - i].index;"),
    "padding_zero": ("for (int i = m; i < M; ++i) idx_out[i] = -1;",
                     "for (int i = m; i < M; ++i) idx_out[i] = 0;"),
    "causal_excludes_self": ("oracle_topm(t + 1, sc, M, set);", "oracle_topm(t, sc, M, set);"),
    "softmax_sign": ("a[i] = exp(a[i] - amax);", "a[i] = exp(amax - a[i]);"),
    "softmax_unscaled": ("a[i] = scale * dot;", "a[i] = dot;"),
    "state_transposed": ("for (int j = 0; j < d; ++j) S[i * d + j] += kt[i] * vt[j];",
                         "for (int j = 0; j < d; ++j) S[i * d + j] += kt[j] * vt[i];"),
    "readout_transposed": ("for (int i = 0; i < d; ++i) acc += qt[i] * S[i * d + j];",
                           "for (int i = 0; i < d; ++i) acc += qt[i] * S[j * d + i];"),
    "decode_state_without_token": ("S[i * d + j] = Sin[i * d + j] + kt[i] * vt[j];",
                                   "S[i * d + j] = Sin[i * d + j];"),
    "gate_swapped": ("o[c] = g * osp[c] + (1.0 - g) * olin[c];",
                     "o[c] = g * olin[c] + (1.0 - g) * osp[c];"),
    "gqa_interleaved": ("return (int)(((long)h * Hkv) / Hq);", "return h % Hkv;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    orig, repl = MUTANTS[name]
    with open(orc.SRC) as f:
        src = f.read()
    assert src.count(orig) >= 1, f"mutation site vanished: {orig}"
    mpath = tmp_path / f"{name}.c"
    mpath.write_text(src.replace(orig, repl))
    so = orc.build(str(mpath), str(tmp_path / f"lib{name}.so"))
    lib = orc.load(so)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
