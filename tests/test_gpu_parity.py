"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every case prints its name, shape and seed before touching the GPU.  The
rules are in tests/parity.py: index sets within the 1e-5 score band of the
M-th score, normwise error <= 1e-2 (bf16) / 1e-4 (fp32) for the sparse
branch, the linear branch, the gated output and the final state.
"""
import sys

import numpy as np
import pytest

from hybrid_linear_top_amd import inputs as gen
from hybrid_linear_top_amd.inputs import LayerConfig
from tests import parity

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_linear_top_amd import lisa  # noqa: F401  (fails loudly if the library is missing)
    yield


def _pcfg(n, Hq, Hkv, d, HI, dI, M, dtype="bf16", B=1, seed=1, w_dist="u01"):
    wtag = "" if w_dist == "u01" else f"_w{w_dist}"
    return LayerConfig(f"p_n{n}_h{Hq}x{Hkv}_d{d}_i{HI}x{dI}_m{M}_{dtype}{wtag}", "prefill", dtype, B=B,
                       n=n, Hq=Hq, Hkv=Hkv, d=d, HI=HI, dI=dI, M=M, seed=seed, w_dist=w_dist)


PREFILL_SMALL = [
    _pcfg(200, 4, 2, 64, 4, 32, 16),
    _pcfg(333, 7, 1, 128, 3, 64, 64),
    _pcfg(130, 6, 2, 128, 8, 64, 300),            # M > n: full causal attention
    _pcfg(257, 4, 4, 64, 5, 32, 1, dtype="f32"),
    _pcfg(1, 4, 2, 128, 4, 64, 256),
    _pcfg(65, 12, 2, 128, 4, 64, 256, B=2, seed=3),
    _pcfg(700, 8, 2, 128, 4, 64, 512, seed=4),    # largest prefill M (1024-entry buffers)
    _pcfg(520, 4, 2, 64, 4, 64, 200, dtype="f32", seed=5),
    _pcfg(900, 14, 2, 128, 2, 64, 96, seed=6),
    _pcfg(1500, 12, 2, 128, 4, 64, 256, seed=7),  # several compactions per query
    _pcfg(300, 8, 2, 128, 4, 64, 130, seed=8),    # index rows not 16-byte aligned (M % 4 = 2)
    _pcfg(180, 6, 3, 64, 4, 32, 37, seed=9),      # d = 64 with odd M
    _pcfg(1300, 4, 2, 128, 4, 64, 1, seed=10),    # M = 1: the argmax of every row (bf16)
    _pcfg(900, 6, 2, 64, 2, 32, 2, seed=12),      # M = 2
]


@pytest.mark.parametrize("cfg", PREFILL_SMALL, ids=lambda c: c.name)
def test_prefill_small(cfg):
    _say("prefill", cfg.name, "seed", cfg.seed)
    inp = gen.make_prefill_inputs(cfg)
    rep = {}
    parity.prefill_parity(cfg, inp, report=rep)
    _say("  ", rep)


def test_prefill_with_initial_state():
    cfg = _pcfg(150, 6, 2, 128, 4, 64, 32, seed=11)
    _say("prefill state_in", cfg.name)
    inp = gen.make_prefill_inputs(cfg)
    S0 = np.random.default_rng(2).standard_normal((1, cfg.Hq, cfg.d, cfg.d)).astype(np.float32)
    rep = {}
    parity.prefill_parity(cfg, inp, state_in=S0, report=rep)
    _say("  ", rep)


def test_prefill_config0_tiny_fp32():
    cfg = gen.TINY_F32_PREFILL
    _say("prefill", cfg.name)
    inp = gen.make_prefill_inputs(cfg)
    rep = {}
    parity.prefill_parity(cfg, inp, report=rep)
    _say("  ", rep)


def test_prefill_config1_full():
    cfg = gen.PREFILL_1P5B_4K
    _say("prefill", cfg.name)
    inp = gen.make_prefill_inputs(cfg)
    rep = {}
    parity.prefill_parity(cfg, inp, report=rep)
    _say("  ", rep)


def test_prefill_max_length_sampled_rows():
    """n = 32768, the longest prefill (candidate indices are 16-bit): rows
    near the end select among every position up to 32767."""
    cfg = _pcfg(32768, 4, 2, 64, 2, 32, 256, seed=11)
    _say("prefill", cfg.name, "(sampled rows, full state)")
    inp = gen.make_prefill_inputs(cfg)
    rng = np.random.default_rng(11)
    rows = sorted(set([0, 255, 256, 16383, 16384, 32700, 32766, 32767]
                      + rng.integers(16384, cfg.n, size=12).tolist()))
    rep = {}
    parity.prefill_parity(cfg, inp, rows=rows, report=rep)
    _say("  ", rep)


def test_prefill_two_sequences_long_sampled_rows():
    """Two sequences of 8400 positions at d = 128, three groups, M = 130
    (index rows not 16-byte aligned), in the group-major unit order of
    batches above one sequence; rows at both ends and across the middle."""
    cfg = _pcfg(8400, 6, 3, 128, 4, 64, 130, B=2, seed=38)
    _say("prefill", cfg.name, "(sampled rows)")
    inp = gen.make_prefill_inputs(cfg)
    rng = np.random.default_rng(38)
    rows = sorted(set([0, 1, 15, 16, 17, 2000, 8191, 8192, 8399] + rng.integers(0, cfg.n, size=8).tolist()))
    rep = {}
    parity.prefill_parity(cfg, inp, rows=rows, report=rep)
    _say("  ", rep)


def test_prefill_config3_all_rows():
    """The 16K 7B-shaped workload in the benchmark's launch configuration,
    every row: index sets of all 16384 x 4 units, all outputs and the state."""
    cfg = gen.PREFILL_7B_16K
    _say("prefill", cfg.name, "(all rows)")
    inp = gen.make_prefill_inputs(cfg)
    rep = {}
    parity.prefill_parity(cfg, inp, report=rep)
    _say("  ", rep)


def _dcfg(Hq, Hkv, d, HI, dI, M, lengths, dtype="bf16", seed=1, w_dist="u01"):
    wtag = "" if w_dist == "u01" else f"_w{w_dist}"
    return LayerConfig(f"d_h{Hq}x{Hkv}_d{d}_i{HI}x{dI}_m{M}_{dtype}{wtag}_L{'-'.join(map(str, lengths))}",
                       "decode", dtype, B=len(lengths), Hq=Hq, Hkv=Hkv, d=d, HI=HI, dI=dI, M=M,
                       seed=seed, w_dist=w_dist), np.asarray(lengths)


DECODE_SMALL = [
    _dcfg(12, 2, 128, 4, 64, 256, [1, 2, 255, 256, 257, 1000]),
    _dcfg(7, 7, 64, 3, 32, 16, [17, 300, 513, 64]),
    _dcfg(28, 4, 128, 4, 64, 512, [4097, 700, 513, 20000], seed=2),
    _dcfg(8, 2, 64, 8, 64, 100, [999, 1001, 5000], dtype="f32", seed=3),
    _dcfg(16, 1, 128, 6, 64, 2048, [3000, 2048, 2049], seed=4),
    _dcfg(4, 1, 64, 4, 32, 256, [40000, 3, 33100], seed=5),   # two-part select and its merge
    # the two-part select with M = 2048 (its parts' exact passes; 4096
    # candidates merged), contexts at its lower edge, between and at the top
    _dcfg(8, 2, 64, 4, 32, 2048, [33793, 47000, 65536], seed=21),
    # the 33-keys-per-thread top-M, at its largest context and just above the
    # 17-keys-per-thread one's
    _dcfg(4, 1, 64, 4, 32, 512, [33792, 17409, 9000], seed=6),
    _dcfg(4, 2, 64, 2, 32, 64, [17409, 25000], seed=7),
    _dcfg(2, 1, 64, 1, 32, 256, [65536, 100], seed=9),         # the longest decode context
    # degenerate set sizes: M = 1 (the argmax, lowest index on ties) and 2,
    # at contexts that take the shortcut, the exact passes and the two parts
    _dcfg(6, 2, 128, 4, 64, 1, [1, 5, 3000, 17000], seed=10),
    _dcfg(4, 2, 64, 3, 32, 2, [2, 9000, 40000], seed=11),
]


@pytest.mark.parametrize("case", DECODE_SMALL, ids=lambda c: c[0].name)
def test_decode_small(case):
    cfg, lengths = case
    _say("decode", cfg.name, "seed", cfg.seed)
    inp = gen.make_decode_inputs(cfg, lengths=lengths)
    rep = {}
    parity.decode_parity(cfg, inp, report=rep)
    _say("  ", rep)


@pytest.mark.parametrize("cfg", [gen.DECODE_1P5B_16K, gen.DECODE_7B_RAGGED], ids=lambda c: c.name)
def test_decode_configs(cfg):
    _say("decode", cfg.name)
    inp = gen.make_decode_inputs(cfg)
    rep = {}
    parity.decode_parity(cfg, inp, report=rep)
    _say("  ", rep)


def test_ties_lowest_index_wins():
    """w = 0 makes every score exactly 0: the sets must be the first m positions."""
    cfg = _pcfg(400, 4, 2, 64, 4, 32, 100)
    _say("prefill all-ties", cfg.name)
    inp = gen.make_prefill_inputs(cfg)
    inp["w_idx"] = np.zeros_like(inp["w_idx"])
    _, _, idx = parity.run_prefill(cfg, inp)
    for t in range(cfg.n):
        m = min(cfg.M, t + 1)
        exp = np.concatenate([np.arange(m), -np.ones(cfg.M - m)]).astype(np.int32)
        assert np.array_equal(idx[0, t, 0], exp) and np.array_equal(idx[0, t, 1], exp), t
    # long enough for the sampled starting threshold (which admits nothing here)
    cfg = _pcfg(2000, 4, 2, 64, 4, 32, 64, seed=2)
    _say("prefill all-ties, sampled threshold", cfg.name)
    inp = gen.make_prefill_inputs(cfg)
    inp["w_idx"] = np.zeros_like(inp["w_idx"])
    _, _, idx = parity.run_prefill(cfg, inp)
    for t in range(cfg.n):
        m = min(cfg.M, t + 1)
        exp = np.concatenate([np.arange(m), -np.ones(cfg.M - m)]).astype(np.int32)
        assert np.array_equal(idx[0, t, 0], exp) and np.array_equal(idx[0, t, 1], exp), t
    dcfg, L = _dcfg(4, 2, 64, 4, 32, 100, [50, 100, 101, 3000])
    _say("decode all-ties", dcfg.name)
    dinp = gen.make_decode_inputs(dcfg, lengths=L)
    dinp["w_idx"] = np.zeros_like(dinp["w_idx"])
    _, _, didx = parity.run_decode(dcfg, dinp)
    for b, Lb in enumerate(L):
        m = min(dcfg.M, Lb)
        exp = np.concatenate([np.arange(m), -np.ones(dcfg.M - m)]).astype(np.int32)
        assert np.array_equal(didx[b, 0], exp) and np.array_equal(didx[b, 1], exp), b


@pytest.mark.parametrize("lengths,M", [([8000, 300], 512), ([17000], 512), ([33792, 18000], 512),
                                       ([40000, 5], 512), ([65536], 512), ([40000, 34000], 2048)],
                         ids=["ctx8000", "ctx17000", "ctx33792", "ctx40000", "ctx65536", "ctx40000_m2048"])
def test_decode_ties_every_select_variant(lengths, M):
    """w = 0 at contexts that pick each top-M kernel variant: every score is
    exactly 0, so each set is the first min(M, L) positions (in the two-part
    select above 33,792 positions both parts hold tied candidates, and the
    merge must keep the first part's)."""
    dcfg, L = _dcfg(4, 2, 64, 4, 32, M, lengths, seed=8)
    _say("decode all-ties", dcfg.name)
    dinp = gen.make_decode_inputs(dcfg, lengths=L)
    dinp["w_idx"] = np.zeros_like(dinp["w_idx"])
    _, _, didx = parity.run_decode(dcfg, dinp)
    for b, Lb in enumerate(L):
        m = min(dcfg.M, Lb)
        exp = np.concatenate([np.arange(m), -np.ones(dcfg.M - m)]).astype(np.int32)
        assert np.array_equal(didx[b, 0], exp) and np.array_equal(didx[b, 1], exp), b


def test_prefill_sampled_threshold_rescan():
    """Every third query has all-zero weights, so it scores every key 0 and a
    sampled starting threshold admits nothing: those queries are rescanned
    exactly (first m positions) while the other queries of the same waves keep
    their candidates."""
    cfg = _pcfg(2100, 4, 2, 64, 4, 32, 64, seed=12)
    _say("prefill mixed rescan", cfg.name)
    inp = gen.make_prefill_inputs(cfg)
    inp["w_idx"][:, ::3] = 0
    rep = {}
    parity.prefill_parity(cfg, inp, report=rep)
    _say("  ", rep)


CONTINUE_CASES = [
    (_pcfg(700, 12, 2, 128, 4, 64, 256, seed=31), 300),     # past not a multiple of 64
    (_pcfg(400, 4, 2, 64, 4, 32, 64, B=2, seed=32), 384),   # 16 new tokens, chunk-aligned past
    (_pcfg(1300, 8, 2, 128, 4, 64, 128, seed=33), 1299),    # one new token (a decode step by prefill)
    (_pcfg(2500, 12, 2, 128, 4, 64, 256, seed=34), 1100),   # sampled threshold active
    (_pcfg(520, 4, 2, 64, 4, 64, 100, dtype="f32", seed=35), 129),
    # 300 new tokens after 8200: sets at the largest prefill M drawn from a
    # long cached context
    (_pcfg(8500, 8, 2, 128, 4, 64, 512, seed=37), 8200),
]


@pytest.mark.parametrize("case", CONTINUE_CASES, ids=lambda c: f"{c[0].name}_past{c[1]}")
def test_prefill_continue(case):
    cfg, past = case
    _say("prefill continue", cfg.name, "past", past, "seed", cfg.seed)
    inp = gen.make_prefill_inputs(cfg)
    rep = {}
    parity.prefill_parity(cfg, inp, past=past, report=rep)
    _say("  ", rep)


def test_prefill_continue_with_state_and_past0():
    """An initial state is carried through both calls, and past = 0 gives
    exactly lisa_prefill's result."""
    cfg = _pcfg(330, 6, 2, 128, 4, 64, 64, seed=36)
    _say("prefill continue, state_in", cfg.name)
    inp = gen.make_prefill_inputs(cfg)
    S0 = np.random.default_rng(5).standard_normal((1, cfg.Hq, cfg.d, cfg.d)).astype(np.float32)
    rep = {}
    parity.prefill_parity(cfg, inp, past=200, state_in=S0, report=rep)
    _say("  ", rep)
    a = parity.run_prefill(cfg, inp, state_in=S0)
    b = parity.run_prefill_continue(cfg, inp, 0, state_in=S0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


WINDOW_PREFILL = [
    (_pcfg(300, 8, 2, 128, 1, 32, 64, seed=41), 0),
    (_pcfg(150, 4, 2, 64, 1, 32, 300, seed=42), 0),               # window > n: full causal
    (_pcfg(900, 12, 2, 128, 1, 32, 256, B=2, seed=43), 500),      # continued, B = 2
    (_pcfg(400, 6, 3, 128, 1, 32, 1000, seed=44), 100),           # window above the indexer's 512
    (_pcfg(260, 4, 2, 64, 1, 32, 50, dtype="f32", seed=45), 70),
]


@pytest.mark.parametrize("case", WINDOW_PREFILL, ids=lambda c: f"{c[0].name}_past{c[1]}")
def test_prefill_window(case):
    cfg, past = case
    _say("prefill window", cfg.name, "past", past, "seed", cfg.seed)
    inp = gen.make_prefill_inputs(cfg)
    rep = {}
    parity.window_prefill_parity(cfg, inp, past=past, report=rep)
    _say("  ", rep)


WINDOW_DECODE = [
    _dcfg(12, 2, 128, 1, 32, 256, [1, 100, 256, 257, 3000]),
    _dcfg(8, 4, 64, 1, 32, 1500, [1499, 1500, 1501, 40]),
    _dcfg(8, 2, 128, 1, 32, 64, [65, 900], dtype="f32", seed=2),
]


@pytest.mark.parametrize("case", WINDOW_DECODE, ids=lambda c: c[0].name)
def test_decode_window(case):
    cfg, lengths = case
    _say("decode window", cfg.name, "seed", cfg.seed)
    inp = gen.make_decode_inputs(cfg, lengths=lengths)
    rep = {}
    parity.window_decode_parity(cfg, inp, report=rep)
    _say("  ", rep)


PAGED_DECODE = [
    (_dcfg(12, 2, 128, 4, 64, 256, [1, 2, 255, 256, 257, 1000]), 16),
    (_dcfg(28, 4, 128, 4, 64, 512, [4097, 700, 513, 20000], seed=2), 64),
    (_dcfg(8, 2, 64, 8, 64, 100, [999, 1001, 5000], dtype="f32", seed=3), 1),
    (_dcfg(4, 1, 64, 4, 32, 256, [40000, 3, 33100], seed=5), 256),  # longest-context select
    (_dcfg(7, 7, 64, 3, 32, 16, [17, 300, 513, 64], seed=6), 4096),
]


@pytest.mark.parametrize("case", PAGED_DECODE, ids=lambda c: f"{c[0][0].name}_bs{c[1]}")
def test_decode_paged(case):
    (cfg, lengths), bs = case
    _say("decode paged", cfg.name, "block", bs, "seed", cfg.seed)
    inp = gen.make_decode_inputs(cfg, lengths=lengths)
    rep = {}
    parity.paged_decode_parity(cfg, inp, bs, seed=cfg.seed, report=rep)
    _say("  ", rep)


def test_deterministic():
    cfg = gen.PREFILL_1P5B_4K
    _say("determinism", cfg.name)
    inp = gen.make_prefill_inputs(cfg)
    a = parity.run_prefill(cfg, inp)
    b = parity.run_prefill(cfg, inp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    dcfg = gen.DECODE_1P5B_16K
    _say("determinism", dcfg.name)
    dinp = gen.make_decode_inputs(dcfg, B=4)
    a = parity.run_decode(dcfg, dinp)
    b = parity.run_decode(dcfg, dinp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_prefill_then_decode_matches_longer_prefill():
    """GPU prefill(n) + GPU decode of token n equals row n of GPU prefill(n+1)."""
    cfg = _pcfg(600, 12, 2, 128, 4, 64, 256, seed=21)
    _say("cross-path", cfg.name)
    full = gen.make_prefill_inputs(cfg)
    n = cfg.n - 1
    short = {k: (v[:, :n] if isinstance(v, np.ndarray) else v) for k, v in full.items()}
    short["n"] = n
    _, st, _ = parity.run_prefill(cfg, short)
    out_full, st_full, idx_full = parity.run_prefill(cfg, full)
    dcfg = LayerConfig("cross", "decode", cfg.dtype, B=1, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d,
                       HI=cfg.HI, dI=cfg.dI, M=cfg.M)
    dec = {"q": full["q"][:, n], "k_cache": full["k"][0], "v_cache": full["v"][0],
           "q_idx": full["q_idx"][:, n], "k_idx_cache": full["k_idx"][0],
           "w_idx": full["w_idx"][:, n], "gate": full["gate"][:, n],
           "state": st.astype(np.float32), "cu_ctx": np.array([0, cfg.n], dtype=np.int64),
           "B": 1, "max_ctx": cfg.n}
    out_d, st_d, idx_d = parity.run_decode(dcfg, dec)
    assert np.array_equal(idx_d[0], idx_full[0, n])
    assert parity.normwise(out_d[0], out_full[0, n]) <= 1e-2
    assert parity.normwise(st_d, st_full) <= 1e-3


# ---- backward ------------------------------------------------------------------
BACKWARD = [
    (_pcfg(200, 4, 2, 64, 4, 32, 16), True),
    (_pcfg(300, 12, 2, 128, 4, 64, 64, seed=2), True),
    (_pcfg(130, 8, 2, 64, 2, 32, 37, dtype="f32", seed=3), True),
    (_pcfg(257, 7, 7, 128, 4, 64, 256, seed=4), False),      # no state in or out, M > n
    (_pcfg(1000, 8, 2, 128, 4, 64, 256, seed=5), True),
    (_pcfg(300, 8, 2, 128, 4, 64, 64, B=2, seed=6), True),     # batch of two
    (_pcfg(700, 4, 2, 128, 4, 64, 512, seed=7), True),         # M = 512: two merge passes
    (_pcfg(600, 6, 3, 64, 4, 32, 300, seed=8), False),         # M not a power of two, d = 64
    (_pcfg(50, 4, 1, 128, 2, 32, 1, seed=9), True),            # M = 1
    (_pcfg(1, 4, 2, 128, 2, 32, 16, seed=10), True),           # one position
    (_pcfg(129, 32, 2, 64, 2, 32, 40, seed=11), True),         # 16 heads per group
]


def test_prefill_backward_16k_sampled():
    """The backward at the benchmark's 16K, 7B-shaped workload and launch
    configuration: dq, dz at sampled query rows and dk, dv at sampled keys
    (the first, the last, both sides of the t = M boundary, mid-sequence)."""
    cfg = gen.PREFILL_7B_16K
    _say("backward 16K sampled", cfg.name)
    inp = gen.make_prefill_inputs(cfg)
    binp = gen.make_backward_inputs(cfg)
    rows = [0, 1, cfg.M - 1, cfg.M, 5000, cfg.n // 2, cfg.n - 1]
    keys = [0, 1, cfg.M, 9000, cfg.n - 2, cfg.n - 1]
    rep = {}
    parity.backward_sampled_parity(cfg, inp, binp, rows, keys, report=rep)
    _say("  ", rep)


@pytest.mark.parametrize("case", BACKWARD, ids=lambda c: c[0].name + ("_states" if c[1] else ""))
def test_prefill_backward(case):
    cfg, states = case
    _say("backward", cfg.name, "states", states, "seed", cfg.seed)
    inp = gen.make_prefill_inputs(cfg)
    binp = gen.make_backward_inputs(cfg, with_states=states)
    rep = {}
    parity.backward_parity(cfg, inp, binp, report=rep)
    _say("  ", rep)


@pytest.mark.parametrize("case", [(_pcfg(400, 8, 2, 128, 4, 64, 96, seed=21), True),
                                  (_pcfg(150, 4, 1, 64, 4, 32, 256, dtype="f32", seed=22), False)],
                         ids=lambda c: c[0].name)
def test_prefill_backward_window_sets(case):
    """The backward of the sliding-window variant: the window's sets passed as
    topm (the backward takes any sets; the window ones are dense bands)."""
    cfg, states = case
    _say("backward window sets", cfg.name, "states", states)
    inp = gen.make_prefill_inputs(cfg)
    binp = gen.make_backward_inputs(cfg, with_states=states)
    rep = {}
    parity.backward_parity(cfg, inp, binp, report=rep,
                           sets=parity.window_sets(cfg.B, cfg.n, cfg.Hkv, cfg.M))
    _say("  ", rep)


def _random_cases(seed, count):
    """Seeded random shapes within the supported ranges (a sweep beside the
    hand-picked cases: ragged n and M, every head-group ratio, both dtypes)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        G = int(rng.choice([1, 2, 4]))
        r = int(rng.choice([1, 2, 3, 5, 7, 8, 16]))
        d = int(rng.choice([64, 128]))
        dI = int(rng.choice([32, 64]))
        HI = int(rng.integers(1, 9))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        out.append((G, r, d, dI, HI, dtype, int(rng.integers(1_000_000))))
    return out


@pytest.mark.parametrize("case", _random_cases(77, 16), ids=lambda c: f"G{c[0]}r{c[1]}d{c[2]}s{c[6]}")
def test_prefill_random_shapes(case):
    G, r, d, dI, HI, dtype, seed = case
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 700))
    M = int(rng.integers(1, 513))
    B = int(rng.choice([1, 1, 2]))
    cfg = _pcfg(n, G * r, G, d, HI, dI, M, dtype=dtype, B=B, seed=seed % 1000)
    _say("prefill random", cfg.name, "B", B, "seed", cfg.seed)
    rep = {}
    parity.prefill_parity(cfg, gen.make_prefill_inputs(cfg), report=rep)
    _say("  ", rep)


@pytest.mark.parametrize("case", _random_cases(78, 16), ids=lambda c: f"G{c[0]}r{c[1]}d{c[2]}s{c[6]}")
def test_decode_random_shapes(case):
    G, r, d, dI, HI, dtype, seed = case
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 6))
    M = int(rng.integers(1, 2049))
    lengths = [int(x) for x in rng.integers(1, 12000, size=B)]
    cfg, L = _dcfg(G * r, G, d, HI, dI, M, lengths, dtype=dtype, seed=seed % 1000)
    _say("decode random", cfg.name, "seed", cfg.seed)
    rep = {}
    parity.decode_parity(cfg, gen.make_decode_inputs(cfg, lengths=L), report=rep)
    _say("  ", rep)


@pytest.mark.parametrize("case", _random_cases(79, 12), ids=lambda c: f"G{c[0]}r{c[1]}d{c[2]}s{c[6]}")
def test_backward_random_shapes(case):
    G, r, d, dI, HI, dtype, seed = case
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 500))
    M = int(rng.integers(1, 513))
    if dtype == "f32":
        M = min(M, 128)  # the fp32 kernel's LDS holds M * r logits
    B = int(rng.choice([1, 2]))
    cfg = _pcfg(n, G * r, G, d, HI, dI, M, dtype=dtype, B=B, seed=seed % 1000)
    states = bool(rng.random() < 0.5)
    _say("backward random", cfg.name, "B", B, "states", states, "seed", cfg.seed)
    rep = {}
    parity.backward_parity(cfg, gen.make_prefill_inputs(cfg), gen.make_backward_inputs(cfg, with_states=states),
                           report=rep)
    _say("  ", rep)


@pytest.mark.parametrize("case", _random_cases(80, 8), ids=lambda c: f"G{c[0]}r{c[1]}d{c[2]}s{c[6]}")
def test_prefill_continue_random_shapes(case):
    G, r, d, dI, HI, dtype, seed = case
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 700))
    past = int(rng.integers(0, n))
    M = int(rng.integers(1, 513))
    cfg = _pcfg(n, G * r, G, d, HI, dI, M, dtype=dtype, B=int(rng.choice([1, 2])), seed=seed % 1000)
    _say("prefill continue random", cfg.name, "past", past, "seed", cfg.seed)
    rep = {}
    parity.prefill_parity(cfg, gen.make_prefill_inputs(cfg), past=past, report=rep)
    _say("  ", rep)


@pytest.mark.parametrize("case", _random_cases(81, 8), ids=lambda c: f"G{c[0]}r{c[1]}d{c[2]}s{c[6]}")
def test_window_random_shapes(case):
    G, r, d, dI, HI, dtype, seed = case
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 700))
    past = int(rng.integers(0, n))
    M = int(rng.integers(1, 2049))
    cfg = _pcfg(n, G * r, G, d, 1, 32, M, dtype=dtype, seed=seed % 1000)
    _say("prefill window random", cfg.name, "past", past, "seed", cfg.seed)
    rep = {}
    parity.window_prefill_parity(cfg, gen.make_prefill_inputs(cfg), past=past, report=rep)
    _say("  ", rep)
    lengths = [int(x) for x in rng.integers(1, 6000, size=int(rng.integers(1, 5)))]
    dcfg, L = _dcfg(G * r, G, d, 1, 32, M, lengths, dtype=dtype, seed=seed % 1000)
    _say("decode window random", dcfg.name, "seed", dcfg.seed)
    rep = {}
    parity.window_decode_parity(dcfg, gen.make_decode_inputs(dcfg, lengths=L), report=rep)
    _say("  ", rep)


@pytest.mark.parametrize("case", _random_cases(82, 8), ids=lambda c: f"G{c[0]}r{c[1]}d{c[2]}s{c[6]}")
def test_decode_paged_random_shapes(case):
    G, r, d, dI, HI, dtype, seed = case
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(1, 9000, size=int(rng.integers(1, 5)))]
    M = int(rng.integers(1, 2049))
    bs = int(2 ** rng.integers(0, 13))
    cfg, L = _dcfg(G * r, G, d, HI, dI, M, lengths, dtype=dtype, seed=seed % 1000)
    _say("decode paged random", cfg.name, "block", bs, "seed", cfg.seed)
    rep = {}
    parity.paged_decode_parity(cfg, gen.make_decode_inputs(cfg, lengths=L), bs, seed=cfg.seed, report=rep)
    _say("  ", rep)


def test_stage_timing_changes_nothing():
    """With stage timing on, the kernels launch through hipExtLaunchKernel with
    events attached: prefill, decode and backward must give the same outputs
    as with it off (bit for bit; dk and dv, summed with fp32 atomics, to
    rounding), and every stage must report positive, finite times."""
    import torch
    from hybrid_linear_top_amd import lisa
    cfg = _pcfg(700, 8, 2, 128, 4, 64, 256, seed=12)
    dcfg, L = _dcfg(12, 2, 128, 4, 64, 256, [3000, 20000, 100], seed=12)
    inp = gen.make_prefill_inputs(cfg)
    dinp = gen.make_decode_inputs(dcfg, lengths=L)
    binp = gen.make_backward_inputs(cfg)
    dims = lisa.dims_from_config(cfg)
    dv_ = lisa.to_device

    def run_all():
        pre = parity.run_prefill(cfg, inp, state_in=binp["state_in"])
        dec = parity.run_decode(dcfg, dinp)
        g = lisa.prefill_backward(dims, dv_(inp["q"]), dv_(inp["k"]), dv_(inp["v"]), dv_(inp["gate"]),
                                  dv_(pre[2]), dv_(binp["d_out"]), state_in=dv_(binp["state_in"]),
                                  d_state_out=dv_(binp["d_state_out"]), want_state_grad=True)
        torch.cuda.synchronize()
        return list(pre) + list(dec) + [lisa.from_device(x) for x in g]

    _say("stage timing off/on", cfg.name, dcfg.name)
    ref = run_all()
    lisa.lisa_stage_timing_read(reset=True)
    lisa.lisa_stage_timing(True)
    try:
        got = run_all()
    finally:
        lisa.lisa_stage_timing(False)
    stages = lisa.lisa_stage_timing_read(reset=True)
    names = ["prefill out", "prefill state", "prefill idx", "decode out", "decode state", "decode idx",
             "dq", "dk", "dv", "dz", "d_state_in"]
    for nm, a, b in zip(names, ref, got):
        if nm in ("dk", "dv"):
            assert parity.normwise(b.astype(np.float64), a.astype(np.float64)) < 1e-6, nm
        else:
            assert np.array_equal(a, b), nm
    for st in ("indexer_topm", "sparse_gate_prefill", "linear_chunk_output", "decode_score_state",
               "decode_select", "sparse_gate_decode", "bwd_sparse_query", "bwd_sparse_keys", "bwd_linear"):
        n, ms = stages[st]
        assert n >= 1 and np.isfinite(ms) and ms > 0.0, (st, n, ms)
    _say("  ", {k: round(v[1], 4) for k, v in stages.items()})


def test_graph_replay():
    """A serving loop captures the calls in a HIP graph: the library enqueues
    only kernels on the caller's stream (no allocation, memset or sync), so a
    captured prefill and a captured decode step replay to the eager results
    bit for bit, replay after replay, with eager work (the decode state reset
    from a saved copy) between the replays."""
    import torch
    from hybrid_linear_top_amd import lisa
    dv = lisa.to_device
    pcfg = _pcfg(700, 8, 2, 128, 4, 64, 128, seed=51)
    pinp = gen.make_prefill_inputs(pcfg)
    dims = lisa.dims_from_config(pcfg)
    x = {k: dv(pinp[k]) for k in ("q", "k", "v", "q_idx", "k_idx", "w_idx", "gate")}
    B, n = pinp["B"], pinp["n"]
    ws = torch.empty(lisa.lisa_prefill_workspace_bytes(dims, B, n), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x["q"])
    st = torch.empty((B, pcfg.Hq, pcfg.d, pcfg.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, n, pcfg.Hkv, pcfg.M), dtype=torch.int32, device="cuda")

    def prefill():
        lisa.prefill(dims, x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], x["w_idx"], x["gate"],
                     out=out, state_out=st, topm_out=idx, workspace=ws)

    prefill()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, st, idx)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        prefill()
    for rep in range(3):
        for t in (out, st, idx):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say("prefill graph replay", rep)
        for a, b in zip((out, st, idx), ref):
            assert torch.equal(a, b)

    dcfg, lengths = _dcfg(12, 2, 128, 4, 64, 256, [300, 1000, 4000], seed=52)
    dinp = gen.make_decode_inputs(dcfg, lengths=lengths)
    ddims = lisa.dims_from_config(dcfg)
    y = {k: dv(dinp[k]) for k in ("cu_ctx", "q", "k_cache", "v_cache", "q_idx", "k_idx_cache", "w_idx", "gate",
                                  "state")}
    state0 = y["state"].clone()
    dws = torch.empty(lisa.lisa_decode_workspace_bytes(ddims, dinp["B"], dinp["max_ctx"]), dtype=torch.uint8,
                      device="cuda")
    dout = torch.empty_like(y["q"])
    didx = torch.empty((dinp["B"], dcfg.Hkv, dcfg.M), dtype=torch.int32, device="cuda")

    def step():
        lisa.decode_step(ddims, y["cu_ctx"], dinp["max_ctx"], y["q"], y["k_cache"], y["v_cache"], y["q_idx"],
                         y["k_idx_cache"], y["w_idx"], y["gate"], y["state"], out=dout, topm_out=didx,
                         workspace=dws)

    step()
    torch.cuda.synchronize()
    dref = [t.clone() for t in (dout, y["state"], didx)]
    y["state"].copy_(state0)
    torch.cuda.synchronize()
    dg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dg):
        step()
    for rep in range(3):
        y["state"].copy_(state0)  # the step advances the state in place
        dout.zero_()
        didx.zero_()
        torch.cuda.synchronize()
        dg.replay()
        torch.cuda.synchronize()
        _say("decode graph replay", rep)
        for a, b in zip((dout, y["state"], didx), dref):
            assert torch.equal(a, b)


# ---- negative indexer scores (w may be negative: scores of either sign) ----
NEG_PREFILL = [
    _pcfg(3000, 8, 2, 128, 4, 64, 256, seed=51, w_dist="signed"),  # n >= 4M: sampled threshold, trims
    _pcfg(2600, 4, 2, 64, 4, 32, 64, seed=52, w_dist="neg"),       # every score <= 0; the zeros tie
    _pcfg(1200, 6, 3, 128, 8, 64, 100, seed=53, w_dist="signed"),  # 8 indexer heads
    _pcfg(600, 4, 1, 64, 3, 32, 512, seed=54, w_dist="neg"),       # t < M and the 1024-entry buffers
    _pcfg(2100, 4, 2, 128, 2, 64, 37, dtype="f32", seed=55, w_dist="signed"),
]


@pytest.mark.parametrize("cfg", NEG_PREFILL, ids=lambda c: c.name)
def test_prefill_negative_scores(cfg):
    _say("prefill", cfg.name, "seed", cfg.seed)
    inp = gen.make_prefill_inputs(cfg)
    rep = {}
    parity.prefill_parity(cfg, inp, report=rep)
    _say("  ", rep)


@pytest.mark.parametrize("case", _random_cases(83, 6), ids=lambda c: f"G{c[0]}r{c[1]}d{c[2]}s{c[6]}")
def test_prefill_random_long_any_sign(case):
    """Random shapes at lengths where late queries start from a sampled
    threshold (and may trim or rescan), with head weights of either sign."""
    G, r, d, dI, HI, dtype, seed = case
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1500, 3500))
    M = int(rng.integers(1, 513))
    w_dist = str(rng.choice(["u01", "signed", "neg"]))
    cfg = _pcfg(n, G * r, G, d, HI, dI, M, dtype=dtype, seed=seed % 1000, w_dist=w_dist)
    _say("prefill random long", cfg.name, "seed", cfg.seed)
    rep = {}
    parity.prefill_parity(cfg, gen.make_prefill_inputs(cfg), report=rep)
    _say("  ", rep)


@pytest.mark.parametrize("w_dist", ["signed", "neg"])
@pytest.mark.parametrize("lengths", [[8000, 300], [17000], [33792, 18000], [40000, 5]],
                         ids=["ctx8000", "ctx17000", "ctx33792", "ctx40000"])
@pytest.mark.parametrize("M", [256, 512])
def test_decode_negative_scores_every_select_variant(lengths, w_dist, M):
    """Scores of both signs (and, with w <= 0, only of one sign with many exact
    zeros) at contexts that pick each top-M kernel variant."""
    cfg, L = _dcfg(4, 2, 64, 4, 32, M, lengths, seed=61, w_dist=w_dist)
    _say("decode", cfg.name)
    inp = gen.make_decode_inputs(cfg, lengths=L)
    rep = {}
    parity.decode_parity(cfg, inp, report=rep)
    _say("  ", rep)


# ---- long prefill at the largest M and with 8 indexer heads -----------------
def test_prefill_m512_long_sampled_rows():
    """M = 512 (1024-entry candidate buffers) at n = 8192: queries past 2048
    start from a sampled threshold, queries between 960 and 2048 trim their
    buffers; rows sampled over both ranges, the state in full."""
    for w_dist, seed in (("u01", 71), ("signed", 72)):
        cfg = _pcfg(8192, 8, 2, 128, 4, 64, 512, seed=seed, w_dist=w_dist)
        _say("prefill", cfg.name, "(sampled rows, full state)")
        inp = gen.make_prefill_inputs(cfg)
        rng = np.random.default_rng(seed)
        rows = sorted(set([0, 511, 512, 959, 960, 1500, 2047, 2048, 2049, 4095, 8191]
                          + rng.integers(960, 2048, size=24).tolist()
                          + rng.integers(2048, cfg.n, size=24).tolist()))
        rep = {}
        parity.prefill_parity(cfg, inp, rows=rows, report=rep)
        _say("  ", rep)


def test_prefill_eight_indexer_heads_long():
    """8 indexer heads (two head halves per query) at n = 4500, all rows."""
    cfg = _pcfg(4500, 8, 2, 128, 8, 64, 256, seed=73)
    _say("prefill", cfg.name)
    inp = gen.make_prefill_inputs(cfg)
    rep = {}
    parity.prefill_parity(cfg, inp, report=rep)
    _say("  ", rep)


def test_prefill_backward_max_length_m512_window():
    """n = 32768 and M = 512: the last key row is selected by the last
    position, in its set's last slot (window sets), which packs the largest
    key, block position and slot into one sort entry.  dk and dv of the last
    keys and dq of the last rows against the oracle's per-row form."""
    cfg = _pcfg(32768, 4, 2, 128, 4, 64, 512, seed=81)
    _say("backward window sets", cfg.name, "(sampled rows and keys)")
    inp = gen.make_prefill_inputs(cfg)
    binp = gen.make_backward_inputs(cfg)
    sets = parity.window_sets(cfg.B, cfg.n, cfg.Hkv, cfg.M)
    rows = [0, 511, 512, 32766, 32767]
    keys = [0, 20000, 32255, 32256, 32766, 32767]
    rep = {}
    parity.backward_sampled_parity(cfg, inp, binp, rows, keys, report=rep, sets=sets)
    _say("  ", rep)
