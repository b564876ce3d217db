"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each pin takes a loaded oracle library (so the same pins can be run against
deliberately broken builds of the oracle, see test_oracle_mutants.py) and
raises AssertionError when the oracle disagrees with:
  * hand-worked examples (tests/golden/*.json, derivations inside),
  * brute force (Python's own sort for the selection, numpy argmax),
  * library routines for special cases (torch SDPA for M >= n, numpy matmul
    for the closed form of the linear branch),
  * exact algebraic identities (gate limits, positive homogeneity).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from hybrid_linear_top_amd.inputs import LayerConfig, make_prefill_inputs, make_decode_inputs
from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _cfg(n=40, Hq=4, Hkv=2, d=16, HI=2, dI=8, M=8, seed=7):
    return LayerConfig("pin", "prefill", "f32", B=1, n=n, Hq=Hq, Hkv=Hkv, d=d, HI=HI, dI=dI, M=M,
                       seed=seed)


def _golden_prefill_inputs(fx):
    a = lambda key: np.asarray(fx[key], dtype=np.float32)[None]  # noqa: E731
    inp = {"q": a("q"), "k": a("k"), "v": a("v"), "q_idx": a("q_idx"), "k_idx": a("k_idx"),
           "w_idx": a("w_idx"), "gate": a("gate"), "B": 1, "n": fx["n"]}
    cfg = LayerConfig("golden", "prefill", "f32", B=1, n=fx["n"], Hq=fx["Hq"], Hkv=fx["Hkv"],
                      d=fx["d"], HI=fx["HI"], dI=fx["dI"], M=fx["M"])
    return inp, cfg


def pin_golden_prefill(lib):
    with open(os.path.join(GOLDEN, "hand_prefill_n5.json")) as f:
        fx = json.load(f)
    inp, cfg = _golden_prefill_inputs(fx)
    r = orc.prefill(inp, cfg, lib=lib)
    assert np.array_equal(r["idx"][0], np.asarray(fx["expect_idx"])), r["idx"][0]
    np.testing.assert_allclose(r["osp"][0], fx["expect_osp"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["olin"][0], fx["expect_olin"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["out"][0], fx["expect_out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["state_out"][0, 0], np.asarray(fx["expect_state_out"])[0],
                               rtol=0, atol=1e-12)


def pin_golden_softmax(lib):
    with open(os.path.join(GOLDEN, "hand_softmax_weights.json")) as f:
        fx = json.load(f)
    out, osp = orc.sparse_given_sets(np.array(fx["q"]), np.array(fx["k_rows"]),
                                     np.array(fx["v_rows"]), np.array([0]), np.array(fx["idx"]),
                                     np.array(fx["z"]), np.array(fx["olin"]), Hq=1, Hkv=1, d=2,
                                     M=2, scale=fx["scale"], lib=lib)
    np.testing.assert_allclose(osp, fx["expect_osp"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, fx["expect_out"], rtol=0, atol=1e-12)


def pin_golden_decode(lib):
    with open(os.path.join(GOLDEN, "hand_decode_step.json")) as f:
        fx = json.load(f)
    cfg = LayerConfig("golden_dec", "decode", "f32", B=1, Hq=fx["Hq"], Hkv=fx["Hkv"], d=fx["d"],
                      HI=fx["HI"], dI=fx["dI"], M=fx["M"])
    f32 = lambda key: np.asarray(fx[key], dtype=np.float32)  # noqa: E731
    inp = {k: f32(k) for k in ("q", "k_cache", "v_cache", "q_idx", "k_idx_cache", "w_idx",
                               "gate", "state")}
    inp["cu_ctx"] = np.asarray(fx["cu_ctx"], dtype=np.int64)
    inp["B"] = 1
    r = orc.decode(inp, cfg, lib=lib)
    assert np.array_equal(r["idx"], np.asarray(fx["expect_idx"])), r["idx"]
    np.testing.assert_allclose(r["osp"], fx["expect_osp"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["olin"], fx["expect_olin"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["out"], fx["expect_out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["state_out"], fx["expect_state_out"], rtol=0, atol=1e-12)


def _brute_topm(scores, M):
    T = len(scores)
    order = sorted(range(T), key=lambda s: (-scores[s], s))
    chosen = sorted(order[:min(M, T)])
    return chosen + [-1] * (M - len(chosen))


def pin_topm_bruteforce(lib):
    rng = np.random.default_rng(11)
    for trial in range(60):
        T = int(rng.integers(1, 70))
        if trial % 3 == 0:      # heavy ties: few distinct values, including both zeros
            vals = np.array([0.0, -0.0, 1.0, 2.0, -1.5])
            scores = vals[rng.integers(0, len(vals), size=T)]
        else:
            scores = rng.standard_normal(T)
        for M in (1, 3, 8, T, T + 5):
            got = orc.topm(scores, M, lib=lib).tolist()
            assert got == _brute_topm(scores.tolist(), M), (T, M, got)


def pin_scores_reductions(lib):
    rng = np.random.default_rng(12)
    HI, dI, T = 3, 8, 25
    qI = rng.standard_normal((HI, dI))
    kI = rng.standard_normal((T, dI))
    # one-hot head weights reduce the score to one ReLU'd dot product
    for j in range(HI):
        w = np.zeros(HI)
        w[j] = 1.0
        got = orc.index_scores(qI, w, kI, lib=lib)
        np.testing.assert_allclose(got, np.maximum(kI @ qI[j], 0.0), rtol=1e-14, atol=1e-14)
    # positive homogeneity: scaling by powers of two is exact
    w = rng.random(HI)
    base = orc.index_scores(qI, w, kI, lib=lib)
    scaled = orc.index_scores(qI * 2.0, w * 0.25, kI * 8.0, lib=lib)
    assert np.array_equal(scaled, base * 4.0)
    # a key anti-aligned with every indexer query scores exactly zero
    qpos = np.abs(qI) + 0.1
    kneg = -(np.abs(kI) + 0.1)
    got = orc.index_scores(qpos, w, kneg, lib=lib)
    assert np.all(got == 0.0)
    # and one aligned with them scores the w-weighted sum of the dot products
    got = orc.index_scores(qpos, w, -kneg, lib=lib)
    np.testing.assert_allclose(got, (-kneg @ qpos.T) @ w, rtol=1e-13)


def _sdpa_causal(q, k, v, scale):
    import torch
    Hq, Hkv = q.shape[2], k.shape[2]
    r = Hq // Hkv
    qt = torch.from_numpy(q[0]).permute(1, 0, 2)[None]                    # [1,Hq,n,d]
    kt = torch.from_numpy(k[0]).permute(1, 0, 2).repeat_interleave(r, 0)[None]
    vt = torch.from_numpy(v[0]).permute(1, 0, 2).repeat_interleave(r, 0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o[0].permute(1, 0, 2).numpy()[None]


def pin_sparse_full_causal(lib):
    cfg = _cfg(n=37, Hq=6, Hkv=2, d=16, HI=2, dI=8, M=64)
    inp = make_prefill_inputs(cfg)
    r = orc.prefill(inp, cfg, lib=lib)
    q, k, v = (orc.widen(inp[x], "f32") for x in ("q", "k", "v"))
    ref = _sdpa_causal(q, k, v, 1.0 / math.sqrt(cfg.d))
    np.testing.assert_allclose(r["osp"], ref, rtol=1e-11, atol=1e-12)
    # every position selects all of 0..t
    for t in range(cfg.n):
        for g in range(cfg.Hkv):
            assert r["idx"][0, t, g, :t + 1].tolist() == list(range(t + 1))
            assert (r["idx"][0, t, g, t + 1:] == -1).all()


def pin_sparse_m1(lib):
    cfg = _cfg(n=30, Hq=4, Hkv=2, d=8, HI=3, dI=8, M=1)
    inp = make_prefill_inputs(cfg)
    r = orc.prefill(inp, cfg, lib=lib)
    v = orc.widen(inp["v"], "f32")
    qI, kI, w = (orc.widen(inp[x], "f32") for x in ("q_idx", "k_idx", "w_idx"))
    for t in range(cfg.n):
        for h in range(cfg.Hq):
            g = h * cfg.Hkv // cfg.Hq
            # scores by numpy: sum_j w_j relu(qI_j . kI_s), first maximum = lowest index
            sc = (w[0, t, g][:, None] * np.maximum(qI[0, t, g] @ kI[0, :t + 1, g].T, 0)).sum(0)
            s = int(np.argmax(sc))
            np.testing.assert_allclose(r["osp"][0, t, h], v[0, s, g], rtol=0, atol=1e-14)


def pin_sparse_zero_query(lib):
    cfg = _cfg(n=33, Hq=4, Hkv=2, d=8, HI=2, dI=8, M=5)
    inp = make_prefill_inputs(cfg)
    inp["q"] = np.zeros_like(inp["q"])
    r = orc.prefill(inp, cfg, lib=lib)
    v = orc.widen(inp["v"], "f32")
    qI, kI, w = (orc.widen(inp[x], "f32") for x in ("q_idx", "k_idx", "w_idx"))
    for t in range(cfg.n):
        for h in range(cfg.Hq):
            g = h * cfg.Hkv // cfg.Hq
            sc = (w[0, t, g][:, None] * np.maximum(qI[0, t, g] @ kI[0, :t + 1, g].T, 0)).sum(0)
            sel = _brute_topm(sc.tolist(), cfg.M)
            sel = [s for s in sel if s >= 0]
            np.testing.assert_allclose(r["osp"][0, t, h], v[0, sel, g].mean(0), rtol=1e-13,
                                       atol=1e-14)
    assert np.all(r["olin"] == 0.0)


def pin_linear_closed_form(lib):
    cfg = _cfg(n=29, Hq=4, Hkv=2, d=8, HI=2, dI=8, M=4)
    inp = make_prefill_inputs(cfg)
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((1, cfg.Hq, cfg.d, cfg.d))
    r = orc.prefill(inp, cfg, state_in=S0, lib=lib)
    q, k, v = (orc.widen(inp[x], "f32") for x in ("q", "k", "v"))
    for h in range(cfg.Hq):
        g = h * cfg.Hkv // cfg.Hq
        Q, K, V = q[0, :, h], k[0, :, g], v[0, :, g]
        o = np.tril(Q @ K.T) @ V + Q @ S0[0, h]        # o_t = sum_{s<=t} (q_t.k_s) v_s + q_t^T S0
        np.testing.assert_allclose(r["olin"][0, :, h], o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r["state_out"][0, h], S0[0, h] + K.T @ V, rtol=1e-12,
                                   atol=1e-12)


def _chunked_linear(Q, K, V, S0, C):
    """Chunked evaluation of the identity-feature-map linear attention
    (gptget.net analysis, method-details section: state S_t, O(1) per step),
    chunk by chunk: O_c = tril(Q_c K_c^T) V_c + Q_c S_{c-1},
    S_c = S_{c-1} + K_c^T V_c.  The last chunk may be short."""
    n = Q.shape[0]
    S = np.array(S0, dtype=np.float64)
    out = np.zeros((n, V.shape[1]))
    for c0 in range(0, n, C):
        Qc, Kc, Vc = Q[c0:c0 + C], K[c0:c0 + C], V[c0:c0 + C]
        out[c0:c0 + C] = np.tril(Qc @ Kc.T) @ Vc + Qc @ S
        S = S + Kc.T @ Vc
    return out, S


def pin_linear_chunked(lib):
    """The oracle's recurrent linear branch (one rank-one update per token)
    equals the chunked form at chunk sizes 1, 4, 16 and 64, with n = 150 not a
    multiple of any of them but 1, with and without an initial state."""
    cfg = _cfg(n=150, Hq=4, Hkv=2, d=8, HI=2, dI=8, M=4)
    inp = make_prefill_inputs(cfg)
    rng = np.random.default_rng(6)
    q, k, v = (orc.widen(inp[x], "f32") for x in ("q", "k", "v"))
    for S0 in (None, rng.standard_normal((1, cfg.Hq, cfg.d, cfg.d))):
        r = orc.prefill(inp, cfg, state_in=S0, lib=lib)
        for h in range(cfg.Hq):
            g = h * cfg.Hkv // cfg.Hq
            init = np.zeros((cfg.d, cfg.d)) if S0 is None else S0[0, h]
            for C in (1, 4, 16, 64):
                o, S = _chunked_linear(q[0, :, h], k[0, :, g], v[0, :, g], init, C)
                np.testing.assert_allclose(r["olin"][0, :, h], o, rtol=1e-11, atol=1e-12)
                np.testing.assert_allclose(r["state_out"][0, h], S, rtol=1e-11, atol=1e-12)


def pin_topm_negative_scores(lib):
    """Selection with head weights of both signs: the oracle's sets equal the
    brute-force sort of its own scores, and a query whose weights are all
    negative selects its exact-zero scores (keys anti-aligned with every
    indexer head) first, in index order, then the negatives closest to 0."""
    cfg = LayerConfig("pin", "prefill", "f32", B=1, n=90, Hq=2, Hkv=2, d=8, HI=3, dI=8, M=12,
                      seed=9, w_dist="signed")
    inp = make_prefill_inputs(cfg)
    r = orc.prefill(inp, cfg, lib=lib)
    qI, kI, w = (orc.widen(inp[x], "f32") for x in ("q_idx", "k_idx", "w_idx"))
    assert (w < 0).any() and (w > 0).any()
    for t in range(cfg.n):
        for g in range(cfg.Hkv):
            sc = (w[0, t, g][:, None] * np.maximum(qI[0, t, g] @ kI[0, :t + 1, g].T, 0)).sum(0)
            assert r["idx"][0, t, g].tolist() == _brute_topm(sc.tolist(), cfg.M), (t, g)
    # every weight negative: zeros first (lowest index), then the least negative
    rng = np.random.default_rng(10)
    HI, dI, T, M = 2, 4, 40, 10
    qIn = np.abs(rng.standard_normal((HI, dI))) + 0.1
    kIn = np.abs(rng.standard_normal((T, dI))) + 0.1   # aligned: every dot > 0, score < 0
    kIn[::4] = -kIn[::4]                                # anti-aligned: these 10 score exactly 0
    wn = -(rng.random(HI) + 0.1)
    sc = orc.index_scores(qIn, wn, kIn, lib=lib)
    assert np.all(sc <= 0.0) and np.count_nonzero(sc == 0.0) == 10
    got = orc.topm(sc, M, lib=lib).tolist()
    assert got == list(range(0, T, 4)), got
    got = orc.topm(sc, M + 3, lib=lib).tolist()
    neg = sorted((s for s in range(T) if sc[s] < 0), key=lambda s: (-sc[s], s))[:3]
    assert got == sorted(list(range(0, T, 4)) + neg), got


def pin_gate_limits(lib):
    cfg = _cfg(n=21, Hq=4, Hkv=2, d=8, HI=2, dI=8, M=4)
    inp = make_prefill_inputs(cfg)
    shp = inp["gate"].shape
    plus = orc.prefill(inp, cfg, z_override=np.full(shp, np.inf), lib=lib)
    assert np.array_equal(plus["out"], plus["osp"])
    minus = orc.prefill(inp, cfg, z_override=np.full(shp, -np.inf), lib=lib)
    assert np.array_equal(minus["out"], minus["olin"])
    zero = orc.prefill(inp, cfg, z_override=np.zeros(shp), lib=lib)
    np.testing.assert_allclose(zero["out"], 0.5 * (zero["osp"] + zero["olin"]), rtol=1e-15,
                               atol=1e-15)


def pin_selection_properties(lib):
    cfg = _cfg(n=64, Hq=2, Hkv=2, d=8, HI=4, dI=8, M=9)
    inp = make_prefill_inputs(cfg)
    r = orc.prefill(inp, cfg, lib=lib)
    r2 = orc.prefill(inp, cfg, M=cfg.M + 1, lib=lib)
    qI, kI, w = (orc.widen(inp[x], "f32") for x in ("q_idx", "k_idx", "w_idx"))
    for t in range(cfg.n):
        for g in range(cfg.Hkv):
            sel = r["idx"][0, t, g]
            m = min(cfg.M, t + 1)
            assert (sel[m:] == -1).all() and (sel[:m] >= 0).all() and (sel[:m] <= t).all()
            assert (np.diff(sel[:m]) > 0).all()
            sc = (w[0, t, g][:, None] * np.maximum(qI[0, t, g] @ kI[0, :t + 1, g].T, 0)).sum(0)
            chosen = set(sel[:m].tolist())
            rest = [s for s in range(t + 1) if s not in chosen]
            if rest:   # dominance, with the lower index winning ties
                worst = min(chosen, key=lambda s: (sc[s], -s))
                for s in rest:
                    assert (sc[s], -s) < (sc[worst], -worst)
            # nesting: the M set is inside the M+1 set
            assert chosen <= set(r2["idx"][0, t, g].tolist())


def pin_rows_subset(lib):
    cfg = _cfg(n=45, Hq=4, Hkv=2, d=8, HI=2, dI=8, M=6)
    inp = make_prefill_inputs(cfg)
    full = orc.prefill(inp, cfg, lib=lib)
    rows = [0, 3, 17, 44]
    part = orc.prefill(inp, cfg, rows=rows, lib=lib)
    for key in ("out", "osp", "olin", "idx"):
        assert np.array_equal(part[key][0], full[key][0, rows]), key
    assert np.array_equal(part["state_out"], full["state_out"])


def pin_decode_matches_prefill(lib):
    cfg = _cfg(n=26, Hq=4, Hkv=2, d=8, HI=2, dI=8, M=5)
    inp = make_prefill_inputs(cfg)
    full = orc.prefill(inp, cfg, lib=lib)
    t = cfg.n - 1
    # state after t-1 tokens comes from a shorter prefill
    short = {k: (v[:, :t] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    short["n"] = t
    pre = orc.prefill(short, cfg, lib=lib)
    dcfg = LayerConfig("pin_dec", "decode", "f32", B=1, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d,
                       HI=cfg.HI, dI=cfg.dI, M=cfg.M)
    dec = {"q": inp["q"][:, t], "k_cache": inp["k"][0], "v_cache": inp["v"][0],
           "q_idx": inp["q_idx"][:, t], "k_idx_cache": inp["k_idx"][0], "w_idx": inp["w_idx"][:, t],
           "gate": inp["gate"][:, t], "state": pre["state_out"],
           "cu_ctx": np.array([0, cfg.n], dtype=np.int64), "B": 1}
    r = orc.decode(dec, dcfg, lib=lib)
    assert np.array_equal(r["idx"][0], full["idx"][0, t])
    np.testing.assert_allclose(r["out"][0], full["out"][0, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["state_out"], full["state_out"], rtol=1e-12, atol=1e-13)


def pin_decode_ragged_groups(lib):
    """Decode on a ragged batch equals per-sequence decode (no cross-talk)."""
    cfg = LayerConfig("pin_rag", "decode", "f32", B=3, Hq=4, Hkv=2, d=8, HI=2, dI=8, M=6,
                      ctx_lo=3, ctx_hi=20, seed=9)
    inp = make_decode_inputs(cfg)
    r = orc.decode(inp, cfg, lib=lib)
    cu = inp["cu_ctx"]
    for b in range(inp["B"]):
        lo, hi = cu[b], cu[b + 1]
        one = {"q": inp["q"][b:b + 1], "k_cache": inp["k_cache"][lo:hi],
               "v_cache": inp["v_cache"][lo:hi], "q_idx": inp["q_idx"][b:b + 1],
               "k_idx_cache": inp["k_idx_cache"][lo:hi], "w_idx": inp["w_idx"][b:b + 1],
               "gate": inp["gate"][b:b + 1], "state": inp["state"][b:b + 1],
               "cu_ctx": np.array([0, hi - lo], dtype=np.int64), "B": 1}
        rb = orc.decode(one, cfg, lib=lib)
        assert np.array_equal(rb["idx"][0], r["idx"][b])
        assert np.array_equal(rb["out"][0], r["out"][b])


def window_sets(positions, M, G):
    """Sliding-window sets: position t takes max(0, t-M+1)..t, ascending, -1 padded."""
    sets = -np.ones((len(positions), G, M), dtype=np.int32)
    for u, t in enumerate(positions):
        m = min(M, t + 1)
        sets[u, :, :m] = np.arange(t - m + 1, t + 1)
    return sets


def pin_window_banded(lib):
    """The oracle's sparse branch on sliding-window sets equals dense attention
    under a banded causal mask (torch SDPA with an explicit mask); with a
    window at least n long it is plain causal attention."""
    import torch
    cfg = _cfg(n=29, Hq=4, Hkv=2, d=16, HI=2, dI=8, M=6)
    inp = make_prefill_inputs(cfg)
    q, k, v = (orc.widen(inp[x], "f32") for x in ("q", "k", "v"))
    n, Hq, Hkv, d = cfg.n, cfg.Hq, cfg.Hkv, cfg.d
    scale = 1.0 / math.sqrt(d)
    zinf = np.full((n, Hq), np.inf)
    for W in (6, 1, 40):
        sets = window_sets(range(n), W, Hkv)
        _, osp = orc.sparse_given_sets(q[0], k[0], v[0], np.zeros(n, dtype=np.int64), sets, zinf,
                                       np.zeros((n, Hq, d)), Hq, Hkv, d, W, lib=lib)
        t = np.arange(n)
        band = (t[None, :] <= t[:, None]) & (t[None, :] > t[:, None] - W)   # [query, key]
        r = Hq // Hkv
        qt = torch.from_numpy(q[0]).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k[0]).permute(1, 0, 2).repeat_interleave(r, 0)[None]
        vt = torch.from_numpy(v[0]).permute(1, 0, 2).repeat_interleave(r, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=torch.from_numpy(band), scale=scale)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(osp, ref, rtol=1e-11, atol=1e-12)
        if W >= n:
            np.testing.assert_allclose(osp, _sdpa_causal(q, k, v, scale)[0], rtol=1e-11, atol=1e-12)


ALL_PINS = [pin_golden_prefill, pin_golden_softmax, pin_golden_decode, pin_topm_bruteforce,
            pin_scores_reductions, pin_sparse_full_causal, pin_sparse_m1, pin_sparse_zero_query,
            pin_linear_closed_form, pin_linear_chunked, pin_topm_negative_scores, pin_gate_limits, pin_selection_properties, pin_rows_subset,
            pin_decode_matches_prefill, pin_decode_ragged_groups, pin_window_banded]
