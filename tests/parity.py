"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare with the fp64 oracle.

Parity rules (the bar the tests enforce):
  * index sets: for every (query, group), |B| = m = min(M, t+1), B is an
    ascending subset of [0, t] padded with -1, and every candidate in the
    symmetric difference of B and the oracle's set A scores within
    eps = 1e-5 * |s_m| of the m-th oracle score s_m (eps = 1e-5 * max I when
    s_m == 0; exact match when every score is 0);
  * outputs: normwise relative error ||x - ref||_F / ||ref||_F <= 1e-2 for bf16
    and <= 1e-4 for fp32, checked separately for the sparse branch alone
    (gate logit +inf), the linear branch alone (-inf), the gated output and
    the final state.  The sparse reference is the oracle evaluated on the
    GPU's own (validated) index sets.
"""
from __future__ import annotations

import numpy as np

from hybrid_linear_top_amd import inputs as gen
from oracle import oracle as orc

TOL = {"bf16": 1e-2, "f32": 1e-4}
# Per-row bound (a row is one (position, head) output vector, or one row of a
# head's d x d state): the normwise rule over a whole tensor averages a bad
# row away (one wrong row of 18,000 adds 0.75 %), so every row must also be
# within ROW_TOL of its reference row.  A bf16 row carries a few roundings of
# relative size 2^-9 (the output, the bf16 MFMA operands P and the prefix
# states), so its error is a few 1e-3 (measured on MI355X over every GPU
# case: at most 3e-3 for the sparse branch, 4e-3 for the linear branch and
# 1.5e-2 for the gated output, where the two branches partly cancel); fp32
# rows differ by summation order.
# A row whose reference norm is under ROW_FLOOR of the tensor's RMS row norm
# is measured against that floor, so that near-zero rows (a lone product
# q.k_0 v_0 that happens to be tiny) do not divide by ~0.
ROW_TOL = {"bf16": 5e-2, "f32": 1e-3}
ROW_FLOOR = 2e-2


def normwise(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


def row_errors(x, ref, d):
    """Per-row relative errors ||x_r - ref_r|| / max(||ref_r||, ROW_FLOOR * rms)
    over rows of length d (the last axis, or d consecutive elements)."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, d)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, d)
    rn = np.linalg.norm(ref, axis=1)
    rms = float(np.sqrt(np.mean(rn * rn))) if len(rn) else 0.0
    den = np.maximum(rn, ROW_FLOOR * rms)
    num = np.linalg.norm(x - ref, axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        e = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return e


def max_row_error(x, ref, d) -> float:
    e = row_errors(x, ref, d)
    return float(e.max()) if e.size else 0.0


def check_sets(idx, ref_idx, T, score_fn, M, rel=1e-5):
    """Band rule for many (query, group) units at once.  idx, ref_idx [U, M]
    (GPU and oracle sets), T [U] candidates per unit (t + 1), score_fn(u) ->
    fp64 oracle scores of unit u's candidates 0..T-1 (called only for units
    whose sets differ).  Returns the number of swapped candidates."""
    idx = np.asarray(idx).reshape(-1, M)
    ref_idx = np.asarray(ref_idx).reshape(-1, M)
    T = np.asarray(T, dtype=np.int64).reshape(-1)
    U = idx.shape[0]
    m = np.minimum(M, T)
    col = np.arange(M)[None, :]
    live = col < m[:, None]
    bad = np.nonzero(np.any(~live & (idx != -1), axis=1))[0]
    assert bad.size == 0, ("padding", bad[:5])
    bad = np.nonzero(np.any(live & ((idx < 0) | (idx >= T[:, None])), axis=1))[0]
    assert bad.size == 0, ("range", bad[:5])
    if M > 1:
        asc = (idx[:, 1:] > idx[:, :-1]) | ~live[:, 1:]
        bad = np.nonzero(~np.all(asc, axis=1))[0]
        assert bad.size == 0, ("ascending and distinct", bad[:5])
    swaps = 0
    for u in np.nonzero(np.any(idx != ref_idx, axis=1))[0]:
        swaps += check_set(idx[u], score_fn(int(u)), M, rel=rel)
    return swaps


def check_set(sel, scores, M, rel=1e-5):
    """Band rule for one (query, group).  scores: fp64 oracle scores of the
    candidates 0..T-1.  Returns the number of swapped candidates."""
    T = len(scores)
    m = min(M, T)
    sel = np.asarray(sel)
    assert len(sel) == M
    assert np.all(sel[m:] == -1), "padding"
    s = sel[:m]
    assert np.all(s >= 0) and np.all(s < T), "range"
    assert np.all(np.diff(s) > 0), "ascending and distinct"
    ref = orc.topm(scores, M)[:m]
    diff = set(ref.tolist()) ^ set(s.tolist())
    if diff:
        s_m = np.sort(scores)[::-1][m - 1]
        eps = rel * abs(s_m) if s_m != 0 else rel * float(np.max(scores))
        for c in diff:
            assert abs(scores[c] - s_m) <= eps, (c, scores[c], s_m, eps)
    return len(diff)


def gate_fill(shape, dtype, value):
    x = np.full(shape, value, dtype=np.float32)
    return gen.round_bf16(x) if dtype == "bf16" else x


def run_prefill(cfg, inp, gate=None, state_in=None, dims=None):
    import torch
    from hybrid_linear_top_amd import lisa
    dims = dims or lisa.dims_from_config(cfg)
    dv = lisa.to_device
    tens = [dv(inp[k]) for k in ("q", "k", "v", "q_idx", "k_idx", "w_idx")]
    g = dv(inp["gate"] if gate is None else gate)
    s0 = None if state_in is None else dv(np.ascontiguousarray(state_in, dtype=np.float32))
    out, st, idx = lisa.prefill(dims, *tens, g, state_in=s0)
    torch.cuda.synchronize()
    return (orc.widen(lisa.from_device(out), cfg.dtype), lisa.from_device(st).astype(np.float64),
            lisa.from_device(idx))


def run_prefill_continue(cfg, inp, past, gate=None, state_in=None, dims=None):
    """GPU prefill of the first `past` tokens (for its final state), then the
    continued prefill of the rest against the full caches.  Returns the
    continued call's (out, state_out, idx) for rows past..n-1."""
    import torch
    from hybrid_linear_top_amd import lisa
    dims = dims or lisa.dims_from_config(cfg)
    dv = lisa.to_device
    gate = inp["gate"] if gate is None else gate
    s0 = None if state_in is None else dv(np.ascontiguousarray(state_in, dtype=np.float32))
    if past > 0:
        head = [dv(np.ascontiguousarray(inp[k][:, :past])) for k in ("q", "k", "v", "q_idx", "k_idx", "w_idx")]
        _, s0, _ = lisa.prefill(dims, *head, dv(np.ascontiguousarray(gate[:, :past])), state_in=s0)
    tail = {k: dv(np.ascontiguousarray(inp[k][:, past:])) for k in ("q", "q_idx", "w_idx")}
    caches = {k: dv(inp[k]) for k in ("k", "v", "k_idx")}
    out, st, idx = lisa.prefill_continue(dims, past, tail["q"], caches["k"], caches["v"], tail["q_idx"],
                                         caches["k_idx"], tail["w_idx"],
                                         dv(np.ascontiguousarray(gate[:, past:])), state_in=s0)
    torch.cuda.synchronize()
    return (orc.widen(lisa.from_device(out), cfg.dtype), lisa.from_device(st).astype(np.float64),
            lisa.from_device(idx))


def run_decode(cfg, inp, gate=None, dims=None):
    import torch
    from hybrid_linear_top_amd import lisa
    dims = dims or lisa.dims_from_config(cfg)
    dv = lisa.to_device
    state = dv(inp["state"])
    out, idx = lisa.decode_step(dims, dv(inp["cu_ctx"]), inp["max_ctx"], dv(inp["q"]),
                                dv(inp["k_cache"]), dv(inp["v_cache"]), dv(inp["q_idx"]),
                                dv(inp["k_idx_cache"]), dv(inp["w_idx"]),
                                dv(inp["gate"] if gate is None else gate), state)
    torch.cuda.synchronize()
    return (orc.widen(lisa.from_device(out), cfg.dtype), lisa.from_device(state).astype(np.float64),
            lisa.from_device(idx))


def to_pages(inp, block_size, seed=0, spare=2, fill=64.0):
    """Scatter packed decode caches into page pools whose pages are shuffled.
    Table entries past a sequence's last block, and `spare` extra pages, point
    at pages holding `fill` everywhere: a kernel that reads a row it should
    not would pick up those values (and, in the indexer, score them highest)
    instead of faulting."""
    rng = np.random.default_rng(seed)
    cu = np.asarray(inp["cu_ctx"], dtype=np.int64)
    B, max_ctx = inp["B"], inp["max_ctx"]
    L = np.diff(cu)
    nblk = (L + block_size - 1) // block_size
    max_blocks = max(int(nblk.max()), -(-max_ctx // block_size))
    num_pages = int(nblk.sum()) + spare
    order = rng.permutation(num_pages)
    junk = int(order[-1])
    table = np.full((B, max_blocks), junk, dtype=np.int32)
    pools = {}
    for name in ("k_cache", "v_cache", "k_idx_cache"):
        src = inp[name]
        pool = np.full((num_pages * block_size,) + src.shape[1:], fill, dtype=src.dtype)
        pools[name] = pool
    nxt = 0
    for b in range(B):
        for j in range(int(nblk[b])):
            page = int(order[nxt])
            nxt += 1
            table[b, j] = page
            lo = j * block_size
            hi = min(int(L[b]), lo + block_size)
            for name, pool in pools.items():
                pool[page * block_size:page * block_size + hi - lo] = inp[name][cu[b] + lo:cu[b] + hi]
    return dict(lengths=L.astype(np.int32), table=table, num_pages=num_pages, **pools)


def run_decode_paged(cfg, inp, paged, block_size, dims=None):
    import torch
    from hybrid_linear_top_amd import lisa
    dims = dims or lisa.dims_from_config(cfg)
    dv = lisa.to_device
    state = dv(inp["state"])
    out, idx = lisa.decode_step_paged(dims, dv(paged["lengths"]), dv(paged["table"]), block_size,
                                      inp["max_ctx"], dv(inp["q"]), dv(paged["k_cache"]),
                                      dv(paged["v_cache"]), dv(inp["q_idx"]),
                                      dv(paged["k_idx_cache"]), dv(inp["w_idx"]), dv(inp["gate"]),
                                      state)
    torch.cuda.synchronize()
    return (orc.widen(lisa.from_device(out), cfg.dtype), lisa.from_device(state).astype(np.float64),
            lisa.from_device(idx))


def paged_decode_parity(cfg, inp, block_size, seed=0, report=None):
    """The packed step against the oracle, then the paged step on the same
    cache contents: same output, state and index sets, bit for bit (the two
    differ only in where a row is fetched from)."""
    decode_parity(cfg, inp, report=report)
    ref = run_decode(cfg, inp)
    paged = to_pages(inp, block_size, seed=seed)
    got = run_decode_paged(cfg, inp, paged, block_size)
    for name, x, y in zip(("out", "state", "idx"), got, ref):
        assert np.array_equal(x, y), f"paged {name} differs from packed"


def prefill_parity(cfg, inp, rows=None, state_in=None, report=None, past=0):
    """Full prefill parity (all four checks) on the listed rows (None = all).
    With past > 0 the GPU side is a prefill of the first `past` tokens followed
    by the continued prefill of the rest; the oracle is one prefill over all n
    tokens, and the rows checked are past..n-1 (or the listed ones)."""
    dt = cfg.dtype
    B, n = inp["B"], inp["n"]
    tol = TOL[dt]
    if rows is None and past > 0:
        rows = list(range(past, n))
    ref = orc.prefill(inp, cfg, rows=rows, state_in=state_in)
    R = ref["rows"] if rows is not None else np.arange(n)
    assert np.all(R >= past)

    def gpu(gate=None):
        if past == 0:
            o, st_, ix = run_prefill(cfg, inp, gate=gate, state_in=state_in)
            return o, st_, ix
        o, st_, ix = run_prefill_continue(cfg, inp, past, gate=gate, state_in=state_in)
        pad = lambda x: np.concatenate([np.zeros((B, past) + x.shape[2:], x.dtype), x], axis=1)
        return pad(o), st_, pad(ix)

    out, st, idx = gpu()
    osp, _, idx_p = gpu(gate=gate_fill(inp["gate"].shape, dt, np.inf))
    olin, _, _ = gpu(gate=gate_fill(inp["gate"].shape, dt, -np.inf))
    assert np.array_equal(idx, idx_p), "index sets differ between two runs"
    qI, kI, w = (orc.widen(inp[x], dt) for x in ("q_idx", "k_idx", "w_idx"))
    G = cfg.Hkv
    Rl = np.asarray(R)

    def score_fn(u):
        b, rem = divmod(u, len(Rl) * G)
        r, g = divmod(rem, G)
        t = int(Rl[r])
        return orc.index_scores(qI[b, t, g], w[b, t, g], kI[b, :t + 1, g])

    Tq = np.broadcast_to((Rl + 1)[None, :, None], (B, len(Rl), G))
    swaps = check_sets(idx[:, Rl], ref["idx"], Tq, score_fn, cfg.M)
    # oracle sparse branch and gate on the GPU's sets
    q = orc.widen(inp["q"], dt)
    kr = orc.widen(inp["k"], dt).reshape(B * n, cfg.Hkv, cfg.d)
    vr = orc.widen(inp["v"], dt).reshape(B * n, cfg.Hkv, cfg.d)
    z = orc.widen(inp["gate"], dt)
    U = B * len(R)
    qs = q[:, R].reshape(U, cfg.Hq, cfg.d)
    row0 = np.repeat(np.arange(B) * n, len(R))
    sets = idx[:, R].reshape(U, cfg.Hkv, cfg.M)
    out_g, osp_g = orc.sparse_given_sets(qs, kr, vr, row0, sets, z[:, R].reshape(U, cfg.Hq),
                                         ref["olin"].reshape(U, cfg.Hq, cfg.d), cfg.Hq, cfg.Hkv,
                                         cfg.d, cfg.M)
    e_sp = normwise(osp[:, R].reshape(U, -1), osp_g.reshape(U, -1))
    e_lin = normwise(olin[:, R], ref["olin"])
    e_out = normwise(out[:, R].reshape(U, -1), out_g.reshape(U, -1))
    e_out_own = normwise(out[:, R], ref["out"])
    e_st = normwise(st, ref["state_out"])
    d = cfg.d
    rows_err = dict(row_sparse=max_row_error(osp[:, R].reshape(U, -1), osp_g.reshape(U, -1), d),
                    row_linear=max_row_error(olin[:, R], ref["olin"], d),
                    row_out=max_row_error(out[:, R].reshape(U, -1), out_g.reshape(U, -1), d),
                    row_state=max_row_error(st, ref["state_out"], d))
    res = dict(e_sparse=e_sp, e_linear=e_lin, e_out=e_out, e_out_vs_oracle_sets=e_out_own,
               e_state=e_st, swaps=swaps, **rows_err)
    if report is not None:
        report.update(res)
    assert e_sp <= tol, res
    assert e_lin <= tol, res
    assert e_out <= tol, res
    assert e_st <= tol, res
    for key, val in rows_err.items():
        assert val <= ROW_TOL[dt], (key, res)
    return res


def decode_parity(cfg, inp, report=None):
    dt = cfg.dtype
    tol = TOL[dt]
    ref = orc.decode(inp, cfg)
    out, st, idx = run_decode(cfg, inp)
    osp, _, idx_p = run_decode(cfg, inp, gate=gate_fill(inp["gate"].shape, dt, np.inf))
    olin, _, _ = run_decode(cfg, inp, gate=gate_fill(inp["gate"].shape, dt, -np.inf))
    assert np.array_equal(idx, idx_p), "index sets differ between two runs"
    cu = inp["cu_ctx"]
    qI, kIc, w = (orc.widen(inp[x], dt) for x in ("q_idx", "k_idx_cache", "w_idx"))
    G = cfg.Hkv

    def score_fn(u):
        b, g = divmod(u, G)
        return orc.index_scores(qI[b, g], w[b, g], kIc[cu[b]:cu[b + 1], g])

    Tq = np.repeat(np.diff(cu), G)
    swaps = check_sets(idx, ref["idx"], Tq, score_fn, cfg.M)
    q = orc.widen(inp["q"], dt)
    kc, vc = orc.widen(inp["k_cache"], dt), orc.widen(inp["v_cache"], dt)
    z = orc.widen(inp["gate"], dt)
    out_g, osp_g = orc.sparse_given_sets(q, kc, vc, cu[:-1], idx, z, ref["olin"], cfg.Hq, cfg.Hkv,
                                         cfg.d, cfg.M)
    d = cfg.d
    rows_err = dict(row_sparse=max_row_error(osp, osp_g, d), row_linear=max_row_error(olin, ref["olin"], d),
                    row_out=max_row_error(out, out_g, d), row_state=max_row_error(st, ref["state_out"], d))
    res = dict(e_sparse=normwise(osp, osp_g), e_linear=normwise(olin, ref["olin"]),
               e_out=normwise(out, out_g), e_out_vs_oracle_sets=normwise(out, ref["out"]),
               e_state=normwise(st, ref["state_out"]), swaps=swaps, **rows_err)
    if report is not None:
        report.update(res)
    for key in ("e_sparse", "e_linear", "e_out", "e_state"):
        assert res[key] <= tol, res
    for key, val in rows_err.items():
        assert val <= ROW_TOL[dt], (key, res)
    return res


# ---- sliding-window variant ------------------------------------------------
def window_prefill_parity(cfg, inp, past=0, state_in=None, report=None):
    """GPU lisa_prefill_window (after a prefill of the first `past` tokens for
    the state) against the oracle: the sparse branch on the window sets
    max(0, t-M+1)..t, the linear branch and state of one oracle prefill."""
    import torch
    from hybrid_linear_top_amd import lisa
    from tests.oracle_pins import window_sets
    dt = cfg.dtype
    B, n = inp["B"], inp["n"]
    tol = TOL[dt]
    rows = list(range(past, n))
    ref = orc.prefill(inp, cfg, rows=rows, state_in=state_in)
    dims = lisa.dims_from_config(cfg)
    dv = lisa.to_device

    def gpu(gate):
        s0 = None if state_in is None else dv(np.ascontiguousarray(state_in, dtype=np.float32))
        if past > 0:
            head = [dv(np.ascontiguousarray(inp[k][:, :past])) for k in ("q", "k", "v")]
            _, s0 = lisa.prefill_window(dims, 0, head[0], head[1], head[2],
                                        dv(np.ascontiguousarray(gate[:, :past])), state_in=s0)
        o, st_ = lisa.prefill_window(dims, past, dv(np.ascontiguousarray(inp["q"][:, past:])),
                                     dv(inp["k"]), dv(inp["v"]), dv(np.ascontiguousarray(gate[:, past:])),
                                     state_in=s0)
        torch.cuda.synchronize()
        return orc.widen(lisa.from_device(o), dt), lisa.from_device(st_).astype(np.float64)

    out, st = gpu(inp["gate"])
    osp, _ = gpu(gate_fill(inp["gate"].shape, dt, np.inf))
    olin, _ = gpu(gate_fill(inp["gate"].shape, dt, -np.inf))
    q = orc.widen(inp["q"], dt)
    kr = orc.widen(inp["k"], dt).reshape(B * n, cfg.Hkv, cfg.d)
    vr = orc.widen(inp["v"], dt).reshape(B * n, cfg.Hkv, cfg.d)
    z = orc.widen(inp["gate"], dt)
    R = np.asarray(rows)
    U = B * len(R)
    sets = np.concatenate([window_sets(R, cfg.M, cfg.Hkv) for _ in range(B)])
    row0 = np.repeat(np.arange(B) * n, len(R))
    out_g, osp_g = orc.sparse_given_sets(q[:, R].reshape(U, cfg.Hq, cfg.d), kr, vr, row0, sets,
                                         z[:, R].reshape(U, cfg.Hq), ref["olin"].reshape(U, cfg.Hq, cfg.d),
                                         cfg.Hq, cfg.Hkv, cfg.d, cfg.M)
    res = dict(e_sparse=normwise(osp.reshape(U, -1), osp_g.reshape(U, -1)),
               e_linear=normwise(olin, ref["olin"]), e_out=normwise(out.reshape(U, -1), out_g.reshape(U, -1)),
               e_state=normwise(st, ref["state_out"]))
    d = cfg.d
    rows_err = dict(row_sparse=max_row_error(osp, osp_g, d), row_linear=max_row_error(olin, ref["olin"], d),
                    row_out=max_row_error(out, out_g, d), row_state=max_row_error(st, ref["state_out"], d))
    if report is not None:
        report.update(res, **rows_err)
    for key in res:
        assert res[key] <= tol, res
    for key, val in rows_err.items():
        assert val <= ROW_TOL[dt], (key, rows_err)
    return res


def window_decode_parity(cfg, inp, report=None):
    """GPU lisa_decode_step_window against the oracle: sparse branch on the
    window set of the new token, the oracle decode's linear branch and state."""
    import torch
    from hybrid_linear_top_amd import lisa
    from tests.oracle_pins import window_sets
    dt = cfg.dtype
    tol = TOL[dt]
    ref = orc.decode(inp, cfg)
    dims = lisa.dims_from_config(cfg)
    dv = lisa.to_device

    def gpu(gate):
        state = dv(inp["state"])
        o = lisa.decode_step_window(dims, dv(inp["cu_ctx"]), inp["max_ctx"], dv(inp["q"]),
                                    dv(inp["k_cache"]), dv(inp["v_cache"]), dv(gate), state)
        torch.cuda.synchronize()
        return orc.widen(lisa.from_device(o), dt), lisa.from_device(state).astype(np.float64)

    out, st = gpu(inp["gate"])
    osp, _ = gpu(gate_fill(inp["gate"].shape, dt, np.inf))
    olin, _ = gpu(gate_fill(inp["gate"].shape, dt, -np.inf))
    cu = inp["cu_ctx"]
    L = np.diff(cu)
    # positions are local to each sequence; rows of the packed cache are cu[b] + s
    sets = window_sets(L - 1, cfg.M, cfg.Hkv)
    q = orc.widen(inp["q"], dt)
    kc, vc = orc.widen(inp["k_cache"], dt), orc.widen(inp["v_cache"], dt)
    z = orc.widen(inp["gate"], dt)
    out_g, osp_g = orc.sparse_given_sets(q, kc, vc, cu[:-1], sets, z, ref["olin"], cfg.Hq, cfg.Hkv,
                                         cfg.d, cfg.M)
    res = dict(e_sparse=normwise(osp, osp_g), e_linear=normwise(olin, ref["olin"]),
               e_out=normwise(out, out_g), e_state=normwise(st, ref["state_out"]))
    d = cfg.d
    rows_err = dict(row_sparse=max_row_error(osp, osp_g, d), row_linear=max_row_error(olin, ref["olin"], d),
                    row_out=max_row_error(out, out_g, d), row_state=max_row_error(st, ref["state_out"], d))
    if report is not None:
        report.update(res, **rows_err)
    for key in res:
        assert res[key] <= tol, res
    for key, val in rows_err.items():
        assert val <= ROW_TOL[dt], (key, rows_err)
    return res


# ---- backward ------------------------------------------------------------------
BWD_TOL = {"bf16": 1e-2, "f32": 1e-4}


def window_sets(B, n, G, M):
    """The sliding-window variant's sets: position t attends to
    max(0, t - M + 1) .. t, ascending, -1 padded."""
    idx = np.full((B, n, G, M), -1, dtype=np.int32)
    for t in range(n):
        lo = max(0, t - M + 1)
        idx[:, t, :, :t + 1 - lo] = np.arange(lo, t + 1, dtype=np.int32)
    return idx


def backward_parity(cfg, inp, binp, report=None, sets=None):
    """GPU forward (for the sets, unless given), GPU backward, oracle backward
    on the same sets; normwise errors of dq, dk, dv, dgate and d_state_in."""
    import torch
    from hybrid_linear_top_amd import lisa
    from oracle import backward as obwd
    dims = lisa.dims_from_config(cfg)
    dv_ = lisa.to_device
    dt = cfg.dtype
    S0 = binp["state_in"]
    idx = sets if sets is not None else run_prefill(cfg, inp, state_in=S0)[2]
    got = lisa.prefill_backward(dims, dv_(inp["q"]), dv_(inp["k"]), dv_(inp["v"]), dv_(inp["gate"]),
                                dv_(idx), dv_(binp["d_out"]),
                                state_in=None if S0 is None else dv_(S0),
                                d_state_out=None if binp["d_state_out"] is None else dv_(binp["d_state_out"]),
                                want_state_grad=True)
    torch.cuda.synchronize()
    got = [lisa.from_device(x).astype(np.float64) for x in got]
    w = lambda x: orc.widen(inp[x], dt)  # noqa: E731
    ref = obwd.prefill_backward(w("q"), w("k"), w("v"), w("gate"), idx, orc.widen(binp["d_out"], dt),
                                state_in=S0, d_state_out=binp["d_state_out"])
    names = ("dq", "dk", "dv", "dz", "d_state_in")
    res = {f"e_{nm}": normwise(g, ref[nm]) for nm, g in zip(names, got)}
    if report is not None:
        report.update(res)
    for key, val in res.items():
        assert val <= BWD_TOL[dt], res
    return res


def backward_sampled_parity(cfg, inp, binp, rows, keys, report=None, sets=None):
    """Full-length backward: GPU forward (for the sets, unless given) and GPU
    backward over all positions, checked against the oracle's per-row form at
    sampled query rows (dq, dz) and key rows (dk, dv); normwise over the
    sampled rows."""
    import torch
    from hybrid_linear_top_amd import lisa
    from oracle import backward as obwd
    dims = lisa.dims_from_config(cfg)
    dv_ = lisa.to_device
    dt = cfg.dtype
    S0, dS = binp["state_in"], binp["d_state_out"]
    idx = sets if sets is not None else run_prefill(cfg, inp, state_in=S0)[2]
    got = lisa.prefill_backward(dims, dv_(inp["q"]), dv_(inp["k"]), dv_(inp["v"]), dv_(inp["gate"]),
                                dv_(idx), dv_(binp["d_out"]),
                                state_in=None if S0 is None else dv_(S0),
                                d_state_out=None if dS is None else dv_(dS), want_state_grad=False)
    torch.cuda.synchronize()
    dq, dk, dv, dz = (lisa.from_device(x).astype(np.float64) for x in got[:4])
    w = lambda x: orc.widen(inp[x], dt)  # noqa: E731
    ref = obwd.prefill_backward_rows(w("q"), w("k"), w("v"), w("gate"), idx, orc.widen(binp["d_out"], dt),
                                     rows, keys, state_in=S0, d_state_out=dS)
    res = {"e_dq": normwise(dq[:, rows], ref["dq"]), "e_dz": normwise(dz[:, rows], ref["dz"]),
           "e_dk": normwise(dk[:, keys], ref["dk"]), "e_dv": normwise(dv[:, keys], ref["dv"])}
    if report is not None:
        report.update(res)
    for key, val in res.items():
        assert val <= BWD_TOL[dt], res
    return res
