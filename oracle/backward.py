"""fp64 CPU oracle of the LISA layer's backward pass.

TEST INFRASTRUCTURE ONLY: used by the tests and the benchmark's CPU baseline,
never by the product path.  Shares no code with the HIP implementation.

The forward pass is the layer of the pages (gptget.net analysis of arXiv
2607.19358, method-details section): per query head h of group g and
position t,
    o_sp  = sum_{s in S_t} p_s v_s,  p = softmax(scale * K_S q)   (selected keys)
    S_t   = S_0 + sum_{s <= t} k_s v_s^T,  o_lin = S_t^T q         (identity map)
    out   = gamma * o_sp + (1 - gamma) * o_lin,  gamma = sigmoid(z)
and state_out = S_n.  This module differentiates
    L = <d_out, out> + <d_state_out, state_out>
by the chain rule, step by step, in the order the forward computes, with the
selected sets S_t held fixed (they are the forward's; a top-M set is a
piecewise-constant function of q_I, k_I and w, so those inputs get no
gradient).  Plain loops over positions and heads; no chunking.
"""
from __future__ import annotations

import math

import numpy as np


def _softmax(x):
    m = np.max(x)
    e = np.exp(x - m)
    return e / np.sum(e)


def prefill_backward(q, k, v, z, idx, d_out, scale=0.0, state_in=None, d_state_out=None):
    """q [B,n,Hq,d]; k, v [B,n,G,d]; z [B,n,Hq]; idx [B,n,G,M] (forward sets,
    ascending, -1 padded); d_out [B,n,Hq,d]; state_in, d_state_out
    [B,Hq,d,d] ([key dim i][value dim j]) or None.  All fp64.

    Returns dq [B,n,Hq,d], dk, dv [B,n,G,d], dz [B,n,Hq], d_state_in
    [B,Hq,d,d], plus the recomputed osp and olin [B,n,Hq,d]."""
    q, k, v, z, d_out = (np.asarray(x, dtype=np.float64) for x in (q, k, v, z, d_out))
    B, n, Hq, d = q.shape
    G = k.shape[2]
    scale = scale if scale else 1.0 / math.sqrt(d)
    gam = 1.0 / (1.0 + np.exp(-z))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dz = np.zeros_like(z)
    dS0 = np.zeros((B, Hq, d, d))
    osp = np.zeros_like(q)
    olin = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            g = (h * G) // Hq
            # forward of the linear branch, keeping every S_t
            S = np.zeros((d, d)) if state_in is None else np.array(state_in[b, h], dtype=np.float64)
            states = []
            for t in range(n):
                S = S + np.outer(k[b, t, g], v[b, t, g])
                states.append(S.copy())
                olin[b, t, h] = S.T @ q[b, t, h]
            for t in range(n):
                sel = np.asarray(idx[b, t, g])
                sel = sel[sel >= 0]
                K, V = k[b, sel, g], v[b, sel, g]
                p = _softmax(scale * (K @ q[b, t, h]))
                osp[b, t, h] = p @ V
                dO = d_out[b, t, h]
                ga = gam[b, t, h]
                # gate
                dz[b, t, h] = ga * (1.0 - ga) * float(dO @ (osp[b, t, h] - olin[b, t, h]))
                d_sp = ga * dO
                d_lin = (1.0 - ga) * dO
                # sparse branch: softmax attention over the selected rows
                dp = V @ d_sp
                dlogit = p * (dp - float(p @ dp))
                dq[b, t, h] += scale * (dlogit @ K)
                dk[b, sel, g] += scale * np.outer(dlogit, q[b, t, h])
                dv[b, sel, g] += np.outer(p, d_sp)
                # linear branch, query side: o_lin = S_t^T q
                dq[b, t, h] += states[t] @ d_lin
            # linear branch, key/value side: H_t = dS_out + sum_{t' >= t} q_t' d_lin_t'^T
            H = np.zeros((d, d)) if d_state_out is None else np.array(d_state_out[b, h], dtype=np.float64)
            for t in range(n - 1, -1, -1):
                d_lin = (1.0 - gam[b, t, h]) * d_out[b, t, h]
                H = H + np.outer(q[b, t, h], d_lin)
                dk[b, t, g] += H @ v[b, t, g]
                dv[b, t, g] += H.T @ k[b, t, g]
            dS0[b, h] = H
    return {"dq": dq, "dk": dk, "dv": dv, "dz": dz, "d_state_in": dS0, "osp": osp, "olin": olin}


def prefill_backward_rows(q, k, v, z, idx, d_out, rows, keys, scale=0.0, state_in=None,
                          d_state_out=None):
    """The same gradients, evaluated one output row at a time (for sequences
    too long for prefill_backward): dq and dz at query positions `rows`, dk
    and dv at key positions `keys`, for every batch entry and head.

    Each gradient is written as its own sum from the chain rule rather than
    accumulated while walking the sequence:
      dq_t  = scale sum_{s in S_t} dlogit_s k_s  +  S_t d_lin_t
      dz_t  = gamma (1 - gamma) dO_t . (o_sp - o_lin)
      dk_s  = sum_h [ H_s v_s + scale sum_{t : s in S_t} dlogit_{t,s} q_t ]
      dv_s  = sum_h [ H_s^T k_s + sum_{t : s in S_t} p_{t,s} d_sp_t ]
    with S_t = S_0 + K_{0..t}^T V_{0..t} and H_s = dS_out + sum_{t >= s}
    q_t d_lin_t^T (library matmuls), and the softmax weights of a position
    recomputed over its whole set.  Returns dq, dz [B,R,Hq(,d)], dk, dv
    [B,K,G,d]."""
    q, k, v, z, d_out = (np.asarray(x, dtype=np.float64) for x in (q, k, v, z, d_out))
    B, n, Hq, d = q.shape
    G = k.shape[2]
    r = Hq // G
    scale = scale if scale else 1.0 / math.sqrt(d)
    gam = 1.0 / (1.0 + np.exp(-z))
    rows = [int(t) for t in rows]
    keys = [int(s) for s in keys]
    dq = np.zeros((B, len(rows), Hq, d))
    dz = np.zeros((B, len(rows), Hq))
    dk = np.zeros((B, len(keys), G, d))
    dv = np.zeros((B, len(keys), G, d))

    def unit(b, t, h):
        """softmax weights, d logits, o_sp and the set of (b, t, head h)"""
        g = (h * G) // Hq
        sel = np.asarray(idx[b, t, g])
        sel = sel[sel >= 0]
        K, V = k[b, sel, g], v[b, sel, g]
        p = _softmax(scale * (K @ q[b, t, h]))
        d_sp = gam[b, t, h] * d_out[b, t, h]
        dp = V @ d_sp
        return sel, p, p * (dp - float(p @ dp)), p @ V

    def state(b, h, t):
        g = (h * G) // Hq
        S = np.zeros((d, d)) if state_in is None else np.array(state_in[b, h], dtype=np.float64)
        return S + k[b, :t + 1, g].T @ v[b, :t + 1, g]

    for b in range(B):
        for i, t in enumerate(rows):
            for h in range(Hq):
                g = (h * G) // Hq
                sel, p, dlogit, osp = unit(b, t, h)
                S_t = state(b, h, t)
                olin = S_t.T @ q[b, t, h]
                ga = gam[b, t, h]
                dz[b, i, h] = ga * (1.0 - ga) * float(d_out[b, t, h] @ (osp - olin))
                dq[b, i, h] = scale * (dlogit @ k[b, sel, g]) + S_t @ ((1.0 - ga) * d_out[b, t, h])
        for i, s in enumerate(keys):
            for g in range(G):
                users = s + np.nonzero(np.any(np.asarray(idx[b, s:, g]) == s, axis=1))[0]
                for h in range(g * r, (g + 1) * r):
                    d_lin = (1.0 - gam[b, s:, h])[:, None] * d_out[b, s:, h]
                    H = q[b, s:, h].T @ d_lin
                    if d_state_out is not None:
                        H = H + d_state_out[b, h]
                    dk[b, i, g] += H @ v[b, s, g]
                    dv[b, i, g] += H.T @ k[b, s, g]
                    for t in users:
                        sel, p, dlogit, _ = unit(b, t, h)
                        j = int(np.nonzero(sel == s)[0][0])
                        dk[b, i, g] += scale * dlogit[j] * q[b, t, h]
                        dv[b, i, g] += p[j] * gam[b, t, h] * d_out[b, t, h]
    return {"dq": dq, "dz": dz, "dk": dk, "dv": dv}
