"""ctypes wrapper of the fp64 CPU oracle (lisa_oracle.c).

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
baseline of the benchmark; never by the product path.  Shares no code with
the HIP implementation.  Inputs are the stored tensors (bf16 bit patterns or
fp32) which are widened exactly to fp64 here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lisa_oracle.c")
LIB = os.path.join(HERE, "liblisa_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)
_lp = ctypes.POINTER(ctypes.c_long)


def build(src: str = SRC, out: str = LIB, extra: tuple = ()) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics kept, OpenMP)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib_cache: dict = {}


def load(path: str = LIB):
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        if path == LIB:
            build()
        else:
            raise FileNotFoundError(path)
    lib = ctypes.CDLL(path)
    lib.oracle_index_scores.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp,
                                        ctypes.c_long, _dp]
    lib.oracle_index_scores.restype = None
    lib.oracle_topm.argtypes = [ctypes.c_int, _dp, ctypes.c_int, _ip]
    lib.oracle_topm.restype = ctypes.c_int
    lib.oracle_sparse_given_sets.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_double, _dp, _dp, _dp, _lp, _ip,
                                             _dp, _dp, _dp, _dp, ctypes.c_int]
    lib.oracle_prefill.argtypes = [ctypes.c_int] * 8 + [ctypes.c_double] + [_dp] * 8 + \
        [_ip, ctypes.c_int, _dp, _dp, _ip, _dp, _dp, ctypes.c_int]
    lib.oracle_decode.argtypes = [ctypes.c_int, _lp] + [ctypes.c_int] * 6 + [ctypes.c_double] + \
        [_dp] * 8 + [_dp, _dp, _ip, _dp, _dp, ctypes.c_int]
    _lib_cache[path] = lib
    return lib


def _d(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, t):
    return None if a is None else a.ctypes.data_as(t)


def widen(arr, dtype):
    if dtype == "bf16" and arr.dtype == np.uint16:
        return (arr.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def index_scores(qI, w, kI, lib=None):
    """qI [HI,dI], w [HI], kI [T,dI] (fp64) -> scores [T]."""
    lib = lib or load()
    qI, w, kI = _d(qI), _d(w), _d(kI)
    T, dI = kI.shape
    HI = qI.shape[0]
    out = np.zeros(T, dtype=np.float64)
    lib.oracle_index_scores(T, HI, dI, _ptr(qI, _dp), _ptr(w, _dp), _ptr(kI, _dp), dI,
                            _ptr(out, _dp))
    return out


def topm(scores, M, lib=None):
    lib = lib or load()
    s = _d(scores)
    out = np.zeros(M, dtype=np.int32)
    lib.oracle_topm(len(s), _ptr(s, _dp), M, _ptr(out, _ip))
    return out


def prefill(inp: dict, cfg, rows=None, M=None, scale=0.0, state_in=None, nthreads=0, lib=None,
            z_override=None):
    """Oracle prefill on generator inputs.  Returns dict with out, osp, olin
    [B,R,Hq,d], idx [B,R,G,M] and state_out [B,Hq,d,d] (R = len(rows) or n)."""
    lib = lib or load()
    dt = cfg.dtype
    B, n = inp["B"], inp["n"]
    M = cfg.M if M is None else M
    q, k, v = widen(inp["q"], dt), widen(inp["k"], dt), widen(inp["v"], dt)
    qI, kI, w = widen(inp["q_idx"], dt), widen(inp["k_idx"], dt), widen(inp["w_idx"], dt)
    z = widen(inp["gate"], dt) if z_override is None else _d(z_override)
    S0 = None if state_in is None else _d(state_in)
    if rows is not None:
        rows = np.ascontiguousarray(np.unique(np.asarray(rows, dtype=np.int32)))
        R = len(rows)
    else:
        R = n
    Hq, G, d = cfg.Hq, cfg.Hkv, cfg.d
    out = np.zeros((B, R, Hq, d))
    osp = np.zeros((B, R, Hq, d))
    olin = np.zeros((B, R, Hq, d))
    st = np.zeros((B, Hq, d, d))
    idx = np.zeros((B, R, G, M), dtype=np.int32)
    t0 = time.perf_counter()
    lib.oracle_prefill(B, n, Hq, cfg.Hkv, d, cfg.HI, cfg.dI, M, float(scale),
                       _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(qI, _dp), _ptr(kI, _dp),
                       _ptr(w, _dp), _ptr(z, _dp), _ptr(S0, _dp),
                       _ptr(rows, _ip), R, _ptr(out, _dp), _ptr(st, _dp), _ptr(idx, _ip),
                       _ptr(osp, _dp), _ptr(olin, _dp), int(nthreads))
    secs = time.perf_counter() - t0
    return {"out": out, "osp": osp, "olin": olin, "idx": idx, "state_out": st, "rows": rows,
            "seconds": secs}


def decode(inp: dict, cfg, M=None, scale=0.0, nthreads=0, lib=None, z_override=None):
    lib = lib or load()
    dt = cfg.dtype
    B = inp["B"]
    M = cfg.M if M is None else M
    Hq, G, d = cfg.Hq, cfg.Hkv, cfg.d
    cu = np.ascontiguousarray(inp["cu_ctx"], dtype=np.int64)
    q = widen(inp["q"], dt)
    kc, vc = widen(inp["k_cache"], dt), widen(inp["v_cache"], dt)
    qI, kIc, w = widen(inp["q_idx"], dt), widen(inp["k_idx_cache"], dt), widen(inp["w_idx"], dt)
    z = widen(inp["gate"], dt) if z_override is None else _d(z_override)
    S = _d(inp["state"])
    out = np.zeros((B, Hq, d))
    osp = np.zeros((B, Hq, d))
    olin = np.zeros((B, Hq, d))
    st = np.zeros((B, Hq, d, d))
    idx = np.zeros((B, G, M), dtype=np.int32)
    t0 = time.perf_counter()
    lib.oracle_decode(B, _ptr(cu, _lp), Hq, cfg.Hkv, d, cfg.HI, cfg.dI, M, float(scale),
                      _ptr(q, _dp), _ptr(kc, _dp), _ptr(vc, _dp), _ptr(qI, _dp), _ptr(kIc, _dp),
                      _ptr(w, _dp), _ptr(z, _dp), _ptr(S, _dp), _ptr(out, _dp), _ptr(st, _dp),
                      _ptr(idx, _ip), _ptr(osp, _dp), _ptr(olin, _dp), int(nthreads))
    secs = time.perf_counter() - t0
    return {"out": out, "osp": osp, "olin": olin, "idx": idx, "state_out": st, "seconds": secs}


def sparse_given_sets(q, k_rows, v_rows, row0, idx, z, olin, Hq, Hkv, d, M, scale=0.0,
                      nthreads=0, lib=None):
    """Sparse branch + gate for U units with given sets.  q [U,Hq,d];
    k_rows/v_rows [R,Hkv,d]; row0 [U] first key row of each unit; idx [U,G,M];
    z [U,Hq]; olin [U,Hq,d].  Returns (out, osp) [U,Hq,d]."""
    lib = lib or load()
    q, kr, vr, z, olin = _d(q), _d(k_rows), _d(v_rows), _d(z), _d(olin)
    row0 = np.ascontiguousarray(row0, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    U = q.shape[0]
    out = np.zeros((U, Hq, d))
    osp = np.zeros((U, Hq, d))
    lib.oracle_sparse_given_sets(U, Hq, Hkv, d, M, float(scale), _ptr(q, _dp), _ptr(kr, _dp),
                                 _ptr(vr, _dp), _ptr(row0, _lp), _ptr(idx, _ip), _ptr(z, _dp),
                                 _ptr(olin, _dp), _ptr(out, _dp), _ptr(osp, _dp), int(nthreads))
    return out, osp
