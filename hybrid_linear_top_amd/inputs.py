"""Seeded synthetic inputs for the LISA layer (prefill and decode).

This module only draws random numbers and rounds them to the storage
precision; it contains none of the layer's arithmetic.  Both the HIP path
(through the Python binding) and the fp64 CPU oracle are fed from here.

Workload recipe (the shapes are the Qwen2.5 attention shapes the LISA pages
name as host models: arxivdaily page for arXiv 2607.19358, English abstract,
"DeepSeek-distilled-Qwen"; gptget.net analysis, experiment-design section,
"Qwen-2.5 series", M = 256):

* generator: ``numpy.random.Generator(PCG64(seed))``, default seed 1000 + id;
* draw order: ragged context lengths (ragged decode only), then q, k, v, q_I,
  k_I, w, z, and the decode-time linear state S;
* every tensor is drawn as float32 (``standard_normal``/``random`` with
  ``dtype=float32``), scaled in float32, then rounded once to bf16 with
  round-to-nearest-even where the configuration is bf16;
* q, k, v ~ N(0,1)/sqrt(d); q_I, k_I ~ N(0,1); w ~ U(0,1); z ~ N(0,1);
  (test cases for negative indexer scores map the same uniform draw u to
  w = 2u - 1 ~ U(-1,1) or w = u - 1 ~ U(-1,0));
  decode state S ~ N(0,1) * sqrt(L_b) / d (the magnitude a zero-start
  prefill of L_b tokens at this input scale produces).

Storage formats: bf16 tensors are ``numpy.uint16`` bit patterns, fp32 tensors
are ``numpy.float32``; the linear state is always fp32.
"""
from __future__ import annotations

import dataclasses
import numpy as np

DT_F32 = 0
DT_BF16 = 1


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    mode: str            # "prefill" or "decode"
    dtype: str           # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    d: int
    HI: int
    dI: int
    M: int
    chunk: int = 64
    n: int = 0           # prefill length
    ctx: int = 0         # decode: cached tokens per sequence (fixed lengths)
    ctx_lo: int = 0      # decode: ragged lengths drawn U[ctx_lo, ctx_hi]
    ctx_hi: int = 0
    seed: int = 1000
    w_dist: str = "u01"  # indexer head weights: "u01" U(0,1), "signed" U(-1,1), "neg" U(-1,0)

    @property
    def dtype_code(self) -> int:
        return DT_BF16 if self.dtype == "bf16" else DT_F32


# The five workloads: a tiny fp32 correctness case; Qwen2.5-1.5B-shaped
# prefill at 4K; 1.5B-shaped decode at 16K context; Qwen2.5-7B-shaped
# prefill at 16K; 7B-shaped ragged decode, 4K..32K context, M = 512.
TINY_F32_PREFILL = LayerConfig("tiny_fp32_prefill_n512", "prefill", "f32", B=1, n=512, Hq=1, Hkv=1,
                               d=64, HI=4, dI=32, M=64, chunk=64, seed=1000)
PREFILL_1P5B_4K = LayerConfig("qwen2.5-1.5b_prefill_n4096", "prefill", "bf16", B=1, n=4096, Hq=12,
                              Hkv=2, d=128, HI=4, dI=64, M=256, chunk=64, seed=1001)
DECODE_1P5B_16K = LayerConfig("qwen2.5-1.5b_decode_b16_ctx16k", "decode", "bf16", B=16, ctx=16384,
                              Hq=12, Hkv=2, d=128, HI=4, dI=64, M=256, seed=1002)
PREFILL_7B_16K = LayerConfig("qwen2.5-7b_prefill_n16384", "prefill", "bf16", B=1, n=16384, Hq=28,
                             Hkv=4, d=128, HI=4, dI=64, M=256, chunk=64, seed=1003)
DECODE_7B_RAGGED = LayerConfig("qwen2.5-7b_ragged_decode_b32_ctx4k-32k", "decode", "bf16", B=32,
                               ctx_lo=4096, ctx_hi=32768, Hq=28, Hkv=4, d=128, HI=4, dI=64, M=512,
                               seed=1004)
WORKLOADS: dict[str, LayerConfig] = {c.name: c for c in (
    TINY_F32_PREFILL, PREFILL_1P5B_4K, DECODE_1P5B_16K, PREFILL_7B_16K, DECODE_7B_RAGGED)}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a stored tensor to float64."""
    if dtype == "bf16" and arr.dtype == np.uint16:
        return bf16_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _weights(rng, shape, cfg):
    u = rng.random(shape, dtype=np.float32)
    if cfg.w_dist == "signed":
        u = u * np.float32(2) - np.float32(1)
    elif cfg.w_dist == "neg":
        u = u - np.float32(1)
    elif cfg.w_dist != "u01":
        raise ValueError(f"unknown w_dist {cfg.w_dist!r}")
    return _store(u, cfg.dtype)


def _normal(rng, shape, scale, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return _store(x, dtype)


def decode_lengths(cfg: LayerConfig, rng=None) -> np.ndarray:
    """Visible lengths L_b (cached tokens + the one new token)."""
    if cfg.ctx_hi:
        if rng is None:
            rng = np.random.Generator(np.random.PCG64(cfg.seed))
        cached = rng.integers(cfg.ctx_lo, cfg.ctx_hi, size=cfg.B, endpoint=True)
    else:
        cached = np.full(cfg.B, cfg.ctx, dtype=np.int64)
    return cached.astype(np.int64) + 1


def make_prefill_inputs(cfg: LayerConfig, seed: int | None = None, n: int | None = None,
                        B: int | None = None) -> dict:
    """Prefill inputs in the layouts the library takes (all row-major):
    q [B,n,Hq,d], k/v [B,n,Hkv,d], q_idx [B,n,G,HI,dI], k_idx [B,n,G,dI],
    w_idx [B,n,G,HI], gate [B,n,Hq]  (G = Hkv)."""
    seed = cfg.seed if seed is None else seed
    n = cfg.n if n is None else n
    B = cfg.B if B is None else B
    rng = np.random.Generator(np.random.PCG64(seed))
    G, dt = cfg.Hkv, cfg.dtype
    s = 1.0 / np.sqrt(cfg.d)
    out = {
        "q": _normal(rng, (B, n, cfg.Hq, cfg.d), s, dt),
        "k": _normal(rng, (B, n, cfg.Hkv, cfg.d), s, dt),
        "v": _normal(rng, (B, n, cfg.Hkv, cfg.d), s, dt),
        "q_idx": _normal(rng, (B, n, G, cfg.HI, cfg.dI), 1.0, dt),
        "k_idx": _normal(rng, (B, n, G, cfg.dI), 1.0, dt),
        "w_idx": _weights(rng, (B, n, G, cfg.HI), cfg),
        "gate": _normal(rng, (B, n, cfg.Hq), 1.0, dt),
    }
    out["B"], out["n"] = B, n
    return out


def make_decode_inputs(cfg: LayerConfig, seed: int | None = None, B: int | None = None,
                       lengths: np.ndarray | None = None) -> dict:
    """Decode inputs: packed token-major caches whose last row per sequence is
    the new token.  cu_ctx [B+1] int64; q [B,Hq,d]; k_cache/v_cache
    [sum L, Hkv, d]; q_idx [B,G,HI,dI]; k_idx_cache [sum L, G, dI];
    w_idx [B,G,HI]; gate [B,Hq]; state [B,Hq,d,d] fp32 (row = key dim)."""
    seed = cfg.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    if lengths is None:
        L = decode_lengths(cfg, rng)
        if B is not None:
            L = L[:B]
    else:
        L = np.asarray(lengths, dtype=np.int64)
    B = len(L)
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(L)
    tot = int(cu[-1])
    G, dt = cfg.Hkv, cfg.dtype
    s = 1.0 / np.sqrt(cfg.d)
    out = {
        "q": _normal(rng, (B, cfg.Hq, cfg.d), s, dt),
        "k_cache": _normal(rng, (tot, cfg.Hkv, cfg.d), s, dt),
        "v_cache": _normal(rng, (tot, cfg.Hkv, cfg.d), s, dt),
        "q_idx": _normal(rng, (B, G, cfg.HI, cfg.dI), 1.0, dt),
        "k_idx_cache": _normal(rng, (tot, G, cfg.dI), 1.0, dt),
        "w_idx": _weights(rng, (B, G, cfg.HI), cfg),
        "gate": _normal(rng, (B, cfg.Hq), 1.0, dt),
    }
    st = rng.standard_normal((B, cfg.Hq, cfg.d, cfg.d), dtype=np.float32)
    st *= (np.sqrt(L.astype(np.float32)) / np.float32(cfg.d))[:, None, None, None]
    out["state"] = np.ascontiguousarray(st, dtype=np.float32)
    out["cu_ctx"] = cu
    out["lengths"] = L
    out["B"] = B
    out["max_ctx"] = int(L.max()) if B else 0
    return out


def make_backward_inputs(cfg: LayerConfig, seed: int | None = None, with_states: bool = True) -> dict:
    """Upstream gradients for the backward pass: d_out [B,n,Hq,d] in the layer
    dtype, d_state_out and an initial state [B,Hq,d,d] fp32 (or None)."""
    seed = (cfg.seed if seed is None else seed) + 1000
    rng = np.random.Generator(np.random.PCG64(seed))
    B, n, d = cfg.B, cfg.n, cfg.d
    out = {"d_out": _normal(rng, (B, n, cfg.Hq, d), 1.0, cfg.dtype), "d_state_out": None, "state_in": None}
    if with_states:
        out["d_state_out"] = (rng.standard_normal((B, cfg.Hq, d, d), dtype=np.float32) * 0.1).astype(np.float32)
        out["state_in"] = (rng.standard_normal((B, cfg.Hq, d, d), dtype=np.float32) * 0.1).astype(np.float32)
    return out
