"""Python binding of liblisa.so (the gfx950 HIP library behind include/lisa.h).

The functions named like the C ABI (``lisa_prefill``, ``lisa_decode_step``,
...) only marshal arguments: every step of the layer runs in the library's
kernels.  ``prefill`` / ``decode_step`` are conveniences that take torch
device tensors and allocate outputs and the workspace with torch (memory
plumbing only).  Importing this module fails if the library is not built:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblisa.so")

LISA_OK = 0
LISA_ERR_INVALID_ARGUMENT = 1
LISA_ERR_UNSUPPORTED = 2
LISA_ERR_WORKSPACE = 3
LISA_ERR_HIP = 4
LISA_F32 = 0
LISA_BF16 = 1

EXPORTS = ["lisa_prefill_workspace_bytes", "lisa_prefill_continue_workspace_bytes", "lisa_prefill",
           "lisa_prefill_continue",
           "lisa_prefill_window", "lisa_decode_step_window", "lisa_decode_step_paged",
           "lisa_decode_workspace_bytes", "lisa_prefill_backward_workspace_bytes",
           "lisa_prefill_backward",
           "lisa_decode_step", "lisa_decode_step_noalloc", "lisa_peak_probe", "lisa_stage_timing", "lisa_stage_timing_read", "lisa_last_error",
           "lisa_build_info"]


class LisaDims(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("idx_heads", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("top_m", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


class LisaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"LISA status {status}: {message}")
        self.status = status
        self.message = message


# Tests set this to fill every buffer the binding allocates (outputs and
# workspaces) with a poison pattern before the call, so that an element the
# library fails to write shows up: 0xFF bytes (NaN) for floating-point and
# workspace bytes, 0x7F bytes for int32 sets (-1 is their padding value).
POISON_FRESH_BUFFERS = False


def _fresh(t):
    if POISON_FRESH_BUFFERS:
        import torch
        t.view(torch.uint8).fill_(0x7F if t.dtype == torch.int32 else 0xFF)
    return t


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m hybrid_linear_top_amd.build`")
    # torch carries its own HIP and HSA runtimes; they must be in the process
    # before the library's ROCm ones.  Loaded the other way round (library
    # first, torch later), the library's launches found no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, sz, i32, i64p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p
    dp = ctypes.POINTER(LisaDims)
    lib.lisa_prefill_workspace_bytes.argtypes = [dp, i32, i32, ctypes.POINTER(sz)]
    lib.lisa_prefill_workspace_bytes.restype = ctypes.c_int
    lib.lisa_prefill_continue_workspace_bytes.argtypes = [dp, i32, i32, i32, ctypes.POINTER(sz)]
    lib.lisa_prefill_continue_workspace_bytes.restype = ctypes.c_int
    lib.lisa_prefill.argtypes = [dp, i32, i32] + [vp] * 7 + [vp, vp, vp, vp, vp, sz, vp]
    lib.lisa_prefill.restype = ctypes.c_int
    lib.lisa_prefill_continue.argtypes = [dp, i32, i32, i32] + [vp] * 7 + [vp, vp, vp, vp, vp, sz, vp]
    lib.lisa_prefill_continue.restype = ctypes.c_int
    lib.lisa_prefill_window.argtypes = [dp, i32, i32, i32] + [vp] * 4 + [vp, vp, vp, vp, sz, vp]
    lib.lisa_prefill_window.restype = ctypes.c_int
    lib.lisa_decode_step_window.argtypes = [dp, i32, i64p, i32] + [vp] * 4 + [vp, vp, vp, sz, vp]
    lib.lisa_decode_step_window.restype = ctypes.c_int
    lib.lisa_decode_step_paged.argtypes = [dp, i32, vp, vp, i32, i32, i32, i32] + [vp] * 7 + \
        [vp, vp, vp, vp, sz, vp]
    lib.lisa_decode_step_paged.restype = ctypes.c_int
    lib.lisa_prefill_backward_workspace_bytes.argtypes = [dp, i32, i32, ctypes.POINTER(sz)]
    lib.lisa_prefill_backward_workspace_bytes.restype = ctypes.c_int
    lib.lisa_prefill_backward.argtypes = [dp, i32, i32] + [vp] * 4 + [vp, vp, vp, vp] + [vp] * 5 + \
        [vp, sz, vp]
    lib.lisa_prefill_backward.restype = ctypes.c_int
    lib.lisa_decode_workspace_bytes.argtypes = [dp, i32, i32, ctypes.POINTER(sz)]
    lib.lisa_decode_workspace_bytes.restype = ctypes.c_int
    lib.lisa_decode_step.argtypes = [dp, i32, i64p, i32] + [vp] * 7 + [vp, vp, vp, vp, sz, vp]
    lib.lisa_decode_step.restype = ctypes.c_int
    lib.lisa_decode_step_noalloc.argtypes = [dp, i32, i64p, i32] + [vp] * 7 + [vp, vp, vp, vp]
    lib.lisa_decode_step_noalloc.restype = ctypes.c_int
    lib.lisa_peak_probe.argtypes = [i32, vp, vp, sz, i32, ctypes.POINTER(ctypes.c_double), vp]
    lib.lisa_peak_probe.restype = ctypes.c_int
    lib.lisa_stage_timing.argtypes = [i32]
    lib.lisa_stage_timing.restype = ctypes.c_int
    lib.lisa_stage_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p),
                                           ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_int32), i32]
    lib.lisa_stage_timing_read.restype = ctypes.c_int
    lib.lisa_last_error.argtypes = []
    lib.lisa_last_error.restype = ctypes.c_char_p
    lib.lisa_build_info.argtypes = []
    lib.lisa_build_info.restype = ctypes.c_char_p
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != LISA_OK:
        raise LisaError(status, _lib.lisa_last_error().decode())


# ---- C-ABI-named wrappers (pointers are Python ints, 0 = NULL) -------------
def lisa_last_error() -> str:
    return _lib.lisa_last_error().decode()


def lisa_build_info() -> str:
    return _lib.lisa_build_info().decode()


def lisa_prefill_continue_workspace_bytes(dims: LisaDims, B: int, past: int, n: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.lisa_prefill_continue_workspace_bytes(ctypes.byref(dims), B, past, n, ctypes.byref(out)))
    return out.value


def lisa_prefill_backward_workspace_bytes(dims: LisaDims, B: int, n: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.lisa_prefill_backward_workspace_bytes(ctypes.byref(dims), B, n, ctypes.byref(out)))
    return out.value


def lisa_prefill_backward(dims, B, n, q, k, v, gate, state_in, topm, d_out, d_state_out, dq, dk, dv,
                          dgate, d_state_in, workspace, workspace_bytes, stream) -> int:
    """Raw call; returns the status code (0 = LISA_OK)."""
    return _lib.lisa_prefill_backward(ctypes.byref(dims), B, n, q, k, v, gate, state_in, topm, d_out,
                                      d_state_out, dq, dk, dv, dgate, d_state_in, workspace,
                                      workspace_bytes, stream)


def lisa_prefill_workspace_bytes(dims: LisaDims, B: int, n: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.lisa_prefill_workspace_bytes(ctypes.byref(dims), B, n, ctypes.byref(out)))
    return out.value


def lisa_decode_workspace_bytes(dims: LisaDims, B: int, max_ctx: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.lisa_decode_workspace_bytes(ctypes.byref(dims), B, max_ctx, ctypes.byref(out)))
    return out.value


def lisa_prefill(dims, B, n, q, k, v, q_idx, k_idx, w_idx, gate, state_in, out, state_out,
                 topm_out, workspace, workspace_bytes, stream) -> int:
    """Raw call; returns the status code (0 = LISA_OK)."""
    return _lib.lisa_prefill(ctypes.byref(dims), B, n, q, k, v, q_idx, k_idx, w_idx, gate,
                             state_in, out, state_out, topm_out, workspace, workspace_bytes, stream)


def lisa_prefill_continue(dims, B, past, n, q, k_cache, v_cache, q_idx, k_idx_cache, w_idx, gate,
                          state_in, out, state_out, topm_out, workspace, workspace_bytes,
                          stream) -> int:
    """Raw call; returns the status code (0 = LISA_OK)."""
    return _lib.lisa_prefill_continue(ctypes.byref(dims), B, past, n, q, k_cache, v_cache, q_idx,
                                      k_idx_cache, w_idx, gate, state_in, out, state_out, topm_out,
                                      workspace, workspace_bytes, stream)


def lisa_prefill_window(dims, B, past, n, q, k_cache, v_cache, gate, state_in, out, state_out,
                        workspace, workspace_bytes, stream) -> int:
    """Raw call; returns the status code (0 = LISA_OK)."""
    return _lib.lisa_prefill_window(ctypes.byref(dims), B, past, n, q, k_cache, v_cache, gate,
                                    state_in, out, state_out, workspace, workspace_bytes, stream)


def lisa_decode_step_window(dims, B, cu_ctx, max_ctx, q, k_cache, v_cache, gate, state, out,
                            workspace, workspace_bytes, stream) -> int:
    """Raw call; returns the status code (0 = LISA_OK)."""
    return _lib.lisa_decode_step_window(ctypes.byref(dims), B, cu_ctx, max_ctx, q, k_cache, v_cache,
                                        gate, state, out, workspace, workspace_bytes, stream)


def lisa_decode_step_paged(dims, B, lengths, block_table, block_size, max_blocks, num_pages, max_ctx,
                           q, k_pages, v_pages, q_idx, k_idx_pages, w_idx, gate, state, out,
                           topm_out, workspace, workspace_bytes, stream) -> int:
    """Raw call; returns the status code (0 = LISA_OK)."""
    return _lib.lisa_decode_step_paged(ctypes.byref(dims), B, lengths, block_table, block_size,
                                       max_blocks, num_pages, max_ctx, q, k_pages, v_pages, q_idx,
                                       k_idx_pages, w_idx, gate, state, out, topm_out, workspace,
                                       workspace_bytes, stream)


def lisa_decode_step(dims, B, cu_ctx, max_ctx, q, k_cache, v_cache, q_idx, k_idx_cache, w_idx,
                     gate, state, out, topm_out, workspace, workspace_bytes, stream) -> int:
    """Raw call; returns the status code (0 = LISA_OK)."""
    return _lib.lisa_decode_step(ctypes.byref(dims), B, cu_ctx, max_ctx, q, k_cache, v_cache,
                                 q_idx, k_idx_cache, w_idx, gate, state, out, topm_out, workspace,
                                 workspace_bytes, stream)


def lisa_decode_step_noalloc(dims, B, cu_ctx, max_ctx, q, k_cache, v_cache, q_idx, k_idx_cache,
                             w_idx, gate, state, out, topm_out, stream) -> int:
    """Raw call; returns the status code (0 = LISA_OK)."""
    return _lib.lisa_decode_step_noalloc(ctypes.byref(dims), B, cu_ctx, max_ctx, q, k_cache, v_cache,
                                         q_idx, k_idx_cache, w_idx, gate, state, out, topm_out, stream)


LISA_PROBE_COPY = 0
LISA_PROBE_MFMA = 1
LISA_PROBE_READ = 2
LISA_PROBE_GATHER = 3


def peak_probe(kind: int, src, dst, nbytes: int, iters: int = 0, stream=None) -> float:
    """Enqueue a calibration kernel (lisa_peak_probe); returns its work (bytes
    moved or flops)."""
    work = ctypes.c_double(0.0)
    st = _lib.lisa_peak_probe(kind, 0 if src is None else _ptr(src), _ptr(dst), int(nbytes), int(iters),
                              ctypes.byref(work), _stream(stream))
    if st != LISA_OK:
        raise LisaError(st, f"lisa_peak_probe(kind={kind}) failed")
    return work.value


def lisa_stage_timing(enable: bool) -> None:
    _check(_lib.lisa_stage_timing(1 if enable else 0))


def lisa_stage_timing_read(reset: bool = True) -> dict:
    """{stage name: (launches, total_ms)} for every stage with launches."""
    N = 32
    names = (ctypes.c_char_p * N)()
    launches = (ctypes.c_int64 * N)()
    total = (ctypes.c_double * N)()
    n = ctypes.c_int32(0)
    _check(_lib.lisa_stage_timing_read(N, names, launches, total, ctypes.byref(n), 1 if reset else 0))
    return {names[i].decode(): (int(launches[i]), float(total[i])) for i in range(n.value)
            if launches[i] > 0}


# ---- torch conveniences ---------------------------------------------------
def make_dims(Hq, Hkv, d, HI, dI, M, dtype, chunk=64, softmax_scale=0.0) -> LisaDims:
    code = dtype if isinstance(dtype, int) else (LISA_BF16 if dtype == "bf16" else LISA_F32)
    return LisaDims(Hq, Hkv, d, HI, dI, M, chunk, softmax_scale, code)


def dims_from_config(cfg, softmax_scale=0.0) -> LisaDims:
    return make_dims(cfg.Hq, cfg.Hkv, cfg.d, cfg.HI, cfg.dI, cfg.M, cfg.dtype, cfg.chunk,
                     softmax_scale)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    return int(getattr(stream, "cuda_stream", stream))


def prefill(dims: LisaDims, q, k, v, q_idx, k_idx, w_idx, gate, state_in=None, out=None,
            state_out=None, topm_out=None, workspace=None, stream=None):
    """q [B,n,Hq,d] etc. as torch device tensors.  Allocates missing outputs.
    Returns (out, state_out, topm_out)."""
    import torch
    B, n = int(q.shape[0]), int(q.shape[1])
    dev = q.device
    if out is None:
        out = _fresh(torch.empty_like(q))
    if state_out is None:
        state_out = _fresh(torch.empty((B, dims.num_q_heads, dims.head_dim, dims.head_dim),
                                dtype=torch.float32, device=dev))
    if topm_out is None:
        topm_out = _fresh(torch.empty((B, n, dims.num_kv_heads, dims.top_m), dtype=torch.int32, device=dev))
    wsb = lisa_prefill_workspace_bytes(dims, B, n)
    if workspace is None:
        workspace = _fresh(torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev))
    _check(lisa_prefill(dims, B, n, _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx),
                        _ptr(w_idx), _ptr(gate), _ptr(state_in), _ptr(out), _ptr(state_out),
                        _ptr(topm_out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, state_out, topm_out


def prefill_continue(dims: LisaDims, past: int, q, k_cache, v_cache, q_idx, k_idx_cache, w_idx,
                     gate, state_in=None, out=None, state_out=None, topm_out=None,
                     workspace=None, stream=None):
    """n new tokens against caches of past + n rows (torch device tensors;
    q [B,n,Hq,d], k_cache [B,past+n,Hkv,d], ...).  Allocates missing outputs.
    Returns (out, state_out, topm_out)."""
    import torch
    B, n = int(q.shape[0]), int(q.shape[1])
    dev = q.device
    if out is None:
        out = _fresh(torch.empty_like(q))
    if state_out is None:
        state_out = _fresh(torch.empty((B, dims.num_q_heads, dims.head_dim, dims.head_dim),
                                dtype=torch.float32, device=dev))
    if topm_out is None:
        topm_out = _fresh(torch.empty((B, n, dims.num_kv_heads, dims.top_m), dtype=torch.int32, device=dev))
    wsb = lisa_prefill_continue_workspace_bytes(dims, B, past, n)
    if workspace is None:
        workspace = _fresh(torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev))
    _check(lisa_prefill_continue(dims, B, past, n, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(q_idx), _ptr(k_idx_cache), _ptr(w_idx), _ptr(gate),
                                 _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(topm_out),
                                 _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, state_out, topm_out


def prefill_window(dims: LisaDims, past: int, q, k_cache, v_cache, gate, state_in=None, out=None,
                   state_out=None, workspace=None, stream=None):
    """Sliding-window prefill of n new tokens against caches of past + n rows.
    Returns (out, state_out)."""
    import torch
    B, n = int(q.shape[0]), int(q.shape[1])
    dev = q.device
    if out is None:
        out = _fresh(torch.empty_like(q))
    if state_out is None:
        state_out = _fresh(torch.empty((B, dims.num_q_heads, dims.head_dim, dims.head_dim),
                                dtype=torch.float32, device=dev))
    wsb = lisa_prefill_workspace_bytes(dims, B, n)
    if workspace is None:
        workspace = _fresh(torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev))
    _check(lisa_prefill_window(dims, B, past, n, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(gate),
                               _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(workspace),
                               workspace.numel(), _stream(stream)))
    return out, state_out


def decode_step_window(dims: LisaDims, cu_ctx, max_ctx: int, q, k_cache, v_cache, gate, state,
                       out=None, workspace=None, stream=None):
    """Sliding-window decode step; `state` is updated in place.  Returns out."""
    import torch
    B = int(q.shape[0])
    if out is None:
        out = _fresh(torch.empty_like(q))
    wsb = lisa_decode_workspace_bytes(dims, B, max_ctx)
    if workspace is None:
        workspace = _fresh(torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device))
    _check(lisa_decode_step_window(dims, B, _ptr(cu_ctx), max_ctx, _ptr(q), _ptr(k_cache),
                                   _ptr(v_cache), _ptr(gate), _ptr(state), _ptr(out),
                                   _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def prefill_backward(dims: LisaDims, q, k, v, gate, topm, d_out, state_in=None, d_state_out=None,
                     want_state_grad=False, workspace=None, stream=None):
    """Gradients of <d_out, out> + <d_state_out, state_out> (torch device
    tensors as for prefill; topm the forward's sets).  Returns (dq, dk, dv,
    dgate, d_state_in or None), all fp32."""
    import torch
    B, n = int(q.shape[0]), int(q.shape[1])
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    dq = _fresh(torch.empty(tuple(q.shape), **f32))
    dk = _fresh(torch.empty(tuple(k.shape), **f32))
    dv = _fresh(torch.empty(tuple(v.shape), **f32))
    dgate = _fresh(torch.empty(tuple(gate.shape), **f32))
    dsi = _fresh(torch.empty((B, dims.num_q_heads, dims.head_dim, dims.head_dim), **f32)) if want_state_grad else None
    wsb = lisa_prefill_backward_workspace_bytes(dims, B, n)
    if workspace is None:
        workspace = _fresh(torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev))
    _check(lisa_prefill_backward(dims, B, n, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(state_in),
                                 _ptr(topm), _ptr(d_out), _ptr(d_state_out), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(dgate), _ptr(dsi), _ptr(workspace), workspace.numel(),
                                 _stream(stream)))
    return dq, dk, dv, dgate, dsi


def decode_step_paged(dims: LisaDims, lengths, block_table, block_size: int, max_ctx: int, q, k_pages,
                      v_pages, q_idx, k_idx_pages, w_idx, gate, state, out=None, topm_out=None,
                      workspace=None, stream=None):
    """Decode step on page pools (torch device tensors; lengths [B] int32,
    block_table [B, max_blocks] int32, pools [num_pages*block_size, ...]).
    `state` is updated in place.  Returns (out, topm_out)."""
    import torch
    B = int(q.shape[0])
    max_blocks = int(block_table.shape[1])
    num_pages = int(k_pages.shape[0]) // block_size
    if out is None:
        out = _fresh(torch.empty_like(q))
    if topm_out is None:
        topm_out = _fresh(torch.empty((B, dims.num_kv_heads, dims.top_m), dtype=torch.int32, device=q.device))
    wsb = lisa_decode_workspace_bytes(dims, B, max_ctx)
    if workspace is None:
        workspace = _fresh(torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device))
    _check(lisa_decode_step_paged(dims, B, _ptr(lengths), _ptr(block_table), block_size, max_blocks,
                                  num_pages, max_ctx, _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                  _ptr(q_idx), _ptr(k_idx_pages), _ptr(w_idx), _ptr(gate),
                                  _ptr(state), _ptr(out), _ptr(topm_out), _ptr(workspace),
                                  workspace.numel(), _stream(stream)))
    return out, topm_out


def decode_step(dims: LisaDims, cu_ctx, max_ctx: int, q, k_cache, v_cache, q_idx, k_idx_cache,
                w_idx, gate, state, out=None, topm_out=None, workspace=None, stream=None):
    """One decode step; `state` is updated in place.  Returns (out, topm_out)."""
    import torch
    B = int(q.shape[0])
    dev = q.device
    if out is None:
        out = _fresh(torch.empty_like(q))
    if topm_out is None:
        topm_out = _fresh(torch.empty((B, dims.num_kv_heads, dims.top_m), dtype=torch.int32, device=dev))
    wsb = lisa_decode_workspace_bytes(dims, B, max_ctx)
    if workspace is None:
        workspace = _fresh(torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev))
    _check(lisa_decode_step(dims, B, _ptr(cu_ctx), int(max_ctx), _ptr(q), _ptr(k_cache),
                            _ptr(v_cache), _ptr(q_idx), _ptr(k_idx_cache), _ptr(w_idx), _ptr(gate),
                            _ptr(state), _ptr(out), _ptr(topm_out), _ptr(workspace),
                            workspace.numel(), _stream(stream)))
    return out, topm_out


def to_device(arr, device="cuda"):
    """numpy storage array (uint16 bf16 bits / float32 / int) -> torch tensor."""
    import numpy as np
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def from_device(t):
    """torch tensor -> numpy storage array (bf16 as uint16 bits)."""
    import numpy as np
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
