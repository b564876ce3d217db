"""C-ABI boundary checks that need no GPU: the library loads, exports every
symbol include/lisa.h declares, and rejects bad arguments with the
documented status before any HIP call."""
import ctypes
import os
import re

import pytest

from hybrid_linear_top_amd import lisa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced on error paths


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "lisa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(lisa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(lisa.LIB_PATH)
    declared = _declared_symbols()
    assert set(declared) == set(lisa.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def _declared_param_counts():
    with open(os.path.join(ROOT, "include", "lisa.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(lisa_[a-z_]+)\s*\(([^;{]*?)\)\s*;", text):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argument_counts_match_header():
    """Every ctypes prototype has as many arguments as the C declaration."""
    counts = _declared_param_counts()
    lib = lisa._lib
    for name in lisa.EXPORTS:
        fn = getattr(lib, name)
        assert fn.argtypes is not None, name
        assert len(fn.argtypes) == counts[name], (name, len(fn.argtypes), counts[name])


def test_build_info_names_target():
    assert "gfx950" in lisa.lisa_build_info()


def _dims(**kw):
    base = dict(Hq=12, Hkv=2, d=128, HI=4, dI=64, M=256, dtype="bf16")
    base.update(kw)
    return lisa.make_dims(base["Hq"], base["Hkv"], base["d"], base["HI"], base["dI"], base["M"],
                          base["dtype"], chunk=base.get("chunk", 64))


def _prefill(d, B=1, n=64, ws_bytes=1 << 40, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, q_idx=FAKE, k_idx=FAKE, w_idx=FAKE, gate=FAKE, state_in=0,
             out=FAKE, state_out=0, topm_out=0, workspace=FAKE)
    p.update(ptrs)
    return lisa.lisa_prefill(d, B, n, p["q"], p["k"], p["v"], p["q_idx"], p["k_idx"], p["w_idx"],
                             p["gate"], p["state_in"], p["out"], p["state_out"], p["topm_out"],
                             p["workspace"], ws_bytes, 0)


def _decode(d, B=2, max_ctx=100, ws_bytes=1 << 40, **ptrs):
    p = dict(cu=FAKE, q=FAKE, kc=FAKE, vc=FAKE, q_idx=FAKE, kic=FAKE, w_idx=FAKE, gate=FAKE,
             state=FAKE, out=FAKE, topm_out=0, workspace=FAKE)
    p.update(ptrs)
    return lisa.lisa_decode_step(d, B, p["cu"], max_ctx, p["q"], p["kc"], p["vc"], p["q_idx"],
                                 p["kic"], p["w_idx"], p["gate"], p["state"], p["out"],
                                 p["topm_out"], p["workspace"], ws_bytes, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), lisa.LISA_ERR_INVALID_ARGUMENT),
    (dict(Hq=12, Hkv=5), lisa.LISA_ERR_INVALID_ARGUMENT),
    (dict(Hq=0), lisa.LISA_ERR_INVALID_ARGUMENT),
    (dict(Hq=34, Hkv=2), lisa.LISA_ERR_UNSUPPORTED),
    (dict(d=96), lisa.LISA_ERR_UNSUPPORTED),
    (dict(dI=48), lisa.LISA_ERR_UNSUPPORTED),
    (dict(HI=0), lisa.LISA_ERR_UNSUPPORTED),
    (dict(HI=9), lisa.LISA_ERR_UNSUPPORTED),
    (dict(M=0), lisa.LISA_ERR_INVALID_ARGUMENT),
    (dict(M=513), lisa.LISA_ERR_UNSUPPORTED),
    (dict(chunk=32), lisa.LISA_ERR_UNSUPPORTED),
])
def test_prefill_rejects_bad_dims(kw, status):
    assert _prefill(_dims(**kw)) == status
    assert lisa.lisa_last_error() != ""


def test_decode_accepts_larger_topm_than_prefill():
    d = _dims(M=2048)
    assert lisa.lisa_decode_workspace_bytes(d, 4, 4096) > 0
    assert _prefill(d) == lisa.LISA_ERR_UNSUPPORTED
    assert _decode(_dims(M=2049)) == lisa.LISA_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["q", "k", "v", "q_idx", "k_idx", "w_idx", "gate", "out", "workspace"])
def test_prefill_null_pointer(name):
    assert _prefill(_dims(), **{name: 0}) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert name in lisa.lisa_last_error()


@pytest.mark.parametrize("name", ["q", "gate", "out", "state_in", "topm_out"])
def test_prefill_misaligned_pointer(name):
    assert _prefill(_dims(), **{name: FAKE + 8}) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert "aligned" in lisa.lisa_last_error()


def test_prefill_workspace_too_small():
    d = _dims()
    need = lisa.lisa_prefill_workspace_bytes(d, 1, 64)
    assert _prefill(d, ws_bytes=need - 1) == lisa.LISA_ERR_WORKSPACE
    assert str(need) in lisa.lisa_last_error()


def test_prefill_empty_is_noop():
    d = _dims()
    assert _prefill(d, B=0, q=0, k=0, workspace=0) == lisa.LISA_OK
    assert _prefill(d, n=0, q=0, k=0, workspace=0) == lisa.LISA_OK
    assert _prefill(d, n=-1) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _prefill(d, n=40000) == lisa.LISA_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["cu", "q", "kc", "vc", "q_idx", "kic", "w_idx", "gate", "state",
                                  "out", "workspace"])
def test_decode_null_pointer(name):
    assert _decode(_dims(), **{name: 0}) == lisa.LISA_ERR_INVALID_ARGUMENT


def test_decode_argument_errors():
    d = _dims()
    assert _decode(d, cu=FAKE + 4) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _decode(d, max_ctx=0) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _decode(d, max_ctx=65537) == lisa.LISA_ERR_UNSUPPORTED
    assert _decode(d, B=-1) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _decode(d, B=0, q=0) == lisa.LISA_OK
    need = lisa.lisa_decode_workspace_bytes(d, 2, 100)
    assert _decode(d, ws_bytes=need - 1) == lisa.LISA_ERR_WORKSPACE


def test_workspace_sizes():
    d = _dims()
    # decode: fp32 scores per (sequence, group, position) dominate
    assert lisa.lisa_decode_workspace_bytes(d, 16, 16385) >= 16 * 2 * 16385 * 4
    a = lisa.lisa_prefill_workspace_bytes(d, 1, 4096)
    b = lisa.lisa_prefill_workspace_bytes(d, 1, 8192)
    assert b > a > 4096 * 2 * 256 * 4
    with pytest.raises(lisa.LisaError):
        lisa.lisa_prefill_workspace_bytes(_dims(d=80), 1, 10)


def _cont(d, B=1, past=10, n=64, ws_bytes=1 << 40, **ptrs):
    p = dict(q=FAKE, kc=FAKE, vc=FAKE, q_idx=FAKE, kic=FAKE, w_idx=FAKE, gate=FAKE, state_in=0,
             out=FAKE, state_out=0, topm_out=0, workspace=FAKE)
    p.update(ptrs)
    return lisa.lisa_prefill_continue(d, B, past, n, p["q"], p["kc"], p["vc"], p["q_idx"], p["kic"],
                                      p["w_idx"], p["gate"], p["state_in"], p["out"], p["state_out"],
                                      p["topm_out"], p["workspace"], ws_bytes, 0)


@pytest.mark.parametrize("name", ["q", "kc", "vc", "q_idx", "kic", "w_idx", "gate", "out", "workspace"])
def test_prefill_continue_null_pointer(name):
    assert _cont(_dims(), **{name: 0}) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert name.replace("kc", "k").replace("vc", "v").replace("kic", "k_idx") in lisa.lisa_last_error()


def test_prefill_continue_limits():
    d = _dims()
    assert _cont(d, past=-1) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _cont(d, past=32768 - 63, n=64) == lisa.LISA_ERR_UNSUPPORTED
    assert _cont(d, n=0, q=0, workspace=0) == lisa.LISA_OK
    assert _cont(d, B=0, q=0, workspace=0) == lisa.LISA_OK
    need = lisa.lisa_prefill_workspace_bytes(d, 1, 64)
    assert _cont(d, ws_bytes=need - 1) == lisa.LISA_ERR_WORKSPACE
    assert _cont(_dims(M=513)) == lisa.LISA_ERR_UNSUPPORTED


def _win(d, B=1, past=0, n=64, ws_bytes=1 << 40, **ptrs):
    p = dict(q=FAKE, kc=FAKE, vc=FAKE, gate=FAKE, state_in=0, out=FAKE, state_out=0, workspace=FAKE)
    p.update(ptrs)
    return lisa.lisa_prefill_window(d, B, past, n, p["q"], p["kc"], p["vc"], p["gate"], p["state_in"],
                                    p["out"], p["state_out"], p["workspace"], ws_bytes, 0)


def _dwin(d, B=2, max_ctx=100, ws_bytes=1 << 40, **ptrs):
    p = dict(cu=FAKE, q=FAKE, kc=FAKE, vc=FAKE, gate=FAKE, state=FAKE, out=FAKE, workspace=FAKE)
    p.update(ptrs)
    return lisa.lisa_decode_step_window(d, B, p["cu"], max_ctx, p["q"], p["kc"], p["vc"], p["gate"],
                                        p["state"], p["out"], p["workspace"], ws_bytes, 0)


@pytest.mark.parametrize("name", ["q", "kc", "vc", "gate", "out", "workspace"])
def test_window_null_pointers(name):
    assert _win(_dims(), **{name: 0}) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _dwin(_dims(), **{name: 0}) == lisa.LISA_ERR_INVALID_ARGUMENT


def test_window_limits():
    # the indexer fields are not used (and not checked); the window may be up to 2048
    assert _win(_dims(HI=0, dI=48, M=2049)) == lisa.LISA_ERR_UNSUPPORTED
    assert _win(_dims(M=0)) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _dwin(_dims(M=2049)) == lisa.LISA_ERR_UNSUPPORTED
    assert _dwin(_dims(), max_ctx=65537) == lisa.LISA_ERR_UNSUPPORTED
    assert _win(_dims(), n=0, q=0, workspace=0) == lisa.LISA_OK
    assert _dwin(_dims(), B=0, q=0) == lisa.LISA_OK
    d = _dims(M=1000)
    need = lisa.lisa_prefill_workspace_bytes(d, 1, 64)
    assert _win(d, ws_bytes=need - 1) == lisa.LISA_ERR_WORKSPACE


def _paged(d, B=2, max_ctx=100, bs=16, max_blocks=8, num_pages=16, ws_bytes=1 << 40, **ptrs):
    p = dict(lengths=FAKE, table=FAKE, q=FAKE, kp=FAKE, vp=FAKE, q_idx=FAKE, kip=FAKE, w_idx=FAKE,
             gate=FAKE, state=FAKE, out=FAKE, topm_out=0, workspace=FAKE)
    p.update(ptrs)
    return lisa.lisa_decode_step_paged(d, B, p["lengths"], p["table"], bs, max_blocks, num_pages,
                                       max_ctx, p["q"], p["kp"], p["vp"], p["q_idx"], p["kip"],
                                       p["w_idx"], p["gate"], p["state"], p["out"], p["topm_out"],
                                       p["workspace"], ws_bytes, 0)


@pytest.mark.parametrize("name", ["lengths", "table", "q", "kp", "vp", "q_idx", "kip", "w_idx",
                                  "gate", "state", "out", "workspace"])
def test_paged_null_pointer(name):
    assert _paged(_dims(), **{name: 0}) == lisa.LISA_ERR_INVALID_ARGUMENT


def test_paged_limits():
    d = _dims()
    assert _paged(d, lengths=FAKE + 2) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _paged(d, table=FAKE + 1) == lisa.LISA_ERR_INVALID_ARGUMENT
    for bs in (0, 3, 24, 8192):
        assert _paged(d, bs=bs) == lisa.LISA_ERR_UNSUPPORTED
    assert _paged(d, max_blocks=6) == lisa.LISA_ERR_INVALID_ARGUMENT      # 6 * 16 < 100
    assert _paged(d, num_pages=0) == lisa.LISA_ERR_INVALID_ARGUMENT
    # 2 GiB pool: 1024 pages of 4096 rows of 2 heads x 128 bf16
    assert _paged(d, bs=4096, max_blocks=1, num_pages=1024) == lisa.LISA_ERR_UNSUPPORTED
    assert _paged(d, max_ctx=0) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _paged(d, max_ctx=65537, max_blocks=4097) == lisa.LISA_ERR_UNSUPPORTED
    assert _paged(_dims(M=2049)) == lisa.LISA_ERR_UNSUPPORTED
    assert _paged(d, B=-1) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _paged(d, B=0, q=0) == lisa.LISA_OK
    need = lisa.lisa_decode_workspace_bytes(d, 2, 100)
    assert _paged(d, ws_bytes=need - 1) == lisa.LISA_ERR_WORKSPACE


def test_continue_workspace_query():
    d = _dims()
    # past == 0 is the prefill query; more cached keys need more workspace
    assert lisa.lisa_prefill_continue_workspace_bytes(d, 1, 0, 512) == lisa.lisa_prefill_workspace_bytes(d, 1, 512)
    assert lisa.lisa_prefill_continue_workspace_bytes(d, 1, 4096, 512) > lisa.lisa_prefill_workspace_bytes(d, 1, 512)
    assert lisa.lisa_prefill_continue_workspace_bytes(d, 2, 4096, 512) > lisa.lisa_prefill_continue_workspace_bytes(d, 1, 4096, 512)
    with pytest.raises(lisa.LisaError):
        lisa.lisa_prefill_continue_workspace_bytes(d, 1, 32768, 1)
    with pytest.raises(lisa.LisaError):
        lisa.lisa_prefill_continue_workspace_bytes(d, 1, -1, 8)
    # a continue call given only the n-token prefill workspace is refused
    need = lisa.lisa_prefill_continue_workspace_bytes(d, 1, 4096, 64)
    assert _cont(d, past=4096, n=64, ws_bytes=need - 1) == lisa.LISA_ERR_WORKSPACE


def _bwd(d, B=1, n=64, ws_bytes=1 << 40, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, state_in=0, topm=FAKE, d_out=FAKE, d_state_out=0,
             dq=FAKE, dk=FAKE, dv=FAKE, dgate=FAKE, d_state_in=0, workspace=FAKE)
    p.update(ptrs)
    return lisa.lisa_prefill_backward(d, B, n, p["q"], p["k"], p["v"], p["gate"], p["state_in"], p["topm"],
                                      p["d_out"], p["d_state_out"], p["dq"], p["dk"], p["dv"], p["dgate"],
                                      p["d_state_in"], p["workspace"], ws_bytes, 0)


@pytest.mark.parametrize("name", ["q", "k", "v", "gate", "topm", "d_out", "dq", "dk", "dv", "dgate",
                                  "workspace"])
def test_backward_null_pointer(name):
    assert _bwd(_dims(), **{name: 0}) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert name in lisa.lisa_last_error()


def test_backward_limits():
    d = _dims()
    assert _bwd(d, state_in=FAKE + 4) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _bwd(d, d_state_in=FAKE + 8) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _bwd(d, n=-1) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert _bwd(d, n=32769) == lisa.LISA_ERR_UNSUPPORTED
    assert _bwd(_dims(Hq=34, Hkv=2)) == lisa.LISA_ERR_UNSUPPORTED
    assert _bwd(_dims(Hq=32, Hkv=1, M=512)) == lisa.LISA_ERR_UNSUPPORTED   # 32 heads per group
    # fp32 keeps M * r logits per wave in LDS; bf16 has no such bound
    assert _bwd(_dims(Hq=16, Hkv=1, M=512, dtype="f32")) == lisa.LISA_ERR_UNSUPPORTED
    assert "LDS" in lisa.lisa_last_error()
    assert _bwd(d, n=0, q=0, workspace=0) == lisa.LISA_OK
    assert _bwd(d, B=0, q=0) == lisa.LISA_OK
    need = lisa.lisa_prefill_backward_workspace_bytes(d, 1, 64)
    assert need > 0
    assert _bwd(d, ws_bytes=need - 1) == lisa.LISA_ERR_WORKSPACE
    # workspace grows with the sequence
    assert lisa.lisa_prefill_backward_workspace_bytes(d, 1, 4096) > need


def test_descriptor_spans_refused():
    """Shapes whose per-sequence row spans or launch sizes do not fit the
    kernels' 32-bit buffer-descriptor extents and thread counts are refused
    with UNSUPPORTED before any HIP call (the pointers are never touched)."""
    # K/V rows of one sequence: 32768 rows x 2048 groups x 128 fp32 = 32 GiB
    big = _dims(Hq=2048, Hkv=2048, dtype="f32")
    assert _prefill(big, n=32768) == lisa.LISA_ERR_UNSUPPORTED
    assert "descriptor" in lisa.lisa_last_error()
    assert _cont(big, past=16384, n=16384) == lisa.LISA_ERR_UNSUPPORTED
    assert _win(big, n=32768) == lisa.LISA_ERR_UNSUPPORTED
    assert _bwd(big, n=32768) == lisa.LISA_ERR_UNSUPPORTED
    with pytest.raises(lisa.LisaError):
        lisa.lisa_prefill_workspace_bytes(big, 1, 32768)
    # decode: 65536 rows x 512 groups x 128 fp32 = 16 GiB per sequence
    dbig = _dims(Hq=512, Hkv=512, dtype="f32", M=256)
    assert _decode(dbig, max_ctx=65536) == lisa.LISA_ERR_UNSUPPORTED
    assert _dwin(dbig, max_ctx=65536) == lisa.LISA_ERR_UNSUPPORTED
    with pytest.raises(lisa.LisaError):
        lisa.lisa_decode_workspace_bytes(dbig, 1, 65536)
    # the same groups at a short context fit
    assert lisa.lisa_decode_workspace_bytes(dbig, 1, 1024) > 0
    # too many (sequence, position, group) units for one launch's thread count
    many = _dims(Hq=64, Hkv=64)
    assert _prefill(many, B=4, n=32768) == lisa.LISA_ERR_UNSUPPORTED
    assert "units" in lisa.lisa_last_error()
    assert _decode(_dims(), B=(1 << 21) + 1) == lisa.LISA_ERR_UNSUPPORTED
    # backward: 256 positions' per-slot coefficients, 8 bytes per slot and head
    assert _bwd(_dims(Hq=4096, Hkv=256, M=512), n=64) == lisa.LISA_ERR_UNSUPPORTED
    assert "coefficient" in lisa.lisa_last_error()
    assert _bwd(_dims(Hq=1024, Hkv=64, M=512), n=64, ws_bytes=1) == lisa.LISA_ERR_WORKSPACE


def test_noalloc_decode_validation():
    """The no-allocation decode step validates like lisa_decode_step and
    refuses a step whose scratch would exceed its static 32 MiB, all before
    any HIP call."""
    d = _dims(Hq=28, Hkv=4, M=512)
    args = [FAKE] * 7
    assert lisa.lisa_decode_step_noalloc(d, 64, FAKE, 65536, *args, FAKE, FAKE, 0, 0) == lisa.LISA_ERR_UNSUPPORTED
    assert "scratch" in lisa.lisa_last_error()
    assert lisa.lisa_decode_step_noalloc(d, 2, 0, 100, *args, FAKE, FAKE, 0, 0) == lisa.LISA_ERR_INVALID_ARGUMENT
    assert lisa.lisa_decode_step_noalloc(d, 2, FAKE, 65537, *args, FAKE, FAKE, 0, 0) == lisa.LISA_ERR_UNSUPPORTED
    assert lisa.lisa_decode_step_noalloc(_dims(M=2049), 2, FAKE, 100, *args, FAKE, FAKE, 0, 0) == \
        lisa.LISA_ERR_UNSUPPORTED
    assert lisa.lisa_decode_step_noalloc(d, 0, 0, 100, *([0] * 7), 0, 0, 0, 0) == lisa.LISA_OK
