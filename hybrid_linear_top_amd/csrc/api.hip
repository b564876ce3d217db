// C ABI of the LISA layer: argument validation, workspace layout and the
// launch sequence of each entry point.  Every check runs before the first
// HIP call, so a rejected call enqueues nothing.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>
#include <vector>

#include "lisa.h"
#include "kernels.hpp"

namespace lisa {
DispatchEvents &dispatch_events() {
    static thread_local DispatchEvents d;
    return d;
}
}  // namespace lisa

namespace {

thread_local char g_err[512] = "";

lisa_status fail(lisa_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

lisa_status ok() {
    g_err[0] = 0;
    return LISA_OK;
}

constexpr size_t kAlign = 256;
constexpr int kMaxDecodeCtx = 65536;  // the select kernel keeps up to 64 keys per thread
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// LISA_LOG=1 in the environment: each call that passed its checks prints its
// entry point and shapes to stderr before it enqueues (read once per process).
bool log_on() {
    static const bool on = [] {
        const char *e = std::getenv("LISA_LOG");
        return e && e[0] == '1';
    }();
    return on;
}
void log_call(const char *what, const lisa_dims *d, int B, const char *k1, int64_t v1, const char *k2, int64_t v2) {
    if (!log_on()) return;
    std::fprintf(stderr,
                 "lisa: %s B=%d %s=%lld %s=%lld heads=%d/%d d=%d indexer=%dx%d top_m=%d chunk=%d %s\n", what, B,
                 k1, (long long)v1, k2, (long long)v2, d->num_q_heads, d->num_kv_heads, d->head_dim, d->idx_heads,
                 d->idx_dim, d->top_m, d->chunk, d->dtype == LISA_BF16 ? "bf16" : "f32");
}

int elt_bytes(int dtype) { return dtype == LISA_BF16 ? 2 : 4; }

// window: the sliding-window variant, which has no indexer (its fields are
// not checked) and no top-M buffers (window up to 2048 in prefill too)
lisa_status check_dims(const lisa_dims *d, bool prefill, bool window = false) {
    if (!d) return fail(LISA_ERR_INVALID_ARGUMENT, "dims is NULL");
    if (d->dtype != LISA_F32 && d->dtype != LISA_BF16)
        return fail(LISA_ERR_INVALID_ARGUMENT, "dtype %d is neither LISA_F32 nor LISA_BF16", d->dtype);
    if (d->num_q_heads < 1 || d->num_kv_heads < 1)
        return fail(LISA_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (Hq=%d, Hkv=%d)",
                    d->num_q_heads, d->num_kv_heads);
    if (d->num_q_heads % d->num_kv_heads != 0)
        return fail(LISA_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    d->num_q_heads, d->num_kv_heads);
    if (d->num_q_heads / d->num_kv_heads > 16)
        return fail(LISA_ERR_UNSUPPORTED, "more than 16 query heads per KV group (%d)",
                    d->num_q_heads / d->num_kv_heads);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(LISA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", d->head_dim);
    if (!window && d->idx_dim != 32 && d->idx_dim != 64)
        return fail(LISA_ERR_UNSUPPORTED, "idx_dim %d not in {32, 64}", d->idx_dim);
    if (!window && (d->idx_heads < 1 || d->idx_heads > 8))
        return fail(LISA_ERR_UNSUPPORTED, "idx_heads %d not in [1, 8]", d->idx_heads);
    const int mmax = prefill && !window ? 512 : 2048;
    if (d->top_m < 1) return fail(LISA_ERR_INVALID_ARGUMENT, "top_m %d must be >= 1", d->top_m);
    if (d->top_m > mmax)
        return fail(LISA_ERR_UNSUPPORTED, "top_m %d above the supported %d", d->top_m, mmax);
    if (d->chunk != 0 && d->chunk != 64)
        return fail(LISA_ERR_UNSUPPORTED, "chunk %d not in {0, 64}", d->chunk);
    if (!std::isfinite(d->softmax_scale))
        return fail(LISA_ERR_INVALID_ARGUMENT, "softmax_scale is not finite");
    return LISA_OK;
}

// Every kernel addresses a sequence's rows through buffer descriptors whose
// byte extent is a 32-bit field, and every launch counts its threads in 32
// bits.  Shapes whose spans do not fit are refused here, before any HIP call
// (they would otherwise wrap and read zeros past the wrapped extent).
constexpr int64_t kSpan32 = 0xFFFFFFFFll;
constexpr int64_t kMaxUnitThreads = 1024;  // the largest work-group one unit gets

// (products in 128 bits: the arguments are unvalidated 32-bit counts whose
// products can pass 2^63)
using wide_t = __int128;

lisa_status check_spans(const lisa_dims *d, int64_t B, int64_t units, int64_t kv_rows, bool indexer) {
    const wide_t G = d->num_kv_heads, eb = elt_bytes(d->dtype);
    // (one row more: the sparse gathers address the row past the last)
    const wide_t kv_span = ((wide_t)kv_rows + 1) * G * d->head_dim * eb;
    if (kv_span > kSpan32)
        return fail(LISA_ERR_UNSUPPORTED,
                    "%lld K/V rows of %d groups span %.4g bytes: a buffer descriptor holds at most %lld",
                    (long long)kv_rows, d->num_kv_heads, (double)kv_span, (long long)kSpan32);
    // (the sparse gathers form row offsets with 24-bit multiplies)
    if (G * d->head_dim * eb >= ((wide_t)1 << 24))
        return fail(LISA_ERR_UNSUPPORTED, "a K/V position of %d groups spans %.4g bytes: at most 2^24 - 1",
                    d->num_kv_heads, (double)(G * d->head_dim * eb));
    const wide_t idx_span = (wide_t)kv_rows * G * d->idx_dim * eb;
    if (indexer && idx_span > kSpan32)
        return fail(LISA_ERR_UNSUPPORTED, "%lld indexer-key rows span %.4g bytes: at most %lld",
                    (long long)kv_rows, (double)idx_span, (long long)kSpan32);
    if ((wide_t)B * units * kMaxUnitThreads > kSpan32)
        return fail(LISA_ERR_UNSUPPORTED, "%.4g (sequence, position, group) units: at most %lld per call",
                    (double)((wide_t)B * units), (long long)(kSpan32 / kMaxUnitThreads));
    return LISA_OK;
}

// decode: kv_rows is max_ctx for packed caches (a sequence's rows) or the
// page pool's rows; the score scan launches a 256-thread work-group per 128
// positions of every sequence
lisa_status check_decode_spans(const lisa_dims *d, int64_t B, int64_t max_ctx, int64_t kv_rows) {
    lisa_status st = check_spans(d, B, d->num_kv_heads, kv_rows, true);
    if (st) return st;
    if (B * ((max_ctx + 127) / 128) * 256 > kSpan32)
        return fail(LISA_ERR_UNSUPPORTED, "B=%lld sequences of max_ctx=%lld: the score launch exceeds 2^32 threads",
                    (long long)B, (long long)max_ctx);
    return LISA_OK;
}

// backward: besides the forward's spans, the key side reads a block of 256
// positions' per-slot coefficients (8 bytes per slot and query head) and
// their q / d_out rows through one descriptor each
lisa_status check_bwd_spans(const lisa_dims *d, int64_t B, int64_t n) {
    lisa_status st = check_spans(d, B, n * d->num_kv_heads, n, false);
    if (st) return st;
    const int64_t coef = 256ll * d->num_q_heads * d->top_m * 8;
    if (coef > kSpan32)
        return fail(LISA_ERR_UNSUPPORTED, "%d query heads x top_m %d: a 256-position coefficient block spans %lld bytes",
                    d->num_q_heads, d->top_m, (long long)coef);
    if (256ll * d->num_q_heads * d->head_dim * 4 > kSpan32)
        return fail(LISA_ERR_UNSUPPORTED, "%d query heads: a 256-position row block exceeds 4 GiB", d->num_q_heads);
    return LISA_OK;
}

float scale_log2(const lisa_dims *d) {
    const double s = d->softmax_scale > 0.0f ? (double)d->softmax_scale : 1.0 / std::sqrt((double)d->head_dim);
    return (float)(s * 1.4426950408889634);
}

// ---- prefill workspace ------------------------------------------------------
struct PrefillWs {
    size_t idx, dS, P, kpk, cand, total;
};
// n query rows against nk key positions (nk = past + n; 0 when the indexer
// does not run)
PrefillWs prefill_ws(const lisa_dims *d, int B, int n, int nk) {
    const size_t G = d->num_kv_heads, Hq = d->num_q_heads, D = d->head_dim;
    const size_t nC = ((size_t)n + 63) / 64;
    PrefillWs w;
    size_t off = 0;
    w.idx = off;
    off += align_up((size_t)B * n * G * d->top_m * 4);
    w.dS = off;
    off += align_up((size_t)B * G * nC * D * D * 4);
    w.P = off;
    off += align_up((size_t)B * Hq * nC * D * D * elt_bytes(d->dtype));
    w.kpk = off;
    off += align_up(nk > 0 ? lisa::indexer_packed_bytes(B, nk, (int)G, d->idx_dim, d->dtype) : 0);
    w.cand = off;
    off += align_up(nk > 0 && d->top_m <= 512 ? lisa::indexer_cand_bytes(B, n, (int)G, d->top_m) : 0);
    w.total = off;
    return w;
}

struct DecodeWs {
    size_t scores, olin, idx, cand, total;
};
DecodeWs decode_ws(const lisa_dims *d, int B, int max_ctx) {
    const size_t G = d->num_kv_heads, Hq = d->num_q_heads, D = d->head_dim;
    DecodeWs w;
    size_t off = 0;
    w.scores = off;
    off += align_up((size_t)B * G * (size_t)max_ctx * 4);
    w.olin = off;
    off += align_up((size_t)B * Hq * D * 4);
    w.idx = off;
    off += align_up((size_t)B * G * d->top_m * 4);
    w.cand = off;  // the two-part select of long contexts
    off += align_up(lisa::decode_cand_bytes(B, (int)G, d->top_m, max_ctx));
    w.total = off;
    return w;
}

// ---- optional per-stage timing (benchmarking) -------------------------------
enum Stage {
    ST_LIN_STATE, ST_LIN_SCAN, ST_LIN_OUT, ST_IDX_PACK, ST_INDEXER, ST_SPARSE_PREFILL,
    ST_DEC_SCORE_STATE, ST_DEC_SELECT, ST_SPARSE_DECODE,
    ST_BWD_OPER, ST_BWD_LINEAR, ST_BWD_COMBINE, ST_BWD_SPARSE, ST_BWD_SPARSE_Q, ST_BWD_SORT, ST_BWD_SPARSE_KV,
    ST_COUNT
};
const char *const kStageNames[ST_COUNT] = {
    "linear_chunk_state", "linear_prefix_scan", "linear_chunk_output", "indexer_pack", "indexer_topm",
    "sparse_gate_prefill", "decode_score_state", "decode_select", "sparse_gate_decode",
    "bwd_operands", "bwd_linear", "bwd_combine", "bwd_sparse", "bwd_sparse_query", "bwd_sparse_sort",
    "bwd_sparse_keys",
};

struct Timing {
    std::mutex mu;
    std::atomic<bool> enabled{false};
    struct Rec { int stage; hipEvent_t a, b; };
    std::vector<Rec> pending;
    std::vector<hipEvent_t> pool;
    double total_ms[ST_COUNT] = {};
    int64_t launches[ST_COUNT] = {};
    hipEvent_t get() {
        if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
};
Timing g_timing;

// Launch through `fn`, bracketed by an event pair when timing is enabled.
// The stage's launches carry the events (lisa::launch_kernel): a = the first
// kernel's start, b = the last kernel's end.  A stage that launched nothing
// records them as plain markers, so every pair completes.
template <typename F>
hipError_t timed(int stage, hipStream_t s, F fn) {
    if (!g_timing.enabled) return fn();
    std::lock_guard<std::mutex> lk(g_timing.mu);
    hipEvent_t a = g_timing.get(), b = g_timing.get();
    if (!a || !b) return hipErrorOutOfMemory;
    lisa::DispatchEvents &de = lisa::dispatch_events();
    de = lisa::DispatchEvents{a, b, 0};
    hipError_t e = fn();
    const int launched = de.launches;
    de = lisa::DispatchEvents{};
    if (e != hipSuccess) return e;
    if (launched == 0) {
        e = hipEventRecord(a, s);
        if (e != hipSuccess) return e;
        e = hipEventRecord(b, s);
        if (e != hipSuccess) return e;
    }
    g_timing.pending.push_back({stage, a, b});
    return hipSuccess;
}

#define LISA_NEED(p, name)                                                                  \
    do {                                                                                    \
        if (!(p)) return fail(LISA_ERR_INVALID_ARGUMENT, "%s is NULL", name);               \
        if (!aligned16(p)) return fail(LISA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name); \
    } while (0)
#define LISA_OPT(p, name)                                                                   \
    do {                                                                                    \
        if ((p) && !aligned16(p))                                                           \
            return fail(LISA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);      \
    } while (0)
#define LISA_HIP(call, what)                                                                \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess)                                                               \
            return fail(LISA_ERR_HIP, "%s: %s", what, hipGetErrorString(e_));               \
    } while (0)

}  // namespace

extern "C" {

const char *lisa_last_error(void) { return g_err; }

const char *lisa_build_info(void) {
    return "lisa-mi355x 0.1 (gfx950)";
}

lisa_status lisa_prefill_workspace_bytes(const lisa_dims *dims, int32_t B, int32_t n,
                                         size_t *bytes) {
    // sized for both prefill variants: the window one allows top_m up to 2048
    lisa_status st = check_dims(dims, true, true);
    if (st) return st;
    if (!bytes) return fail(LISA_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (B < 0 || n < 0) return fail(LISA_ERR_INVALID_ARGUMENT, "B=%d, n=%d must be >= 0", B, n);
    if (n > 32768) return fail(LISA_ERR_UNSUPPORTED, "n=%d above the supported 32768", n);
    if ((st = check_spans(dims, B, (int64_t)n * dims->num_kv_heads, n, false))) return st;
    *bytes = prefill_ws(dims, B, n, n).total;
    return ok();
}

lisa_status lisa_prefill_continue_workspace_bytes(const lisa_dims *dims, int32_t B, int32_t past,
                                                  int32_t n, size_t *bytes) {
    lisa_status st = check_dims(dims, true, true);
    if (st) return st;
    if (!bytes) return fail(LISA_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (B < 0 || n < 0 || past < 0)
        return fail(LISA_ERR_INVALID_ARGUMENT, "B=%d, past=%d, n=%d must be >= 0", B, past, n);
    if ((int64_t)past + n > 32768)
        return fail(LISA_ERR_UNSUPPORTED, "past + n = %lld above the supported 32768", (long long)past + n);
    if ((st = check_spans(dims, B, (int64_t)n * dims->num_kv_heads, (int64_t)past + n, false))) return st;
    *bytes = prefill_ws(dims, B, n, past + n).total;
    return ok();
}

lisa_status lisa_decode_workspace_bytes(const lisa_dims *dims, int32_t B, int32_t max_ctx,
                                        size_t *bytes) {
    lisa_status st = check_dims(dims, false);
    if (st) return st;
    if (!bytes) return fail(LISA_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (B < 0 || max_ctx < 1)
        return fail(LISA_ERR_INVALID_ARGUMENT, "B=%d must be >= 0 and max_ctx=%d >= 1", B, max_ctx);
    if (max_ctx > kMaxDecodeCtx)
        return fail(LISA_ERR_UNSUPPORTED, "max_ctx=%d above the supported %d", max_ctx, kMaxDecodeCtx);
    if ((st = check_decode_spans(dims, B, max_ctx, max_ctx))) return st;
    *bytes = decode_ws(dims, B, max_ctx).total;
    return ok();
}

lisa_status lisa_prefill(const lisa_dims *dims, int32_t B, int32_t n, const void *q,
                         const void *k, const void *v, const void *q_idx, const void *k_idx,
                         const void *w_idx, const void *gate, const float *state_in, void *out,
                         float *state_out, int32_t *topm_out, void *workspace,
                         size_t workspace_bytes, lisa_stream_t stream) {
    return lisa_prefill_continue(dims, B, 0, n, q, k, v, q_idx, k_idx, w_idx, gate, state_in, out,
                                 state_out, topm_out, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The prefill path: window = false runs the indexer and top-M; window = true
// is the sliding-window variant (set of position t = max(0, t-M+1)..t), where
// q_idx, k_idx, w_idx and topm_out are unused.
lisa_status prefill_impl(const lisa_dims *dims, int32_t B, int32_t past, int32_t n, const void *q,
                         const void *k, const void *v, const void *q_idx, const void *k_idx,
                         const void *w_idx, const void *gate, const float *state_in, void *out,
                         float *state_out, int32_t *topm_out, void *workspace,
                         size_t workspace_bytes, lisa_stream_t stream, bool window) {
    lisa_status st = check_dims(dims, true, window);
    if (st) return st;
    if (B < 0 || n < 0 || past < 0)
        return fail(LISA_ERR_INVALID_ARGUMENT, "B=%d, past=%d, n=%d must be >= 0", B, past, n);
    if ((int64_t)past + n > 32768)
        return fail(LISA_ERR_UNSUPPORTED, "past + n = %lld above the supported 32768",
                    (long long)past + n);
    if ((st = check_spans(dims, B, (int64_t)n * dims->num_kv_heads, (int64_t)past + n, false))) return st;
    if (B == 0 || n == 0) return ok();
    LISA_NEED(q, "q");
    LISA_NEED(k, "k");
    LISA_NEED(v, "v");
    if (!window) {
        LISA_NEED(q_idx, "q_idx");
        LISA_NEED(k_idx, "k_idx");
        LISA_NEED(w_idx, "w_idx");
    }
    LISA_NEED(gate, "gate");
    LISA_NEED(out, "out");
    LISA_OPT(state_in, "state_in");
    LISA_OPT(state_out, "state_out");
    LISA_OPT(topm_out, "topm_out");
    LISA_NEED(workspace, "workspace");
    // the window variant asks for what lisa_prefill_workspace_bytes gives (it needs less)
    const PrefillWs w = prefill_ws(dims, B, n, window ? n : past + n);
    if (workspace_bytes < w.total)
        return fail(LISA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, w.total);
    log_call(window ? "prefill_window" : "prefill", dims, B, "past", past, "n", n);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const int G = dims->num_kv_heads, Hq = dims->num_q_heads, D = dims->head_dim;
    int32_t *idx = topm_out ? topm_out : reinterpret_cast<int32_t *>(ws + w.idx);

    lisa::LinearArgs la{};
    la.q = q;
    la.k = k;
    la.v = v;
    la.state_in = state_in;
    la.state_out = state_out;
    la.dS = reinterpret_cast<float *>(ws + w.dS);
    la.P = ws + w.P;
    la.out = out;
    la.B = B;
    la.n = n;
    la.Hq = Hq;
    la.G = G;
    la.r = Hq / G;
    la.nC = (n + 63) / 64;
    la.kv_rows = past + n;
    la.kv_off = past;
    la.per_head = state_in != nullptr;
    LISA_HIP(timed(ST_LIN_STATE, s, [&] { return lisa::launch_linear_chunk_state(la, dims->dtype, D, s); }),
             "linear chunk-state launch");
    LISA_HIP(timed(ST_LIN_SCAN, s, [&] { return lisa::launch_linear_prefix_scan(la, dims->dtype, D, s); }),
             "linear prefix-scan launch");
    LISA_HIP(timed(ST_LIN_OUT, s, [&] { return lisa::launch_linear_chunk_output(la, dims->dtype, D, s); }),
             "linear chunk-output launch");

    lisa::IndexerArgs ia{};
    ia.q_idx = q_idx;
    ia.k_idx = k_idx;
    ia.w_idx = w_idx;
    ia.idx = idx;
    ia.B = B;
    ia.n = n;
    ia.G = G;
    ia.HI = dims->idx_heads;
    ia.M = dims->top_m;
    ia.past = past;
    ia.k_packed = ws + w.kpk;
    ia.cand = ws + w.cand;
    if (!window) {
        LISA_HIP(timed(ST_IDX_PACK, s, [&] { return lisa::launch_indexer_pack(ia, dims->dtype, dims->idx_dim, s); }),
                 "indexer key-pack launch");
        LISA_HIP(timed(ST_INDEXER, s, [&] { return lisa::launch_indexer_prefill(ia, dims->dtype, dims->idx_dim, s); }),
                 "indexer launch");
    }

    lisa::SparseArgs sa{};
    sa.q = q;
    sa.k = k;
    sa.v = v;
    sa.cu = nullptr;
    sa.idx = window ? nullptr : idx;
    sa.window = window ? 1 : 0;
    sa.lin = out;
    sa.gate = gate;
    sa.out = out;
    sa.B = B;
    sa.n = n;
    sa.Hq = Hq;
    sa.G = G;
    sa.r = Hq / G;
    sa.M = dims->top_m;
    sa.max_ctx = past + n;
    sa.past = past;
    sa.scale_log2 = scale_log2(dims);
    sa.units = B * n * G;
    LISA_HIP(timed(ST_SPARSE_PREFILL, s, [&] { return lisa::launch_sparse_gate(sa, dims->dtype, D, false, s); }),
             "sparse-attention launch");
    return ok();
}

// ---- static scratch for lisa_decode_step_noalloc ------------------------------
// A file-scope device array stands in for the caller's workspace.  In host
// code its name is only a stand-in for the symbol: every host use goes
// through the device address hipGetSymbolAddress returns, resolved once per
// device on the first call there (with that device current) and kept.
constexpr size_t kScratchBytes = size_t{32} << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

lisa_status device_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(LISA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(LISA_ERR_UNSUPPORTED, "device %d: the scratch table holds %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(LISA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LISA_OK;
}

// The decode path; window as in prefill_impl.  map.table == nullptr: packed
// caches described by cu_ctx; otherwise paged caches (pool_rows rows).
lisa_status decode_impl(const lisa_dims *dims, int32_t B, const int64_t *cu_ctx, int32_t max_ctx,
                        const void *q, const void *k_cache, const void *v_cache, const void *q_idx,
                        const void *k_idx_cache, const void *w_idx, const void *gate, float *state,
                        void *out, int32_t *topm_out, void *workspace, size_t workspace_bytes,
                        lisa_stream_t stream, bool window, lisa::CacheMap map = lisa::CacheMap{},
                        int64_t pool_rows = 0, bool use_scratch = false) {
    const bool paged = map.table != nullptr;
    lisa_status st = check_dims(dims, false, window);
    if (st) return st;
    if (B < 0) return fail(LISA_ERR_INVALID_ARGUMENT, "B=%d must be >= 0", B);
    if (max_ctx < 1) return fail(LISA_ERR_INVALID_ARGUMENT, "max_ctx=%d must be >= 1", max_ctx);
    if (max_ctx > kMaxDecodeCtx)
        return fail(LISA_ERR_UNSUPPORTED, "max_ctx=%d above the supported %d", max_ctx, kMaxDecodeCtx);
    if ((st = check_decode_spans(dims, B, max_ctx, paged ? pool_rows : max_ctx))) return st;
    if (B == 0) return ok();
    if (!paged) {
        if (!cu_ctx) return fail(LISA_ERR_INVALID_ARGUMENT, "cu_ctx is NULL");
        if (reinterpret_cast<uintptr_t>(cu_ctx) & 7u)
            return fail(LISA_ERR_INVALID_ARGUMENT, "cu_ctx is not 8-byte aligned");
        map.cu = cu_ctx;
    }
    LISA_NEED(q, "q");
    LISA_NEED(k_cache, "k_cache");
    LISA_NEED(v_cache, "v_cache");
    if (!window) {
        LISA_NEED(q_idx, "q_idx");
        LISA_NEED(k_idx_cache, "k_idx_cache");
        LISA_NEED(w_idx, "w_idx");
    }
    LISA_NEED(gate, "gate");
    LISA_NEED(state, "state");
    LISA_NEED(out, "out");
    LISA_OPT(topm_out, "topm_out");
    const DecodeWs w = decode_ws(dims, B, max_ctx);
    if (use_scratch) {
        // the kernels overwrite every scratch byte they read (no zero start)
        if (w.total > kScratchBytes)
            return fail(LISA_ERR_UNSUPPORTED, "this step needs %zu bytes of scratch; the static scratch holds %zu",
                        w.total, kScratchBytes);
        if ((st = device_scratch(&workspace))) return st;
        workspace_bytes = kScratchBytes;
    } else {
        LISA_NEED(workspace, "workspace");
        if (workspace_bytes < w.total)
            return fail(LISA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, w.total);
    }
    log_call(window ? "decode_step_window" : paged ? "decode_step_paged" : use_scratch ? "decode_step_noalloc"
                                                                             : "decode_step",
             dims, B, "max_ctx", max_ctx, "pool_rows", pool_rows);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const int G = dims->num_kv_heads, Hq = dims->num_q_heads, D = dims->head_dim;
    float *scores = reinterpret_cast<float *>(ws + w.scores);
    float *olin = reinterpret_cast<float *>(ws + w.olin);
    int32_t *idx = topm_out ? topm_out : reinterpret_cast<int32_t *>(ws + w.idx);

    lisa::DecodeScoreArgs da{};
    da.q = q;
    da.k_cache = k_cache;
    da.v_cache = v_cache;
    da.q_idx = q_idx;
    da.k_idx_cache = k_idx_cache;
    da.w_idx = w_idx;
    da.cu = cu_ctx;
    da.map = map;
    da.pool_rows = pool_rows;
    da.state = state;
    da.olin = olin;
    da.scores = scores;
    da.B = B;
    da.Hq = Hq;
    da.G = G;
    da.HI = dims->idx_heads;
    da.max_ctx = max_ctx;
    // the window variant launches the state groups only (no indexer scan)
    da.tiles_per_seq = window ? 0 : (max_ctx + lisa::kDecodeTile - 1) / lisa::kDecodeTile;
    const int dI = window ? 64 : dims->idx_dim;  // any supported width: no score groups run
    // with the indexer, the state step runs in the select's launch, beside
    // the selects (it does not need the scores)
    LISA_HIP(timed(ST_DEC_SCORE_STATE, s,
                   [&] { return lisa::launch_decode_score_state(da, dims->dtype, D, dI, window, s); }),
             "indexer-scan/state launch");
    if (!window)
        LISA_HIP(timed(ST_DEC_SELECT, s, [&] {
                     return lisa::launch_decode_select(scores, map, B, G, dims->top_m, max_ctx, idx,
                                                       reinterpret_cast<int32_t *>(ws + w.cand), &da, dims->dtype, D,
                                                       s);
                 }),
                 "top-M select launch");

    lisa::SparseArgs sa{};
    sa.q = q;
    sa.k = k_cache;
    sa.v = v_cache;
    sa.cu = cu_ctx;
    sa.map = map;
    sa.pool_rows = pool_rows;
    sa.idx = window ? nullptr : idx;
    sa.window = window ? 1 : 0;
    sa.lin = olin;
    sa.gate = gate;
    sa.out = out;
    sa.B = B;
    sa.n = 1;
    sa.Hq = Hq;
    sa.G = G;
    sa.r = Hq / G;
    sa.M = dims->top_m;
    sa.max_ctx = max_ctx;
    sa.scale_log2 = scale_log2(dims);
    sa.units = B * G;
    LISA_HIP(timed(ST_SPARSE_DECODE, s, [&] { return lisa::launch_sparse_gate(sa, dims->dtype, D, true, s); }),
             "sparse-attention launch");
    return ok();
}

}  // namespace

extern "C" {

lisa_status lisa_prefill_continue(const lisa_dims *dims, int32_t B, int32_t past, int32_t n,
                                  const void *q, const void *k, const void *v, const void *q_idx,
                                  const void *k_idx, const void *w_idx, const void *gate,
                                  const float *state_in, void *out, float *state_out,
                                  int32_t *topm_out, void *workspace, size_t workspace_bytes,
                                  lisa_stream_t stream) {
    return prefill_impl(dims, B, past, n, q, k, v, q_idx, k_idx, w_idx, gate, state_in, out,
                        state_out, topm_out, workspace, workspace_bytes, stream, false);
}

lisa_status lisa_prefill_window(const lisa_dims *dims, int32_t B, int32_t past, int32_t n,
                                const void *q, const void *k_cache, const void *v_cache,
                                const void *gate, const float *state_in, void *out,
                                float *state_out, void *workspace, size_t workspace_bytes,
                                lisa_stream_t stream) {
    return prefill_impl(dims, B, past, n, q, k_cache, v_cache, nullptr, nullptr, nullptr, gate,
                        state_in, out, state_out, nullptr, workspace, workspace_bytes, stream, true);
}

lisa_status lisa_decode_step(const lisa_dims *dims, int32_t B, const int64_t *cu_ctx,
                             int32_t max_ctx, const void *q, const void *k_cache,
                             const void *v_cache, const void *q_idx, const void *k_idx_cache,
                             const void *w_idx, const void *gate, float *state, void *out,
                             int32_t *topm_out, void *workspace, size_t workspace_bytes,
                             lisa_stream_t stream) {
    return decode_impl(dims, B, cu_ctx, max_ctx, q, k_cache, v_cache, q_idx, k_idx_cache, w_idx,
                       gate, state, out, topm_out, workspace, workspace_bytes, stream, false);
}

lisa_status lisa_decode_step_noalloc(const lisa_dims *dims, int32_t B, const int64_t *cu_ctx,
                                     int32_t max_ctx, const void *q, const void *k_cache,
                                     const void *v_cache, const void *q_idx, const void *k_idx_cache,
                                     const void *w_idx, const void *gate, float *state, void *out,
                                     int32_t *topm_out, lisa_stream_t stream) {
    return decode_impl(dims, B, cu_ctx, max_ctx, q, k_cache, v_cache, q_idx, k_idx_cache, w_idx,
                       gate, state, out, topm_out, nullptr, 0, stream, false, lisa::CacheMap{}, 0, true);
}

lisa_status lisa_decode_step_paged(const lisa_dims *dims, int32_t B, const int32_t *lengths,
                                   const int32_t *block_table, int32_t block_size,
                                   int32_t max_blocks, int32_t num_pages, int32_t max_ctx,
                                   const void *q, const void *k_pages, const void *v_pages,
                                   const void *q_idx, const void *k_idx_pages, const void *w_idx,
                                   const void *gate, float *state, void *out, int32_t *topm_out,
                                   void *workspace, size_t workspace_bytes, lisa_stream_t stream) {
    lisa_status st = check_dims(dims, false);
    if (st) return st;
    if (B < 0) return fail(LISA_ERR_INVALID_ARGUMENT, "B=%d must be >= 0", B);
    if (B == 0) return ok();
    if (!lengths || !block_table) return fail(LISA_ERR_INVALID_ARGUMENT, "lengths or block_table is NULL");
    if ((reinterpret_cast<uintptr_t>(lengths) | reinterpret_cast<uintptr_t>(block_table)) & 3u)
        return fail(LISA_ERR_INVALID_ARGUMENT, "lengths or block_table is not 4-byte aligned");
    if (block_size < 1 || block_size > 4096 || (block_size & (block_size - 1)))
        return fail(LISA_ERR_UNSUPPORTED, "block_size %d is not a power of two in [1, 4096]", block_size);
    if (max_ctx < 1) return fail(LISA_ERR_INVALID_ARGUMENT, "max_ctx=%d must be >= 1", max_ctx);
    if ((int64_t)max_blocks * block_size < max_ctx)
        return fail(LISA_ERR_INVALID_ARGUMENT, "max_blocks %d x block_size %d < max_ctx %d", max_blocks,
                    block_size, max_ctx);
    if (num_pages < 1) return fail(LISA_ERR_INVALID_ARGUMENT, "num_pages=%d must be >= 1", num_pages);
    const int64_t row_bytes = (int64_t)dims->num_kv_heads * dims->head_dim * (dims->dtype == LISA_BF16 ? 2 : 4);
    const wide_t pool_bytes = (wide_t)num_pages * block_size * row_bytes;
    if (pool_bytes >= ((wide_t)1 << 31))
        return fail(LISA_ERR_UNSUPPORTED, "K/V page pool of %.4g bytes: at most 2 GiB is supported",
                    (double)pool_bytes);
    lisa::CacheMap map{};
    map.table = block_table;
    map.lengths = lengths;
    map.max_blocks = max_blocks;
    map.log2_block = __builtin_ctz((unsigned)block_size);
    return decode_impl(dims, B, nullptr, max_ctx, q, k_pages, v_pages, q_idx, k_idx_pages, w_idx, gate,
                       state, out, topm_out, workspace, workspace_bytes, stream, false, map,
                       (int64_t)num_pages * block_size);
}

lisa_status lisa_decode_step_window(const lisa_dims *dims, int32_t B, const int64_t *cu_ctx,
                                    int32_t max_ctx, const void *q, const void *k_cache,
                                    const void *v_cache, const void *gate, float *state, void *out,
                                    void *workspace, size_t workspace_bytes,
                                    lisa_stream_t stream) {
    return decode_impl(dims, B, cu_ctx, max_ctx, q, k_cache, v_cache, nullptr, nullptr, nullptr,
                       gate, state, out, nullptr, workspace, workspace_bytes, stream, true);
}

// ---- backward --------------------------------------------------------------------
namespace {
struct BwdWs {
    size_t Grev, qrev, vrep, krep, dqlin, ok, ov, sinT, dS, P, coef, sorted, total;
};
BwdWs bwd_ws(const lisa_dims *d, int B, int n) {
    const size_t Hq = d->num_q_heads, D = d->head_dim, eb = elt_bytes(d->dtype);
    const size_t nC = ((size_t)n + 63) / 64;
    const size_t act = align_up((size_t)B * n * Hq * D * eb);
    const size_t st = align_up((size_t)B * Hq * D * D * 4);
    BwdWs w;
    size_t off = 0;
    size_t *acts[] = {&w.Grev, &w.qrev, &w.vrep, &w.krep, &w.dqlin, &w.ok, &w.ov};
    for (size_t *x : acts) {
        *x = off;
        off += act;
    }
    w.sinT = off;
    off += st;
    // the chunked passes: up to Hq groups (each head its own group in the reversed passes)
    w.dS = off;
    off += align_up((size_t)B * Hq * nC * D * D * 4);
    w.P = off;
    off += align_up((size_t)B * Hq * nC * D * D * eb);
    // bf16: per-slot coefficients of the sparse branch, [B,n,G,M,r,2] fp32
    w.coef = off;
    if (d->dtype == LISA_BF16) off += align_up((size_t)B * n * Hq * d->top_m * 2 * 4);
    w.sorted = off;
    if (d->dtype == LISA_BF16) off += align_up(lisa::sparse_bwd_sorted_bytes(B, n, d->num_kv_heads, d->top_m));
    w.total = off;
    return w;
}

// one causal chunked linear-attention pass: out = o_lin of (q, k, v, state_in)
// output_only: the chunk-output kernel alone, on the prefix states the previous
// pass left in the workspace, read transposed (they are those of the
// transposed recurrence)
hipError_t linear_pass(const lisa_dims *dims, int B, int n, int Hq, int G, const void *q, const void *k,
                        const void *v, const float *state_in, float *state_out, void *out,
                        unsigned char *ws, const BwdWs &w, hipStream_t s, bool output_only = false) {
    lisa::LinearArgs la{};
    la.q = q;
    la.k = k;
    la.v = v;
    la.state_in = state_in;
    la.state_out = state_out;
    la.dS = reinterpret_cast<float *>(ws + w.dS);
    la.P = ws + w.P;
    la.out = out;
    la.B = B;
    la.n = n;
    la.Hq = Hq;
    la.G = G;
    la.r = Hq / G;
    la.nC = (n + 63) / 64;
    la.kv_rows = n;
    la.kv_off = 0;
    la.per_head = state_in != nullptr;
    const int D = dims->head_dim;
    if (output_only) {
        la.state_t = 1;
        return lisa::launch_linear_chunk_output(la, dims->dtype, D, s);
    }
    hipError_t e = lisa::launch_linear_chunk_state(la, dims->dtype, D, s);
    if (e == hipSuccess) e = lisa::launch_linear_prefix_scan(la, dims->dtype, D, s);
    if (e == hipSuccess) e = lisa::launch_linear_chunk_output(la, dims->dtype, D, s);
    return e;
}
}  // namespace

lisa_status lisa_prefill_backward_workspace_bytes(const lisa_dims *dims, int32_t B, int32_t n,
                                                  size_t *bytes) {
    lisa_status st = check_dims(dims, true);
    if (st) return st;
    if (!bytes) return fail(LISA_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (B < 0 || n < 0) return fail(LISA_ERR_INVALID_ARGUMENT, "B=%d, n=%d must be >= 0", B, n);
    if (n > 32768) return fail(LISA_ERR_UNSUPPORTED, "n=%d above the supported 32768", n);
    if ((st = check_bwd_spans(dims, B, n))) return st;
    *bytes = bwd_ws(dims, B, n).total;
    return ok();
}

lisa_status lisa_prefill_backward(const lisa_dims *dims, int32_t B, int32_t n, const void *q,
                                  const void *k, const void *v, const void *gate,
                                  const float *state_in, const int32_t *topm, const void *d_out,
                                  const float *d_state_out, float *dq, float *dk, float *dv,
                                  float *dgate, float *d_state_in, void *workspace,
                                  size_t workspace_bytes, lisa_stream_t stream) {
    lisa_status st = check_dims(dims, true);
    if (st) return st;
    if (B < 0 || n < 0) return fail(LISA_ERR_INVALID_ARGUMENT, "B=%d, n=%d must be >= 0", B, n);
    if (n > 32768) return fail(LISA_ERR_UNSUPPORTED, "n=%d above the supported 32768", n);
    const int G = dims->num_kv_heads, Hq = dims->num_q_heads, D = dims->head_dim, M = dims->top_m;
    if (Hq / G > 16)
        return fail(LISA_ERR_UNSUPPORTED, "%d query heads per group: the backward handles up to 16", Hq / G);
    if (dims->dtype != LISA_BF16 && lisa::sparse_bwd_lds_bytes(Hq / G, M, D) > 65536)
        return fail(LISA_ERR_UNSUPPORTED, "top_m %d with %d heads per group exceeds the backward's LDS", M, Hq / G);
    if ((st = check_bwd_spans(dims, B, n))) return st;
    if ((int64_t)B * n == 0) return ok();
    LISA_NEED(q, "q");
    LISA_NEED(k, "k");
    LISA_NEED(v, "v");
    LISA_NEED(gate, "gate");
    LISA_NEED(topm, "topm");
    LISA_NEED(d_out, "d_out");
    LISA_NEED(dq, "dq");
    LISA_NEED(dk, "dk");
    LISA_NEED(dv, "dv");
    LISA_NEED(dgate, "dgate");
    LISA_OPT(state_in, "state_in");
    LISA_OPT(d_state_out, "d_state_out");
    LISA_OPT(d_state_in, "d_state_in");
    LISA_NEED(workspace, "workspace");
    const BwdWs w = bwd_ws(dims, B, n);
    if (workspace_bytes < w.total)
        return fail(LISA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, w.total);
    log_call("prefill_backward", dims, B, "n", n, "state_grad", d_state_in != nullptr);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    unsigned char *ws = static_cast<unsigned char *>(workspace);

    lisa::BwdPrepArgs pa{};
    pa.q = q;
    pa.k = k;
    pa.v = v;
    pa.z = gate;
    pa.dout = d_out;
    pa.Grev = ws + w.Grev;
    pa.qrev = ws + w.qrev;
    pa.vrep = ws + w.vrep;
    pa.krep = ws + w.krep;
    pa.B = B;
    pa.n = n;
    pa.Hq = Hq;
    pa.G = G;
    pa.d = D;
    float *sinT = state_in ? reinterpret_cast<float *>(ws + w.sinT) : nullptr;
    LISA_HIP(timed(ST_BWD_OPER, s, [&] {
                 hipError_t e = lisa::launch_bwd_prep(pa, dims->dtype, s);
                 if (e == hipSuccess && sinT) e = lisa::launch_transpose_states(state_in, sinT, (int64_t)B * Hq, D, s);
                 return e;
             }),
             "backward operand launch");
    // three passes: R_t = S_t d_out (dq_lin = (1 - gamma) R, and q . R = d_out . o_lin
    // for the gate), then dk and dv of the linear branch in reversed time
    LISA_HIP(timed(ST_BWD_LINEAR, s, [&] {
                 hipError_t e = linear_pass(dims, B, n, Hq, G, d_out, v, k, sinT, nullptr, ws + w.dqlin, ws, w, s);
                 // dv: H_s = dS_out + sum_{t >= s} q_t G_t^T is the state of the
                 // reversed recurrence k' = q, v' = G; dk reads the same prefixes
                 // transposed (k' = G, v' = q), so it needs only the output kernel
                 if (e == hipSuccess)
                     e = linear_pass(dims, B, n, Hq, Hq, ws + w.krep, ws + w.qrev, ws + w.Grev, d_state_out,
                                     d_state_in, ws + w.ov, ws, w, s);
                 if (e == hipSuccess)
                     e = linear_pass(dims, B, n, Hq, Hq, ws + w.vrep, ws + w.Grev, ws + w.qrev, d_state_out,
                                     nullptr, ws + w.ok, ws, w, s, true);
                 return e;
             }),
             "backward linear-pass launch");

    lisa::BwdCombineArgs ca{};
    ca.z = gate;
    ca.dq_lin = ws + w.dqlin;
    ca.o_k = ws + w.ok;
    ca.o_v = ws + w.ov;
    ca.dq = dq;
    ca.dk = dk;
    ca.dv = dv;
    ca.B = B;
    ca.n = n;
    ca.Hq = Hq;
    ca.G = G;
    ca.d = D;
    LISA_HIP(timed(ST_BWD_COMBINE, s, [&] { return lisa::launch_bwd_combine(ca, dims->dtype, s); }),
             "backward combine launch");

    lisa::SparseBwdArgs sb{};
    sb.q = q;
    sb.k = k;
    sb.v = v;
    sb.z = gate;
    sb.dout = d_out;
    sb.rlin = ws + w.dqlin;
    sb.idx = topm;
    sb.dq = dq;
    sb.dk = dk;
    sb.dv = dv;
    sb.dgate = dgate;
    sb.B = B;
    sb.n = n;
    sb.Hq = Hq;
    sb.G = G;
    sb.r = Hq / G;
    sb.M = M;
    sb.scale = (float)(dims->softmax_scale > 0.0f ? (double)dims->softmax_scale : 1.0 / std::sqrt((double)D));
    if (dims->dtype == LISA_BF16) {
        sb.coef = reinterpret_cast<float *>(ws + w.coef);
        sb.sorted = reinterpret_cast<uint32_t *>(ws + w.sorted);
        LISA_HIP(timed(ST_BWD_SPARSE_Q, s, [&] { return lisa::launch_sparse_bwd_split(sb, D, 0, s); }),
                 "sparse backward (query side) launch");
        LISA_HIP(timed(ST_BWD_SORT, s, [&] { return lisa::launch_sparse_bwd_split(sb, D, 1, s); }),
                 "sparse backward (key sort) launch");
        LISA_HIP(timed(ST_BWD_SPARSE_KV, s, [&] { return lisa::launch_sparse_bwd_split(sb, D, 2, s); }),
                 "sparse backward (key side) launch");
    } else {
        LISA_HIP(timed(ST_BWD_SPARSE, s, [&] { return lisa::launch_sparse_bwd(sb, dims->dtype, D, s); }),
                 "sparse backward launch");
    }
    return ok();
}

lisa_status lisa_stage_timing(int32_t enable) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.enabled = enable != 0;
    return ok();
}

lisa_status lisa_stage_timing_read(int32_t max_stages, const char **names, int64_t *launches,
                                   double *total_ms, int32_t *n_stages, int32_t reset) {
    if (max_stages < 0) return fail(LISA_ERR_INVALID_ARGUMENT, "max_stages < 0");
    std::lock_guard<std::mutex> lk(g_timing.mu);
    for (auto &r : g_timing.pending) {
        float ms = 0.0f;
        LISA_HIP(hipEventSynchronize(r.b), "event synchronize");
        LISA_HIP(hipEventElapsedTime(&ms, r.a, r.b), "event elapsed time");
        g_timing.total_ms[r.stage] += ms;
        g_timing.launches[r.stage] += 1;
        g_timing.pool.push_back(r.a);
        g_timing.pool.push_back(r.b);
    }
    g_timing.pending.clear();
    for (int i = 0; i < ST_COUNT && i < max_stages; ++i) {
        if (names) names[i] = kStageNames[i];
        if (launches) launches[i] = g_timing.launches[i];
        if (total_ms) total_ms[i] = g_timing.total_ms[i];
    }
    if (n_stages) *n_stages = ST_COUNT;
    if (reset) {
        for (int i = 0; i < ST_COUNT; ++i) { g_timing.total_ms[i] = 0.0; g_timing.launches[i] = 0; }
    }
    return ok();
}

}  // extern "C"

