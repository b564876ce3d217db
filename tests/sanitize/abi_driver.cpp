// Host-side driver for the C ABI's argument validation, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the
// device code is not instrumented).  Every call below is one that must
// return before any HIP call: workspace queries, rejected arguments, and
// empty (B == 0 or n == 0) calls.  Exits non-zero on the first status that
// differs from the expected one; a sanitizer report aborts the process.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "lisa.h"

namespace {
int failures = 0;

void expect(const char *what, lisa_status got, lisa_status want) {
    if (got != want) {
        std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want, lisa_last_error());
        ++failures;
    }
    // the message must be a terminated string on every path
    (void)std::strlen(lisa_last_error());
}

lisa_dims dims(int Hq, int Hkv, int d, int HI, int dI, int M, int dtype) {
    lisa_dims x;
    x.num_q_heads = Hq;
    x.num_kv_heads = Hkv;
    x.head_dim = d;
    x.idx_heads = HI;
    x.idx_dim = dI;
    x.top_m = M;
    x.chunk = 64;
    x.softmax_scale = 0.0f;
    x.dtype = dtype;
    return x;
}

// a 16-byte aligned address that is never dereferenced on these paths
void *const P = reinterpret_cast<void *>(uintptr_t{1} << 20);
float *const F = reinterpret_cast<float *>(P);
int32_t *const I = reinterpret_cast<int32_t *>(P);
const int64_t *const L64 = reinterpret_cast<const int64_t *>(P);
void *const MIS = reinterpret_cast<void *>((uintptr_t{1} << 20) + 8);
constexpr size_t BIG = size_t{1} << 40;
}  // namespace

int main() {
    const lisa_dims ok = dims(12, 2, 128, 4, 64, 256, LISA_BF16);
    size_t bytes = 0;

    // workspace queries
    expect("prefill ws", lisa_prefill_workspace_bytes(&ok, 1, 4096, &bytes), LISA_OK);
    expect("prefill ws null out", lisa_prefill_workspace_bytes(&ok, 1, 4096, nullptr), LISA_ERR_INVALID_ARGUMENT);
    expect("prefill ws null dims", lisa_prefill_workspace_bytes(nullptr, 1, 4096, &bytes), LISA_ERR_INVALID_ARGUMENT);
    expect("prefill ws n", lisa_prefill_workspace_bytes(&ok, 1, 32769, &bytes), LISA_ERR_UNSUPPORTED);
    expect("continue ws", lisa_prefill_continue_workspace_bytes(&ok, 2, 4096, 512, &bytes), LISA_OK);
    expect("continue ws past", lisa_prefill_continue_workspace_bytes(&ok, 1, 32768, 1, &bytes), LISA_ERR_UNSUPPORTED);
    expect("decode ws", lisa_decode_workspace_bytes(&ok, 16, 16385, &bytes), LISA_OK);
    expect("decode ws ctx", lisa_decode_workspace_bytes(&ok, 16, 65537, &bytes), LISA_ERR_UNSUPPORTED);
    expect("backward ws", lisa_prefill_backward_workspace_bytes(&ok, 1, 16384, &bytes), LISA_OK);

    // bad dims on every entry point
    const lisa_dims bad[] = {dims(12, 5, 128, 4, 64, 256, LISA_BF16), dims(12, 2, 96, 4, 64, 256, LISA_BF16),
                             dims(12, 2, 128, 9, 64, 256, LISA_BF16), dims(12, 2, 128, 4, 48, 256, LISA_BF16),
                             dims(12, 2, 128, 4, 64, 0, LISA_BF16), dims(12, 2, 128, 4, 64, 256, 7),
                             dims(34, 2, 128, 4, 64, 256, LISA_BF16)};
    for (const lisa_dims &d : bad) {
        expect("prefill bad dims",
               lisa_prefill(&d, 1, 64, P, P, P, P, P, P, P, nullptr, P, nullptr, nullptr, P, BIG, nullptr),
               d.num_kv_heads == 5 || d.top_m == 0 || d.dtype == 7 ? LISA_ERR_INVALID_ARGUMENT : LISA_ERR_UNSUPPORTED);
        lisa_status st = lisa_decode_step(&d, 2, L64, 100, P, P, P, P, P, P, P, F, P, nullptr, P, BIG, nullptr);
        if (st == LISA_OK) { std::fprintf(stderr, "decode accepted bad dims\n"); ++failures; }
        st = lisa_prefill_backward(&d, 1, 64, P, P, P, P, nullptr, I, P, nullptr, F, F, F, F, nullptr, P, BIG, nullptr);
        if (st == LISA_OK) { std::fprintf(stderr, "backward accepted bad dims\n"); ++failures; }
    }

    // null and misaligned pointers
    expect("prefill null q",
           lisa_prefill(&ok, 1, 64, nullptr, P, P, P, P, P, P, nullptr, P, nullptr, nullptr, P, BIG, nullptr),
           LISA_ERR_INVALID_ARGUMENT);
    expect("prefill misaligned out",
           lisa_prefill(&ok, 1, 64, P, P, P, P, P, P, P, nullptr, MIS, nullptr, nullptr, P, BIG, nullptr),
           LISA_ERR_INVALID_ARGUMENT);
    expect("prefill small workspace",
           lisa_prefill(&ok, 1, 64, P, P, P, P, P, P, P, nullptr, P, nullptr, nullptr, P, 16, nullptr),
           LISA_ERR_WORKSPACE);
    expect("continue null k", lisa_prefill_continue(&ok, 1, 10, 64, P, nullptr, P, P, P, P, P, nullptr, P, nullptr,
                                                    nullptr, P, BIG, nullptr),
           LISA_ERR_INVALID_ARGUMENT);
    expect("window null v",
           lisa_prefill_window(&ok, 1, 0, 64, P, P, nullptr, P, nullptr, P, nullptr, P, BIG, nullptr),
           LISA_ERR_INVALID_ARGUMENT);
    expect("decode misaligned cu",
           lisa_decode_step(&ok, 2, reinterpret_cast<const int64_t *>((uintptr_t{1} << 20) + 4), 100, P, P, P, P,
                            P, P, P, F, P, nullptr, P, BIG, nullptr),
           LISA_ERR_INVALID_ARGUMENT);
    expect("decode small workspace",
           lisa_decode_step(&ok, 2, L64, 100, P, P, P, P, P, P, P, F, P, nullptr, P, 16, nullptr), LISA_ERR_WORKSPACE);
    expect("decode window null state",
           lisa_decode_step_window(&ok, 2, L64, 100, P, P, P, P, nullptr, P, P, BIG, nullptr),
           LISA_ERR_INVALID_ARGUMENT);
    expect("paged block size",
           lisa_decode_step_paged(&ok, 2, I, I, 24, 8, 16, 100, P, P, P, P, P, P, P, F, P, nullptr, P, BIG, nullptr),
           LISA_ERR_UNSUPPORTED);
    expect("paged pool",
           lisa_decode_step_paged(&ok, 2, I, I, 4096, 1, 1024, 100, P, P, P, P, P, P, P, F, P, nullptr, P, BIG,
                                  nullptr),
           LISA_ERR_UNSUPPORTED);
    expect("backward null topm",
           lisa_prefill_backward(&ok, 1, 64, P, P, P, P, nullptr, nullptr, P, nullptr, F, F, F, F, nullptr, P, BIG,
                                 nullptr),
           LISA_ERR_INVALID_ARGUMENT);

    // spans beyond the 32-bit descriptor extents and launch sizes
    const lisa_dims wide = dims(2048, 2048, 128, 4, 64, 256, LISA_F32);
    expect("prefill span",
           lisa_prefill(&wide, 1, 32768, P, P, P, P, P, P, P, nullptr, P, nullptr, nullptr, P, BIG, nullptr),
           LISA_ERR_UNSUPPORTED);
    const lisa_dims dwide = dims(512, 512, 128, 4, 64, 256, LISA_F32);
    expect("decode span", lisa_decode_step(&dwide, 1, L64, 65536, P, P, P, P, P, P, P, F, P, nullptr, P, BIG, nullptr),
           LISA_ERR_UNSUPPORTED);
    const lisa_dims coef = dims(4096, 256, 128, 4, 64, 512, LISA_BF16);
    expect("backward coefficient span",
           lisa_prefill_backward(&coef, 1, 64, P, P, P, P, nullptr, I, P, nullptr, F, F, F, F, nullptr, P, BIG,
                                 nullptr),
           LISA_ERR_UNSUPPORTED);

    // empty calls enqueue nothing and succeed with null buffers
    expect("prefill empty",
           lisa_prefill(&ok, 0, 64, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr, nullptr, 0, nullptr),
           LISA_OK);
    expect("decode empty",
           lisa_decode_step(&ok, 0, nullptr, 100, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           LISA_OK);
    expect("backward empty",
           lisa_prefill_backward(&ok, 1, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           LISA_OK);

    // products of the largest 32-bit counts (checked in 128 bits)
    const lisa_dims many = dims(1 << 24, 1 << 24, 128, 4, 64, 256, LISA_BF16);
    expect("units product", lisa_prefill(&many, 2147483647, 1, P, P, P, P, P, P, P, nullptr, P, nullptr, nullptr, P,
                                         BIG, nullptr),
           LISA_ERR_UNSUPPORTED);
    expect("decode units product",
           lisa_decode_step(&many, 2147483647, L64, 65536, P, P, P, P, P, P, P, F, P, nullptr, P, BIG, nullptr),
           LISA_ERR_UNSUPPORTED);
    expect("paged pool product",
           lisa_decode_step_paged(&ok, 1, I, I, 4096, 2147483647, 2147483647, 65536, P, P, P, P, P, P, P, F, P,
                                  nullptr, P, BIG, nullptr),
           LISA_ERR_UNSUPPORTED);
    // every rejection message fits the thread-local buffer (long arguments)
    const lisa_dims huge = dims(2147483646, 1, 128, 4, 64, 256, LISA_BF16);
    (void)lisa_prefill(&huge, 2147483647, 2147483647, P, P, P, P, P, P, P, nullptr, P, nullptr, nullptr, P, BIG,
                       nullptr);
    std::printf("%s\n", lisa_build_info());
    std::printf(failures ? "FAILED %d\n" : "ok\n", failures);
    return failures ? 1 : 0;
}
