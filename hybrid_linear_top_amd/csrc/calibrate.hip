// Roofline calibration kernels, for measurement only (not on the LISA path):
// a plain streaming copy and a read stream, which measure the HBM bandwidth
// a kernel can reach on this part, an MFMA loop, which measures the bf16
// matrix-core rate a kernel can reach, and random row gathers, which measure
// the rate at which the vector memory path delivers scattered 256-byte rows
// from a table of a given size (the sparse kernels' access pattern).  The benchmark reports each path's roofline fraction
// against these measured peaks next to the published ones.
#include "common.hpp"
#include "kernels.hpp"
#include "lisa.h"

namespace lisa {
namespace {

// 16-byte loads and stores, grid-stride, every wave reading whole lines,
// four loads in flight per thread
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                         int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        dst[i] = a;
        dst[i + stride] = b;
        dst[i + 2 * stride] = c;
        dst[i + 3 * stride] = d;
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

// The read-only stream: the same loads, folded into one word per thread that
// is stored only if it matches a value these inputs never produce.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4 *__restrict__ src, uint32_t *sink,
                                                         int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride)
        acc ^= src[i] ^ src[i + stride] ^ src[i + 2 * stride] ^ src[i + 3 * stride];
    for (; i < n16; i += stride) acc ^= src[i];
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x9E3779B9u) sink[blockIdx.x * 256 + threadIdx.x] = x;
}

// Each wave: iters rounds of 8 independent v_mfma_f32_16x16x32_bf16 on
// register operands.  The accumulators feed one store, made only when their
// sum is not finite (never, for these small operands), so nothing is dead.
constexpr int kChains = 8;
__global__ __launch_bounds__(256) void probe_mfma_kernel(float *sink, int iters) {
    const int lane = threadIdx.x & 63;
    Frag<uint16_t> a, b;
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 1e-3f * (float)((lane + 3 * i) & 7);
    a.set(x);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 1e-3f * (float)((lane * 5 + i) & 3);
    b.set(x);
    f32x4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = mma16(a, b, acc[c]);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    if (!__builtin_isfinite(s)) sink[blockIdx.x * 256 + threadIdx.x] = s;
}

constexpr int kMfmaBlocks = 2048;  // 8192 waves: 8 per SIMD

// Row gathers: random 256-byte rows of a table of nrows (a power of two),
// 16 lanes per row, each wave `iters` batches of 16 loads (64 rows, 16 KB)
// in flight together -- the access pattern of the sparse kernels' K/V
// gathers.  Rows come from a counter-based hash of (wave, load).
constexpr int kGatherBlocks = 16384;  // 65536 waves
constexpr int kGatherDepth = 16;
__global__ __launch_bounds__(256) void probe_gather_kernel(const u32x4 *__restrict__ table, uint32_t *sink,
                                                           uint32_t row_mask, int iters) {
    const int lane = threadIdx.x & 63;
    const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) >> 6;
    const uint32_t piece = lane & 15, rsub = lane >> 4;
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    for (int it = 0; it < iters; ++it) {
        u32x4 v[kGatherDepth];
#pragma unroll
        for (int i = 0; i < kGatherDepth; ++i) {
            uint32_t x = (wave * 0x9E3779B1u) ^ ((uint32_t)(it * kGatherDepth + i) * 0x85EBCA77u) ^ (rsub * 0xC2B2AE3Du);
            x ^= x >> 15;
            x *= 0x2C1B3C6Du;
            x ^= x >> 12;
            v[i] = table[(size_t)(x & row_mask) * 16 + piece];
        }
#pragma unroll
        for (int i = 0; i < kGatherDepth; ++i) acc ^= v[i];
    }
    const uint32_t y = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (y == 0x9E3779B9u) sink[threadIdx.x] = y;
}

}  // namespace
}  // namespace lisa

extern "C" lisa_status lisa_peak_probe(int32_t kind, const void *src, void *dst, size_t bytes, int32_t iters,
                                       double *work, lisa_stream_t stream) {
    if (!work) return LISA_ERR_INVALID_ARGUMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (kind == LISA_PROBE_COPY) {
        if (!src || !dst || bytes == 0 || bytes % 16 != 0 || ((reinterpret_cast<uintptr_t>(src) |
                                                               reinterpret_cast<uintptr_t>(dst)) & 15u))
            return LISA_ERR_INVALID_ARGUMENT;
        const int64_t n16 = (int64_t)(bytes / 16);
        const int64_t blocks = n16 / 256 < 8192 ? (n16 + 255) / 256 : 8192;
        lisa::launch_kernel(lisa::probe_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                            reinterpret_cast<const lisa::u32x4 *>(src), reinterpret_cast<lisa::u32x4 *>(dst), n16);
        *work = 2.0 * (double)bytes;
    } else if (kind == LISA_PROBE_READ) {
        if (!src || !dst || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u))
            return LISA_ERR_INVALID_ARGUMENT;
        const int64_t n16 = (int64_t)(bytes / 16);
        lisa::launch_kernel(lisa::probe_read_kernel, dim3(8192), dim3(256), 0, s,
                            reinterpret_cast<const lisa::u32x4 *>(src), static_cast<uint32_t *>(dst), n16);
        *work = (double)bytes;
    } else if (kind == LISA_PROBE_MFMA) {
        if (!dst || iters < 1 || bytes < (size_t)lisa::kMfmaBlocks * 256 * 4) return LISA_ERR_INVALID_ARGUMENT;
        lisa::launch_kernel(lisa::probe_mfma_kernel, dim3(lisa::kMfmaBlocks), dim3(256), 0, s,
                            static_cast<float *>(dst), (int)iters);
        *work = (double)lisa::kMfmaBlocks * 4 * iters * lisa::kChains * (2.0 * 16 * 16 * 32);
    } else if (kind == LISA_PROBE_GATHER) {
        const size_t rows = bytes / 256;
        if (!src || !dst || iters < 1 || bytes % 256 != 0 || rows == 0 || (rows & (rows - 1)) != 0 ||
            rows > ((size_t)1 << 31) || (reinterpret_cast<uintptr_t>(src) & 15u))
            return LISA_ERR_INVALID_ARGUMENT;
        lisa::launch_kernel(lisa::probe_gather_kernel, dim3(lisa::kGatherBlocks), dim3(256), 0, s,
                            reinterpret_cast<const lisa::u32x4 *>(src), static_cast<uint32_t *>(dst),
                            (uint32_t)(rows - 1), (int)iters);
        *work = (double)lisa::kGatherBlocks * 4 * iters * lisa::kGatherDepth * 1024.0;
    } else {
        return LISA_ERR_INVALID_ARGUMENT;
    }
    return hipGetLastError() == hipSuccess ? LISA_OK : LISA_ERR_HIP;
}
