// Chunked linear attention for prefill (identity feature map, state matrix
// S_t: gptget.net analysis of arXiv 2607.19358, method-details section).
//
// The recurrence S_t = S_{t-1} + k_t v_t^T, o_t = q_t^T S_t is evaluated in
// chunks of C = 64 tokens, an exact rearrangement of it:
//   O_c = tril(Q_c K_c^T) V_c + Q_c S_{c-1},   S_c = S_{c-1} + K_c^T V_c.
// Three launches:
//   chunk_state   dS_c = K_c^T V_c per (batch, group, chunk)      [MFMA]
//   prefix_scan   S_{c-1} = S0 + sum_{c'<c} dS_c' (fp32 running sum), stored in
//                 the activation dtype for the MFMA consumer; state_out = S_n
//   chunk_output  O_c for the r heads of a group                  [MFMA]
// Within a group the r query heads share k and v, so with a zero initial
// state their states are equal and one prefix per group serves all r heads;
// with a caller-supplied initial state the prefix is kept per head.
// All states are stored transposed ([j][i], j = value dim) because that is
// the A-operand layout the output MFMA reads.
#include "common.hpp"
#include "kernels.hpp"

namespace lisa {
namespace {

constexpr int kC = 64;  // chunk length
#ifndef LISA_SCAN_U
#define LISA_SCAN_U 32
#endif

// Half-fragment helpers: 4 consecutive elements into the low / high half.
__device__ __forceinline__ void load_halves(Frag<uint16_t> &f, const uint16_t *p0, const uint16_t *p1) {
    const u32x2 a = *reinterpret_cast<const u32x2 *>(p0);
    const u32x2 b = *reinterpret_cast<const u32x2 *>(p1);
    f.v = u32x4{a[0], a[1], b[0], b[1]};
}
__device__ __forceinline__ void load_halves(Frag<float> &f, const float *p0, const float *p1) {
    f.lo = *reinterpret_cast<const f32x4 *>(p0);
    f.hi = *reinterpret_cast<const f32x4 *>(p1);
}

// The staging copies below issue all of a thread's loads before any LDS
// write, unconditionally (rows past `valid` re-read row valid - 1 and are
// zeroed afterwards; valid >= 1): a guarded load in the loop had compiled to
// one full wait per iteration.

// Copy a [64 tokens x D] tile (rows rstride apart in global memory; rows
// >= valid are zero) into LDS transposed: dst[dim * ts + tok].
template <typename T, int D>
__device__ __forceinline__ void stage_transposed(T *dst, int ts, const T *src, size_t rstride, int valid) {
    constexpr int EPC = 16 / Elt<T>::kBytes, CPR = D / EPC, N = kC * CPR / 256;
    static_assert(kC * CPR % 256 == 0, "whole rounds of 256 threads");
    u32x4 raw[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int q = threadIdx.x + k * 256, tok = q % kC, cc = q / kC;
        raw[k] = *reinterpret_cast<const u32x4 *>(src + (size_t)min(tok, valid - 1) * rstride + cc * EPC);
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int q = threadIdx.x + k * 256, tok = q % kC, cc = q / kC;
        const u32x4 v = tok < valid ? raw[k] : u32x4{0u, 0u, 0u, 0u};
        const T *e = reinterpret_cast<const T *>(&v);
#pragma unroll
        for (int i = 0; i < EPC; ++i) dst[(cc * EPC + i) * ts + tok] = e[i];
    }
}

// Copy a D x D matrix transposed into LDS rows ds apart: dst[j][i] = src[i][j].
template <typename T, int D>
__device__ __forceinline__ void stage_square_transposed(T *dst, int ds, const T *src) {
    constexpr int EPC = 16 / Elt<T>::kBytes, CPR = D / EPC, N = D * CPR / 256;
    static_assert(D * CPR % 256 == 0, "whole rounds of 256 threads");
    u32x4 raw[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int q = threadIdx.x + k * 256, row = q % D, cc = q / D;
        raw[k] = *reinterpret_cast<const u32x4 *>(src + (size_t)row * D + cc * EPC);
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int q = threadIdx.x + k * 256, row = q % D, cc = q / D;
        const T *e = reinterpret_cast<const T *>(&raw[k]);
#pragma unroll
        for (int i = 0; i < EPC; ++i) dst[(cc * EPC + i) * ds + row] = e[i];
    }
}

// Copy ROWS x D (row-major, rows rstride apart) into LDS rows ds apart; rows
// >= valid are zero.
template <typename T, int D, int ROWS>
__device__ __forceinline__ void stage_rows(T *dst, int ds, const T *src, size_t rstride, int valid) {
    constexpr int EPC = 16 / Elt<T>::kBytes, CPR = D / EPC, N = ROWS * CPR / 256;
    static_assert(ROWS * CPR % 256 == 0, "whole rounds of 256 threads");
    u32x4 raw[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int q = threadIdx.x + k * 256, row = q / CPR, cc = q % CPR;
        raw[k] = *reinterpret_cast<const u32x4 *>(src + (size_t)min(row, valid - 1) * rstride + cc * EPC);
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int q = threadIdx.x + k * 256, row = q / CPR, cc = q % CPR;
        *reinterpret_cast<u32x4 *>(dst + row * ds + cc * EPC) = row < valid ? raw[k] : u32x4{0u, 0u, 0u, 0u};
    }
}

template <typename T> constexpr int pad16() { return 16 / Elt<T>::kBytes; }  // 16-byte row pad

// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void chunk_state_kernel(LinearArgs a) {
    constexpr int TS = kC + pad16<T>();
    __shared__ __attribute__((aligned(16))) T kt[D * TS];
    __shared__ __attribute__((aligned(16))) T vt[D * TS];
    const int blk = blockIdx.x, c = blk % a.nC, bg = blk / a.nC, g = bg % a.G, b = bg / a.G;
    const int t0 = c * kC, valid = min(kC, a.n - t0);
    const size_t rstride = (size_t)a.G * D;
    const T *kp = reinterpret_cast<const T *>(a.k) + (((size_t)b * a.kv_rows + a.kv_off + t0) * a.G + g) * D;
    const T *vp = reinterpret_cast<const T *>(a.v) + (((size_t)b * a.kv_rows + a.kv_off + t0) * a.G + g) * D;
    stage_transposed<T, D>(kt, TS, kp, rstride, valid);
    stage_transposed<T, D>(vt, TS, vp, rstride, valid);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15, grp = lane >> 4;
    constexpr int NB = D / 16, TILES = NB * NB, TPW = TILES / 4;
    float *dst = a.dS + (size_t)blk * D * D;
    for (int tt = 0; tt < TPW; ++tt) {
        const int tile = wave * TPW + tt, mb = tile / NB, nb = tile % NB;
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < kC / 32; ++ks) {
            Frag<T> fa, fb;
            fa.load(vt + (mb * 16 + col) * TS + ks * 32 + grp * 8);  // V^T rows j
            fb.load(kt + (nb * 16 + col) * TS + ks * 32 + grp * 8);  // K columns i
            acc = mma16(fa, fb, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(mb * 16 + grp * 4 + i) * D + nb * 16 + col] = acc[i];
    }
}

// ---------------------------------------------------------------------------
template <typename T, int D, bool PH>  // PH: per-head prefixes (a.per_head)
__global__ __launch_bounds__(256) void prefix_scan_kernel(LinearArgs a) {
    constexpr int Q4 = D * D / 4;  // float4 columns per state
    constexpr int BPG = (Q4 + 255) / 256;
    const int bg = blockIdx.x / BPG, part = blockIdx.x % BPG;
    const int e4 = part * 256 + threadIdx.x;
    if (e4 >= Q4) return;
    const int g = bg % a.G, b = bg / a.G;
    const int j = (4 * e4) / D, i0 = (4 * e4) % D;  // transposed layout: element (j, i0..i0+3)
    // chunk c's float4 e4 of this group's dS: loads past the last chunk read
    // zeros through the descriptor, so a batch of U loads is always in flight
    const rsrc_t srs = make_rsrc(a.dS + (size_t)bg * a.nC * D * D, (uint32_t)a.nC * D * D * 4u);
    T *P = reinterpret_cast<T *>(a.P);
    f32x4 run = {0, 0, 0, 0};
    const size_t pbase = PH ? ((size_t)b * a.Hq + g * a.r) : ((size_t)b * a.G + g);
    // per-head initial states: this thread's four elements of each head's S0
    // (read transposed from [i][j] once) kept in a thread-private LDS slot
    extern __shared__ f32x4 s0l[];  // [r][256] when per_head
    if (PH) {
        for (int hh = 0; hh < a.r; ++hh) {
            const float *S0 = a.state_in + (pbase + hh) * D * D;
            f32x4 t;
#pragma unroll
            for (int q = 0; q < 4; ++q) t[q] = S0[(size_t)(i0 + q) * D + j];
            s0l[hh * 256 + threadIdx.x] = t;
        }
    }
    constexpr int U = LISA_SCAN_U;
#pragma unroll 1
    for (int c0 = 0; c0 < a.nC; c0 += U) {
        f32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            x[u] = __builtin_bit_cast(f32x4, buf_load16(srs, ((uint32_t)(c0 + u) * Q4 + (uint32_t)e4) * 16u));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u;
            if (c < a.nC) {
                if (!PH) {
                    T *dst = P + (pbase * a.nC + c) * D * D + 4 * e4;
#pragma unroll
                    for (int q = 0; q < 4; ++q) dst[q] = Elt<T>::from_f32(run[q]);
                } else {
                    // S_{c-1} = S0 + running sum
                    for (int hh = 0; hh < a.r; ++hh) {
                        const f32x4 s0 = s0l[hh * 256 + threadIdx.x];
                        T *dst = P + ((pbase + hh) * a.nC + c) * D * D + 4 * e4;
#pragma unroll
                        for (int q = 0; q < 4; ++q) dst[q] = Elt<T>::from_f32(run[q] + s0[q]);
                    }
                }
            }
            run += x[u];
        }
    }
    if (a.state_out) {
        for (int hh = 0; hh < a.r; ++hh) {
            const size_t h = (size_t)g * a.r + hh;
            float *so = a.state_out + ((size_t)b * a.Hq + h) * D * D;
            const float *S0 = a.state_in ? a.state_in + ((size_t)b * a.Hq + h) * D * D : nullptr;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t at = (size_t)(i0 + q) * D + j;
                so[at] = run[q] + (S0 ? S0[at] : 0.0f);
            }
        }
    }
}

// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void chunk_output_kernel(LinearArgs a) {
    constexpr int PD = pad16<T>();
    constexpr int KS = D + PD;    // K rows (natural)
    // bf16: V rows natural (32-byte pad), read transposed by ds_read_b64_tr_b16;
    // fp32: V^T staged transposed
    constexpr bool TRV = sizeof(T) == 2;
    constexpr int VRS = D + 32 / (int)sizeof(T);
    constexpr int VTS = kC + PD;
    constexpr int VBUF = TRV ? kC * VRS : D * VTS;
    constexpr int SS = D + PD;    // S^T rows
    __shared__ __attribute__((aligned(16))) T ks_[kC * KS];
    __shared__ __attribute__((aligned(16))) T vt_[VBUF];
    __shared__ __attribute__((aligned(16))) T st_[D * SS];
    const int blk = blockIdx.x, c = blk % a.nC, bg = blk / a.nC, g = bg % a.G, b = bg / a.G;
    const int t0 = c * kC, valid = min(kC, a.n - t0);
    const size_t rstride = (size_t)a.G * D;
    const T *kp = reinterpret_cast<const T *>(a.k) + (((size_t)b * a.kv_rows + a.kv_off + t0) * a.G + g) * D;
    const T *vp = reinterpret_cast<const T *>(a.v) + (((size_t)b * a.kv_rows + a.kv_off + t0) * a.G + g) * D;
    const T *P = reinterpret_cast<const T *>(a.P);
    stage_rows<T, D, kC>(ks_, KS, kp, rstride, valid);
    if constexpr (TRV) stage_rows<T, D, kC>(vt_, VRS, vp, rstride, valid);
    else stage_transposed<T, D>(vt_, VTS, vp, rstride, valid);
    const size_t pgrp = a.per_head ? ((size_t)b * a.Hq + g * a.r) : ((size_t)b * a.G + g);
    if (a.state_t) stage_square_transposed<T, D>(st_, SS, P + (pgrp * a.nC + c) * D * D);
    else stage_rows<T, D, D>(st_, SS, P + (pgrp * a.nC + c) * D * D, D, D);
    __syncthreads();

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, grp = lane >> 4;
    constexpr int MB = D / 16, KD = D / 32;
    const int tq = w * 16 + col;  // this lane's query row in the chunk (B-operand column)
    const T *qbase = reinterpret_cast<const T *>(a.q);
    T *obase = reinterpret_cast<T *>(a.out);
    // this lane's query row of every head: head hh + 1's fragments load while
    // head hh is computed
    const T *qrow = qbase + (((size_t)b * a.n + t0 + min(tq, valid - 1)) * a.Hq + g * a.r) * D + grp * 8;
    Frag<T> qn[KD];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) qn[ks].load(qrow + ks * 32);
    for (int hh = 0; hh < a.r; ++hh) {
        const int h = g * a.r + hh;
        if (a.per_head && hh > 0) {
            __syncthreads();
            if (a.state_t) stage_square_transposed<T, D>(st_, SS, P + ((pgrp + hh) * a.nC + c) * D * D);
            else stage_rows<T, D, D>(st_, SS, P + ((pgrp + hh) * a.nC + c) * D * D, D, D);
            __syncthreads();
        }
        Frag<T> qb[KD];
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
            qb[ks] = qn[ks];
            if (tq >= valid) qb[ks].zero();  // rows past the chunk end (their loads read row valid - 1)
        }
        // (unconditional: the last head loads its own row again)
        const int hn = min(hh + 1, a.r - 1);
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) qn[ks].load(qrow + (size_t)hn * D + ks * 32);
        // A^T[tk][tq] = K Q^T for key blocks at or below the diagonal
        f32x4 att[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            att[mt] = f32x4{0, 0, 0, 0};
            if (mt > w) continue;
#pragma unroll
            for (int ks = 0; ks < KD; ++ks) {
                Frag<T> kf;
                kf.load(ks_ + (mt * 16 + col) * KS + ks * 32 + grp * 8);
                att[mt] = mma16(kf, qb[ks], att[mt]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (mt * 16 + grp * 4 + i > tq) att[mt][i] = 0.0f;
        }
        f32x4 o[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) o[mb] = f32x4{0, 0, 0, 0};
        // intra-chunk: O^T += V^T A^T
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            if (2 * k2 > w) continue;
            float pv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pv[e] = att[2 * k2][e];
                pv[4 + e] = att[2 * k2 + 1][e];
            }
            Frag<T> pf;
            pf.set(pv);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                Frag<T> vf;
                if constexpr (TRV) {
                    // lane (col, grp): keys k2*32 + 4 grp .. +3 and +16.. of dim 16 mb + col
                    const T *p0 = vt_ + (k2 * 32 + grp * 4 + (col >> 2)) * VRS + mb * 16 + (col & 3) * 4;
                    const u32x2 lo = lds_read_tr16(p0), hi = lds_read_tr16(p0 + 16 * VRS);
                    vf.v = u32x4{lo[0], lo[1], hi[0], hi[1]};
                } else {
                    const T *row = vt_ + (mb * 16 + col) * VTS + k2 * 32 + grp * 4;
                    load_halves(vf, row, row + 16);
                }
                o[mb] = mma16(vf, pf, o[mb]);
            }
        }
        // inter-chunk: O^T += S^T Q^T
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                Frag<T> sf;
                sf.load(st_ + (mb * 16 + col) * SS + ks * 32 + grp * 8);
                o[mb] = mma16(sf, qb[ks], o[mb]);
            }
        }
        if (tq < valid) {
            T *dst = obase + (((size_t)b * a.n + t0 + tq) * a.Hq + h) * D;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[mb * 16 + grp * 4 + i] = Elt<T>::from_f32(o[mb][i]);
        }
    }
}

template <typename T, int D>
hipError_t run_state(const LinearArgs &a, hipStream_t s) {
    launch_kernel((chunk_state_kernel<T, D>), dim3(a.B * a.G * a.nC), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <typename T, int D>
hipError_t run_scan(const LinearArgs &a, hipStream_t s) {
    constexpr int BPG = (D * D / 4 + 255) / 256;
    if (a.per_head)
        launch_kernel((prefix_scan_kernel<T, D, true>), dim3(a.B * a.G * BPG), dim3(256),
                           (size_t)a.r * 256 * sizeof(f32x4), s, a);
    else
        launch_kernel((prefix_scan_kernel<T, D, false>), dim3(a.B * a.G * BPG), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <typename T, int D>
hipError_t run_output(const LinearArgs &a, hipStream_t s) {
    launch_kernel((chunk_output_kernel<T, D>), dim3(a.B * a.G * a.nC), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

#define LISA_LIN_DISPATCH(fn)                                                            \
    if (a.B * a.nC == 0) return hipSuccess;                                              \
    if (dtype == 1) return d == 128 ? fn<uint16_t, 128>(a, s) : fn<uint16_t, 64>(a, s);  \
    return d == 128 ? fn<float, 128>(a, s) : fn<float, 64>(a, s);

hipError_t launch_linear_chunk_state(const LinearArgs &a, int dtype, int d, hipStream_t s) {
    LISA_LIN_DISPATCH(run_state)
}
hipError_t launch_linear_prefix_scan(const LinearArgs &a, int dtype, int d, hipStream_t s) {
    LISA_LIN_DISPATCH(run_scan)
}
hipError_t launch_linear_chunk_output(const LinearArgs &a, int dtype, int d, hipStream_t s) {
    LISA_LIN_DISPATCH(run_output)
}
#undef LISA_LIN_DISPATCH

}  // namespace lisa
