// Sparse softmax attention over the selected rows, fused with the gate.
//
// The Lightning Indexer's top-M tokens feed a sparse self-attention, and a
// gate fuses its output with the linear branch (arxivdaily page for arXiv
// 2607.19358, English abstract; gptget.net analysis, method-details section:
// learned gate g).  For one query position and one KV group (a "unit") the
// r query heads of the group share the selected K/V rows, so each gathered
// row is read once and used by all r heads:
//
//   S^T[key][head] = K_sel Q^T     (MFMA, A = gathered K rows, B = Q^T)
//   online softmax over keys per head (fp32, exp2 with the scale folded in)
//   O^T[dim][head] += V_sel^T P^T  (MFMA, A = V rows staged in LDS, B = P^T
//                                   taken straight from the S^T accumulators)
//
// The r heads are padded to the 16 columns of a 16x16x32 MFMA tile.  The M
// selected slots are split over the NW waves of the work-group (32 slots per
// step; prefill uses 4 waves per unit, decode 4 or 8, and 16 only for
// M > 512, since it has few units); the waves' partial (max, sum, O) are
// merged in LDS, then the gate gamma = sigmoid(z) mixes o_sparse with o_lin
// and the result is stored.
// Each step issues the gathered K fragment loads and the V row loads
// together, so both gathers are in flight before the first MFMA.
#include "common.hpp"
#include "kernels.hpp"

namespace lisa {
namespace {

constexpr int kChunk = 32;  // selected slots per wave step

typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2 f32x2_lo(f32x4 v) { return f32x2{v[0], v[1]}; }
__device__ __forceinline__ f32x2 f32x2_hi(f32x4 v) { return f32x2{v[2], v[3]}; }

template <typename T, int D, int NW>
struct SparseSmem {
    // row pad: bf16 32 bytes (the 4-row transposing reads of V^T are then
    // conflict-free), fp32 8 bytes
    static constexpr int kVStride = D + (Elt<T>::kBytes == 2 ? 16 : 2);
    static constexpr int kVBytes = NW * kChunk * kVStride * Elt<T>::kBytes;
    static constexpr int kMergeStride = 32 + 16 * (D + 1);  // max[16] sum[16] O[head][D+1]
    static constexpr int kMergeBytes = NW * kMergeStride * 4;
    static constexpr int kBytes = kVBytes > kMergeBytes ? kVBytes : kMergeBytes;
};

template <typename T, int D, bool DECODE, int NW>
__global__ __launch_bounds__(NW * 64) void sparse_gate_kernel(SparseArgs a) {
    using S = SparseSmem<T, D, NW>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::kBytes];
    constexpr int VS = S::kVStride;
    constexpr int KC = D / 32;  // K-steps of 32 over the head dim
    constexpr int MB = D / 16;  // 16-row blocks of O^T
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    // Logical unit: decode (b, g) -> b*G + g.  Prefill units are taken
    // group-major, and the XCD remap hands each XCD a contiguous range, so an
    // XCD's L2 only ever holds the K/V rows of one or two groups.
    const int lu = xcd_remap(blockIdx.x, gridDim.x);
    const int G = a.G, r = a.r, M = a.M;
    const int u = DECODE ? lu : (lu % (a.B * a.n)) * G + lu / (a.B * a.n);
    // The wave's slot range, and the selected positions of its first step,
    // loaded before anything that waits on the sequence length (a descriptor
    // over the unit's M entries; none for the window sets, which use no idx).
    const int per_wave = ((M + NW - 1) / NW + kChunk - 1) / kChunk * kChunk;
    const int s_begin = wave * per_wave, s_end = min(M, s_begin + per_wave);
    // (the 16-wave variant, at its register limit, reads them in the loop)
    constexpr bool kEarlyIdx = NW <= 8;
    int32_t idx0[2] = {0, 0};
    if constexpr (kEarlyIdx) {
        const rsrc_t irs = make_rsrc(a.window ? a.q : (const void *)(a.idx + (size_t)u * M),
                                     a.window ? 0u : (uint32_t)M * 4u);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            idx0[kb] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
                irs, (uint32_t)(s_begin + kb * 16 + (lane & 15)) * 4u, 0u, 0);
    }

    const T *qrows, *kbase, *vbase;
    int smax;    // largest valid key position of the unit (defensive bound on gathered rows)
    int nvalid;  // selected slots of the unit: min(M, visible tokens); the rest are -1
    const void *linp;
    const T *zp;
    T *outp;
    size_t lin_off;
    const int32_t *tb = nullptr;  // paged decode: this sequence's page-table row
    {
        if (DECODE) {
            const int b = u / G, g = u % G;
            // paged caches: rows are relative to the pool, packed: to the sequence
            const int64_t row0 = a.map.table ? 0 : a.cu[b];
            if (a.map.table) tb = a.map.table + (size_t)b * a.map.max_blocks;
            smax = cache_len(a.map, b, a.max_ctx) - 1;
            nvalid = min(M, smax + 1);
            qrows = reinterpret_cast<const T *>(a.q) + ((size_t)b * a.Hq + g * r) * D;
            kbase = reinterpret_cast<const T *>(a.k) + ((size_t)row0 * G + g) * D;
            vbase = reinterpret_cast<const T *>(a.v) + ((size_t)row0 * G + g) * D;
            zp = reinterpret_cast<const T *>(a.gate) + (size_t)b * a.Hq + g * r;
            lin_off = ((size_t)b * a.Hq + g * r) * D;
            outp = reinterpret_cast<T *>(a.out) + lin_off;
        } else {
            const int g = u % G, bt = u / G, b = bt / a.n;
            smax = a.past + bt % a.n;  // the query's position: keys 0..smax are visible
            nvalid = min(M, smax + 1);
            qrows = reinterpret_cast<const T *>(a.q) + ((size_t)bt * a.Hq + g * r) * D;
            kbase = reinterpret_cast<const T *>(a.k) + ((size_t)b * (a.past + a.n) * G + g) * D;
            vbase = reinterpret_cast<const T *>(a.v) + ((size_t)b * (a.past + a.n) * G + g) * D;
            zp = reinterpret_cast<const T *>(a.gate) + (size_t)bt * a.Hq + g * r;
            lin_off = ((size_t)bt * a.Hq + g * r) * D;
            outp = reinterpret_cast<T *>(a.out) + lin_off;
        }
        linp = a.lin;
    }
    const size_t rstride = (size_t)G * D;  // elements between consecutive token rows
    const int32_t *idxp = a.idx + (size_t)u * M;

    // Q^T fragments: column = head (zero beyond r), K = head dim.
    Frag<T> qf[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        if (col < r) qf[kc].load(qrows + (size_t)col * D + kc * 32 + grp * 8);
        else qf[kc].zero();
    }

    // The epilogue's gate logits and o_lin (thread t mixes elements
    // t + j*NW*64 of the unit's r x D outputs), through descriptors that read
    // zeros past the end.  Up to 8 waves they load now, in flight during the
    // gathers instead of after the merge; the 16-wave variant has no
    // registers to spare (1024 threads) and loads them in the epilogue.
    constexpr int NPF = (16 * D + NW * 64 - 1) / (NW * 64);  // r <= 16
    constexpr bool kEarly = NW <= 8;
    float zv[NPF], linv[NPF];
    constexpr uint32_t LB = DECODE ? 4u : Elt<T>::kBytes;  // o_lin is fp32 in decode
    const rsrc_t lrs = make_rsrc(reinterpret_cast<const unsigned char *>(linp) + lin_off * LB,
                                 (uint32_t)(r * D) * LB);
    const rsrc_t zrs = make_rsrc(zp, (uint32_t)r * Elt<T>::kBytes);
    auto load_epilogue = [&](int j) {
        const uint32_t e = (uint32_t)(threadIdx.x + j * NW * 64);
        const uint32_t hh = e / D;
        if constexpr (Elt<T>::kBytes == 2)
            zv[j] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(zrs, hh * 2u, 0u, 0) << 16);
        else
            zv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(zrs, hh * 4u, 0u, 0));
        if constexpr (LB == 4)
            linv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lrs, e * 4u, 0u, 0));
        else
            linv[j] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(lrs, e * 2u, 0u, 0) << 16);
    };
    if constexpr (kEarly) {
#pragma unroll
        for (int j = 0; j < NPF; ++j) load_epilogue(j);
    }

    f32x4 o[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] = f32x4{0, 0, 0, 0};
    float m_run = -INFINITY, l_run = 0.0f;

    T *vs = reinterpret_cast<T *>(smem) + (size_t)wave * kChunk * VS;
    const int s_stop = min(s_end, nvalid);
    // buffer descriptors over the unit's visible K and V rows: slots that are
    // padding or out of range read as zeros without a branch
    constexpr uint32_t EB = Elt<T>::kBytes;
    const uint32_t row_bytes = (uint32_t)rstride * EB;
    const uint32_t vis_bytes = DECODE && a.map.table ? (uint32_t)a.pool_rows * row_bytes
                                                     : (uint32_t)(smax + 1) * row_bytes;
    const rsrc_t krs = make_rsrc(kbase, vis_bytes), vrs = make_rsrc(vbase, vis_bytes);
    for (int cs = s_begin; cs < s_stop; cs += kChunk) {
        // --- issue both gathers: lane (grp, col) fetches, for key block kb,
        // 16-byte pieces kc*32 + grp*8 of the K row and of the V row of slot
        // cs + 16*kb + col -- the K pieces are MFMA A fragments as loaded ----
        Frag<T> kf[2][KC], vf8[2][KC];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int slot = cs + kb * 16 + col;
            const int s = slot >= s_stop ? -1
                          : a.window ? max(0, smax - M + 1) + slot
                                     : (kEarlyIdx && cs == s_begin ? idx0[kb] : idxp[slot]);
            const uint32_t rrow = DECODE && tb ? (uint32_t)cache_row(a.map, 0, tb, min(max(s, 0), max(smax, 0))) : (uint32_t)s;
            const uint32_t roff = (s >= 0 && s <= smax) ? rrow * row_bytes + grp * 8 * EB : kOffNone;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                frag_buf_load(kf[kb][kc], krs, roff + kc * 32 * EB);
                frag_buf_load(vf8[kb][kc], vrs, roff + kc * 32 * EB);
            }
        }
        // --- logits S^T for two 16-slot key blocks --------------------------
        f32x4 acc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            acc[kb] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) acc[kb] = mma16(kf[kb][kc], qf[kc], acc[kb]);
        }
        // rows of acc[kb] are slots cs + 16*kb + 4*grp + i; slots >= s_stop are padding
        float x[8];
        float cmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = cs + kb * 16 + grp * 4 + i < s_stop;
                const float v = ok ? acc[kb][i] * a.scale_log2 : -INFINITY;
                x[kb * 4 + i] = v;
                cmax = fmaxf(cmax, v);
            }
        }
        cmax = wave_max_across16(cmax);
        const float m_new = fmaxf(m_run, cmax);
        float p[8];
        float psum = 0.0f;
        float alpha = 1.0f;
        if (m_new == -INFINITY) {
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = 0.0f;
        } else {
            alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = __builtin_amdgcn_exp2f(x[e] - m_new);
                psum += p[e];
            }
        }
        psum = wave_sum_across16(psum);
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;

        // --- stage the 32 V rows in LDS (row-major, padded rows) ------------
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            unsigned char *row = reinterpret_cast<unsigned char *>(vs + (kb * 16 + col) * VS);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                unsigned char *dst = row + (kc * 32 + grp * 8) * Elt<T>::kBytes;
                if constexpr (Elt<T>::kBytes == 2) {
                    *reinterpret_cast<u32x4 *>(dst) = reinterpret_cast<const Frag<uint16_t> &>(vf8[kb][kc]).v;
                } else {
                    const Frag<float> &ff = reinterpret_cast<const Frag<float> &>(vf8[kb][kc]);
                    reinterpret_cast<u32x2 *>(dst)[0] = __builtin_bit_cast(u32x2, f32x2_lo(ff.lo));
                    reinterpret_cast<u32x2 *>(dst)[1] = __builtin_bit_cast(u32x2, f32x2_hi(ff.lo));
                    reinterpret_cast<u32x2 *>(dst)[2] = __builtin_bit_cast(u32x2, f32x2_lo(ff.hi));
                    reinterpret_cast<u32x2 *>(dst)[3] = __builtin_bit_cast(u32x2, f32x2_hi(ff.hi));
                }
            }
        }
        wave_lds_sync();
        // --- O^T += V^T P^T --------------------------------------------------
        Frag<T> pf;
        pf.set(p);  // K-slot e <-> chunk slot (e<4 ? 4*grp+e : 16+4*grp+e-4)
        if constexpr (Elt<T>::kBytes == 2 && NW <= 8) {
            // V^T fragments by the transposing read (as in the prefill
            // kernel): lane (col, grp) gets V[row][16 mb + col] for the rows
            // of its K-slots, 4 grp .. +3 and 16 + 4 grp .. +3 (the 16-wave
            // variant, at 128 VGPRs, keeps the element reads: this form
            // spilled 35 registers there)
            const unsigned char *vb = reinterpret_cast<const unsigned char *>(vs);
            constexpr int VRB = VS * 2;  // row bytes
            const int vr_base = (grp * 4 + (col >> 2)) * VRB + (col & 3) * 8;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const u32x2 lo = lds_read_tr16(vb + vr_base + mb * 32);
                const u32x2 hi = lds_read_tr16(vb + vr_base + 16 * VRB + mb * 32);
                Frag<T> vf;
                vf.v = u32x4{lo[0], lo[1], hi[0], hi[1]};
                o[mb] = mma16(vf, pf, o[mb]);
            }
        } else {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int dim = mb * 16 + col;
                T vv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int row = (e < 4) ? (grp * 4 + e) : (16 + grp * 4 + e - 4);
                    vv[e] = vs[row * VS + dim];
                }
                Frag<T> vf;
                vf.set_bits(vv);
                o[mb] = mma16(vf, pf, o[mb]);
            }
        }
        wave_lds_sync();
    }

    // --- merge the 4 waves -------------------------------------------------
    __syncthreads();
    float *mrg = reinterpret_cast<float *>(smem);
    constexpr int MS = S::kMergeStride;
    float *wm = mrg + wave * MS;  // [0..15] max, [16..31] sum, then O[head][D+1]
    if (grp == 0) {
        wm[col] = m_run;
        wm[16 + col] = l_run;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) wm[32 + col * (D + 1) + mb * 16 + grp * 4 + i] = o[mb][i];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NPF; ++j) {
        const int e = threadIdx.x + j * NW * 64;
        if (e >= r * D) break;
        if constexpr (!kEarly) load_epilogue(j);
        const int hh = e / D, dim = e % D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) mx = fmaxf(mx, mrg[w * MS + hh]);
        float num = 0.0f, den = 0.0f;
        if (mx != -INFINITY) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float *ww = mrg + w * MS;
                const float sc = __builtin_amdgcn_exp2f(ww[hh] - mx);
                den += ww[16 + hh] * sc;
                num += ww[32 + hh * (D + 1) + dim] * sc;
            }
        }
        const float osp = den > 0.0f ? num / den : 0.0f;
        const float gam = 1.0f / (1.0f + expf(-zv[j]));
        outp[e] = Elt<T>::from_f32(gam * osp + (1.0f - gam) * linv[j]);
    }
}

// ---- prefill, bf16: one wave per unit ------------------------------------
//
// Prefill has B*n*G units, far more than the chip has waves, so a unit gets
// a single wave that walks its M slots in steps of 32 with no cross-wave
// merge.
//
// Gathers are row-coalesced: D*2/16 consecutive lanes fetch one whole K (or
// V) row, so every group of four lanes reads one contiguous 64-byte piece.
// (Loading rows straight into MFMA fragment order instead puts four
// different rows under every four lanes, which the address path handles at
// well under half the rate.)  The rows are staged in LDS and read back in
// fragment order: K with plain 16-byte reads, V through the gfx950
// transposing read ds_read_b64_tr_b16.  In each 16-lane block that read
// gives lane l element l%4 of the 4-element row piece addressed by lane
// 4e + l/4, e = 0..3; with lane j addressing slot row (base + j/4), dims
// 16*mb + 4*(j%4), lane l receives V[base + e][16*mb + l%16] -- four
// K-elements of the A operand of O^T += V^T P^T, in the slot order P^T has
// in the S^T accumulators.  K and V of a step share one LDS region (K is
// read into registers before V overwrites it), and the next step's gathers
// are issued as soon as both have been copied out of their registers.

template <int D>
struct WaveSmem {
    static constexpr int kLPR = D * 2 / 16;      // lanes per gathered row
    static constexpr int kRPI = 64 / kLPR;       // rows per load instruction
    static constexpr int kNI = kChunk / kRPI;    // load instructions per 32 rows (per tensor)
    // row strides: 16-byte pad makes the 16-row fragment reads of K
    // conflict-free, 32-byte pad the 4-row transposing reads of V
    static constexpr int kKRow = D * 2 + 16;
    static constexpr int kVRow = D * 2 + 32;
    static constexpr int kBytes = kChunk * kVRow;
};

template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3)))
void sparse_prefill_wave_kernel(SparseArgs a) {
    using S = WaveSmem<D>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[S::kBytes];
    constexpr int KRB = S::kKRow, VRB = S::kVRow, NI = S::kNI, LPR = S::kLPR;
    constexpr int KC = D / 32;
    constexpr int MB = D / 16;
    const int lane = threadIdx.x;
    const int col = lane & 15, grp = lane >> 4;
    // group-major logical units, each XCD taking a contiguous range
    const int G = a.G, r = a.r, M = a.M;
    int u;
    if (a.split_lo > 0) {
        // one sequence, two XCDs per group: the first takes queries
        // [0, split_lo), whose rows span a smaller L2 footprint and gather
        // faster, the second [split_lo, n); blocks past an XCD's share exit
        const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3, sub = xcd & 1;
        const int cnt = sub ? a.n - a.split_lo : a.split_lo;
        if (j >= cnt) return;
        u = ((sub ? a.split_lo : 0) + j) * G + (xcd >> 1);
    } else {
        // group-major logical units, each XCD taking a contiguous range
        const int lu = xcd_remap(blockIdx.x, gridDim.x);
        u = (lu % (a.B * a.n)) * G + lu / (a.B * a.n);
    }
    const int g = u % G, bt = u / G, b = bt / a.n;
    const int smax = a.past + bt % a.n;       // the query's position: keys 0..smax are visible
    const int nvalid = min(M, smax + 1);
    const uint16_t *qrows = reinterpret_cast<const uint16_t *>(a.q) + ((size_t)bt * a.Hq + g * r) * D;
    const uint16_t *kbase = reinterpret_cast<const uint16_t *>(a.k) + ((size_t)b * (a.past + a.n) * G + g) * D;
    const uint16_t *vbase = reinterpret_cast<const uint16_t *>(a.v) + ((size_t)b * (a.past + a.n) * G + g) * D;
    const uint32_t row_bytes = (uint32_t)G * D * 2;
    const uint32_t vis_bytes = (uint32_t)(smax + 1) * row_bytes;
    const rsrc_t krs = make_rsrc(kbase, vis_bytes), vrs = make_rsrc(vbase, vis_bytes);
    const rsrc_t irs = make_rsrc(a.idx + (size_t)u * M, (uint32_t)M * 4u);

    Frag<uint16_t> qf[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        if (col < r) qf[kc].load(qrows + (size_t)col * D + kc * 32 + grp * 8);
        else qf[kc].zero();
    }

    // this lane fetches piece (lane % LPR) of the step's LDS rows
    // rho = (lane / LPR) * NI + i, i = 0..NI-1 (slot 32*j + rho)
    const int rsub = lane / LPR, piece = lane % LPR;
    const int rho0 = rsub * NI;
    const int nsteps = (nvalid + kChunk - 1) / kChunk;
    struct Idx { u32x4 v[NI / 4]; };
    const bool idx16 = (M & 3) == 0;  // index rows 16-byte aligned: vector loads
    const int wbase = max(0, smax - M + 1);  // window mode: slot i is position wbase + i
    auto load_idx = [&](int j) {
        Idx x;
        const uint32_t o = (uint32_t)(j * kChunk + rho0) * 4u;
        if (a.window) {
#pragma unroll
            for (int i = 0; i < NI; ++i) x.v[i / 4][i % 4] = (uint32_t)(wbase + j * kChunk + rho0 + i);
        } else if (idx16) {
#pragma unroll
            for (int h = 0; h < NI / 4; ++h) x.v[h] = buf_load16(irs, o + 16u * h);
        } else {
#pragma unroll
            for (int i = 0; i < NI; ++i)
                x.v[i / 4][i % 4] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(irs, o + 4u * i, 0u, 0);
        }
        return x;
    };
    u32x4 kp[NI], vp[NI];
    // Row offsets by 24-bit multiplies (positions and row bytes are below
    // 2^24).  An index past smax, -1 padding included, is clamped to smax + 1,
    // whose row starts at the descriptor's end and reads zeros (the host keeps
    // one row past the last inside 32 bits).  Slots past nvalid hold such
    // indices: -1 padding, or window positions past smax.
    const uint32_t uend = (uint32_t)smax + 1u;
    auto gather = [&](int j, const Idx &x) {
        uint32_t off[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) off[i] = __umul24(min(x.v[i / 4][i % 4], uend), row_bytes) + piece * 16;
#pragma unroll
        for (int i = 0; i < NI; ++i) kp[i] = buf_load16(krs, off[i]);
#pragma unroll
        for (int i = 0; i < NI; ++i) vp[i] = buf_load16(vrs, off[i]);
    };
    // gathers run one step ahead of the compute and index loads two steps
    // ahead; an index becomes an offset only when its gather is issued, so
    // waiting for it never waits for a gather still in flight
    gather(0, load_idx(0));
    Idx inext = load_idx(1);  // reads past the row return zeros, masked by slot < nvalid

    f32x4 o[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] = f32x4{0, 0, 0, 0};
    float m_run = -INFINITY, l_part = 0.0f;  // l_part: this lane's share of the row sum

    const uint32_t kw_base = (uint32_t)rho0 * KRB + piece * 16;   // K row writes
    const uint32_t vw_base = (uint32_t)rho0 * VRB + piece * 16;   // V row writes
    const uint32_t kr_base = (uint32_t)col * KRB + grp * 16;      // K fragment reads
    const uint32_t vr_base = (uint32_t)(grp * 4 + (col >> 2)) * VRB + (col & 3) * 8;  // V^T reads

    for (int j = 0; j < nsteps; ++j) {
        // K rows through LDS into fragment order, then V rows into the same
        // region (a wave's LDS accesses complete in issue order)
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4 *>(lds + kw_base + i * KRB) = kp[i];
        wave_lds_sync();
        Frag<uint16_t> kf[2][KC];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                kf[kb][kc].v = *reinterpret_cast<const u32x4 *>(lds + kr_base + kb * 16 * KRB + kc * 64);
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4 *>(lds + vw_base + i * VRB) = vp[i];
        if (j + 1 < nsteps) {
            gather(j + 1, inext);
            inext = load_idx(j + 2);
        }
        // logits S^T for the two 16-slot blocks
        f32x4 acc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            acc[kb] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) acc[kb] = mma16(kf[kb][kc], qf[kc], acc[kb]);
        }
        // online softmax over the 32 slots, per head (column); slots past
        // nvalid (only in the last step) get -inf
        float x[8];
        if ((j + 1) * kChunk <= nvalid) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = acc[e / 4][e % 4] * a.scale_log2;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[e] = j * kChunk + (e / 4) * 16 + grp * 4 + e % 4 < nvalid ? acc[e / 4][e % 4] * a.scale_log2
                                                                              : -INFINITY;
        }
        float cmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        cmax = wave_max_across16(cmax);
        // The reference m_run moves only when a logit passes it by more than
        // 8 (log2 units): p stays below 256, O / l does not depend on the
        // reference, and the rescale of O runs on few steps.  m_run is finite
        // from the first step on (slot 0 is valid).
        if (__ballot(cmax > m_run + 8.0f)) {
            const float m_new = fmaxf(m_run, cmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_part *= alpha;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
            m_run = m_new;
        }
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(x[e] - m_run);
            l_part += p[e];
        }
        Frag<uint16_t> pf;
        pf.set(p);  // K-element e <-> slot (e < 4 ? 4*grp + e : 16 + 4*grp + e - 4)
        wave_lds_sync();
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const u32x2 lo = lds_read_tr16(lds + vr_base + mb * 32);
            const u32x2 hi = lds_read_tr16(lds + vr_base + 16 * VRB + mb * 32);
            Frag<uint16_t> vt;
            vt.v = u32x4{lo[0], lo[1], hi[0], hi[1]};
            o[mb] = mma16(vt, pf, o[mb]);
        }
    }

    // gate epilogue: lane (col = head, grp) holds dims 16*mb + 4*grp + i
    const float l = wave_sum_across16(l_part);
    if (col < r) {
        const size_t base = ((size_t)bt * a.Hq + g * r + col) * D;
        const float z = bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(a.gate)[(size_t)bt * a.Hq + g * r + col]);
        const float gam = 1.0f / (1.0f + expf(-z));
        const float inv = l > 0.0f ? gam / l : 0.0f;
        const uint16_t *lin = reinterpret_cast<const uint16_t *>(a.lin) + base;
        uint16_t *outp = reinterpret_cast<uint16_t *>(a.out) + base;
        // o_lin lives in the output buffer: read all of it before any store
        u32x2 lvs[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) lvs[mb] = *reinterpret_cast<const u32x2 *>(lin + mb * 16 + grp * 4);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int d0 = mb * 16 + grp * 4;
            const u32x2 lv = lvs[mb];
            float res[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t bits = (lv[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                res[i] = o[mb][i] * inv + (1.0f - gam) * bf16_bits_to_f32(bits);
            }
            *reinterpret_cast<u32x2 *>(outp + d0) =
                u32x2{f32_to_bf16_bits(res[0]) | (f32_to_bf16_bits(res[1]) << 16),
                      f32_to_bf16_bits(res[2]) | (f32_to_bf16_bits(res[3]) << 16)};
        }
    }
}

// Share of a group's queries the first of its two XCDs takes (one
// sequence): the early queries' rows span less of the group's K/V, so that
// XCD gathers a little faster (16K, 7B shapes: 0.5 -> 0.577 ms, 0.52 ->
// 0.558 ms, 0.54 -> 0.563 ms, 0.58 -> 0.607 ms).
constexpr double kSplitFrac = 0.52;

template <typename T, int D>
hipError_t dispatch_d(const SparseArgs &a, bool decode, hipStream_t s) {
    const dim3 grid(a.units);
    if (!decode) {
        if constexpr (sizeof(T) == 2) {
            SparseArgs b = a;
            b.split_lo = 0;
            dim3 g2 = grid;
            if (a.B == 1 && a.G == 4 && a.n >= 4096) {  // see the kernel: two XCDs per group
                b.split_lo = (int)((double)a.n * kSplitFrac);
                g2 = dim3(8u * (unsigned)max(b.split_lo, a.n - b.split_lo));
            }
            launch_kernel((sparse_prefill_wave_kernel<D>), g2, dim3(64), 0, s, b);
        } else {
            launch_kernel((sparse_gate_kernel<T, D, false, 4>), grid, dim3(256), 0, s, a);
        }
    } else if (a.M <= 4 * kChunk) {
        launch_kernel((sparse_gate_kernel<T, D, true, 4>), grid, dim3(256), 0, s, a);
    } else if (a.M <= 16 * kChunk) {
        launch_kernel((sparse_gate_kernel<T, D, true, 8>), grid, dim3(512), 0, s, a);
    } else if constexpr (sizeof(T) == 4 && D == 128) {  // 16 waves of fp32 rows exceed the LDS
        launch_kernel((sparse_gate_kernel<T, D, true, 8>), grid, dim3(512), 0, s, a);
    } else {
        launch_kernel((sparse_gate_kernel<T, D, true, 16>), grid, dim3(1024), 0, s, a);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const SparseArgs &a, int d, bool decode, hipStream_t s) {
    if (a.units == 0) return hipSuccess;
    if (d == 128) return dispatch_d<T, 128>(a, decode, s);
    if (d == 64) return dispatch_d<T, 64>(a, decode, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_sparse_gate(const SparseArgs &a, int dtype, int d, bool decode, hipStream_t s) {
    return dtype == 1 ? dispatch<uint16_t>(a, d, decode, s) : dispatch<float>(a, d, decode, s);
}

}  // namespace lisa
