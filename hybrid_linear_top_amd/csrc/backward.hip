// Backward pass of the LISA layer for prefill (past = 0) on gfx950.
//
// The gradients of L = <d_out, out> + <d_state_out, state_out> follow the
// forward of the pages (gptget.net analysis of arXiv 2607.19358,
// method-details section) by the chain rule, with the selected sets held at
// the forward's (a top-M set is piecewise constant in q_I, k_I and w, which
// therefore get no gradient).  With G_t = (1 - gamma_t) d_out_t per head:
//
//  * gate:   dz = gamma (1 - gamma) (d_out . o_sp - d_out . o_lin), where
//            d_out . o_lin = q . (S_t d_out);
//  * linear branch, causal linear-attention passes run by the forward
//    chunked kernels on rearranged operands:
//      R_t  = S_t d_out_t               = attention(q'=d_out, k'=v, v'=k, S0'=S0^T),
//      dq_t = (1 - gamma) R_t;
//      dk_s = H_s v_s,  dv_s = H_s^T k_s, H_s = dS_out + sum_{t >= s} q_t G_t^T
//        -- in reversed time these are causal too, per head (each head its
//           own group there, then summed over the heads of a group):
//           dv: q'=k, k'=q, v'=G, S0'=dS_out, whose final state is d_state_in;
//           dk: q'=v, k'=G, v'=q carries the transposed state, so it is the
//           output kernel alone on dv's prefix states read transposed;
//  * sparse branch: ds = gamma p (d_out . v_s - d_out . o_sp),
//      dq += scale sum_s ds k_s,
//      dk_s += scale sum_h ds_h q_h,  dv_s += sum_h gamma_h p_h d_out_h.
//    bf16: a query-side kernel on MFMA (softmax statistics, ds, dq and the
//    per-slot coefficients) and a key side that sorts the entries of blocks
//    of positions by key and walks them, adding each key row about once per
//    block with fp32 atomics (details at the kernels).  fp32: one wave per
//    (position, group) with the atomics per selected key (sparse_bwd_kernel).
#include "common.hpp"
#include "kernels.hpp"

namespace lisa {
namespace {

constexpr int kMaxR = 16;  // query heads per group the sparse backward handles

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);  // row_half_mirror
    v += dpp_f32<0x140>(v);  // row_mirror
    return wave_sum_across16(v);
}

__device__ __forceinline__ float sigmoidf(float z) { return 1.0f / (1.0f + expf(-z)); }

// ---- operands of the linear-branch passes ------------------------------------
// One thread per 8 consecutive elements of [B, n, Hq, d] (d is a multiple of 8):
//   Grev = (1 - gamma) d_out,  qrev = q,  vrep = v of the head's group,
//          krep = k of the group, all at position n - 1 - t (reversed time).
template <typename T>
struct alignas(16) Vec8 {
    T x[8];
};

template <typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdPrepArgs a) {
    const int64_t total = (int64_t)a.B * a.n * a.Hq * a.d / 8;
    const int64_t e8 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e8 >= total) return;
    const int64_t e = e8 * 8;
    const int dd = (int)(e % a.d);
    int64_t r = e / a.d;
    const int h = (int)(r % a.Hq);
    r /= a.Hq;
    const int t = (int)(r % a.n), b = (int)(r / a.n);
    const int g = (int)(((int64_t)h * a.G) / a.Hq);
    using V = Vec8<T>;
    const float gam = sigmoidf(Elt<T>::to_f32(reinterpret_cast<const T *>(a.z)[((size_t)b * a.n + t) * a.Hq + h]));
    const V dov = *reinterpret_cast<const V *>(reinterpret_cast<const T *>(a.dout) + e);
    const V qv = *reinterpret_cast<const V *>(reinterpret_cast<const T *>(a.q) + e);
    const size_t kv = (((size_t)b * a.n + t) * a.G + g) * a.d + dd;
    const V kvv = *reinterpret_cast<const V *>(reinterpret_cast<const T *>(a.k) + kv);
    const V vvv = *reinterpret_cast<const V *>(reinterpret_cast<const T *>(a.v) + kv);
    V gv;
#pragma unroll
    for (int i = 0; i < 8; ++i) gv.x[i] = Elt<T>::from_f32((1.0f - gam) * Elt<T>::to_f32(dov.x[i]));
    const size_t rev = (((size_t)b * a.n + (a.n - 1 - t)) * a.Hq + h) * a.d + dd;
    *reinterpret_cast<V *>(reinterpret_cast<T *>(a.Grev) + rev) = gv;
    *reinterpret_cast<V *>(reinterpret_cast<T *>(a.qrev) + rev) = qv;
    *reinterpret_cast<V *>(reinterpret_cast<T *>(a.vrep) + rev) = vvv;
    *reinterpret_cast<V *>(reinterpret_cast<T *>(a.krep) + rev) = kvv;
}

// [B*H] d x d fp32 matrices transposed (dst[m][j][i] = src[m][i][j])
__global__ __launch_bounds__(256) void transpose_states_kernel(const float *src, float *dst, int64_t nmat, int d) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= nmat * d * d) return;
    const int64_t m = e / ((int64_t)d * d);
    const int i = (int)((e / d) % d), j = (int)(e % d);
    dst[(m * d + j) * d + i] = src[e];
}

// dq = (1 - gamma) dq_lin; dk[b,t,g] = sum_{h in g} o_k[b, n-1-t, h]; dv
// likewise (fp32); one thread per 8 consecutive elements
template <typename T>
__global__ __launch_bounds__(256) void bwd_combine_kernel(BwdCombineArgs a) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    const int64_t nq = (int64_t)a.B * a.n * a.Hq * a.d;
    const int64_t nk = (int64_t)a.B * a.n * a.G * a.d;
    using V = Vec8<T>;
    if (e < nq) {
        const V x = *reinterpret_cast<const V *>(reinterpret_cast<const T *>(a.dq_lin) + e);
        const float om = 1.0f - sigmoidf(Elt<T>::to_f32(reinterpret_cast<const T *>(a.z)[e / a.d]));
        f32x4 lo, hi;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo[i] = om * Elt<T>::to_f32(x.x[i]);
            hi[i] = om * Elt<T>::to_f32(x.x[4 + i]);
        }
        *reinterpret_cast<f32x4 *>(a.dq + e) = lo;
        *reinterpret_cast<f32x4 *>(a.dq + e + 4) = hi;
    }
    if (e >= nk) return;
    const int dd = (int)(e % a.d);
    int64_t r = e / a.d;
    const int g = (int)(r % a.G);
    r /= a.G;
    const int t = (int)(r % a.n), b = (int)(r / a.n);
    const int rr = a.Hq / a.G;
    float sk[8], sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sk[i] = sv[i] = 0.0f;
    for (int j = 0; j < rr; ++j) {
        const size_t at = (((size_t)b * a.n + (a.n - 1 - t)) * a.Hq + g * rr + j) * a.d + dd;
        const V ok = *reinterpret_cast<const V *>(reinterpret_cast<const T *>(a.o_k) + at);
        const V ov = *reinterpret_cast<const V *>(reinterpret_cast<const T *>(a.o_v) + at);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sk[i] += Elt<T>::to_f32(ok.x[i]);
            sv[i] += Elt<T>::to_f32(ov.x[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; i += 4) {
        *reinterpret_cast<f32x4 *>(a.dk + e + i) = f32x4{sk[i], sk[i + 1], sk[i + 2], sk[i + 3]};
        *reinterpret_cast<f32x4 *>(a.dv + e + i) = f32x4{sv[i], sv[i + 1], sv[i + 2], sv[i + 3]};
    }
}

// ---- sparse branch and gate ----------------------------------------------------
// One wave per unit (b, t, g).  LDS: q and d_out rows of the r heads (fp32),
// then per slot and head the logit / softmax weight and d_out . v / ds.
//  A. lane = slot: each lane reads its key's K and V rows and forms the r
//     logits and the r dot products d_out_h . v_s;
//  B. per head: max, normaliser, E_h = d_out . o_sp = sum_s p d_out . v_s,
//     ds = gamma p (d_out . v_s - E_h); the gate gradient;
//  C. lane = head dims: a loop over the slots accumulates dq and adds the
//     key rows' dk, dv with fp32 atomics.
template <typename T, int D>
__global__ __launch_bounds__(64) void sparse_bwd_kernel(SparseBwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int DPL = D / 64;  // head dims per lane in part C
    const int lane = threadIdx.x;
    const int u = blockIdx.x;
    const int G = a.G, r = a.r, M = a.M, n = a.n, Hq = a.Hq;
    const int g = u % G, bt = u / G, t = bt % n, b = bt / n;
    float *qs = lds, *dos = qs + r * D, *pl = dos + r * D, *dl = pl + M * r;
    const size_t hrow = ((size_t)bt * Hq + g * r) * D;  // row of the group's first head
    const T *qp = reinterpret_cast<const T *>(a.q) + hrow;
    const T *dop = reinterpret_cast<const T *>(a.dout) + hrow;
    for (int e = lane; e < r * D; e += 64) {
        qs[e] = Elt<T>::to_f32(qp[e]);
        dos[e] = Elt<T>::to_f32(dop[e]);
    }
    float gam[kMaxR];
#pragma unroll
    for (int h = 0; h < kMaxR; ++h)
        gam[h] = h < r ? sigmoidf(Elt<T>::to_f32(reinterpret_cast<const T *>(a.z)[(size_t)bt * Hq + g * r + h])) : 0.0f;
    wave_lds_sync();
    const int32_t *idxp = a.idx + (size_t)u * M;
    const size_t rs = (size_t)G * D;  // elements between consecutive key rows
    const T *kb = reinterpret_cast<const T *>(a.k) + ((size_t)b * n * G + g) * D;
    const T *vb = reinterpret_cast<const T *>(a.v) + ((size_t)b * n * G + g) * D;

    // ---- A: logits and d_out . v per slot ------------------------------------------
    float mrun[kMaxR];
#pragma unroll
    for (int h = 0; h < kMaxR; ++h) mrun[h] = -INFINITY;
    for (int c0 = 0; c0 < M; c0 += 64) {
        const int slot = c0 + lane;
        const int s = slot < M ? idxp[slot] : -1;
        const bool ok = s >= 0 && s <= t;  // sets are the forward's; anything else is skipped
        float lg[kMaxR], ov[kMaxR];
#pragma unroll
        for (int h = 0; h < kMaxR; ++h) lg[h] = ov[h] = 0.0f;
        if (ok) {
            const T *kr = kb + (size_t)s * rs, *vr = vb + (size_t)s * rs;
            for (int p = 0; p < D; p += 4) {
                float kf[4], vf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kf[i] = Elt<T>::to_f32(kr[p + i]);
                    vf[i] = Elt<T>::to_f32(vr[p + i]);
                }
#pragma unroll
                for (int h = 0; h < kMaxR; ++h) {
                    if (h < r) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            lg[h] = fmaf(qs[h * D + p + i], kf[i], lg[h]);
                            ov[h] = fmaf(dos[h * D + p + i], vf[i], ov[h]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < kMaxR; ++h) {
            if (h < r) {
                const float x = ok ? lg[h] * a.scale : -INFINITY;
                if (slot < M) {
                    pl[slot * r + h] = x;
                    dl[slot * r + h] = ov[h];
                }
                mrun[h] = fmaxf(mrun[h], wave_max(x));
            }
        }
    }
    wave_lds_sync();

    // ---- B: softmax weights, E_h, ds, the gate ---------------------------------
    float lsum[kMaxR], eh[kMaxR];
#pragma unroll
    for (int h = 0; h < kMaxR; ++h) lsum[h] = eh[h] = 0.0f;
    for (int slot = lane; slot < M; slot += 64) {
#pragma unroll
        for (int h = 0; h < kMaxR; ++h) {
            if (h < r) {
                const float x = pl[slot * r + h];
                const float p = x == -INFINITY ? 0.0f : expf(x - mrun[h]);
                pl[slot * r + h] = p;
                lsum[h] += p;
            }
        }
    }
#pragma unroll
    for (int h = 0; h < kMaxR; ++h)
        if (h < r) lsum[h] = wave_sum(lsum[h]);
    for (int slot = lane; slot < M; slot += 64) {
#pragma unroll
        for (int h = 0; h < kMaxR; ++h) {
            if (h < r) {
                const float p = lsum[h] > 0.0f ? pl[slot * r + h] / lsum[h] : 0.0f;
                pl[slot * r + h] = p;
                eh[h] = fmaf(p, dl[slot * r + h], eh[h]);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < kMaxR; ++h)
        if (h < r) eh[h] = wave_sum(eh[h]);
    for (int slot = lane; slot < M; slot += 64) {
#pragma unroll
        for (int h = 0; h < kMaxR; ++h)
            if (h < r) dl[slot * r + h] = gam[h] * pl[slot * r + h] * (dl[slot * r + h] - eh[h]);
    }
    {
        // d_out . o_lin = d_out . S_t^T q = q . (S_t d_out)
        const T *rlp = reinterpret_cast<const T *>(a.rlin) + hrow;
#pragma unroll
        for (int h = 0; h < kMaxR; ++h) {
            if (h < r) {
                float dot = 0.0f;
                for (int dd = lane; dd < D; dd += 64) dot = fmaf(qs[h * D + dd], Elt<T>::to_f32(rlp[h * D + dd]), dot);
                dot = wave_sum(dot);
                if (lane == 0) a.dgate[(size_t)bt * Hq + g * r + h] = gam[h] * (1.0f - gam[h]) * (eh[h] - dot);
            }
        }
    }
    wave_lds_sync();

    // ---- C: dq of the r heads, dk / dv of every selected key -------------------
    // lane covers dims lane + 64 j, so each atomic instruction adds one
    // contiguous run of 64 floats; the K rows of kU slots load together
    constexpr int kU = 8;
    float qd[kMaxR][DPL], sd[kMaxR][DPL], dqa[kMaxR][DPL];
#pragma unroll
    for (int h = 0; h < kMaxR; ++h)
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
            const int dd = lane + 64 * j;
            qd[h][j] = h < r ? qs[h * D + dd] : 0.0f;
            sd[h][j] = h < r ? gam[h] * dos[h * D + dd] : 0.0f;
            dqa[h][j] = 0.0f;
        }
    for (int slot0 = 0; slot0 < M; slot0 += kU) {
        int sv[kU];
        float kd[kU][DPL];
#pragma unroll
        for (int uu = 0; uu < kU; ++uu) {
            const int slot = slot0 + uu;
            const int s = slot < M ? idxp[slot] : -1;
            sv[uu] = (s >= 0 && s <= t) ? s : -1;
#pragma unroll
            for (int j = 0; j < DPL; ++j)
                kd[uu][j] = Elt<T>::to_f32(kb[(size_t)max(sv[uu], 0) * rs + lane + 64 * j]);
        }
#pragma unroll
        for (int uu = 0; uu < kU; ++uu) {
            const int s = sv[uu];
            if (s < 0) continue;
            const int slot = slot0 + uu;
            float gk[DPL], gv[DPL];
#pragma unroll
            for (int j = 0; j < DPL; ++j) gk[j] = gv[j] = 0.0f;
#pragma unroll
            for (int h = 0; h < kMaxR; ++h) {
                if (h < r) {
                    const float ds = dl[slot * r + h], p = pl[slot * r + h];
#pragma unroll
                    for (int j = 0; j < DPL; ++j) {
                        dqa[h][j] = fmaf(ds, kd[uu][j], dqa[h][j]);
                        gk[j] = fmaf(ds, qd[h][j], gk[j]);
                        gv[j] = fmaf(p, sd[h][j], gv[j]);
                    }
                }
            }
            const size_t row = (((size_t)b * n + s) * G + g) * D + lane;
#pragma unroll
            for (int j = 0; j < DPL; ++j) {
                unsafeAtomicAdd(a.dk + row + 64 * j, a.scale * gk[j]);
                unsafeAtomicAdd(a.dv + row + 64 * j, gv[j]);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < kMaxR; ++h)
        if (h < r)
#pragma unroll
            for (int j = 0; j < DPL; ++j) a.dq[hrow + h * D + lane + 64 * j] += a.scale * dqa[h][j];
}

// ---- sparse branch, bf16: query side on MFMA, key side by a sorted walk -----
//
// Query side (sparse_bwd_q_kernel), one wave per unit (b, t, g), two sweeps
// over the unit's selected slots in steps of 32, each step gathering the K
// and V rows into LDS (row-coalesced, as the forward does):
//   sweep 1: S^T = K_sel Q^T and DP^T = V_sel dO^T on MFMA; per head the
//            running max, the normaliser l and E = sum p (dO . v) (= dO . o_sp)
//            with online rescaling;
//   sweep 2: the same two products again, p = exp(x - m) / l,
//            ds = gamma p (dO . v - E); the per-slot coefficients (scale ds,
//            gamma p) of every head go to the workspace for the key side, and
//            dq^T += K_sel^T ds^T on MFMA (K read back transposed from LDS).
// The gate gradient is gamma (1 - gamma) (E - dO . o_lin).
//
// Key side (sparse_bwd_sort_kernel, sparse_bwd_walk_kernel): the
// (key, position, slot) entries of a block of consecutive positions of one
// group are sorted by key, and waves walk contiguous stretches of them:
//   dk_s += sum_h (scale ds_h) q_h,  dv_s += sum_h (gamma p_h) dO_h
// accumulating while the key stays the same and adding the sum into the key's
// row with fp32 atomics when it changes.  Neighbouring positions share many
// selected keys, so a key row is added about once per block instead of once
// per selecting position (the atomics' throughput is what bounds the
// one-wave-per-position form).

template <int D>
__global__ __launch_bounds__(64) void sparse_bwd_q_kernel(SparseBwdArgs a) {
    constexpr int LPR = D * 2 / 16;   // lanes per gathered row (16 bytes each)
    constexpr int RPI = 64 / LPR;     // rows per load instruction
    constexpr int NI = 32 / RPI;      // load instructions per 32 rows (per tensor)
    constexpr int KC = D / 32, MB = D / 16;
    constexpr int KRB = D * 2 + 32;   // K rows: fragment reads and transposed reads
    constexpr int VRB = D * 2 + 16;   // V rows: fragment reads
    __shared__ __attribute__((aligned(16))) unsigned char lds[32 * KRB + 32 * VRB + 32 * 4];
    unsigned char *ldk = lds, *ldv = lds + 32 * KRB;
    uint32_t *flg = reinterpret_cast<uint32_t *>(lds + 32 * KRB + 32 * VRB);
    const int lane = threadIdx.x, col = lane & 15, grp = lane >> 4;
    const int G = a.G, r = a.r, M = a.M, n = a.n;
    // group-major units, a contiguous range per XCD (as in the forward)
    const int lu = xcd_remap(blockIdx.x, gridDim.x);
    const int u = (lu % (a.B * n)) * G + lu / (a.B * n);
    const int g = u % G, bt = u / G, b = bt / n, t = bt % n;
    const int nvalid = min(M, t + 1);
    const size_t hrow = ((size_t)bt * a.Hq + g * r) * D;
    const uint16_t *qrows = reinterpret_cast<const uint16_t *>(a.q) + hrow;
    const uint16_t *dorows = reinterpret_cast<const uint16_t *>(a.dout) + hrow;
    const uint16_t *kbase = reinterpret_cast<const uint16_t *>(a.k) + ((size_t)b * n * G + g) * D;
    const uint16_t *vbase = reinterpret_cast<const uint16_t *>(a.v) + ((size_t)b * n * G + g) * D;
    const uint32_t row_bytes = (uint32_t)G * D * 2;
    const uint32_t vis_bytes = (uint32_t)(t + 1) * row_bytes;
    const rsrc_t krs = make_rsrc(kbase, vis_bytes), vrs = make_rsrc(vbase, vis_bytes);
    const rsrc_t irs = make_rsrc(a.idx + (size_t)u * M, (uint32_t)M * 4u);
    const float scale_log2 = a.scale * 1.4426950408889634f;

    Frag<uint16_t> qf[KC], dof[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        if (col < r) {
            qf[kc].load(qrows + (size_t)col * D + kc * 32 + grp * 8);
            dof[kc].load(dorows + (size_t)col * D + kc * 32 + grp * 8);
        } else {
            qf[kc].zero();
            dof[kc].zero();
        }
    }
    const float gam = col < r ? sigmoidf(bf16_bits_to_f32(
                                    reinterpret_cast<const uint16_t *>(a.z)[(size_t)bt * a.Hq + g * r + col]))
                              : 0.0f;

    // this lane fetches piece (lane % LPR) of rows rho0 .. rho0 + NI - 1 of a step
    const int rsub = lane / LPR, piece = lane % LPR, rho0 = rsub * NI;
    const int nsteps = (nvalid + 31) / 32;
    u32x4 kp[NI], vp[NI];
    // the slots' indices load two steps ahead of their gathers (vector loads
    // when the rows are 16-byte aligned), so no gather waits on an index load
    struct Idx { u32x4 v[NI / 4]; };
    const bool idx16 = (M & 3) == 0;
    auto load_idx = [&](int j) {
        Idx x;
        const uint32_t o = (uint32_t)(j * 32 + rho0) * 4u;
        if (idx16) {
#pragma unroll
            for (int h = 0; h < NI / 4; ++h) x.v[h] = buf_load16(irs, o + 16u * h);
        } else {
#pragma unroll
            for (int i = 0; i < NI; ++i)
                x.v[i / 4][i % 4] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(irs, o + 4u * i, 0u, 0);
        }
        return x;
    };
    Idx inext;
    uint32_t okbits = 0;  // bit i: row rho0 + i of the step in flight is a valid slot
    // row offsets by clamped 24-bit products: an index past t (or -1) reads
    // the row past the last, zeros through the descriptor
    const uint32_t uend = (uint32_t)t + 1u;
    auto gather = [&](int j, const Idx &x) {
        okbits = 0;
        uint32_t off[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t si = x.v[i / 4][i % 4];
            const bool ok = j * 32 + rho0 + i < nvalid && si <= (uint32_t)t;
            okbits |= ok ? (1u << i) : 0u;
            off[i] = __umul24(min(si, uend), row_bytes) + piece * 16;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) kp[i] = buf_load16(krs, off[i]);
#pragma unroll
        for (int i = 0; i < NI; ++i) vp[i] = buf_load16(vrs, off[i]);
    };
    auto start = [&]() {  // a sweep's first gather, and the next step's indices in flight
        gather(0, load_idx(0));
        inext = load_idx(1);
    };
    const uint32_t kw = (uint32_t)rho0 * KRB + piece * 16, vw = (uint32_t)rho0 * VRB + piece * 16;
    const uint32_t kfr = (uint32_t)col * KRB + grp * 16, vfr = (uint32_t)col * VRB + grp * 16;
    const uint32_t ktr = (uint32_t)(grp * 4 + (col >> 2)) * KRB + (col & 3) * 8;
    // stage the gathered rows of step j, issue the gather of step j + 1, and
    // form S^T (acc) and DP^T (dacc) of the step's two 16-slot blocks; valid[e]
    // tells whether slot kb*16 + 4*grp + i (e = 4 kb + i) is a selected key
    f32x4 acc[2], dacc[2];
    bool valid[8];
    auto step = [&](int j) {
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            *reinterpret_cast<u32x4 *>(ldk + kw + i * KRB) = kp[i];
            *reinterpret_cast<u32x4 *>(ldv + vw + i * VRB) = vp[i];
            if (piece == 0) flg[rho0 + i] = (okbits >> i) & 1u;
        }
        if (j + 1 < nsteps) {
            gather(j + 1, inext);
            inext = load_idx(j + 2);
        }
        wave_lds_sync();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            acc[kb] = f32x4{0, 0, 0, 0};
            dacc[kb] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                Frag<uint16_t> kf, vf;
                kf.v = *reinterpret_cast<const u32x4 *>(ldk + kfr + kb * 16 * KRB + kc * 64);
                vf.v = *reinterpret_cast<const u32x4 *>(ldv + vfr + kb * 16 * VRB + kc * 64);
                acc[kb] = mma16(kf, qf[kc], acc[kb]);
                dacc[kb] = mma16(vf, dof[kc], dacc[kb]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) valid[kb * 4 + i] = flg[kb * 16 + grp * 4 + i] != 0u;
        }
    };

    // ---- sweep 1: max, normaliser and E per head (column) ----------------------
    float m_run = -INFINITY, l_part = 0.0f, e_part = 0.0f;
    start();
    for (int j = 0; j < nsteps; ++j) {
        step(j);
        float x[8], cmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[e] = valid[e] ? acc[e >> 2][e & 3] * scale_log2 : -INFINITY;
            cmax = fmaxf(cmax, x[e]);
        }
        cmax = wave_max_across16(cmax);
        const float m_new = fmaxf(m_run, cmax);
        if (m_new != -INFINITY) {
            const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_part *= alpha;
            e_part *= alpha;
            m_run = m_new;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = valid[e] ? __builtin_amdgcn_exp2f(x[e] - m_run) : 0.0f;
                l_part += p;
                e_part = fmaf(p, dacc[e >> 2][e & 3], e_part);
            }
        }
    }
    const float l = wave_sum_across16(l_part);
    const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
    const float E = wave_sum_across16(e_part) * inv_l;

    // ---- sweep 2: coefficients and dq ---------------------------------------------
    f32x4 o[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] = f32x4{0, 0, 0, 0};
    float *coefu = a.coef + (size_t)u * M * 2 * r;
    start();
    for (int j = 0; j < nsteps; ++j) {
        step(j);
        float dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = valid[e] ? __builtin_amdgcn_exp2f(acc[e >> 2][e & 3] * scale_log2 - m_run) * inv_l : 0.0f;
            const float ds = gam * p * (dacc[e >> 2][e & 3] - E);
            dsv[e] = ds;
            if (valid[e] && col < r) {
                const int slot = j * 32 + (e >> 2) * 16 + grp * 4 + (e & 3);
                *reinterpret_cast<float2 *>(coefu + ((size_t)slot * r + col) * 2) = float2{a.scale * ds, gam * p};
            }
        }
        Frag<uint16_t> dsf;
        dsf.set(dsv);  // K-element e <-> slot (e < 4 ? 4*grp + e : 16 + 4*grp + e - 4)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const u32x2 lo = lds_read_tr16(ldk + ktr + mb * 32);
            const u32x2 hi = lds_read_tr16(ldk + ktr + 16 * KRB + mb * 32);
            Frag<uint16_t> kt;
            kt.v = u32x4{lo[0], lo[1], hi[0], hi[1]};
            o[mb] = mma16(kt, dsf, o[mb]);
        }
    }

    // ---- epilogue: dq (lane (col = head, grp) holds dims 16 mb + 4 grp + i), dgate
    float dot = 0.0f;
    if (col < r) {
        float *dqp = a.dq + hrow + (size_t)col * D;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x4 *pp = reinterpret_cast<f32x4 *>(dqp + mb * 16 + grp * 4);
            *pp = *pp + o[mb] * a.scale;
        }
        // d_out . o_lin = d_out . S_t^T q = q . (S_t d_out)
        const uint16_t *dor = qrows + (size_t)col * D + grp * (D / 4);
        const uint16_t *olr = reinterpret_cast<const uint16_t *>(a.rlin) + hrow + (size_t)col * D + grp * (D / 4);
#pragma unroll
        for (int c = 0; c < D / 4; c += 8) {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(dor + c);
            const u32x4 y = *reinterpret_cast<const u32x4 *>(olr + c);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                dot = fmaf(bf16_bits_to_f32(x[w] & 0xFFFFu), bf16_bits_to_f32(y[w] & 0xFFFFu), dot);
                dot = fmaf(bf16_bits_to_f32(x[w] >> 16), bf16_bits_to_f32(y[w] >> 16), dot);
            }
        }
    }
    dot = wave_sum_across16(dot);
    if (col < r && grp == 0) a.dgate[(size_t)bt * a.Hq + g * r + col] = gam * (1.0f - gam) * (E - dot);
}

// Key side, step 1: the entries of each walk block of Qw = 256 consecutive
// positions of one group, sorted by key.  An entry is
// key << 17 | position-in-block << 9 | slot (key <= 32767, position < 256,
// slot < 512: the fields fill the word).  kNoEntry marks no entry: key 32767
// with block position 0, which no real entry can be (a key is at most its
// position t = t0 + position, and a block's first position t0 is a multiple of
// 256, at most 32512).  Where kNoEntry sorts does not matter: the walk skips
// it without ending the key run it is in.  sparse_bwd_sort_kernel sorts Qs = min(Qw, 32768 / Mp)
// positions in LDS (Mp = M rounded up to a power of two): each position's
// run of Mp entries is already ascending, so the runs are merged pairwise,
// level by level, in place (each thread computes its outputs of a level by
// merge path into registers, then all write back).  Pairs of sorted lists
// are then merged in global memory (sparse_bwd_merge_kernel) until a list
// covers Qw positions.
constexpr int kSortThreads = 1024;
constexpr int kSortMaxEntries = 32768;  // 128 KB of LDS
constexpr uint32_t kNoEntry = 0x7FFFu << 17;
constexpr uint32_t kUsedUp = 0xFFFFFFFFu;  // merge placeholder for a used-up run (never compared)

constexpr int kWalkBlock = 256;  // Qw
constexpr int kSortPer = kSortMaxEntries / kSortThreads;  // outputs per thread and level at most

// number of entries of A among the first d outputs of merge(A, B), |A| = |B| = L
template <typename P>
__device__ __forceinline__ int merge_split(P A, P Bl, int L, int d) {
    int lo = max(0, d - L), hi = min(d, L);
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (A[mid] <= Bl[d - mid - 1]) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}


__global__ __launch_bounds__(kSortThreads) void sparse_bwd_sort_kernel(SparseBwdArgs a, int Qs, int lgMp,
                                                                       uint32_t *sorted) {
    // entry i lives at word i + i / 16: threads of a merge level read about 16
    // entries apart, which unpadded would put a wave on four LDS banks
    __shared__ uint32_t ent[kSortMaxEntries + kSortMaxEntries / 16];
    struct View {
        uint32_t *w;
        int o;
        __device__ uint32_t operator[](int i) const { return w[o + i + ((o + i) >> 4)]; }
    };
    const int tid = threadIdx.x;
    const int G = a.G, M = a.M, n = a.n;
    const int Mp = 1 << lgMp, E = Qs * Mp;
    const int per = kWalkBlock / Qs;                       // sort blocks per walk block
    const int nrun = (n + kWalkBlock - 1) / kWalkBlock * per;
    const int bg = blockIdx.x / nrun, rr = blockIdx.x % nrun;
    const int g = bg % G, b = bg / G;
    const int sub = rr % per;
    const int t0 = (rr / per) * kWalkBlock + sub * Qs, nq = min(Qs, n - t0);  // nq <= 0: padding run
    // the block's index rows through one descriptor, every load unconditional
    // (a guarded load compiles to a branch with a full wait per load)
    const rsrc_t irs = make_rsrc(a.idx + (((size_t)b * n + max(t0, 0)) * G + g) * M,
                                 nq > 0 ? (uint32_t)nq * G * M * 4u : 0u);
    uint32_t sv[kSortPer];
#pragma unroll
    for (int k = 0; k < kSortPer; ++k) {
        const int i = tid + k * kSortThreads;
        const int tl = i >> lgMp, slot = i & (Mp - 1);
        const bool in = i < E && tl < nq && slot < min(M, t0 + tl + 1);
        sv[k] = __builtin_amdgcn_raw_buffer_load_b32(irs, in ? (uint32_t)(tl * G * M + slot) * 4u : kOffNone, 0u, 0);
    }
#pragma unroll
    for (int k = 0; k < kSortPer; ++k) {
        const int i = tid + k * kSortThreads;
        const int tl = i >> lgMp, slot = i & (Mp - 1), t = t0 + tl;
        const int s = (int)sv[k];
        const bool in = i < E && tl < nq && slot < min(M, t + 1) && s >= 0 && s <= t;
        if (i < E)
            ent[i + (i >> 4)] = in ? ((uint32_t)s << 17) | ((uint32_t)(sub * Qs + tl) << 9) | (uint32_t)slot : kNoEntry;
    }
    __syncthreads();
    // merge levels: runs of R into runs of 2R; thread tid makes outputs
    // [tid * per, (tid + 1) * per) of the level
    const int opt = E >= kSortThreads ? E / kSortThreads : 1;
    const int o0 = tid * opt;
    for (int R = Mp; R < E; R <<= 1) {
        uint32_t out[kSortPer];
        if (o0 < E) {
            int i = 0, j = 0;
            View A{ent, 0}, Bl{ent, 0};
            uint32_t ha = 0, hb = 0;  // the heads A[i], B[j] (kUsedUp when a side is used up)
#pragma unroll
            for (int k = 0; k < kSortPer; ++k) {
                if (k < opt) {
                    const int o = o0 + k;
                    if (k == 0 || (o & (2 * R - 1)) == 0) {  // first output, or a new pair of runs
                        const int p = o / (2 * R), d = o - p * 2 * R;
                        A = View{ent, p * 2 * R};
                        Bl = View{ent, p * 2 * R + R};
                        i = merge_split(A, Bl, R, d);
                        j = d - i;
                        ha = i < R ? A[i] : kUsedUp;
                        hb = j < R ? Bl[j] : kUsedUp;
                    }
                    // ties take A; a used-up side never wins (i + j < 2R here)
                    const bool takeA = j >= R || (i < R && ha <= hb);
                    if (takeA) {
                        out[k] = ha;
                        ++i;
                        ha = i < R ? A[i] : kUsedUp;
                    } else {
                        out[k] = hb;
                        ++j;
                        hb = j < R ? Bl[j] : kUsedUp;
                    }
                }
            }
        }
        __syncthreads();
        if (o0 < E) {
#pragma unroll
            for (int k = 0; k < kSortPer; ++k)
                if (k < opt) ent[o0 + k + ((o0 + k) >> 4)] = out[k];
        }
        __syncthreads();
    }
    uint32_t *dst = sorted + (size_t)blockIdx.x * E;
    for (int i = tid; i < E; i += kSortThreads) dst[i] = ent[i + (i >> 4)];
}

// Merge neighbouring sorted lists of L entries into lists of 2L (merge
// path; ties take the first list).  A work-group makes kMergeTile consecutive
// outputs: two lanes find where the tile starts and ends on both inputs by a
// binary search in global memory, the work-group stages those input ranges
// (kMergeTile entries in all) in LDS, and each thread merges its kMergePer
// outputs from LDS after a second search there.  2L is a multiple of
// kMergeTile.
constexpr int kMergePer = 16;
constexpr int kMergeTile = 256 * kMergePer;

__global__ __launch_bounds__(256) void sparse_bwd_merge_kernel(const uint32_t *src, uint32_t *dst, int L,
                                                               int64_t total) {
    __shared__ uint32_t buf[kMergeTile];
    __shared__ int split[2];
    const int64_t t0 = (int64_t)blockIdx.x * kMergeTile;
    if (t0 >= total) return;
    const int64_t pair = t0 / (2 * (int64_t)L);
    const int d0 = (int)(t0 - pair * 2 * L);
    const uint32_t *A = src + pair * 2 * L, *Bl = A + L;
    if (threadIdx.x < 2) split[threadIdx.x] = merge_split(A, Bl, L, d0 + (int)threadIdx.x * kMergeTile);
    __syncthreads();
    const int a0 = split[0], a1 = split[1];
    const int b0 = d0 - a0, b1 = d0 + kMergeTile - a1;
    const int na = a1 - a0, nb = b1 - b0;  // na + nb = kMergeTile
    for (int i = threadIdx.x; i < kMergeTile; i += 256) buf[i] = i < na ? A[a0 + i] : Bl[b0 + i - na];
    __syncthreads();
    // this thread's outputs: local diagonal dl of merge(buf[0, na), buf[na, na + nb))
    const int dl = threadIdx.x * kMergePer;
    int lo = max(0, dl - nb), hi = min(dl, na);
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (buf[mid] <= buf[na + dl - mid - 1]) lo = mid + 1;
        else hi = mid;
    }
    int i = lo, j = dl - lo;
    uint32_t out[kMergePer];
#pragma unroll
    for (int k = 0; k < kMergePer; ++k) {
        const bool takeA = j >= nb || (i < na && buf[i] <= buf[na + j]);
        out[k] = takeA ? buf[i++] : buf[na + j++];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMergePer; ++k) buf[dl + k] = out[k];
    __syncthreads();
    for (int k = threadIdx.x; k < kMergeTile; k += 256) dst[t0 + k] = buf[k];
}

// Key side, step 2 (sparse_bwd_walk_kernel): the sorted entries of a block
// are split over the waves of kWalkSlices consecutive work-groups, which the
// XCD remap places on one XCD, so the block's q and d_out rows (Qb * r * D
// * 4 bytes) are fetched into that XCD's L2 once and then served from it.
// Each wave walks a contiguous stretch: while the key stays the same it
// accumulates in registers, and when it changes it adds the row once.
constexpr int kWalkThreads = 256;
constexpr int kWalkPerWave = 256;  // sorted entries per wave

template <int D, int RMAX>
__global__ __launch_bounds__(kWalkThreads) void sparse_bwd_walk_kernel(SparseBwdArgs a, int Qb, int E,
                                                                       const uint32_t *sorted) {
    constexpr int DPL = D / 64;  // dims per lane while accumulating: 2 lane + c (D = 128) or lane
    constexpr int U = 8;         // entries whose loads are issued together
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = a.G, r = a.r, M = a.M, n = a.n, Hq = a.Hq;
    const int slices = (E + kWalkPerWave * (kWalkThreads / 64) - 1) / (kWalkPerWave * (kWalkThreads / 64));
    const int lu = xcd_remap(blockIdx.x, gridDim.x);
    const int blk = lu / slices, slice = lu % slices;
    const int nblk = (n + Qb - 1) / Qb;
    const int bg = blk / nblk, tb = blk % nblk;
    const int g = bg % G, b = bg / G;
    const int t0 = tb * Qb, nq = min(Qb, n - t0);
    const int start = (slice * (kWalkThreads / 64) + wave) * kWalkPerWave;
    if (start >= E) return;
    const int len = min(kWalkPerWave, E - start);
    // len is 256 (E = 256 Mp and a stretch starts at a multiple of 256), so
    // batches of U never pass the end; entries are wave-uniform
    const uint32_t *__restrict__ ent = sorted + (size_t)blk * E + start;
    const size_t unit0 = ((size_t)b * n + t0) * G + g;                          // unit of position t0
    const uint16_t *q0 = reinterpret_cast<const uint16_t *>(a.q) + (((size_t)b * n + t0) * Hq + g * r) * D;
    const uint16_t *d0 = reinterpret_cast<const uint16_t *>(a.dout) + (((size_t)b * n + t0) * Hq + g * r) * D;
    const int loff = D == 128 ? 2 * lane : lane;
    // every load goes through a buffer descriptor unconditionally (offsets of
    // missing entries and heads fall outside and read zeros): a guarded load
    // compiles to a branch with a full wait, serializing the batch
    const rsrc_t qrs = make_rsrc(q0, (uint32_t)nq * Hq * D * 2u), drs = make_rsrc(d0, (uint32_t)nq * Hq * D * 2u);
    const rsrc_t crs = make_rsrc(a.coef + unit0 * M * 2 * r, (uint32_t)nq * G * M * 2 * r * 4u);

    float gk[DPL], gv[DPL];
#pragma unroll
    for (int c = 0; c < DPL; ++c) gk[c] = gv[c] = 0.0f;
    int cur = -1;
    // D = 128: lane m accumulates dims 2m, 2m + 1; the atomics want lane l to
    // hold dims l and l + 64, so each instruction adds one contiguous 256-byte run
    auto flush = [&]() {
        if (cur < 0) return;
        const size_t row = (((size_t)b * n + cur) * G + g) * D;
        if constexpr (D == 128) {
            const int src0 = lane >> 1, src1 = 32 + (lane >> 1);
            const bool odd = lane & 1;
            const float k0 = __shfl(gk[0], src0), k1 = __shfl(gk[1], src0);
            const float k2 = __shfl(gk[0], src1), k3 = __shfl(gk[1], src1);
            const float v0 = __shfl(gv[0], src0), v1 = __shfl(gv[1], src0);
            const float v2 = __shfl(gv[0], src1), v3 = __shfl(gv[1], src1);
            unsafeAtomicAdd(a.dk + row + lane, odd ? k1 : k0);
            unsafeAtomicAdd(a.dk + row + 64 + lane, odd ? k3 : k2);
            unsafeAtomicAdd(a.dv + row + lane, odd ? v1 : v0);
            unsafeAtomicAdd(a.dv + row + 64 + lane, odd ? v3 : v2);
        } else {
            unsafeAtomicAdd(a.dk + row + lane, gk[0]);
            unsafeAtomicAdd(a.dv + row + lane, gv[0]);
        }
#pragma unroll
        for (int c = 0; c < DPL; ++c) gk[c] = gv[c] = 0.0f;
    };
    // the entry words of the next batch load while this batch's rows do
    uint32_t evn[U];
#pragma unroll
    for (int x = 0; x < U; ++x) evn[x] = ent[x];
    for (int base = 0; base < len; base += U) {
        uint32_t ev[U];
        float cv[U];
        uint32_t qv[U][RMAX], dv[U][RMAX];
#pragma unroll
        for (int x = 0; x < U; ++x) {
            ev[x] = __builtin_amdgcn_readfirstlane(evn[x]);
            evn[x] = ent[min(base + U + x, len - 1)];
        }
#pragma unroll
        for (int x = 0; x < U; ++x) {
            const bool ok = ev[x] != kNoEntry;
            const uint32_t tl = (ev[x] >> 9) & 255u, slot = ev[x] & 511u;
            const uint32_t coff = ok && lane < 2 * r ? ((tl * G * M + slot) * 2 * r + lane) * 4u : kOffNone;
            cv[x] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(crs, coff, 0u, 0));
            const uint32_t roff = (tl * Hq * D + loff) * 2u;
#pragma unroll
            for (int h = 0; h < RMAX; ++h) {
                const uint32_t off = ok && h < r ? roff + h * D * 2u : kOffNone;
                if constexpr (D == 128) {
                    qv[x][h] = __builtin_amdgcn_raw_buffer_load_b32(qrs, off, 0u, 0);
                    dv[x][h] = __builtin_amdgcn_raw_buffer_load_b32(drs, off, 0u, 0);
                } else {
                    qv[x][h] = __builtin_amdgcn_raw_buffer_load_b16(qrs, off, 0u, 0);
                    dv[x][h] = __builtin_amdgcn_raw_buffer_load_b16(drs, off, 0u, 0);
                }
            }
        }
#pragma unroll
        for (int x = 0; x < U; ++x) {
            if (ev[x] == kNoEntry) continue;
            const int s = (int)(ev[x] >> 17);
            if (s != cur) {
                flush();
                cur = s;
            }
#pragma unroll
            for (int h = 0; h < RMAX; ++h) {
                if (h < r) {
                    const float cds = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cv[x]), 2 * h));
                    const float cpv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cv[x]), 2 * h + 1));
                    if constexpr (D == 128) {
                        gk[0] = fmaf(cds, bf16_bits_to_f32(qv[x][h] & 0xFFFFu), gk[0]);
                        gk[DPL - 1] = fmaf(cds, bf16_bits_to_f32(qv[x][h] >> 16), gk[DPL - 1]);
                        gv[0] = fmaf(cpv, bf16_bits_to_f32(dv[x][h] & 0xFFFFu), gv[0]);
                        gv[DPL - 1] = fmaf(cpv, bf16_bits_to_f32(dv[x][h] >> 16), gv[DPL - 1]);
                    } else {
                        gk[0] = fmaf(cds, bf16_bits_to_f32(qv[x][h]), gk[0]);
                        gv[0] = fmaf(cpv, bf16_bits_to_f32(dv[x][h]), gv[0]);
                    }
                }
            }
        }
    }
    flush();
}

template <typename T>
hipError_t prep_t(const BwdPrepArgs &a, hipStream_t s) {
    const int64_t total = (int64_t)a.B * a.n * a.Hq * a.d / 8;
    launch_kernel((bwd_prep_kernel<T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <typename T>
hipError_t combine_t(const BwdCombineArgs &a, hipStream_t s) {
    const int64_t total = (int64_t)a.B * a.n * a.Hq * a.d / 8;  // >= the dk / dv count / 8
    launch_kernel((bwd_combine_kernel<T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <typename T, int D>
hipError_t sparse_t(const SparseBwdArgs &a, hipStream_t s) {
    const size_t lds = sparse_bwd_lds_bytes(a.r, a.M, D);
    launch_kernel((sparse_bwd_kernel<T, D>), dim3((unsigned)((int64_t)a.B * a.n * a.G)), dim3(64), lds, s, a);
    return hipGetLastError();
}

}  // namespace

size_t sparse_bwd_lds_bytes(int r, int M, int d) { return (size_t)4 * (2 * r * d + 2 * M * r); }

hipError_t launch_bwd_prep(const BwdPrepArgs &a, int dtype, hipStream_t s) {
    if ((int64_t)a.B * a.n == 0) return hipSuccess;
    return dtype == 1 ? prep_t<uint16_t>(a, s) : prep_t<float>(a, s);
}
hipError_t launch_transpose_states(const float *src, float *dst, int64_t nmat, int d, hipStream_t s) {
    const int64_t total = nmat * d * d;
    if (total == 0) return hipSuccess;
    launch_kernel(transpose_states_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, src, dst, nmat, d);
    return hipGetLastError();
}
hipError_t launch_bwd_combine(const BwdCombineArgs &a, int dtype, hipStream_t s) {
    if ((int64_t)a.B * a.n == 0) return hipSuccess;
    return dtype == 1 ? combine_t<uint16_t>(a, s) : combine_t<float>(a, s);
}
int sparse_bwd_key_block(int r, int M, int d) {
    (void)r;
    (void)d;
    return M >= 1 && M <= 512 ? kWalkBlock : 0;
}

namespace {
int lg_mp(int M) {
    int lg = 0;
    while ((1 << lg) < M) ++lg;
    return lg;
}
int sort_block(int M) { return min(kWalkBlock, kSortMaxEntries >> lg_mp(M)); }
}  // namespace

size_t sparse_bwd_sorted_bytes(int B, int n, int G, int M) {
    const size_t one = (size_t)B * G * ((n + kWalkBlock - 1) / kWalkBlock) * kWalkBlock * ((size_t)1 << lg_mp(M)) * 4;
    return sort_block(M) < kWalkBlock ? 2 * one : one;  // merge passes ping-pong
}

template <int D>
hipError_t launch_walk(const SparseBwdArgs &a, int Qb, int E, const uint32_t *sorted, dim3 grid, hipStream_t s) {
    if (a.r <= 4) launch_kernel((sparse_bwd_walk_kernel<D, 4>), grid, dim3(kWalkThreads), 0, s, a, Qb, E, sorted);
    else if (a.r <= 8) launch_kernel((sparse_bwd_walk_kernel<D, 8>), grid, dim3(kWalkThreads), 0, s, a, Qb, E, sorted);
    else launch_kernel((sparse_bwd_walk_kernel<D, 16>), grid, dim3(kWalkThreads), 0, s, a, Qb, E, sorted);
    return hipGetLastError();
}

hipError_t launch_sparse_bwd_split(const SparseBwdArgs &a, int d, int part, hipStream_t s) {
    if ((int64_t)a.B * a.n == 0) return hipSuccess;
    if (part == 0) {
        const dim3 grid((unsigned)((int64_t)a.B * a.n * a.G));
        if (d == 128) launch_kernel((sparse_bwd_q_kernel<128>), grid, dim3(64), 0, s, a);
        else launch_kernel((sparse_bwd_q_kernel<64>), grid, dim3(64), 0, s, a);
        return hipGetLastError();
    }
    if (sparse_bwd_key_block(a.r, a.M, d) == 0 || !a.sorted) return hipErrorInvalidValue;
    const int lgMp = lg_mp(a.M), Qs = sort_block(a.M);
    const int E = kWalkBlock << lgMp;                       // entries per walk block
    const int nb = a.B * a.G * ((a.n + kWalkBlock - 1) / kWalkBlock);
    const int64_t total = (int64_t)nb * E;
    uint32_t *buf[2] = {a.sorted, a.sorted + total};
    int cur = 0;  // the buffer the last merge pass writes
    for (int L = Qs << lgMp; L < E; L *= 2) cur ^= 1;
    if (part == 1) {
        launch_kernel(sparse_bwd_sort_kernel, dim3((unsigned)(nb * (kWalkBlock / Qs))), dim3(kSortThreads), 0,
                           s, a, Qs, lgMp, buf[0]);
        hipError_t e = hipGetLastError();
        int from = 0;
        for (int L = Qs << lgMp; e == hipSuccess && L < E; L *= 2, from ^= 1) {
            launch_kernel(sparse_bwd_merge_kernel, dim3((unsigned)((total + kMergeTile - 1) / kMergeTile)),
                               dim3(256), 0, s, buf[from], buf[from ^ 1], L, total);
            e = hipGetLastError();
        }
        return e;
    }
    const int per_wg = kWalkPerWave * (kWalkThreads / 64);
    const dim3 grid((unsigned)((int64_t)nb * ((E + per_wg - 1) / per_wg)));
    return d == 128 ? launch_walk<128>(a, kWalkBlock, E, buf[cur], grid, s)
                    : launch_walk<64>(a, kWalkBlock, E, buf[cur], grid, s);
}

hipError_t launch_sparse_bwd(const SparseBwdArgs &a, int dtype, int d, hipStream_t s) {
    if ((int64_t)a.B * a.n == 0) return hipSuccess;
    if (a.r > kMaxR) return hipErrorInvalidValue;
    if (dtype == 1) return d == 128 ? sparse_t<uint16_t, 128>(a, s) : sparse_t<uint16_t, 64>(a, s);
    return d == 128 ? sparse_t<float, 128>(a, s) : sparse_t<float, 64>(a, s);
}

}  // namespace lisa
