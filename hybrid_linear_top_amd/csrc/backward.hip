// Backward pass of the LISA layer for prefill (past = 0) on gfx950.
//
// The gradients of L = <d_out, out> + <d_state_out, state_out> follow the
// forward of the pages (gptget.net analysis of arXiv 2607.19358,
// method-details section) by the chain rule, with the selected sets held at
// the forward's (a top-M set is piecewise constant in q_I, k_I and w, which
// therefore get no gradient).  With G_t = (1 - gamma_t) d_out_t per head:
//
//  * gate:   dz = gamma (1 - gamma) (d_out . o_sp - d_out . o_lin);
//  * linear branch, three causal linear-attention passes run by the forward
//    chunked kernels on rearranged operands:
//      dq_t = S_t G_t                   = attention(q'=G, k'=v, v'=k, S0'=S0^T)
//      dk_s = H_s v_s,  dv_s = H_s^T k_s, H_s = dS_out + sum_{t >= s} q_t G_t^T
//        -- in reversed time these are causal too: per head,
//           dk: q'=v, k'=G, v'=q, S0'=dS_out^T;  dv: q'=k, k'=q, v'=G,
//           S0'=dS_out, whose final state is d_state_in;
//        each head its own group there, then summed over the heads of a group;
//  * sparse branch, one wave per (position, group) (sparse_bwd_kernel): the
//    softmax weights p of the r heads are recomputed from the gathered K rows,
//    ds = gamma p (d_out . v_s - d_out . o_sp), dq += scale sum_s ds k_s, and
//    dk_s += scale sum_h ds q_h, dv_s += sum_h p gamma d_out_h are added
//    into the key rows with fp32 atomics (the selected keys of different
//    positions collide at random, so no other owner exists for a key row).
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
//   G    = (1 - gamma) d_out                 (same position and head)
//   Grev = G,  qrev = q,  vrep = v of the head's group, krep = k of the group,
//          all at position n - 1 - t (reversed time).
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
    *reinterpret_cast<V *>(reinterpret_cast<T *>(a.Gl) + e) = gv;
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

// dq = dq_lin; dk[b,t,g] = sum_{h in g} o_k[b, n-1-t, h]; dv likewise (fp32);
// one thread per 8 consecutive elements
template <typename T>
__global__ __launch_bounds__(256) void bwd_combine_kernel(BwdCombineArgs a) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    const int64_t nq = (int64_t)a.B * a.n * a.Hq * a.d;
    const int64_t nk = (int64_t)a.B * a.n * a.G * a.d;
    using V = Vec8<T>;
    if (e < nq) {
        const V x = *reinterpret_cast<const V *>(reinterpret_cast<const T *>(a.dq_lin) + e);
        f32x4 lo, hi;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo[i] = Elt<T>::to_f32(x.x[i]);
            hi[i] = Elt<T>::to_f32(x.x[4 + i]);
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
        const T *olp = reinterpret_cast<const T *>(a.olin) + hrow;
#pragma unroll
        for (int h = 0; h < kMaxR; ++h) {
            if (h < r) {
                float dot = 0.0f;
                for (int dd = lane; dd < D; dd += 64) dot = fmaf(dos[h * D + dd], Elt<T>::to_f32(olp[h * D + dd]), dot);
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

template <typename T>
hipError_t prep_t(const BwdPrepArgs &a, hipStream_t s) {
    const int64_t total = (int64_t)a.B * a.n * a.Hq * a.d / 8;
    hipLaunchKernelGGL((bwd_prep_kernel<T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <typename T>
hipError_t combine_t(const BwdCombineArgs &a, hipStream_t s) {
    const int64_t total = (int64_t)a.B * a.n * a.Hq * a.d / 8;  // >= the dk / dv count / 8
    hipLaunchKernelGGL((bwd_combine_kernel<T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <typename T, int D>
hipError_t sparse_t(const SparseBwdArgs &a, hipStream_t s) {
    const size_t lds = sparse_bwd_lds_bytes(a.r, a.M, D);
    hipLaunchKernelGGL((sparse_bwd_kernel<T, D>), dim3((unsigned)((int64_t)a.B * a.n * a.G)), dim3(64), lds, s, a);
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
    hipLaunchKernelGGL(transpose_states_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, src, dst, nmat, d);
    return hipGetLastError();
}
hipError_t launch_bwd_combine(const BwdCombineArgs &a, int dtype, hipStream_t s) {
    if ((int64_t)a.B * a.n == 0) return hipSuccess;
    return dtype == 1 ? combine_t<uint16_t>(a, s) : combine_t<float>(a, s);
}
hipError_t launch_sparse_bwd(const SparseBwdArgs &a, int dtype, int d, hipStream_t s) {
    if ((int64_t)a.B * a.n == 0) return hipSuccess;
    if (a.r > kMaxR) return hipErrorInvalidValue;
    if (dtype == 1) return d == 128 ? sparse_t<uint16_t, 128>(a, s) : sparse_t<uint16_t, 64>(a, s);
    return d == 128 ? sparse_t<float, 128>(a, s) : sparse_t<float, 64>(a, s);
}

}  // namespace lisa
