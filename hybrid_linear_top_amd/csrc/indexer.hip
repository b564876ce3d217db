// Prefill Lightning Indexer fused with a streaming top-M select.
//
// For each query t and KV group g the indexer scores every candidate s <= t,
//   I[t,s] = sum_j w[t,j] * max(0, q_idx[t,j] . k_idx[s])
// (query/key projections and a ReLU'd dot product: gptget.net analysis of
// arXiv 2607.19358, method-details section), and keeps the top-M candidates
// of the full context (arxivdaily page, English abstract), the lower index
// winning ties.  The n^2/2 scores never leave the chip:
//
//  * A work-group owns QB consecutive queries of one group; each wave owns 8.
//    Key tiles of 64 keys are staged in LDS (double buffered, XOR-swizzled
//    16-byte chunks) and scored with v_mfma_f32_16x16x32_bf16.  The A operand
//    rows are (query, indexer head) pairs laid out so that the four
//    accumulator rows a lane receives are the four heads of one query: the
//    ReLU and the w-weighted head sum are lane-local.
//  * Each query keeps a candidate buffer in LDS, always sorted by key index:
//    candidates are appended in ascending key order (ballot + mbcnt give
//    positions, no atomics) if their score beats the query's threshold tau.
//  * When a buffer could overflow on the next tile, the wave selects the
//    exact current top-M of it (radix select on order-preserving keys, ties
//    to the lower index = earlier buffer position) and compacts it stably;
//    tau becomes the M-th score.  Later keys have larger indices, so a later
//    key must score strictly above tau to enter: equal scores lose, which is
//    the lowest-index tie-break.
//  * At the end the same select trims each buffer to min(M, t+1) entries,
//    which are already in ascending index order, and writes them out.
#include "common.hpp"
#include "kernels.hpp"

namespace lisa {
namespace {

constexpr int kKT = 64;  // keys per tile
constexpr int kQW = 8;   // queries per wave

struct Cand {
    float score;
    int32_t s;
};

__device__ __forceinline__ float key_to_float(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Keep exactly the first m of the c buffered candidates in the order
// (higher score, lower index); stable, so the buffer stays sorted by index.
// Whole wave, uniform control flow.  Returns the order key of the m-th.
template <int NE>
__device__ uint32_t wave_select(Cand *buf, int c, int m, uint32_t *hist) {
    const int lane = threadIdx.x & 63;
    c = min(c, NE * 64);
    float sc[NE];
    int32_t ss[NE];
    uint32_t u[NE];
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const int e = k * 64 + lane;
        if (e < c) {
            const Cand x = buf[e];
            sc[k] = x.score;
            ss[k] = x.s;
            u[k] = order_key(x.score);
        } else {
            sc[k] = 0.0f;
            ss[k] = 0;
            u[k] = 0u;
        }
    }
    uint32_t prefix = 0u, need = (uint32_t)m;
#pragma unroll 1
    for (int p = 0; p < 4; ++p) {
        const int sh = 24 - 8 * p;
        *reinterpret_cast<u32x4 *>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < NE; ++k) {
            const bool match = (k * 64 + lane < c) && (p == 0 || (u[k] >> (sh + 8)) == prefix);
            if (match) atomicAdd(&hist[(u[k] >> sh) & 255u], 1u);
        }
        wave_lds_sync();
        const u32x4 h = *reinterpret_cast<const u32x4 *>(hist + 4 * lane);
        const uint32_t lsum = h[0] + h[1] + h[2] + h[3];
        const uint32_t incl = wave_inclusive_scan(lsum);
        const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        uint32_t run = total - incl;  // candidates in bins above this lane's four
        int fb = -1;
        uint32_t fneed = 0;
#pragma unroll
        for (int bb = 3; bb >= 0; --bb) {
            const uint32_t hb = h[bb];
            if (fb < 0 && run < need && run + hb >= need) {
                fb = 4 * lane + bb;
                fneed = need - run;
            }
            run += hb;
        }
        const uint64_t fm = __ballot(fb >= 0);
        const int src = __ffsll((unsigned long long)fm) - 1;
        fb = __builtin_amdgcn_readlane(fb, src);
        fneed = (uint32_t)__builtin_amdgcn_readlane((int)fneed, src);
        prefix = (prefix << 8) | (uint32_t)fb;
        need = fneed;
        wave_lds_sync();
    }
    const uint32_t theta = prefix, take_eq = need;
    uint32_t base = 0u, eq_seen = 0u;
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const bool valid = k * 64 + lane < c;
        const bool gt = valid && u[k] > theta;
        const bool eq = valid && u[k] == theta;
        const uint64_t em = __ballot(eq);
        const uint32_t er = eq_seen + mbcnt64(em);
        eq_seen += (uint32_t)__popcll(em);
        const bool keep = gt || (eq && er < take_eq);
        const uint64_t km = __ballot(keep);
        const uint32_t pos = base + mbcnt64(km);
        base += (uint32_t)__popcll(km);
        if (keep && pos < (uint32_t)(NE * 64)) buf[pos] = Cand{sc[k], ss[k]};
    }
    wave_lds_sync();
    return theta;
}

template <typename T, int DI, int HH, int W, int CAP>
struct IdxCfg {
    static constexpr int EB = Elt<T>::kBytes;
    static constexpr int EPC = 16 / EB;     // elements per 16-byte chunk
    static constexpr int CPRK = DI / EPC;   // chunks per key row
    static constexpr int SWM = (CPRK < 8 ? CPRK : 8) - 1;
    static constexpr int KD = DI / 32;      // MFMA K-steps
    static constexpr int QB = W * kQW;      // queries per work-group
    static constexpr int NE = CAP / 64;
    static constexpr int TILE_ELEMS = kKT * DI;
};

template <typename T, int DI, int HH, int W, int CAP>
__global__ __launch_bounds__(W * 64) void indexer_topm_kernel(IndexerArgs a) {
    using C = IdxCfg<T, DI, HH, W, CAP>;
    __shared__ __attribute__((aligned(16))) Cand cand[C::QB * CAP];
    __shared__ __attribute__((aligned(16))) T ktile[2 * C::TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) uint32_t hist[W * 256];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int G = a.G, n = a.n, HI = a.HI, M = a.M;
    const int nqb = (n + C::QB - 1) / C::QB;
    // Block order: group fastest (with G | 8 every XCD sees a single group's
    // keys), heaviest (latest) query blocks first.
    const int L = blockIdx.x;
    const int g = L % G, rest = L / G, b = rest % a.B, qblk = nqb - 1 - rest / a.B;
    const int q0 = qblk * C::QB;
    const int qw0 = q0 + wave * kQW;
    const int t_hi = min(n, q0 + C::QB) - 1;  // last query of the block
    const int ntiles = t_hi / kKT + 1;

    const T *qI = reinterpret_cast<const T *>(a.q_idx);
    const T *kI = reinterpret_cast<const T *>(a.k_idx) + ((size_t)b * n * G + g) * DI;
    const T *wI = reinterpret_cast<const T *>(a.w_idx);
    const size_t krs = (size_t)G * DI;  // key row stride

    // ---- per-lane constants: A fragments, head weights, query rows -----------
    Frag<T> af[2][HH][C::KD];
    float wv[2][HH][4];
    int tq[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        tq[qb] = qw0 + qb * 4 + grp;  // the query whose four heads this lane accumulates
        const int tA = qw0 + qb * 4 + col / 4;  // the query of this lane's A row
#pragma unroll
        for (int hh = 0; hh < HH; ++hh) {
            const int headA = hh * 4 + (col & 3);
#pragma unroll
            for (int kc = 0; kc < C::KD; ++kc) {
                if (tA < n && headA < HI)
                    af[qb][hh][kc].load(qI + ((((size_t)b * n + tA) * G + g) * HI + headA) * DI +
                                        kc * 32 + grp * 8);
                else
                    af[qb][hh][kc].zero();
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int head = hh * 4 + i;
                wv[qb][hh][i] = (tq[qb] < n && head < HI)
                                    ? Elt<T>::to_f32(wI[(((size_t)b * n + tq[qb]) * G + g) * HI + head])
                                    : 0.0f;
            }
        }
    }
    int cnt[2] = {0, 0};
    float tau[2] = {-INFINITY, -INFINITY};
    Cand *mybuf[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) mybuf[qb] = cand + (size_t)(wave * kQW + qb * 4 + grp) * CAP;
    uint32_t *whist = hist + wave * 256;

    // ---- cooperative key-tile loads -------------------------------------------
    constexpr int CH_PER_T = kKT * C::CPRK / (W * 64) > 0 ? kKT * C::CPRK / (W * 64) : 1;
    auto load_tile = [&](int kt, u32x4 *regs) {
#pragma unroll
        for (int i = 0; i < CH_PER_T; ++i) {
            const int q = i * W * 64 + threadIdx.x;
            const int row = q / C::CPRK, cc = q % C::CPRK;
            const int s = kt * kKT + row;
            if (q < kKT * C::CPRK && s < n)
                regs[i] = *reinterpret_cast<const u32x4 *>(kI + (size_t)s * krs + cc * C::EPC);
            else
                regs[i] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_tile = [&](int buf, const u32x4 *regs) {
        u32x4 *dst = reinterpret_cast<u32x4 *>(ktile + buf * C::TILE_ELEMS);
#pragma unroll
        for (int i = 0; i < CH_PER_T; ++i) {
            const int q = i * W * 64 + threadIdx.x;
            if (q < kKT * C::CPRK) {
                const int row = q / C::CPRK, cc = q % C::CPRK;
                dst[row * C::CPRK + (cc ^ (row & C::SWM))] = regs[i];
            }
        }
    };

    u32x4 pre[CH_PER_T];
    load_tile(0, pre);
    store_tile(0, pre);
    __syncthreads();

    for (int kt = 0; kt < ntiles; ++kt) {
        const bool more = kt + 1 < ntiles;
        if (more) load_tile(kt + 1, pre);
        const int k0 = kt * kKT;
        if (qw0 + kQW - 1 >= k0 && qw0 < n) {  // this wave has a query that sees the tile
            const u32x4 *tb = reinterpret_cast<const u32x4 *>(ktile + (kt & 1) * C::TILE_ELEMS);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int krow = cb * 16 + col;
                Frag<T> bf[C::KD];
#pragma unroll
                for (int kc = 0; kc < C::KD; ++kc) {
                    const int c0 = (kc * 32 + grp * 8) / C::EPC;
                    if constexpr (C::EB == 2) {
                        bf[kc].v = tb[krow * C::CPRK + (c0 ^ (krow & C::SWM))];
                    } else {
                        const u32x4 x0 = tb[krow * C::CPRK + (c0 ^ (krow & C::SWM))];
                        const u32x4 x1 = tb[krow * C::CPRK + ((c0 + 1) ^ (krow & C::SWM))];
                        reinterpret_cast<Frag<float> &>(bf[kc]).lo = __builtin_bit_cast(f32x4, x0);
                        reinterpret_cast<Frag<float> &>(bf[kc]).hi = __builtin_bit_cast(f32x4, x1);
                    }
                }
                const int s = k0 + krow;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    float score = 0.0f;
#pragma unroll
                    for (int hh = 0; hh < HH; ++hh) {
                        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
                        for (int kc = 0; kc < C::KD; ++kc) acc = mma16(af[qb][hh][kc], bf[kc], acc);
#pragma unroll
                        for (int i = 0; i < 4; ++i) score = fmaf(wv[qb][hh][i], fmaxf(acc[i], 0.0f), score);
                    }
                    const bool ok = (s <= tq[qb]) && (tq[qb] < n) && (score > tau[qb]);
                    const uint64_t mask = __ballot(ok);
                    if (mask) {
                        const uint64_t gm = mask & (0xFFFFull << (16 * grp));
                        const int pos = cnt[qb] + (int)mbcnt64(gm);
                        if (ok && pos < CAP) mybuf[qb][pos] = Cand{score, s};
                        cnt[qb] += __popcll(gm);
                    }
                }
            }
            // trim any buffer that could overflow on the next tile
            wave_lds_sync();
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const uint64_t full = __ballot(cnt[qb] > CAP - kKT);
#pragma unroll 1
                for (int gg = 0; gg < 4; ++gg) {
                    if (!((full >> (16 * gg)) & 1ull)) continue;
                    Cand *qbuf = cand + (size_t)(wave * kQW + qb * 4 + gg) * CAP;
                    const int c = __builtin_amdgcn_readlane(cnt[qb], 16 * gg);
                    const uint32_t th = wave_select<C::NE>(qbuf, c, M, whist);
                    if (grp == gg) {
                        cnt[qb] = M;
                        tau[qb] = key_to_float(th);
                    }
                }
            }
        }
        if (more) store_tile((kt + 1) & 1, pre);
        __syncthreads();
    }

    // ---- final trim and ordered write-out ---------------------------------------
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll 1
        for (int gg = 0; gg < 4; ++gg) {
            const int t = qw0 + qb * 4 + gg;
            if (t >= n) continue;
            Cand *qbuf = cand + (size_t)(wave * kQW + qb * 4 + gg) * CAP;
            const int c = __builtin_amdgcn_readlane(cnt[qb], 16 * gg);
            const int m = min(M, t + 1);
            if (c > m) wave_select<C::NE>(qbuf, c, m, whist);
            int32_t *dst = a.idx + (((size_t)b * n + t) * G + g) * M;
            for (int i = lane; i < M; i += 64) dst[i] = i < m ? qbuf[i].s : -1;
        }
    }
}

template <typename T, int DI, int HH, int W, int CAP>
hipError_t launch(const IndexerArgs &a, hipStream_t s) {
    using C = IdxCfg<T, DI, HH, W, CAP>;
    const int nqb = (a.n + C::QB - 1) / C::QB;
    hipLaunchKernelGGL((indexer_topm_kernel<T, DI, HH, W, CAP>), dim3(a.B * a.G * nqb), dim3(W * 64),
                       0, s, a);
    return hipGetLastError();
}

template <typename T, int DI, int HH>
hipError_t by_m(const IndexerArgs &a, hipStream_t s) {
    // candidate buffers: QB * CAP * 8 bytes; key tiles 2 * 64 * DI * sizeof(T)
    constexpr bool big_tile = (2 * kKT * DI * Elt<T>::kBytes) > 16384;
    if (a.M <= 128) return launch<T, DI, HH, 4, 256>(a, s);
    if constexpr (big_tile) {
        if (a.M <= 256) return launch<T, DI, HH, 2, 512>(a, s);
        return launch<T, DI, HH, 1, 1024>(a, s);
    } else {
        if (a.M <= 256) return launch<T, DI, HH, 4, 512>(a, s);
        return launch<T, DI, HH, 2, 1024>(a, s);
    }
}

template <typename T>
hipError_t by_shape(const IndexerArgs &a, int dI, hipStream_t s) {
    const bool h2 = a.HI > 4;
    if (dI == 64) return h2 ? by_m<T, 64, 2>(a, s) : by_m<T, 64, 1>(a, s);
    return h2 ? by_m<T, 32, 2>(a, s) : by_m<T, 32, 1>(a, s);
}

}  // namespace

hipError_t launch_indexer_prefill(const IndexerArgs &a, int dtype, int dI, hipStream_t s) {
    if (a.B * a.n == 0) return hipSuccess;
    return dtype == 1 ? by_shape<uint16_t>(a, dI, s) : by_shape<float>(a, dI, s);
}

}  // namespace lisa
