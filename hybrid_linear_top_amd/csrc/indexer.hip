// Prefill Lightning Indexer fused with a streaming top-M select.
//
// For each query t and KV group g the indexer scores every candidate s <= t,
//   I[t,s] = sum_j w[t,j] * max(0, q_idx[t,j] . k_idx[s])
// (query/key projections and a ReLU'd dot product: gptget.net analysis of
// arXiv 2607.19358, method-details section), and keeps the top-M candidates
// of the full context (arxivdaily page, English abstract), the lower index
// winning ties.  The n^2/2 scores never leave the chip:
//
//  * A work-group is one wave that owns 4 consecutive queries of one group.
//    It streams the group's keys (L2-resident: every XCD serves a single
//    group) in tiles of 64, loading the MFMA B fragments straight from memory
//    one tile ahead, and scores each tile with 8 v_mfma_f32_16x16x32_bf16
//    issued back to back.  Four queries per wave and two fragment buffers keep
//    a wave at 166 VGPRs and 12 KB of LDS, so 12 waves share a CU.  The keys are first re-laid out (pack_keys_kernel)
//    so that every fragment load of a wave reads 1 KB of consecutive bytes:
//    read in place, each load touches 16 key rows for 64 bytes each, and the
//    scan is then bound by the address units rather than by anything else.  The A operand rows are (query, indexer head) pairs
//    laid out so that the four accumulator rows a lane receives are the four
//    heads of one query: the ReLU and the w-weighted head sum are lane-local.
//  * Column n of key block cb holds key k0 + 4n + cb, so each lane scores
//    four consecutive keys of its query.  Each query keeps a candidate buffer
//    in LDS, always sorted by key index: a lane's accepted keys go to
//    consecutive positions after an exclusive scan of the per-lane counts
//    over the query's 16-lane row (DPP row shifts, row_newbcast for the row
//    total).  A candidate is accepted when its score is strictly above the
//    query's threshold tau.
//  * When a buffer could overflow on the next tile it is trimmed: a one-pass
//    256-bin histogram over the buffered scores finds the bin holding the
//    M-th largest; the lower bins are dropped and tau becomes the largest
//    dropped score, so at least M kept candidates beat everything rejected.
//    When that frees too little (exact ties) the exact select below is used.
//  * The exact select (radix select on order-preserving keys, ties to the
//    lower index = earlier buffer position, stable compaction) trims each
//    buffer to min(M, t+1) entries at the end; they are already in ascending
//    index order and are written out.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lisa {
namespace {

constexpr int kKT = 64;  // keys per tile
#ifndef LISA_IDX_QB
#define LISA_IDX_QB 1  // query quads per wave (4 queries each)
#endif

__device__ __forceinline__ float key_to_float(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}


// Candidate buffers are two LDS arrays: fp32 scores and 16-bit key indices
// (prefill n <= 32768).
struct CandBuf {
    float *sc;
    uint16_t *key;
};

// Keep exactly the first m of the c buffered candidates in the order
// (higher score, lower index); stable, so the buffer stays sorted by index.
// Whole wave, uniform control flow.  Returns the order key of the m-th.
// The threshold is found by 256-bin histogram passes over the live range of
// order keys, [min, max] first (buffered candidates sit in a narrow band, so
// fixed 8-bit digits of the key would waste passes on common high bits); a
// pass stops as soon as the bin holding the m-th key is taken whole, or holds
// a single key value (ties: the earliest buffer positions win).
template <int NE>
__device__ uint32_t wave_select(CandBuf buf, int c, int m, uint32_t *hist) {
    const int lane = threadIdx.x & 63;
    c = min(c, NE * 64);
    float sc[NE];
    uint32_t ss[NE];
    uint32_t u[NE];
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const int e = k * 64 + lane;
        if (e < c) {
            sc[k] = buf.sc[e];
            ss[k] = buf.key[e];
            u[k] = order_key(sc[k]);
            kmin = min(kmin, u[k]);
            kmax = max(kmax, u[k]);
        } else {
            sc[k] = 0.0f;
            ss[k] = 0u;
            u[k] = 0u;
        }
    }
    uint32_t lo = wave_min_u32(kmin);
    const uint32_t span = wave_max_u32(kmax) - lo;
    int width = span == 0 ? 0 : 32 - __builtin_clz(span);  // bits of key - lo
    uint32_t need = (uint32_t)m;
    uint32_t theta;      // keys > theta are kept, and keys == theta up to take_eq,
    uint32_t take_eq;    // or (whole_bin) every key >= theta
    bool whole_bin;
#pragma unroll 1
    for (;;) {
        const int shift = width > 8 ? width - 8 : 0;
        *reinterpret_cast<u32x4 *>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
        wave_lds_sync();
        const uint64_t hi_excl = (uint64_t)lo + ((uint64_t)1 << width);
#pragma unroll
        for (int k = 0; k < NE; ++k) {
            if (k * 64 + lane < c && u[k] >= lo && (uint64_t)u[k] < hi_excl)
                atomicAdd(&hist[(u[k] - lo) >> shift], 1u);
        }
        wave_lds_sync();
        const u32x4 h = *reinterpret_cast<const u32x4 *>(hist + 4 * lane);
        const uint32_t lsum = h[0] + h[1] + h[2] + h[3];
        const uint32_t incl = wave_inclusive_scan(lsum);
        const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        uint32_t run = total - incl;  // keys in the bins of higher lanes
        int fb = -1;
        uint32_t fneed = 0, fcnt = 0;
#pragma unroll
        for (int bb = 3; bb >= 0; --bb) {
            if (fb < 0 && run < need && run + h[bb] >= need) {
                fb = 4 * lane + bb;
                fneed = need - run;
                fcnt = h[bb];
            }
            run += h[bb];
        }
        const int src = __ffsll((unsigned long long)__ballot(fb >= 0)) - 1;
        fb = __builtin_amdgcn_readlane(fb, src);
        fneed = (uint32_t)__builtin_amdgcn_readlane((int)fneed, src);
        fcnt = (uint32_t)__builtin_amdgcn_readlane((int)fcnt, src);
        wave_lds_sync();
        const uint32_t blo = lo + ((uint32_t)fb << shift);
        if (fneed == fcnt) {  // the whole bin is kept: keys >= blo are exactly the first m
            theta = blo;
            take_eq = 0u;
            whole_bin = true;
            break;
        }
        if (shift == 0) {  // one key value: the earliest fneed of them
            theta = blo;
            take_eq = fneed;
            whole_bin = false;
            break;
        }
        lo = blo;
        width = shift;
        need = fneed;
    }
    uint32_t base = 0u, eq_seen = 0u, kth = 0xFFFFFFFFu;
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const bool valid = k * 64 + lane < c;
        const bool gt = valid && (whole_bin ? u[k] >= theta : u[k] > theta);
        const bool eq = valid && !whole_bin && u[k] == theta;
        const uint64_t em = __ballot(eq);
        const uint32_t er = eq_seen + mbcnt64(em);
        eq_seen += (uint32_t)__popcll(em);
        const bool keep = gt || (eq && er < take_eq);
        if (keep) kth = min(kth, u[k]);
        const uint64_t km = __ballot(keep);
        const uint32_t pos = base + mbcnt64(km);
        base += (uint32_t)__popcll(km);
        if (keep && pos < (uint32_t)(NE * 64)) {
            buf.sc[pos] = sc[k];
            buf.key[pos] = (uint16_t)ss[k];
        }
    }
    wave_lds_sync();
    return wave_min_u32(kth);
}

template <int NE>
__device__ bool wave_trim(CandBuf buf, int &c_io, int M, int need_free, uint32_t *hist, float &tau) {
    const int lane = threadIdx.x & 63;
    const int c = min(c_io, NE * 64);
    float sc[NE];
    uint16_t ss[NE];
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const int e = k * 64 + lane;
        if (e < c) {
            sc[k] = buf.sc[e];
            ss[k] = buf.key[e];
            mn = fminf(mn, sc[k]);
            mx = fmaxf(mx, sc[k]);
        } else {
            sc[k] = 0.0f;
            ss[k] = 0;
        }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (!(mx > mn)) return false;
    const float scale = 255.99f / (mx - mn);
    *reinterpret_cast<u32x4 *>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
    wave_lds_sync();
    int bin[NE];
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        bin[k] = -1;
        if (k * 64 + lane < c) {
            bin[k] = min(255, (int)((sc[k] - mn) * scale));
            atomicAdd(&hist[bin[k]], 1u);
        }
    }
    wave_lds_sync();
    const u32x4 h = *reinterpret_cast<const u32x4 *>(hist + 4 * lane);
    const uint32_t lsum = h[0] + h[1] + h[2] + h[3];
    const uint32_t incl = wave_inclusive_scan(lsum);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    uint32_t run = total - incl;
    int fb = -1;
    uint32_t kept = 0;
#pragma unroll
    for (int bb = 3; bb >= 0; --bb) {
        const uint32_t hb = h[bb];
        if (fb < 0 && run < (uint32_t)M && run + hb >= (uint32_t)M) {
            fb = 4 * lane + bb;
            kept = run + hb;
        }
        run += hb;
    }
    const uint64_t fm = __ballot(fb >= 0);
    const int src = __ffsll((unsigned long long)fm) - 1;
    fb = __builtin_amdgcn_readlane(fb, src);
    kept = (uint32_t)__builtin_amdgcn_readlane((int)kept, src);
    wave_lds_sync();
    if (fb <= 0 || (int)kept > c - need_free) return false;
    float dmax = -INFINITY;
#pragma unroll
    for (int k = 0; k < NE; ++k)
        if (bin[k] >= 0 && bin[k] < fb) dmax = fmaxf(dmax, sc[k]);
    dmax = wave_max(dmax);
    uint32_t base = 0u;
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const bool keep = bin[k] >= fb;
        const uint64_t km = __ballot(keep);
        const uint32_t pos = base + mbcnt64(km);
        base += (uint32_t)__popcll(km);
        if (keep && pos < (uint32_t)(NE * 64)) {
            buf.sc[pos] = sc[k];
            buf.key[pos] = ss[k];
        }
    }
    wave_lds_sync();
    c_io = (int)base;
    tau = dmax;
    return true;
}

// Trim one query's buffer of c candidates to about M (one histogram pass, or
// the exact select when that frees too little).  Kept out of line: trims are
// rare and the tile loop stays small enough for the instruction cache.
struct TrimResult {
    int c;
    float tau;
};
template <int NE>
__device__ __attribute__((noinline)) TrimResult trim_buffer(CandBuf buf, int c, int M, int need_free,
                                                            uint32_t *hist) {
    float th = -INFINITY;
    if (!wave_trim<NE>(buf, c, M, need_free, hist, th)) {
        th = key_to_float(wave_select<NE>(buf, c, M, hist));
        c = M;
    }
    return TrimResult{c, th};
}

// Packed key tiles: for batch b and group g, tile kt holds keys 64kt..64kt+63
// as 4 x KD fragments (key block cb, K step kc), each 64 lanes x 8 elements in
// lane order, where lane (grp, col) carries elements kc*32 + grp*8 .. +7 of key
// 64kt + 4col + cb -- exactly what that lane feeds the MFMA.  Keys past the
// last one are zeros.
template <typename T, int DI>
__global__ __launch_bounds__(256) void pack_keys_kernel(const T *__restrict__ k_idx, T *__restrict__ packed,
                                                        int64_t total, int nk, int G, int ntiles) {
    constexpr int KD = DI / 32;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one lane-fragment of 8 elements
    if (i >= total) return;
    const int lane = (int)(i & 63);
    int64_t r = i >> 6;
    const int kc = (int)(r % KD);
    r /= KD;
    const int cb = (int)(r & 3);
    r >>= 2;
    const int kt = (int)(r % ntiles);
    r /= ntiles;
    const int g = (int)(r % G), b = (int)(r / G);
    const int key = kt * kKT + 4 * (lane & 15) + cb;
    Frag<T> f;
    if (key < nk) f.load(k_idx + (((size_t)b * nk + key) * G + g) * DI + kc * 32 + (lane >> 4) * 8);
    else f.zero();
    T *dst = packed + (size_t)i * 8;
    if constexpr (std::is_same<T, uint16_t>::value) {
        *reinterpret_cast<u32x4 *>(dst) = f.v;
    } else {
        reinterpret_cast<f32x4 *>(dst)[0] = f.lo;
        reinterpret_cast<f32x4 *>(dst)[1] = f.hi;
    }
}

template <typename T, int DI, int HH, int CAP, int QB>
struct IdxCfg {
    static constexpr int KD = DI / 32;      // MFMA K-steps
    static constexpr int QW = 4 * QB;       // queries per wave: QB quads of 4
    static constexpr int NE = CAP / 64;
};

template <typename T, int DI, int HH, int CAP, int QB>
__global__ __launch_bounds__(64) void indexer_topm_kernel(IndexerArgs a) {
    using C = IdxCfg<T, DI, HH, CAP, QB>;
    constexpr int kQW = C::QW;
    __shared__ __attribute__((aligned(16))) float cand_sc[kQW * CAP];
    __shared__ __attribute__((aligned(16))) uint16_t cand_key[kQW * CAP];
    __shared__ __attribute__((aligned(16))) uint32_t hist[256];
    // per-lane sink for the writes of rejected keys (appends are straight-line
    // code, so the two query quads' scans and writes interleave).  It lives in
    // the histogram, which every trim and select clears before use.
    float *const sink_sc = reinterpret_cast<float *>(hist);
    uint16_t *const sink_key = reinterpret_cast<uint16_t *>(hist + 64);
    auto qbuf_of = [&](int q) { return CandBuf{cand_sc + q * CAP, cand_key + q * CAP}; };

    const int lane = threadIdx.x & 63;
    const int col = lane & 15, grp = lane >> 4;
    // queries are the rows 0..nq-1 of q_idx / w_idx / idx; query row t sits at
    // position p0 + t, and the keys are positions 0..nk-1 (nk = p0 + nq)
    const int G = a.G, nq = a.n, p0 = a.past, nk = a.past + a.n, HI = a.HI, M = a.M;
    const int nqb = (nq + kQW - 1) / kQW;
    // Block order: group fastest (with G | 8 every XCD sees a single group's
    // keys), latest (heaviest) query blocks first.
    const int L = blockIdx.x;
    const int g = L % G, rest = L / G, b = rest % a.B, qblk = nqb - 1 - rest / a.B;
    const int qw0 = p0 + qblk * kQW;          // position of the wave's first query
    const int t_hi = min(nk, qw0 + kQW) - 1;  // position of its last query
    const int ntiles = t_hi / kKT + 1;

    const T *qI = reinterpret_cast<const T *>(a.q_idx);
    const int ntk = (nk + kKT - 1) / kKT;  // key tiles
    const T *kI = reinterpret_cast<const T *>(a.k_packed) + ((size_t)b * G + g) * ntk * kKT * DI;
    const T *wI = reinterpret_cast<const T *>(a.w_idx);

    // ---- per-lane constants: A fragments, head weights, query rows -----------
    Frag<T> af[QB][HH][C::KD];
    float wv[QB][HH][4];
    int tq[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        tq[qb] = qw0 + qb * 4 + grp;  // position of the query whose four heads this lane accumulates
        const int tA = qw0 - p0 + qb * 4 + col / 4;  // row of the query of this lane's A row
#pragma unroll
        for (int hh = 0; hh < HH; ++hh) {
            const int headA = hh * 4 + (col & 3);
#pragma unroll
            for (int kc = 0; kc < C::KD; ++kc) {
                if (tA < nq && headA < HI)
                    af[qb][hh][kc].load(qI + ((((size_t)b * nq + tA) * G + g) * HI + headA) * DI +
                                        kc * 32 + grp * 8);
                else
                    af[qb][hh][kc].zero();
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int head = hh * 4 + i;
                wv[qb][hh][i] = (tq[qb] < nk && head < HI)
                                    ? Elt<T>::to_f32(wI[(((size_t)b * nq + tq[qb] - p0) * G + g) * HI + head])
                                    : 0.0f;
            }
        }
    }
    int cnt[QB];
    float tau[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        cnt[qb] = 0;
        tau[qb] = tq[qb] < nk ? -INFINITY : INFINITY;  // padding queries accept nothing
    }

    // B fragments of one packed key tile: key 4*col + cb, dims 32*kc + 8*grp
    // .. +7, through a per-tile buffer descriptor (tiles past the last read
    // as zeros)
    constexpr uint32_t EB = Elt<T>::kBytes;
    constexpr uint32_t kTileBytes = kKT * DI * EB, kFragBytes = 64 * 8 * EB;
    const uint32_t all_bytes = (uint32_t)ntk * kTileBytes;
    const uint32_t voff = (uint32_t)lane * 8 * EB;
    auto load_b = [&](int kt, Frag<T> (&bf)[4][C::KD]) {
        const uint32_t tile_off = (uint32_t)kt * kTileBytes;
        const rsrc_t r = make_rsrc(reinterpret_cast<const unsigned char *>(kI) + tile_off,
                                   all_bytes > tile_off ? all_bytes - tile_off : 0u);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int kc = 0; kc < C::KD; ++kc)
                frag_buf_load(bf[cb][kc], r, voff + (uint32_t)(cb * C::KD + kc) * kFragBytes);
    };


    // scores of one tile: score[qb][cb] for key k0 + 4*col + cb of query tq[qb]
    auto tile_scores = [&](const Frag<T> (&bcur)[4][C::KD], float (&score)[QB][4]) {
        // all MFMAs of the tile first
        f32x4 acc[QB][HH][4];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int hh = 0; hh < HH; ++hh)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    f32x4 x = {0, 0, 0, 0};
#pragma unroll
                    for (int kc = 0; kc < C::KD; ++kc) x = mma16(af[qb][hh][kc], bcur[cb][kc], x);
                    acc[qb][hh][cb] = x;
                }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                float sc = 0.0f;
#pragma unroll
                for (int hh = 0; hh < HH; ++hh)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sc = fmaf(wv[qb][hh][i], fmaxf(acc[qb][hh][cb][i], 0.0f), sc);
                score[qb][cb] = sc;
            }
    };

    auto tile_step = [&](int kt, const Frag<T> (&bcur)[4][C::KD], auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;  // tile reaches past the first query
        const int k0 = kt * kKT;
        float score[QB][4];
        tile_scores(bcur, score);
        // threshold tests
        bool ok[QB][4];
        uint64_t any = 0;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const float sc = score[qb][cb];
                if constexpr (DIAG) ok[qb][cb] = (k0 + 4 * col + cb <= tq[qb]) && sc > tau[qb];
                else ok[qb][cb] = sc > tau[qb];
                any |= __ballot(ok[qb][cb]);
            }
        if (!any) return;
        // Append in ascending key order: a query's accepted keys are ordered by
        // (col, cb), so a lane's first position is the query's count plus the
        // exclusive scan of the per-lane counts over its 16-lane row.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const uint32_t c4 = (uint32_t)ok[qb][0] + (uint32_t)ok[qb][1] + (uint32_t)ok[qb][2] +
                                (uint32_t)ok[qb][3];
            const uint32_t incl = row_inclusive_scan(c4);
            const uint32_t tot = row_broadcast15(incl);
            int pos = cnt[qb] + (int)(incl - c4);
            const CandBuf qbuf = qbuf_of(qb * 4 + grp);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                float *psc = ok[qb][cb] ? qbuf.sc + pos : sink_sc + lane;
                uint16_t *pkey = ok[qb][cb] ? qbuf.key + pos : sink_key + lane;
                *psc = score[qb][cb];
                *pkey = (uint16_t)(k0 + 4 * col + cb);
                pos += ok[qb][cb] ? 1 : 0;
            }
            cnt[qb] += (int)tot;
        }
        // trim any buffer that could overflow on the next tile
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const uint64_t full = __ballot(cnt[qb] > CAP - kKT);
            if (!full) continue;
            wave_lds_sync();
#pragma unroll 1
            for (int gg = 0; gg < 4; ++gg) {
                if (!((full >> (16 * gg)) & 1ull)) continue;
                const TrimResult tr = trim_buffer<C::NE>(qbuf_of(qb * 4 + gg),
                                                         __builtin_amdgcn_readlane(cnt[qb], 16 * gg), M,
                                                         CAP / 4, hist);
                if (grp == gg) {
                    cnt[qb] = tr.c;
                    tau[qb] = tr.tau;
                }
            }
        }
    };

    Frag<T> b0[4][C::KD], b1[4][C::KD];
    // tiles below kd hold only keys < qw0 <= every query of the wave
    const int kd = qw0 / kKT;
    // Prefetches are never skipped: a tile past the end is fetched through an
    // empty descriptor (all zeros, no memory access).  A skipped load on one
    // path would make the wait counts of the merged paths wait for the
    // prefetched tiles as well.
    const int knull = (nk + kKT - 1) / kKT;
    auto tile_or_null = [&](int kt, int lim) { return kt < lim ? kt : knull; };

    // ---- starting threshold from a key sample ---------------------------------
    // With tau starting at -inf a late query appends about M*ln(t/M) keys and
    // trims its buffer several times.  Instead, ns tiles spread over the keys
    // below qw0 are scored first; each lane keeps its four best sample scores
    // per query, and tau starts at (about) the R-th largest of a query's 64
    // kept values, R chosen so that about kSlack*M of the query's t+1 keys are
    // expected above it.  This is only a starting point: the scan below
    // accepts what beats it, and a query left with fewer than min(M, t+1)
    // candidates (tau was too high) is scanned again from tau = -inf, so the
    // result is exact whatever the sample says.
    constexpr float kSlack = 1.5f;
    constexpr int kRank = 32;
    int ns = 0;
    if (qw0 >= 4 * M) {
        ns = (int)ceilf((float)kRank * (float)(qw0 + 1) / (kSlack * (float)M * (float)kKT));
        ns = min(ns, kd / 2);
    }
    if (ns > 0) {
        float top[QB][4];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) top[qb][i] = -INFINITY;
        auto sample_tile = [&](const Frag<T> (&bc)[4][C::KD]) {
            float score[QB][4];
            tile_scores(bc, score);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    float x = score[qb][cb];  // insert into the descending top-4
#pragma unroll
                    for (int i = 0; i < 3; ++i) {
                        const float hi = fmaxf(top[qb][i], x);
                        x = fminf(top[qb][i], x);
                        top[qb][i] = hi;
                    }
                    top[qb][3] = fmaxf(top[qb][3], x);
                }
        };
        auto ks = [&](int i) { return ((2 * i + 1) * kd) / (2 * ns); };
        load_b(ks(0), b0);
        for (int i = 0; i < ns; i += 2) {
            load_b(i + 1 < ns ? ks(i + 1) : knull, b1);
            sample_tile(b0);
            if (i + 1 >= ns) break;
            load_b(i + 2 < ns ? ks(i + 2) : knull, b0);
            sample_tile(b1);
        }
        const float S = (float)(ns * kKT);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float R = fminf(48.0f, fmaxf(1.0f, rintf(kSlack * (float)M * S / (float)(tq[qb] + 1))));
            auto count_ge = [&](float x) {
                const uint32_t c = (uint32_t)(top[qb][0] >= x) + (uint32_t)(top[qb][1] >= x) +
                                   (uint32_t)(top[qb][2] >= x) + (uint32_t)(top[qb][3] >= x);
                return (float)row_broadcast15(row_inclusive_scan(c));
            };
            float lo = row_min(top[qb][3]), hi = row_max(top[qb][0]);
            if (count_ge(hi) >= R) lo = hi;
#pragma unroll 1
            for (int it = 0; it < 12; ++it) {
                const float mid = 0.5f * (lo + hi);
                const bool up = count_ge(mid) >= R;
                lo = up ? mid : lo;
                hi = up ? hi : mid;
            }
            if (tq[qb] < nk) tau[qb] = lo;
        }
    }

    // ---- scan: every tile, two fragment buffers alternating (tile kt+1 loads
    // while kt computes); a second pass redoes exactly the queries whose
    // sampled threshold turned out too high --------------------------------------
    auto step = [&](int kt, const Frag<T> (&bc)[4][C::KD]) {
        if (kt >= kd) tile_step(kt, bc, std::true_type{});
        else tile_step(kt, bc, std::false_type{});
    };
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        load_b(0, b0);
        for (int kt = 0; kt < ntiles; kt += 2) {
            load_b(tile_or_null(kt + 1, ntiles), b1);
            step(kt, b0);
            if (kt + 1 >= ntiles) break;
            load_b(tile_or_null(kt + 2, ntiles), b0);
            step(kt + 1, b1);
        }
        if (ns == 0) break;  // started from -inf: already exact
        uint64_t redo = 0;
        bool fail[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            fail[qb] = tq[qb] < nk && cnt[qb] < min(M, tq[qb] + 1);
            redo |= __ballot(fail[qb]);
        }
        if (!redo || pass == 1) break;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            // kept queries take nothing more (their counts stay below a trim)
            tau[qb] = fail[qb] ? -INFINITY : INFINITY;
            cnt[qb] = fail[qb] ? 0 : cnt[qb];
        }
    }

    // ---- final trim and ordered write-out ---------------------------------------
    wave_lds_sync();  // the last tiles' appends are read by other lanes below
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll 1
        for (int gg = 0; gg < 4; ++gg) {
            const int t = qw0 + qb * 4 + gg;
            if (t >= nk) continue;
            const CandBuf qbuf = qbuf_of(qb * 4 + gg);
            const int c = __builtin_amdgcn_readlane(cnt[qb], 16 * gg);
            const int m = min(M, t + 1);
            if (c > m) wave_select<C::NE>(qbuf, c, m, hist);
            int32_t *dst = a.idx + (((size_t)b * nq + t - p0) * G + g) * M;
            for (int i = lane; i < M; i += 64) dst[i] = i < m ? (int32_t)qbuf.key[i] : -1;
        }
    }
}

template <typename T, int DI, int HH, int CAP>
hipError_t launch(const IndexerArgs &a, hipStream_t s) {
    constexpr int QB = LISA_IDX_QB;
    constexpr int QW = 4 * QB;
    const int nqb = (a.n + QW - 1) / QW;
    launch_kernel((indexer_topm_kernel<T, DI, HH, CAP, QB>), dim3(a.B * a.G * nqb), dim3(64), 0, s, a);
    return hipGetLastError();
}

template <typename T, int DI, int HH>
hipError_t by_m(const IndexerArgs &a, hipStream_t s) {
    // per-wave LDS: 4 candidate buffers of CAP 6-byte entries
    if (a.M <= 128) return launch<T, DI, HH, 256>(a, s);
    if (a.M <= 256) return launch<T, DI, HH, 448>(a, s);
    return launch<T, DI, HH, 1024>(a, s);
}

template <typename T>
hipError_t by_shape(const IndexerArgs &a, int dI, hipStream_t s) {
    const bool h2 = a.HI > 4;
    if (dI == 64) return h2 ? by_m<T, 64, 2>(a, s) : by_m<T, 64, 1>(a, s);
    return h2 ? by_m<T, 32, 2>(a, s) : by_m<T, 32, 1>(a, s);
}

}  // namespace

template <typename T>
hipError_t pack(const IndexerArgs &a, int dI, hipStream_t s) {
    const int nk = a.past + a.n, ntiles = (nk + kKT - 1) / kKT;
    const int64_t total = (int64_t)a.B * a.G * ntiles * kKT * dI / 8;  // lane-fragments
    const dim3 grid((unsigned)((total + 255) / 256));
    const T *src = reinterpret_cast<const T *>(a.k_idx);
    T *dst = reinterpret_cast<T *>(a.k_packed);
    if (dI == 64) launch_kernel((pack_keys_kernel<T, 64>), grid, dim3(256), 0, s, src, dst, total, nk, a.G, ntiles);
    else launch_kernel((pack_keys_kernel<T, 32>), grid, dim3(256), 0, s, src, dst, total, nk, a.G, ntiles);
    return hipGetLastError();
}

size_t indexer_packed_bytes(int B, int nk, int G, int dI, int dtype) {
    const size_t ntiles = ((size_t)nk + kKT - 1) / kKT;
    return (size_t)B * G * ntiles * kKT * dI * (dtype == 1 ? 2 : 4);
}

hipError_t launch_indexer_pack(const IndexerArgs &a, int dtype, int dI, hipStream_t s) {
    if (a.B * a.n == 0) return hipSuccess;
    return dtype == 1 ? pack<uint16_t>(a, dI, s) : pack<float>(a, dI, s);
}

hipError_t launch_indexer_prefill(const IndexerArgs &a, int dtype, int dI, hipStream_t s) {
    if (a.B * a.n == 0) return hipSuccess;
    return dtype == 1 ? by_shape<uint16_t>(a, dI, s) : by_shape<float>(a, dI, s);
}

}  // namespace lisa
