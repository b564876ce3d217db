// Prefill Lightning Indexer fused with a streaming top-M select.
//
// For each query t and KV group g the indexer scores every candidate s <= t,
//   I[t,s] = sum_j w[t,j] * max(0, q_idx[t,j] . k_idx[s])
// (query/key projections and a ReLU'd dot product: gptget.net analysis of
// arXiv 2607.19358, method-details section), and keeps the top-M candidates
// of the full context (arxivdaily page, English abstract), the lower index
// winning ties.  The n^2/2 scores never leave the chip:
//
//  * A work-group is one wave that owns QW = 4 * QB consecutive queries of
//    one group (16 for bf16 with up to 4 indexer heads).  It streams the
//    group's keys (L2-resident: every XCD serves a single group) in tiles of
//    64, loading the MFMA B fragments one tile ahead, and scores each tile
//    with 8 v_mfma_f32_16x16x32_bf16 per quad of 4 queries.  The keys are
//    first re-laid out (pack_keys_kernel) so that every fragment load reads
//    1 KB of consecutive bytes.  One loaded tile serves all QW queries: the
//    address unit, which bounds a wave that holds only 4 queries, then has
//    room to spare, and the VALU epilogue is the limit.
//  * A operand rows are (query, indexer head) pairs laid out so that the four
//    accumulator rows a lane receives are the four heads of one query: the
//    ReLU and the w-weighted head sum are lane-local.  Column n of key block
//    cb holds key k0 + 4n + cb, so each lane scores four consecutive keys of
//    its query.
//  * A candidate is accepted when its score is strictly above the query's
//    threshold tau (a later equal score loses: the lowest-index tie-break).
//    Accepted (score, key) pairs go, in key order, to a per-query staging
//    ring in LDS (positions from an exclusive scan of the per-lane counts over
//    the query's 16-lane row, by DPP), and from there in blocks of 64 to the
//    query's candidate buffer in global memory (workspace).  A query's
//    candidates are thus always in ascending key order.
//  * When a buffer could overflow on the next tile it is trimmed in place: a
//    256-bin histogram over the buffered scores finds the bin holding the
//    M-th largest; the lower bins are dropped and tau becomes the largest
//    dropped score, so at least M kept candidates beat everything rejected.
//    When that frees too little (exact ties) an exact select keeps M.
//  * Late queries start from a threshold estimated from a sample of key
//    tiles, so that only about 2 M candidates are appended; a query left
//    with fewer than min(M, t+1) candidates (the estimate was too high) is
//    scanned again from tau = -inf, so the result is exact whatever the
//    sample says.
//  * The exact select (radix select on order-preserving keys, ties to the
//    lower buffer position = lower index) keeps min(M, t+1) candidates at the
//    end; they are written out in buffer order, which is ascending.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lisa {
namespace {

constexpr int kKT = 64;     // keys per tile
constexpr int kRing = 128;  // staging-ring entries per query (LDS)

__device__ __forceinline__ float key_to_float(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// Make this wave's global-memory writes visible to its other lanes' reads
// (the candidate buffers are written and read back by different lanes).
__device__ __forceinline__ void wave_global_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// A query's buffered candidates in registers: entry k*64 + lane in slot k.
template <int NE>
struct Cands {
    float sc[NE];
    uint32_t key[NE];
};

template <int NE>
__device__ __forceinline__ void load_cands(const u32x2 *qbuf, int c, Cands<NE> &x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const int e = k * 64 + lane;
        u32x2 v = u32x2{0u, 0u};
        if (e < c) v = qbuf[e];
        x.sc[k] = __uint_as_float(v[0]);
        x.key[k] = v[1];
    }
}

// Mark exactly the first m of the c candidates in the order (higher score,
// lower buffer position).  Whole wave, uniform control flow.  Returns the
// order key of the m-th.  The threshold is found by 256-bin histogram passes
// over the live range of order keys, [min, max] first (buffered candidates
// sit in a narrow band, so fixed 8-bit digits would waste passes on common
// high bits); a pass stops as soon as the bin holding the m-th key is taken
// whole, or holds a single key value (ties: the earliest positions win).
template <int NE>
__device__ uint32_t select_first(const Cands<NE> &x, int c, int m, bool (&keep)[NE], uint32_t *hist) {
    const int lane = threadIdx.x & 63;
    // order keys are recomputed where needed rather than held (registers)
    auto u = [&](int k) { return order_key(x.sc[k]); };
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        if (k * 64 + lane < c) {
            kmin = min(kmin, u(k));
            kmax = max(kmax, u(k));
        }
    }
    uint32_t lo = wave_min_u32(kmin);
    const uint32_t span = wave_max_u32(kmax) - lo;
    int width = span == 0 ? 0 : 32 - __builtin_clz(span);  // bits of key - lo
    uint32_t need = (uint32_t)m;
    uint32_t theta;    // keys > theta are kept, and keys == theta up to take_eq,
    uint32_t take_eq;  // or (whole_bin) every key >= theta
    bool whole_bin;
#pragma unroll 1
    for (;;) {
        const int shift = width > 8 ? width - 8 : 0;
        *reinterpret_cast<u32x4 *>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
        wave_lds_sync();
        const uint64_t hi_excl = (uint64_t)lo + ((uint64_t)1 << width);
#pragma unroll
        for (int k = 0; k < NE; ++k) {
            const uint32_t uk = u(k);
            if (k * 64 + lane < c && uk >= lo && (uint64_t)uk < hi_excl) atomicAdd(&hist[(uk - lo) >> shift], 1u);
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
    uint32_t eq_seen = 0u, kth = 0xFFFFFFFFu;
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const bool valid = k * 64 + lane < c;
        const uint32_t uk = u(k);
        const bool gt = valid && (whole_bin ? uk >= theta : uk > theta);
        const bool eq = valid && !whole_bin && uk == theta;
        const uint64_t em = __ballot(eq);
        const uint32_t er = eq_seen + mbcnt64(em);
        eq_seen += (uint32_t)__popcll(em);
        keep[k] = gt || (eq && er < take_eq);
        if (keep[k]) kth = min(kth, uk);
    }
    return wave_min_u32(kth);
}

// Stable compaction of the kept entries to positions 0.. (slot order =
// buffer order); returns how many were kept.
template <int NE, typename F>
__device__ __forceinline__ int compact(const bool (&keep)[NE], F &&put) {
    uint32_t base = 0u;
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const uint64_t km = __ballot(keep[k]);
        const uint32_t pos = base + mbcnt64(km);
        base += (uint32_t)__popcll(km);
        if (keep[k]) put(k, pos);
    }
    return (int)base;
}

// ---- trims: streaming passes over a query's buffer in global memory --------
// A trim runs on the rare occasions a buffer fills up (a query rescanned from
// tau = -inf, or adversarial scores), so it reads the buffer in chunks of 256
// entries per pass rather than holding it in registers: the scan's own
// registers stay live across it.
constexpr int kChunkL = 4;  // entries per lane and chunk

// f(e, valid, score, key) for every entry e < c, in order; the chunk's loads
// are all issued before f sees any of them
template <typename F>
__device__ __forceinline__ void stream_cands(const u32x2 *qbuf, int c, F &&f) {
    const int lane = threadIdx.x & 63;
#pragma unroll 1
    for (int base = 0; base < c; base += 64 * kChunkL) {
        u32x2 v[kChunkL];
#pragma unroll
        for (int j = 0; j < kChunkL; ++j) {
            const int e = base + j * 64 + lane;
            v[j] = e < c ? qbuf[e] : u32x2{0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kChunkL; ++j) {
            const int e = base + j * 64 + lane;
            f(e, e < c, __uint_as_float(v[j][0]), v[j][1]);
        }
    }
}

// In-place stable compaction of the entries keep(score, key, rank) marks,
// where rank counts the earlier entries for which eq(score) holds.  A kept
// entry moves to a position at or below its own, and every position a chunk
// writes was read by that chunk or an earlier one, so reads and writes do not
// collide.
template <typename K, typename E>
__device__ int compact_stream(u32x2 *qbuf, int c, K &&keep, E &&eq) {
    uint32_t base = 0u, eq_seen = 0u;
    stream_cands(qbuf, c, [&](int, bool valid, float sc, uint32_t key) {
        const bool is_eq = valid && eq(sc);
        const uint64_t em = __ballot(is_eq);
        const uint32_t er = eq_seen + mbcnt64(em);
        eq_seen += (uint32_t)__popcll(em);
        const bool kp = valid && keep(sc, is_eq, er);
        const uint64_t km = __ballot(kp);
        const uint32_t pos = base + mbcnt64(km);
        base += (uint32_t)__popcll(km);
        if (kp) qbuf[pos] = u32x2{__float_as_uint(sc), key};
    });
    return (int)base;
}

struct TrimResult {
    int c;
    float tau;
};

// Trim one query's c buffered candidates to about M, in place.  First a
// 256-bin histogram over [min, max] of the scores: every bin from the one
// holding the M-th largest up is kept, and tau becomes the largest dropped
// score, so at least M kept candidates beat everything rejected.  When that
// would keep more than c - need_free (exact ties, or a spread too narrow for
// the bins), radix passes over the order keys find the M-th exactly and
// exactly M are kept (ties: the earliest positions, the lower indices).
__device__ __attribute__((noinline)) TrimResult trim_buffer(u32x2 *qbuf, int c, int M, int need_free,
                                                            uint32_t *hist) {
    const int lane = threadIdx.x & 63;
    float mn = INFINITY, mx = -INFINITY;
    stream_cands(qbuf, c, [&](int, bool valid, float sc, uint32_t) {
        if (valid) {
            mn = fminf(mn, sc);
            mx = fmaxf(mx, sc);
        }
    });
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (mx > mn) {
        const float scale = 255.99f / (mx - mn);
        auto bin_of = [&](float sc) { return min(255, (int)((sc - mn) * scale)); };
        *reinterpret_cast<u32x4 *>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
        wave_lds_sync();
        stream_cands(qbuf, c, [&](int, bool valid, float sc, uint32_t) {
            if (valid) atomicAdd(&hist[bin_of(sc)], 1u);
        });
        wave_lds_sync();
        const u32x4 h = *reinterpret_cast<const u32x4 *>(hist + 4 * lane);
        const uint32_t incl = wave_inclusive_scan(h[0] + h[1] + h[2] + h[3]);
        const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        uint32_t run = total - incl;
        int fb = -1;
        uint32_t kept = 0;
#pragma unroll
        for (int bb = 3; bb >= 0; --bb) {
            if (fb < 0 && run < (uint32_t)M && run + h[bb] >= (uint32_t)M) {
                fb = 4 * lane + bb;
                kept = run + h[bb];
            }
            run += h[bb];
        }
        const int src = __ffsll((unsigned long long)__ballot(fb >= 0)) - 1;
        fb = __builtin_amdgcn_readlane(fb, src);
        kept = (uint32_t)__builtin_amdgcn_readlane((int)kept, src);
        wave_lds_sync();
        if (fb > 0 && (int)kept <= c - need_free) {
            float dmax = -INFINITY;
            stream_cands(qbuf, c, [&](int, bool valid, float sc, uint32_t) {
                if (valid && bin_of(sc) < fb) dmax = fmaxf(dmax, sc);
            });
            dmax = wave_max(dmax);
            const int nk = compact_stream(
                qbuf, c, [&](float sc, bool, uint32_t) { return bin_of(sc) >= fb; }, [](float) { return false; });
            wave_global_sync();
            return TrimResult{nk, dmax};
        }
    }
    // exact: radix passes over the live range of order keys, as select_first
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    stream_cands(qbuf, c, [&](int, bool valid, float sc, uint32_t) {
        if (valid) {
            kmin = min(kmin, order_key(sc));
            kmax = max(kmax, order_key(sc));
        }
    });
    uint32_t lo = wave_min_u32(kmin);
    const uint32_t span = wave_max_u32(kmax) - lo;
    int width = span == 0 ? 0 : 32 - __builtin_clz(span);
    uint32_t need = (uint32_t)M, theta, take_eq;
    bool whole_bin;
#pragma unroll 1
    for (;;) {
        const int shift = width > 8 ? width - 8 : 0;
        *reinterpret_cast<u32x4 *>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
        wave_lds_sync();
        const uint64_t hi_excl = (uint64_t)lo + ((uint64_t)1 << width);
        stream_cands(qbuf, c, [&](int, bool valid, float sc, uint32_t) {
            const uint32_t u = order_key(sc);
            if (valid && u >= lo && (uint64_t)u < hi_excl) atomicAdd(&hist[(u - lo) >> shift], 1u);
        });
        wave_lds_sync();
        const u32x4 h = *reinterpret_cast<const u32x4 *>(hist + 4 * lane);
        const uint32_t incl = wave_inclusive_scan(h[0] + h[1] + h[2] + h[3]);
        const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        uint32_t run = total - incl;
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
        if (fneed == fcnt || shift == 0) {
            theta = blo;
            whole_bin = fneed == fcnt;
            take_eq = whole_bin ? 0u : fneed;
            break;
        }
        lo = blo;
        width = shift;
        need = fneed;
    }
    const int nk = compact_stream(
        qbuf, c,
        [&](float sc, bool is_eq, uint32_t er) {
            const uint32_t u = order_key(sc);
            return (whole_bin ? u >= theta : u > theta) || (is_eq && er < take_eq);
        },
        [&](float sc) { return !whole_bin && order_key(sc) == theta; });
    wave_global_sync();
    // the M-th kept key bounds every later candidate: equal scores lose
    return TrimResult{nk, key_to_float(theta)};
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

template <typename T, int DI, int HH, int QB, int CAPG>
struct IdxCfg {
    static constexpr int KD = DI / 32;  // MFMA K-steps
    static constexpr int QW = 4 * QB;   // queries per wave: QB quads of 4
    static constexpr int NE = CAPG / 64;
};

template <typename T, int DI, int HH, int QB, int CAPG>
__global__ __launch_bounds__(64) void indexer_topm_kernel(IndexerArgs a) {
    using C = IdxCfg<T, DI, HH, QB, CAPG>;
    constexpr int kQW = C::QW;
    __shared__ __attribute__((aligned(16))) u32x2 ring[kQW * kRing];
    __shared__ __attribute__((aligned(16))) uint32_t hist[256];

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
    // candidate buffer of query row tr: unit (b, tr, g)
    u32x2 *const cand = reinterpret_cast<u32x2 *>(a.cand);
    auto qbuf_of = [&](int qq) { return cand + (((size_t)b * nq + (qw0 - p0 + qq)) * G + g) * CAPG; };

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
    // per quad, for this lane's query: candidates so far (cnt), how many of
    // them are already in the global buffer (fl), and the threshold
    int cnt[QB], fl[QB];
    float tau[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        cnt[qb] = 0;
        fl[qb] = 0;
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

    // scores of one quad for one tile: score[cb] for key k0 + 4*col + cb of query tq[qb]
    auto quad_scores = [&](int qb, const Frag<T> (&bcur)[4][C::KD], float (&score)[4]) {
        f32x4 acc[HH][4];
#pragma unroll
        for (int hh = 0; hh < HH; ++hh)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                f32x4 x = {0, 0, 0, 0};
#pragma unroll
                for (int kc = 0; kc < C::KD; ++kc) x = mma16(af[qb][hh][kc], bcur[cb][kc], x);
                acc[hh][cb] = x;
            }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            float sc = 0.0f;
#pragma unroll
            for (int hh = 0; hh < HH; ++hh)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc = fmaf(wv[qb][hh][i], fmaxf(acc[hh][cb][i], 0.0f), sc);
            score[cb] = sc;
        }
    };

    // Move entries [fl, fl + 64) of query qq from its ring to its global buffer.
    auto flush64 = [&](int qq, int f) {
        const u32x2 e = ring[qq * kRing + ((f + lane) & (kRing - 1))];
        qbuf_of(qq)[f + lane] = e;
    };
    // Move the ring's remaining entries [f, c) (fewer than 64) to the buffer.
    auto flush_rest = [&](int qq, int f, int c) {
        if (lane < c - f) {
            const u32x2 e = ring[qq * kRing + ((f + lane) & (kRing - 1))];
            qbuf_of(qq)[f + lane] = e;
        }
    };

    // The rejected keys of an append write to a per-lane sink (in the
    // histogram, which every trim and select clears before use), so appends
    // are straight-line code with no exec-mask branches.
    u32x2 *const sink = reinterpret_cast<u32x2 *>(hist) + lane;

    auto tile_step = [&](int kt, const Frag<T> (&bcur)[4][C::KD], auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;  // tile reaches past the first query
        const int k0 = kt * kKT;
        // every quad's MFMAs first, so that the matrix core runs ahead of the
        // epilogues instead of each epilogue waiting for its quad's results
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
        uint64_t flushq = 0;  // quads with a query to flush (64+ ring entries) or to trim
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float score[4];
            bool ok[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                float sc = 0.0f;
#pragma unroll
                for (int hh = 0; hh < HH; ++hh)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sc = fmaf(wv[qb][hh][i], fmaxf(acc[qb][hh][cb][i], 0.0f), sc);
                score[cb] = sc;
                if constexpr (DIAG) ok[cb] = (k0 + 4 * col + cb <= tq[qb]) && sc > tau[qb];
                else ok[cb] = sc > tau[qb];
            }
            // Append in ascending key order: a query's accepted keys are
            // ordered by (col, cb), so a lane's first position is the query's
            // count plus the exclusive scan of the per-lane counts over its
            // 16-lane row.
            const uint32_t c4 = (uint32_t)ok[0] + (uint32_t)ok[1] + (uint32_t)ok[2] + (uint32_t)ok[3];
            const uint32_t incl = row_inclusive_scan(c4);
            const uint32_t tot = row_broadcast15(incl);
            int pos = cnt[qb] + (int)(incl - c4);
            u32x2 *qring = ring + (qb * 4 + grp) * kRing;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                u32x2 *dst = ok[cb] ? qring + (pos & (kRing - 1)) : sink;
                *dst = u32x2{__float_as_uint(score[cb]), (uint32_t)(k0 + 4 * col + cb)};
                pos += ok[cb] ? 1 : 0;
            }
            cnt[qb] += (int)tot;
            flushq |= __ballot(cnt[qb] - fl[qb] >= 64 || cnt[qb] > CAPG - kKT) ? (1ull << qb) : 0ull;
        }
        if (!flushq) return;
        wave_lds_sync();  // the appends are read by other lanes below
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if (!((flushq >> qb) & 1ull)) continue;
            const uint64_t need = __ballot(cnt[qb] - fl[qb] >= 64);
#pragma unroll 1
            for (int gg = 0; gg < 4; ++gg) {
                if (!((need >> (16 * gg)) & 1ull)) continue;
                flush64(qb * 4 + gg, __builtin_amdgcn_readlane(fl[qb], 16 * gg));
            }
#pragma unroll
            for (int gg = 0; gg < 4; ++gg)
                if (grp == gg && ((need >> (16 * gg)) & 1ull)) fl[qb] += 64;
            // trim any buffer that could overflow on the next tile
            const uint64_t full = __ballot(cnt[qb] > CAPG - kKT);
            if (!full) continue;
#pragma unroll 1
            for (int gg = 0; gg < 4; ++gg) {
                if (!((full >> (16 * gg)) & 1ull)) continue;
                const int qq = qb * 4 + gg;
                const int c = __builtin_amdgcn_readlane(cnt[qb], 16 * gg);
                flush_rest(qq, __builtin_amdgcn_readlane(fl[qb], 16 * gg), c);
                wave_global_sync();
                const TrimResult tr = trim_buffer(qbuf_of(qq), c, M, CAPG / 4, hist);
                if (grp == gg) {
                    cnt[qb] = tr.c;
                    fl[qb] = tr.c;
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
    // candidates (tau was too high) is scanned again from tau = -inf.
    constexpr float kSlack = 2.0f;
    constexpr int kRank = 32;
    float tau1[QB];  // a lower start for queries the first estimate starves
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) tau1[qb] = -INFINITY;
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
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float score[4];
                quad_scores(qb, bc, score);
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    float x = score[cb];  // insert into the descending top-4
#pragma unroll
                    for (int i = 0; i < 3; ++i) {
                        const float hi = fmaxf(top[qb][i], x);
                        x = fminf(top[qb][i], x);
                        top[qb][i] = hi;
                    }
                    top[qb][3] = fmaxf(top[qb][3], x);
                }
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
            const float R = fminf(30.0f, fmaxf(1.0f, rintf(kSlack * (float)M * S / (float)(tq[qb] + 1))));
            auto count_ge = [&](float x) {
                const uint32_t c = (uint32_t)(top[qb][0] >= x) + (uint32_t)(top[qb][1] >= x) +
                                   (uint32_t)(top[qb][2] >= x) + (uint32_t)(top[qb][3] >= x);
                return (float)row_broadcast15(row_inclusive_scan(c));
            };
            // the largest x with at least R kept sample values >= x, by bisection
            auto rank_value = [&](float R) {
                float lo = row_min(top[qb][3]), hi = row_max(top[qb][0]);
                if (count_ge(hi) >= R) lo = hi;
#pragma unroll 1
                for (int it = 0; it < 12; ++it) {
                    const float mid = 0.5f * (lo + hi);
                    const bool up = count_ge(mid) >= R;
                    lo = up ? mid : lo;
                    hi = up ? hi : mid;
                }
                return lo;
            };
            if (tq[qb] < nk) {
                tau[qb] = rank_value(R);
                tau1[qb] = rank_value(fminf(60.0f, 2.0f * R));
            }
        }
    }

    // ---- scan: every tile, two fragment buffers alternating (tile kt+1 loads
    // while kt computes).  A query left with fewer than min(M, t+1) candidates
    // had its threshold at or above its M-th score: it is scanned again from
    // the lower sample estimate tau1, and if that starves it too, from -inf;
    // the wave's other queries take nothing in those passes. --------------------
    auto step = [&](int kt, const Frag<T> (&bc)[4][C::KD]) {
        if (kt >= kd) tile_step(kt, bc, std::true_type{});
        else tile_step(kt, bc, std::false_type{});
    };
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
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
        if (!redo || pass == 2) break;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            // kept queries take nothing more (their counts stay below a trim)
            tau[qb] = fail[qb] ? (pass == 0 ? tau1[qb] : -INFINITY) : INFINITY;
            cnt[qb] = fail[qb] ? 0 : cnt[qb];
            fl[qb] = fail[qb] ? 0 : fl[qb];
        }
    }

    // ---- final select and ordered write-out --------------------------------------
    wave_lds_sync();  // the last tiles' appends are read by other lanes below
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll 1
        for (int gg = 0; gg < 4; ++gg) {
            const int t = qw0 + qb * 4 + gg;
            if (t >= nk) continue;
            const int qq = qb * 4 + gg;
            const int c = __builtin_amdgcn_readlane(cnt[qb], 16 * gg);
            flush_rest(qq, __builtin_amdgcn_readlane(fl[qb], 16 * gg), c);
            wave_global_sync();
            const int m = min(M, t + 1);
            Cands<C::NE> x;
            load_cands<C::NE>(qbuf_of(qq), c, x);
            bool keep[C::NE];
            if (c > m) {
                select_first<C::NE>(x, c, m, keep, hist);
            } else {
#pragma unroll
                for (int k = 0; k < C::NE; ++k) keep[k] = k * 64 + lane < c;
            }
            int32_t *dst = a.idx + (((size_t)b * nq + t - p0) * G + g) * M;
            const int kept = compact<C::NE>(keep, [&](int k, uint32_t pos) { dst[pos] = (int32_t)x.key[k]; });
            for (int i = kept + lane; i < M; i += 64) dst[i] = -1;
        }
    }
}

// Candidate-buffer entries per query, 4 M' + 128 for M up to M' (a query is
// trimmed when it holds more than CAPG - 64): a query below 4 M starts from
// -inf and appends every key, so it never trims; a later one starts from a
// sampled threshold expected to admit about 2 M keys.
int cand_entries(int M) { return M <= 64 ? 384 : M <= 128 ? 640 : M <= 256 ? 1152 : 2176; }

template <typename T, int DI, int HH, int QB>
hipError_t launch_q(const IndexerArgs &a, hipStream_t s) {
    constexpr int QW = 4 * QB;
    const int nqb = (a.n + QW - 1) / QW;
    const dim3 grid((unsigned)(a.B * a.G * nqb));
    switch (cand_entries(a.M)) {
        case 384: launch_kernel((indexer_topm_kernel<T, DI, HH, QB, 384>), grid, dim3(64), 0, s, a); break;
        case 640: launch_kernel((indexer_topm_kernel<T, DI, HH, QB, 640>), grid, dim3(64), 0, s, a); break;
        case 1152: launch_kernel((indexer_topm_kernel<T, DI, HH, QB, 1152>), grid, dim3(64), 0, s, a); break;
        default: launch_kernel((indexer_topm_kernel<T, DI, HH, QB, 2176>), grid, dim3(64), 0, s, a); break;
    }
    return hipGetLastError();
}

// Queries per wave (4 * QB).  More queries share each loaded key tile (the
// address unit's load), fewer leave registers for more waves per SIMD and
// give short prompts enough waves to fill the chip: QB = 2 (8 queries, 3
// waves per SIMD) unless that leaves fewer than 2048 waves, then QB = 1.
// fp32 fragments take twice the registers: QB = 1.
template <typename T, int DI>
hipError_t by_heads(const IndexerArgs &a, hipStream_t s) {
    if constexpr (std::is_same<T, float>::value) {
        return a.HI > 4 ? launch_q<T, DI, 2, 1>(a, s) : launch_q<T, DI, 1, 1>(a, s);
    } else {
        const int64_t units = (int64_t)a.B * a.G * a.n;
        const bool wide = units / 8 >= 2048;
        if (a.HI > 4) return wide ? launch_q<T, DI, 2, 2>(a, s) : launch_q<T, DI, 2, 1>(a, s);
        return wide ? launch_q<T, DI, 1, 2>(a, s) : launch_q<T, DI, 1, 1>(a, s);
    }
}

template <typename T>
hipError_t by_shape(const IndexerArgs &a, int dI, hipStream_t s) {
    return dI == 64 ? by_heads<T, 64>(a, s) : by_heads<T, 32>(a, s);
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

size_t indexer_cand_bytes(int B, int n, int G, int M) {
    return (size_t)B * n * G * cand_entries(M) * sizeof(u32x2);
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
