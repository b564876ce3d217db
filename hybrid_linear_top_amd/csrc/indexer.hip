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
//    Each lane stages its accepted (score, key) pairs per query in LDS, up to
//    kLane of them, with straight-line code (every key is written at the next
//    free slot, which advances only past accepted ones).  When a lane could
//    overflow on the next tile, the quad's staged pairs go to the queries'
//    candidate buffers in global memory (workspace), each lane after the lower
//    lanes of its query's row (a DPP scan of the counts).  Buffer order is
//    therefore arbitrary; indices in it are distinct.
//  * When a buffer could overflow on the next flush it is trimmed in place by
//    streaming passes: a 256-bin histogram over the buffered scores finds the
//    bin holding the M-th largest; the lower bins are dropped and tau becomes
//    the largest dropped score, so at least M kept candidates beat everything
//    rejected.  When that frees too little (exact ties) an exact select
//    keeps M.
//  * Late queries start from a threshold estimated from a sample of key
//    tiles, so that only about 2 M candidates are appended; a query left
//    with fewer than min(M, t+1) candidates (the estimate was too high) is
//    scanned again, first from a lower sample estimate, then from -inf, so
//    the result is exact whatever the sample says.
//  * At the end an exact select (radix select on order-preserving 64-bit
//    keys: score, then the lower index) keeps min(M, t+1) candidates; they
//    are marked in an LDS bitmap over positions 0..t and written out in
//    position order, -1 padded.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lisa {
namespace {

constexpr int kKT = 64;    // keys per tile
constexpr int kLane = 8;   // staging entries per lane and query (LDS)

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

// The candidate order as one 64-bit key: higher score first (order-preserving
// bits, -0.0 = +0.0), then lower index.  A query's candidates have distinct
// indices, so their keys are distinct.
__device__ __forceinline__ uint64_t cand_key(float sc, uint32_t idx) {
    return ((uint64_t)order_key(sc) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

// Radix select over 32-bit values: for_each(f) presents f(valid, v) (v may
// repeat); with 1 <= m <= the number of valid values, returns lo such that
// the values >= lo are the m largest -- exactly m of them (*need = 0) or,
// when the m-th largest value is tied, the ones above it plus *need of those
// equal to it (then lo is that value).  256-bin passes over [min, max] (the
// values sit in a narrow band), each narrowing to the bin that holds the
// m-th value, until a bin is taken whole or holds one value.  Whole wave,
// uniform control flow.
template <typename ForEach>
__device__ uint32_t select32(ForEach &&for_each, int m, uint32_t *hist, uint32_t *need_out) {
    const int lane = threadIdx.x & 63;
    uint32_t vmin = 0xFFFFFFFFu, vmax = 0u;
    for_each([&](bool valid, uint32_t v) {
        if (valid) {
            vmin = min(vmin, v);
            vmax = max(vmax, v);
        }
    });
    uint32_t lo = wave_min_u32(vmin);
    const uint32_t span = wave_max_u32(vmax) - lo;
    int width = span == 0 ? 0 : 32 - __builtin_clz(span);  // bits of v - lo
    uint32_t need = (uint32_t)m;
#pragma unroll 1
    for (;;) {
        const int shift = width > 8 ? width - 8 : 0;
        const uint32_t last = width >= 32 ? 0xFFFFFFFFu : (1u << width) - 1u;  // the range is [lo, lo + last]
        *reinterpret_cast<u32x4 *>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
        wave_lds_sync();
        for_each([&](bool valid, uint32_t v) {
            if (valid && v >= lo && v - lo <= last) atomicAdd(&hist[(v - lo) >> shift], 1u);
        });
        wave_lds_sync();
        const u32x4 h = *reinterpret_cast<const u32x4 *>(hist + 4 * lane);
        const uint32_t incl = wave_inclusive_scan(h[0] + h[1] + h[2] + h[3]);
        const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        uint32_t run = total - incl;  // values in the bins of higher lanes
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
        if (fneed == fcnt) {  // the bin taken whole
            *need_out = 0u;
            return blo;
        }
        if (shift == 0) {  // a single tied value
            *need_out = fneed;
            return blo;
        }
        lo = blo;
        width = shift;
        need = fneed;
    }
}

// theta = the m-th largest of the distinct 64-bit candidate keys (score
// order key above, complemented index below) that for_each(f) presents as
// f(valid, order_key(score), index): exactly m keys are >= theta.  A select
// on the scores first; only a tie at the M-th score needs a second one, on
// the indices of the tied candidates (lower index first).
template <typename ForEach>
__device__ uint64_t select_theta(ForEach &&for_each, int m, uint32_t *hist) {
    uint32_t need = 0u;
    const uint32_t hi = select32(
        [&](auto &&f) { for_each([&](bool valid, uint32_t ok, uint32_t) { f(valid, ok); }); }, m, hist, &need);
    if (need == 0u) return (uint64_t)hi << 32;
    uint32_t none = 0u;
    const uint32_t lo = select32(
        [&](auto &&f) { for_each([&](bool valid, uint32_t ok, uint32_t idx) { f(valid && ok == hi, ~idx); }); },
        (int)need, hist, &none);
    return ((uint64_t)hi << 32) | lo;
}

// ---- trims: streaming passes over a query's buffer in global memory --------
// A trim runs on the rare occasions a buffer fills up (a query rescanned from
// a low threshold, or adversarial scores), so it reads the buffer in chunks
// of 256 entries per pass rather than holding it in registers: the scan's own
// registers stay live across it.
constexpr int kChunkL = 4;  // entries per lane and chunk

// f(valid, score, index) for every entry e < c; a chunk's loads are all
// issued before f sees any of them
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
        for (int j = 0; j < kChunkL; ++j) f(base + j * 64 + lane < c, __uint_as_float(v[j][0]), v[j][1]);
    }
}

// In-place stable compaction of the entries keep(score, index) marks.  A
// kept entry moves to a position at or below its own, and every position a
// chunk writes was read by that chunk or an earlier one.
template <typename K>
__device__ int compact_stream(u32x2 *qbuf, int c, K &&keep) {
    uint32_t base = 0u;
    stream_cands(qbuf, c, [&](bool valid, float sc, uint32_t idx) {
        const bool kp = valid && keep(sc, idx);
        const uint64_t km = __ballot(kp);
        const uint32_t pos = base + mbcnt64(km);
        base += (uint32_t)__popcll(km);
        if (kp) qbuf[pos] = u32x2{__float_as_uint(sc), idx};
    });
    return (int)base;
}

struct TrimResult {
    int c;
    float tau;
};

// Trim one query's c buffered candidates (all in its global buffer) to at
// most max_keep and at least M, in place.  First a 256-bin histogram over
// [min, max] of the scores: every bin from the one holding the M-th largest
// up is kept, and tau becomes the largest dropped score, so at least M kept
// candidates beat everything rejected.  When that would keep more than
// max_keep (exact ties, or a spread too narrow for the bins), the exact M are
// kept (select_theta on the candidate keys) and tau is the M-th score: a later
// key with that score has a higher index and loses.
__device__ __attribute__((noinline)) TrimResult trim_buffer(u32x2 *qbuf, int c, int M, int max_keep,
                                                            uint32_t *hist) {
    const int lane = threadIdx.x & 63;
    float mn = INFINITY, mx = -INFINITY;
    stream_cands(qbuf, c, [&](bool valid, float sc, uint32_t) {
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
        stream_cands(qbuf, c, [&](bool valid, float sc, uint32_t) {
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
        if (fb > 0 && (int)kept <= max_keep) {
            float dmax = -INFINITY;
            stream_cands(qbuf, c, [&](bool valid, float sc, uint32_t) {
                if (valid && bin_of(sc) < fb) dmax = fmaxf(dmax, sc);
            });
            dmax = wave_max(dmax);
            const int nk = compact_stream(qbuf, c, [&](float sc, uint32_t) { return bin_of(sc) >= fb; });
            wave_global_sync();
            return TrimResult{nk, dmax};
        }
    }
    const uint64_t theta = select_theta(
        [&](auto &&f) {
            stream_cands(qbuf, c, [&](bool valid, float sc, uint32_t idx) { f(valid, order_key(sc), idx); });
        },
        M, hist);
    const int nk = compact_stream(qbuf, c, [&](float sc, uint32_t idx) { return cand_key(sc, idx) >= theta; });
    wave_global_sync();
    return TrimResult{nk, key_to_float((uint32_t)(theta >> 32))};
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
    // entries per lane of the final select: room for 2 M + 128 candidates
    static constexpr int NF = CAPG <= 512 ? 4 : CAPG <= 768 ? 6 : CAPG <= 1280 ? 10 : 18;
};

template <typename T, int DI, int HH, int QB, int CAPG>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 4 : 1))) void indexer_topm_kernel(IndexerArgs a) {
    using C = IdxCfg<T, DI, HH, QB, CAPG>;
    constexpr int kQW = C::QW;
    // per query, per lane of its 16-lane row: kLane staged candidates; the
    // area doubles as the final select's bitmap with a rank per word (1024
    // words: positions up to 32767)
    constexpr int kListEntries = kQW * 16 * kLane > 1024 ? kQW * 16 * kLane : 1024;
    __shared__ __attribute__((aligned(16))) u32x2 lists[kListEntries];
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
    // candidate buffer of query qq of the wave: unit (b, row, g)
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
    // per quad: this lane's staged candidates (cl), its query's candidates in
    // the global buffer (gc, the same on the query's 16 lanes) and threshold
    int cl[QB], gc[QB];
    float tau[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        cl[qb] = 0;
        gc[qb] = 0;
        tau[qb] = tq[qb] < nk ? -INFINITY : INFINITY;  // padding queries accept nothing
    }
    // this lane's staging list for the query of quad qb: entry j at
    // list_of(qb)[64 j] (slot-major over the wave's lanes, so that the lanes'
    // writes of one slot index fall in distinct LDS banks)
    auto list_of = [&](int qb) { return lists + qb * kLane * 64 + lane; };

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
                frag_buf_load(bf[cb][kc], r, voff, (uint32_t)(cb * C::KD + kc) * kFragBytes);
    };

    // One tile in two halves: every quad's MFMAs (the caller then reuses the
    // fragment registers for the next tile's loads, in flight during the
    // epilogue), and the epilogue, score[qb][cb] for key k0 + 4*col + cb of
    // query tq[qb].
    using Acc = f32x4[QB][HH][4];
    auto tile_mfma = [&](const Frag<T> (&bcur)[4][C::KD], Acc &acc) {
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
    };
    auto tile_epilogue = [&](const Acc &acc, float (&score)[QB][4]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                float sc = 0.0f;
#pragma unroll
                for (int hh = 0; hh < HH; ++hh)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sc = fmaf(wv[qb][hh][i], fmaxf(acc[qb][hh][cb][i], 0.0f), sc);
                score[qb][cb] = sc;
            }
    };

    // Move quad qb's staged candidates to its queries' global buffers: a
    // lane's entries go after those of the lower lanes of its row (exclusive
    // scan of the counts over the row).  Then trim any buffer that another
    // flush could overflow.
    // The wave's candidate buffers through one descriptor: query qq's entry e
    // is entry qq * G * CAPG + e; stores at offsets past the end are dropped,
    // so a lane's flush needs no branch per entry.
    const uint32_t qstride = (uint32_t)G * CAPG;
    const rsrc_t crs = make_rsrc(qbuf_of(0), ((uint32_t)(kQW - 1) * qstride + CAPG) * 8u);
    auto flush_quad = [&](int qb) {
        const uint32_t incl = row_inclusive_scan((uint32_t)cl[qb]);
        const int tot = (int)row_broadcast15(incl);
        const uint32_t off = (uint32_t)(qb * 4 + grp) * qstride + (uint32_t)(gc[qb] + (int)incl - cl[qb]);
        const u32x2 *const my = list_of(qb);
        u32x2 e[kLane];
#pragma unroll
        for (int j = 0; j < kLane; ++j) e[j] = my[64 * j];  // all reads first: one wait
#pragma unroll
        for (int j = 0; j < kLane; ++j)
            __builtin_amdgcn_raw_buffer_store_b64(e[j], crs, j < cl[qb] ? (off + (uint32_t)j) * 8u : kOffNone, 0u, 0);
        gc[qb] += tot;
        cl[qb] = 0;
        const uint64_t full = __ballot(gc[qb] > CAPG - 16 * kLane);
        if (!full) return;
        wave_global_sync();
#pragma unroll 1
        for (int gg = 0; gg < 4; ++gg) {
            if (!((full >> (16 * gg)) & 1ull)) continue;
            const TrimResult tr = trim_buffer(qbuf_of(qb * 4 + gg), __builtin_amdgcn_readlane(gc[qb], 16 * gg), M,
                                              CAPG - 2 * 16 * kLane, hist);
            if (grp == gg) {
                gc[qb] = tr.c;
                tau[qb] = tr.tau;
            }
        }
    };

    auto tile_step = [&](int kt, const Acc &acc, auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;  // tile reaches past the first query
        const int k0 = kt * kKT;
        float score[QB][4];
        tile_epilogue(acc, score);
        uint64_t flushq = 0;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            u32x2 *const my = list_of(qb);
            // Every key is written at the lane's next free slot, and the slot
            // advances only past accepted ones: a rejected key is overwritten
            // by the next key or left past the end, so staging is
            // straight-line code (slots cl .. cl + 3 are at most 7 here).
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const uint32_t key = (uint32_t)(k0 + 4 * col + cb);
                bool ok = score[qb][cb] > tau[qb];
                if constexpr (DIAG) ok = ok && (int)key <= tq[qb];
                my[64 * cl[qb]] = u32x2{__float_as_uint(score[qb][cb]), key};
                cl[qb] += ok ? 1 : 0;
            }
            // a lane can stage 4 more next tile
            flushq |= __ballot(cl[qb] > kLane - 4) ? (1ull << qb) : 0ull;
        }
        if (!flushq) return;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            if ((flushq >> qb) & 1ull) flush_quad(qb);
    };

    Frag<T> bf[4][C::KD];
    // tiles below kd hold only keys < qw0 <= every query of the wave
    const int kd = qw0 / kKT;
    // Prefetches are never skipped: a tile past the end is fetched through an
    // empty descriptor (all zeros, no memory access).  A skipped load on one
    // path would make the wait counts of the merged paths wait for the
    // prefetched tiles as well.
    const int knull = (nk + kKT - 1) / kKT;
    auto tile_or_null = [&](int kt, int lim) { return kt < lim ? kt : knull; };

    // ---- starting threshold from a key sample ---------------------------------
    // With tau starting at -inf a late query would stage every key.  Instead,
    // ns tiles spread over the keys below qw0 are scored first; each lane keeps
    // its four best sample scores per query, and tau starts at (about) the
    // R-th largest of a query's 64 kept values, R chosen so that about
    // kSlack*M of the query's t+1 keys are expected above it (tau1, for a
    // second attempt, about twice as many).  This is only a starting point:
    // the scan accepts what beats it, and a query left with fewer than
    // min(M, t+1) candidates is scanned again from a lower threshold.
    constexpr float kSlack = 2.0f;
    constexpr int kRank = 32;
    float tau1[QB];
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
        auto sample_tile = [&](const Acc &acc) {
            float score[QB][4];
            tile_epilogue(acc, score);
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
        load_b(ks(0), bf);
        for (int i = 0; i < ns; ++i) {
            Acc acc;
            tile_mfma(bf, acc);
            load_b(i + 1 < ns ? ks(i + 1) : knull, bf);
            sample_tile(acc);
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
            auto rank_value = [&](float Rk) {
                float lo = row_min(top[qb][3]), hi = row_max(top[qb][0]);
                if (count_ge(hi) >= Rk) lo = hi;
#pragma unroll 1
                for (int it = 0; it < 12; ++it) {
                    const float mid = 0.5f * (lo + hi);
                    const bool up = count_ge(mid) >= Rk;
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

    // ---- scan: every tile; tile kt+1 loads while the epilogue of kt runs.
    // A query left with fewer than min(M, t+1) candidates
    // had its threshold at or above its M-th score: it is scanned again from
    // the lower sample estimate tau1, and if that starves it too, from -inf;
    // the wave's other queries take nothing in those passes. --------------------
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        load_b(0, bf);
#pragma unroll 1
        for (int kt = 0; kt < ntiles; ++kt) {
            Acc acc;
            tile_mfma(bf, acc);
            load_b(tile_or_null(kt + 1, ntiles), bf);
            if (kt >= kd) tile_step(kt, acc, std::true_type{});
            else tile_step(kt, acc, std::false_type{});
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) flush_quad(qb);
        if (ns == 0) break;  // started from -inf: already exact
        uint64_t redo = 0;
        bool fail[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            fail[qb] = tq[qb] < nk && gc[qb] < min(M, tq[qb] + 1);
            redo |= __ballot(fail[qb]);
        }
        if (!redo || pass == 2) break;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            // kept queries take nothing more (their counts stay below a trim)
            tau[qb] = fail[qb] ? (pass == 0 ? tau1[qb] : -INFINITY) : INFINITY;
            gc[qb] = fail[qb] ? 0 : gc[qb];
        }
    }

    // ---- final select and ordered write-out --------------------------------------
    // For each query: keep the first min(M, t+1) of its c buffered candidates
    // (any order, distinct indices) in the order (higher score, lower index),
    // mark them in a bitmap over positions 0..t (the staging area, free now),
    // give every bitmap word the number of kept positions below it, and store
    // each kept index at its rank, -1 padded.  The wave takes its queries in
    // turn; the chip's other waves keep scanning meanwhile.
    wave_global_sync();
    // per bitmap word: {bits, kept positions in the lower words}; lane l owns
    // words [l * per, (l + 1) * per), per even and at most 16
    uint32_t *const bw = reinterpret_cast<uint32_t *>(lists);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll 1
        for (int gg = 0; gg < 4; ++gg) {
            const int t = qw0 + qb * 4 + gg;
            if (t >= nk) continue;
            int c = __builtin_amdgcn_readlane(gc[qb], 16 * gg);
            const int m = min(M, t + 1);
            u32x2 *const gb = qbuf_of(qb * 4 + gg);
            // the select holds C::NF entries per lane; a larger buffer (a
            // query started from -inf, or a loose threshold) is trimmed first
            if (c > C::NF * 64) c = trim_buffer(gb, c, m, C::NF * 64, hist).c;
            uint32_t ok[C::NF], xi[C::NF];  // order key of the score, index
#pragma unroll
            for (int k = 0; k < C::NF; ++k) {
                const int e = k * 64 + lane;
                u32x2 v = u32x2{0u, 0u};
                if (e < c) v = gb[e];
                ok[k] = order_key(__uint_as_float(v[0]));
                xi[k] = v[1];
            }
            auto valid = [&](int k) { return k * 64 + lane < c; };
            uint64_t theta = 0;  // every valid candidate is kept when c <= m
            if (c > m)
                theta = select_theta(
                    [&](auto &&f) {
#pragma unroll
                        for (int k = 0; k < C::NF; ++k) f(valid(k), ok[k], xi[k]);
                    },
                    m, hist);
            uint32_t kept_mask = 0u;
#pragma unroll
            for (int k = 0; k < C::NF; ++k)
                if (valid(k) && ((((uint64_t)ok[k]) << 32) | (uint64_t)~xi[k]) >= theta) kept_mask |= 1u << k;
            const int per = (((t / 32 + 1) + 63) / 64 + 1) & ~1;
            uint32_t *const mine = bw + 2 * lane * per;
#pragma unroll
            for (int j = 0; j < 16; j += 2)
                if (j < per) *reinterpret_cast<u32x4 *>(mine + 2 * j) = u32x4{0u, 0u, 0u, 0u};
            wave_lds_sync();
#pragma unroll
            for (int k = 0; k < C::NF; ++k)
                if ((kept_mask >> k) & 1u) atomicOr(&bw[2 * (xi[k] >> 5)], 1u << (xi[k] & 31));
            wave_lds_sync();
            uint32_t own = 0u;
#pragma unroll
            for (int j = 0; j < 16; j += 2)
                if (j < per) {
                    const u32x4 w2 = *reinterpret_cast<const u32x4 *>(mine + 2 * j);
                    own += (uint32_t)(__popc(w2[0]) + __popc(w2[2]));
                }
            const uint32_t incl = wave_inclusive_scan(own);
            const int kept = __builtin_amdgcn_readlane((int)incl, 63);
            uint32_t run = incl - own;
#pragma unroll
            for (int j = 0; j < 16; j += 2)
                if (j < per) {
                    u32x4 w2 = *reinterpret_cast<const u32x4 *>(mine + 2 * j);
                    w2[1] = run;
                    run += (uint32_t)__popc(w2[0]);
                    w2[3] = run;
                    run += (uint32_t)__popc(w2[2]);
                    *reinterpret_cast<u32x4 *>(mine + 2 * j) = w2;
                }
            wave_lds_sync();
            int32_t *dst = a.idx + (((size_t)b * nq + t - p0) * G + g) * M;
#pragma unroll
            for (int k = 0; k < C::NF; ++k)
                if ((kept_mask >> k) & 1u) {
                    const u32x2 e = *reinterpret_cast<const u32x2 *>(bw + 2 * (xi[k] >> 5));
                    dst[e[1] + (uint32_t)__popc(e[0] & ((1u << (xi[k] & 31)) - 1u))] = (int32_t)xi[k];
                }
            for (int i = kept + lane; i < M; i += 64) dst[i] = -1;
            wave_lds_sync();  // the bitmap is read before the next query clears it
        }
    }
}

// Candidate-buffer entries per query, 4 M' + 256 for M up to M' (a query is
// trimmed when it holds more than CAPG - 128, room for one more flush): a
// query below 4 M starts from -inf and stages every key, so it never trims;
// a later one starts from a sampled threshold expected to admit about 2 M.
int cand_entries(int M) { return M <= 64 ? 512 : M <= 128 ? 768 : M <= 256 ? 1280 : 2304; }

template <typename T, int DI, int HH, int QB>
hipError_t launch_q(const IndexerArgs &a, hipStream_t s) {
    constexpr int QW = 4 * QB;
    const int nqb = (a.n + QW - 1) / QW;
    const dim3 grid((unsigned)(a.B * a.G * nqb));
    switch (cand_entries(a.M)) {
        case 512: launch_kernel((indexer_topm_kernel<T, DI, HH, QB, 512>), grid, dim3(64), 0, s, a); break;
        case 768: launch_kernel((indexer_topm_kernel<T, DI, HH, QB, 768>), grid, dim3(64), 0, s, a); break;
        case 1280: launch_kernel((indexer_topm_kernel<T, DI, HH, QB, 1280>), grid, dim3(64), 0, s, a); break;
        default: launch_kernel((indexer_topm_kernel<T, DI, HH, QB, 2304>), grid, dim3(64), 0, s, a); break;
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
