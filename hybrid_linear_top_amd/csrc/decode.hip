// Decode-step kernels of the LISA layer on gfx950.
//
// (1) decode_score_state: one launch with two kinds of work-groups.
//   * score groups stream the packed indexer-key cache k_idx and write, for
//     the new token t = L_b - 1 of every sequence, the Lightning Indexer score
//     I(s) = sum_j w_j * max(0, q_idx_j . k_idx_s) of every visible token s
//     (the indexer scans the full context with a ReLU'd dot product: arxivdaily
//     page for arXiv 2607.19358, English abstract; gptget.net analysis,
//     method-details section).  This stream is the largest HBM consumer of a
//     decode step; the dot products run on MFMA in the prefill indexer's
//     layout, so the per-token work is a few VALU operations and the groups
//     stay bound by memory.
//   * state groups do the linear-attention step of one query head:
//     S_t = S_{t-1} + k_t v_t^T in place and o_lin = q_t^T S_t (identity
//     feature map and state matrix S_t, O(1) per token: gptget.net,
//     method-details section), one read-modify-write pass over the fp32 state.
//   Both halves are HBM streams of similar size per group, so they share a
//   grid and fill the chip together.
// (2) decode_select: per (sequence, group) radix select of the top-M scores
//   (M = 256 in the paper's runs: gptget.net, experiment-design section)
//   with the lower index winning ties; the set is written in ascending order.
#include "common.hpp"
#include "kernels.hpp"

namespace lisa {

namespace {

// Scores of one 128-token tile of one sequence, all groups.  A wave task is
// 64 tokens of one group: four 16x16x32 MFMA blocks per K step with the
// query's indexer heads as the A rows (rows past H_I are zero) and 16 tokens
// as the B columns, exactly as the prefill indexer lays out a query and its
// keys; lane (0, col) then holds the heads' dot products for token col and
// forms the score with the same ReLU'd, weighted sum in the same order.
// The key rows are read whole -- each load instruction covers complete
// 128-byte lines, which streams HBM about 1.5x faster than the fragment
// layout's half lines -- and pass through the wave's LDS slice (XOR-swizzled
// 16-byte pieces, conflict-free both ways) on their way to the B fragments.
template <typename T, int DI, int HIPAD>
__device__ void score_group(const DecodeScoreArgs &a, int sb, u32x4 *stage) {
    constexpr int KD = DI / 32;
    constexpr int TPW = 64;                  // tokens per wave task
    constexpr uint32_t EB = Elt<T>::kBytes;
    constexpr int PPR = DI * (int)EB / 16;   // 16-byte pieces per key row (4, 8 or 16)
    constexpr int RPI = 64 / PPR;            // key rows per load instruction
    constexpr int NLD = TPW / RPI;           // load instructions per task
    constexpr int SWS = PPR == 4 ? 2 : PPR == 8 ? 1 : 0;  // swizzle: piece ^ ((row >> SWS) & (PPR - 1))
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int b = sb / a.tiles_per_seq, tile = sb % a.tiles_per_seq;
    const bool paged = a.map.table != nullptr;
    const int64_t row0 = paged ? 0 : a.cu[b];
    const int L = cache_len(a.map, b, a.max_ctx);
    const int tok0 = tile * kDecodeTile;
    if (tok0 >= L) return;
    const int tok_end = min(tok0 + kDecodeTile, L);
    const int G = a.G, HI = a.HI;
    const int ntask = G * (kDecodeTile / TPW);
    // Every load below is unconditional, through a buffer descriptor that
    // turns the lanes with nothing to read into zeros: a load under a branch
    // would make the compiler wait for all loads in flight.
    const uint32_t row_bytes = (uint32_t)G * DI * EB;
    const rsrc_t krs = make_rsrc(reinterpret_cast<const T *>(a.k_idx_cache) + (size_t)row0 * G * DI,
                                 (uint32_t)(paged ? a.pool_rows : L) * row_bytes);
    // the page-table row (empty for packed caches: those lookups read zeros)
    const rsrc_t trs = make_rsrc(paged ? (const void *)(a.map.table + (size_t)b * a.map.max_blocks) : (const void *)a.cu,
                                 paged ? (uint32_t)a.map.max_blocks * 4u : 0u);
    const int lb = a.map.log2_block;
    float *out_b = a.scores + (size_t)b * G * a.max_ctx;
    u32x4 *slice = stage + wave * TPW * PPR;  // this wave's 64 rows
    const int lrow = lane / PPR, lpc = lane % PPR;  // row and piece this lane loads

    for (int task = wave; task < ntask; task += 4) {
        const int g = task % G, tb = tok0 + (task / G) * TPW;
        const size_t qrow = ((size_t)b * G + g) * HI;
        // query heads and weights (rows past H_I read as zeros), page lookups
        const rsrc_t qrs = make_rsrc(reinterpret_cast<const T *>(a.q_idx) + qrow * DI, (uint32_t)HI * DI * EB);
        const rsrc_t wrs = make_rsrc(reinterpret_cast<const T *>(a.w_idx) + qrow, (uint32_t)HI * EB);
        Frag<T> af[KD];
#pragma unroll
        for (int kc = 0; kc < KD; ++kc) frag_buf_load(af[kc], qrs, (uint32_t)(col * DI + kc * 32 + grp * 8) * EB);
        float wv[HIPAD];
#pragma unroll
        for (int j = 0; j < HIPAD; ++j) {
            if constexpr (EB == 2)
                wv[j] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(wrs, (uint32_t)j * 2u, 0u, 0) << 16);
            else
                wv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wrs, (uint32_t)j * 4u, 0u, 0));
        }
        int32_t blk[NLD];
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int tok = min(tb + j * RPI + lrow, L - 1);
            blk[j] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(trs, (uint32_t)(tok >> lb) * 4u, 0u, 0);
        }
        // whole key rows: instruction j reads rows j*RPI .. j*RPI + RPI - 1
        u32x4 raw[NLD];
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int tok = tb + j * RPI + lrow;
            const uint32_t rrow = paged ? ((uint32_t)blk[j] << lb) + (uint32_t)(tok & ((1 << lb) - 1)) : (uint32_t)tok;
            const uint32_t off = tok < tok_end ? rrow * row_bytes + (uint32_t)g * DI * EB + (uint32_t)lpc * 16u : kOffNone;
            raw[j] = buf_load16(krs, off);
        }
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int r = j * RPI + lrow;
            slice[r * PPR + (lpc ^ ((r >> SWS) & (PPR - 1)))] = raw[j];
        }
        wave_lds_sync();
        float *out = out_b + (size_t)g * a.max_ctx;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int r = 16 * cb + col;
            const int sw = (r >> SWS) & (PPR - 1);
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kc = 0; kc < KD; ++kc) {
                Frag<T> bfr;
                if constexpr (EB == 2) {
                    bfr.v = slice[r * PPR + ((kc * 4 + grp) ^ sw)];
                } else {
                    bfr.lo = __builtin_bit_cast(f32x4, slice[r * PPR + ((kc * 8 + 2 * grp) ^ sw)]);
                    bfr.hi = __builtin_bit_cast(f32x4, slice[r * PPR + ((kc * 8 + 2 * grp + 1) ^ sw)]);
                }
                acc = mma16(af[kc], bfr, acc);
            }
            float sc = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) sc = fmaf(wv[i], fmaxf(acc[i], 0.0f), sc);
            if constexpr (HIPAD > 4) {
                // heads 4..7 sit in the rows of lane col + 16: continue the same chain
#pragma unroll
                for (int i = 0; i < 4; ++i) sc = fmaf(wv[4 + i], fmaxf(__shfl_down(acc[i], 16), 0.0f), sc);
            }
            const int tok = tb + r;
            if (grp == 0 && tok < tok_end) out[tok] = sc;
        }
        wave_lds_sync();  // the slice is rewritten by the next task
    }
}

// Linear-attention step of one query head, one column slice of its state:
// state group uu is (sequence b, head h, slice part), the slice being value
// columns [part*D/CS, (part+1)*D/CS) of S (all D rows), so o_lin's columns
// of the slice are complete within the group.  It runs on 256 threads (tid
// 0..255), which may be a quarter of a larger work-group: sync() is a
// barrier every thread of the work-group reaches the same number of times,
// so an inactive group (active false: past the last) still takes part.  The
// state loads are issued before anything else, as they wait for nothing.
template <typename T, int D, typename Sync>
__device__ void state_group(const DecodeScoreArgs &a, int uu, float *smem, int tid, bool active, Sync &&sync) {
    constexpr int CS = D / 32;        // column slices per head
    constexpr int NQ = D / 4;         // float4 columns of a state row
    constexpr int NQP = NQ / CS;      // float4 columns of the slice
    constexpr int RG = 256 / NQP;     // row groups
    constexpr int RPT = D / RG;       // rows per thread
    const int part = uu % CS, u = uu / CS;
    const int Hq = a.Hq, b = active ? u / Hq : 0, h = u % Hq;
    const int g = (int)(((int64_t)h * a.G) / Hq);
    const int jq = part * NQP + tid % NQP, rg = tid / NQP;
    f32x4 *S = reinterpret_cast<f32x4 *>(a.state + ((size_t)b * Hq + h) * D * D);
    f32x4 sv[RPT];
    if (active) {
#pragma unroll
        for (int s = 0; s < RPT; ++s) sv[s] = __builtin_nontemporal_load(&S[(rg + RG * s) * NQ + jq]);
    }
    const int64_t row0 = a.map.table ? 0 : a.cu[b];
    const int32_t *ptab = a.map.table ? a.map.table + (size_t)b * a.map.max_blocks : nullptr;
    const int L = active ? cache_len(a.map, b, a.max_ctx) : 0;
    float *olin = a.olin + ((size_t)b * Hq + h) * D + part * NQP * 4;
    const bool work = active && L >= 1;
    if (active && !work && tid < NQP * 4) olin[tid] = 0.0f;
    float *kk = smem, *vv = smem + D, *qq = smem + 2 * D, *red = smem + 3 * D;
    if (work && tid < D) {
        const int64_t trow = cache_row(a.map, row0, ptab, L - 1);
        const T *kc = reinterpret_cast<const T *>(a.k_cache);
        const T *vc = reinterpret_cast<const T *>(a.v_cache);
        const T *qp = reinterpret_cast<const T *>(a.q);
        kk[tid] = Elt<T>::to_f32(kc[((size_t)trow * a.G + g) * D + tid]);
        vv[tid] = Elt<T>::to_f32(vc[((size_t)trow * a.G + g) * D + tid]);
        qq[tid] = Elt<T>::to_f32(qp[((size_t)b * Hq + h) * D + tid]);
    }
    sync();
    if (work) {
        const f32x4 v4 = *reinterpret_cast<const f32x4 *>(vv + 4 * jq);
        f32x4 o = {0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < RPT; ++s) {
            const int i = rg + RG * s;
            const float ki = kk[i], qi = qq[i];
            f32x4 x = sv[s];
            x[0] = fmaf(ki, v4[0], x[0]);
            x[1] = fmaf(ki, v4[1], x[1]);
            x[2] = fmaf(ki, v4[2], x[2]);
            x[3] = fmaf(ki, v4[3], x[3]);
            __builtin_nontemporal_store(x, &S[i * NQ + jq]);
            o[0] = fmaf(qi, x[0], o[0]);
            o[1] = fmaf(qi, x[1], o[1]);
            o[2] = fmaf(qi, x[2], o[2]);
            o[3] = fmaf(qi, x[3], o[3]);
        }
        *reinterpret_cast<f32x4 *>(red + rg * (NQP * 4) + 4 * (tid % NQP)) = o;
    }
    sync();
    if (work && tid < NQP * 4) {
        float acc = 0.0f;
        for (int r = 0; r < RG; ++r) acc += red[r * (NQP * 4) + tid];
        olin[tid] = acc;
    }
}
constexpr int kStateFloats = 3 * 128 + 1024;  // a state group's LDS (D <= 128)

// the state groups of a launch of 1024-thread work-groups: four per group
// state groups first + 4 wg + sub (sub = 0..3) of a launch of 1024-thread
// work-groups, up to n_state
template <typename T, int D>
__device__ void state_quads(const DecodeScoreArgs &a, int first, int wg, int n_state, float *smem) {
    const int sub = threadIdx.x >> 8, uu = first + 4 * wg + sub;
    state_group<T, D>(a, uu, smem + sub * kStateFloats, threadIdx.x & 255, uu < n_state, [] { __syncthreads(); });
}
__device__ __forceinline__ void state_quads_any(const DecodeScoreArgs &a, int dtype, int d, int first, int wg,
                                                int n_state, float *smem) {
    if (dtype == 1) {
        if (d == 128) state_quads<uint16_t, 128>(a, first, wg, n_state, smem);
        else state_quads<uint16_t, 64>(a, first, wg, n_state, smem);
    } else {
        if (d == 128) state_quads<float, 128>(a, first, wg, n_state, smem);
        else state_quads<float, 64>(a, first, wg, n_state, smem);
    }
}

template <typename T, int D, int DI, int HIPAD>
__global__ __launch_bounds__(256) void decode_score_state_kernel(DecodeScoreArgs a, int n_state) {
    // state groups: 3 vectors + the reduction rows; score groups: 64 key rows per wave
    constexpr int kStateBytes = kStateFloats * 4;
    constexpr int kStageBytes = 4 * 64 * DI * (int)Elt<T>::kBytes;
    __shared__ u32x4 smem[(kStateBytes > kStageBytes ? kStateBytes : kStageBytes) / 16];
    if ((int)blockIdx.x < n_state)
        state_group<T, D>(a, blockIdx.x, reinterpret_cast<float *>(smem), threadIdx.x, true, [] { __syncthreads(); });
    else
        score_group<T, DI, HIPAD>(a, blockIdx.x - n_state, smem);
}

// ---------------------------------------------------------------------------
// One wave: the m-th largest of c 32-bit keys kr[e] (element e*64 + lane),
// all of them in [lo, lo + 2^width), by radix passes of up to 8 bits over
// key - lo from bit width - 1 down, with a 256-bin LDS histogram.  theta is
// that key; take_eq is how many keys equal to theta belong to the top m (the
// earliest elements, as ties go to the lower position).  Passing the live
// range skips the high bits every key shares (and the pile-up of all keys in
// one bin that those passes cause).
template <int NE>
__device__ void wave_kth_u32(const uint32_t (&kr)[NE], int c, uint32_t m, uint32_t *hist, uint32_t lo,
                             int width, uint32_t &theta, uint32_t &take_eq) {
    const int lane = threadIdx.x & 63;
    uint32_t prefix = 0u, need = m;  // prefix: the bits of key - lo above `top`
#pragma unroll 1
    for (int top = width; top > 0; top -= 8) {
        const int sh = top > 8 ? top - 8 : 0;
        const uint32_t digit_mask = (1u << (top - sh)) - 1u;
        *reinterpret_cast<u32x4 *>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < NE; ++k) {
            const uint32_t x = kr[k] - lo;
            const bool live = k * 64 + lane < c && (top >= 32 || (x >> top) == prefix);
            if (live) atomicAdd(&hist[(x >> sh) & digit_mask], 1u);
        }
        wave_lds_sync();
        const u32x4 h = *reinterpret_cast<const u32x4 *>(hist + 4 * lane);
        const uint32_t lsum = h[0] + h[1] + h[2] + h[3];
        const uint32_t incl = wave_inclusive_scan(lsum);
        const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        uint32_t run = total - incl;  // keys in the bins of higher lanes
        int fb = -1;
        uint32_t fneed = 0;
#pragma unroll
        for (int bb = 3; bb >= 0; --bb) {
            if (fb < 0 && run < need && run + h[bb] >= need) {
                fb = 4 * lane + bb;
                fneed = need - run;
            }
            run += h[bb];
        }
        const int src = __ffsll((unsigned long long)__ballot(fb >= 0)) - 1;
        fb = __builtin_amdgcn_readlane(fb, src);
        fneed = (uint32_t)__builtin_amdgcn_readlane((int)fneed, src);
        prefix = (prefix << (top - sh)) | (uint32_t)fb;
        need = fneed;
        wave_lds_sync();
    }
    theta = lo + prefix;
    take_eq = need;
}

// ---------------------------------------------------------------------------
// Top-M select of one (sequence, group) with few block barriers: NT threads,
// the keys in registers, thread t holding positions k*NT + t (k < EPT), so
// every load instruction reads consecutive scores and (k, thread) order is
// position order.
//  0. a shortcut first, when 2M <= CAP (described at the code);
//  1. key range by wave reductions (one barrier);
//  2. 2048-bin histogram passes over the live key range (bins are
//     (key - lo) >> shift), the bin holding the M-th largest key found by
//     wave 0 alone (32 bins a lane, one wave scan) -- three barriers a pass;
//     passes stop as soon as that bin is taken whole or holds at most 64 keys;
//  3. those boundary keys (key, position) are appended to LDS and wave 0
//     ranks them exactly (higher key, then lower position) and marks the
//     `need` best in an LDS bitmap of positions, while every thread marks its
//     keys above the boundary bin; when the boundary bin is a single key value
//     (ties, any number of them) its keys go to a second bitmap instead and
//     the lowest `need` positions of it are taken;
//  4. wave 0 walks the bitmaps in position order (contiguous words per lane,
//     one wave scan of their counts) and writes the set ascending.
// A launch with gridDim.y = 2 selects within one of two position ranges of
// part_len positions (part blockIdx.y covers [part_len * part,
// part_len * (part + 1))),
// writing the part's set (positions, ascending) to row 2 bg + part of idx;
// decode_merge_kernel then merges the two.
// Work-groups past the first nbg of the launch (in part 0) do state groups
// state_first .. n_state - 1 of the linear-attention step instead, four each
// (state_quads): that step does not need the scores, so it runs beside the
// selects, off the scan's critical path (16K decode, 1.5B shapes: 36.9 ->
// 34.2 us per step; ragged 7B batch: 103 -> 98 us, where the state stream
// is longer than the selects).
template <int NT, int EPT, int CAP>
__global__ __launch_bounds__(NT) void decode_topm_kernel(const float *scores, CacheMap map,
                                                         int G, int M, int max_ctx, int part_len, int32_t *idx,
                                                         int nbg, DecodeScoreArgs sa, int state_first,
                                                         int n_state, int dtype, int d) {
    static_assert(NT == 1024, "state groups run four to a work-group");
    __shared__ __attribute__((aligned(16))) float st_smem[4 * kStateFloats];
    if ((int)blockIdx.x >= nbg) {
        if (blockIdx.y == 0) state_quads_any(sa, dtype, d, state_first, (int)blockIdx.x - nbg, n_state, st_smem);
        return;
    }
    constexpr int NW = NT / 64;
    constexpr int NWORD = (NT * EPT + 31) / 32;  // bitmap words
    constexpr int WPL = (NWORD + 63) / 64;       // bitmap words per lane of wave 0
    __shared__ __attribute__((aligned(16))) uint32_t hist[2048];
    __shared__ uint32_t bitmap[NWORD];   // selected outright
    __shared__ uint32_t eqmap[NWORD];    // boundary keys that are all equal (ties)
    __shared__ uint32_t red[2 * NW + 2];
    __shared__ uint32_t cand_key[64], cand_pos[64];
    __shared__ uint32_t found[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bg = blockIdx.x, b = bg / G;
    const int p0 = part_len * (int)blockIdx.y;  // first position of this part
    const float *sc = scores + (size_t)bg * max_ctx + p0;
    // The score loads are issued first, before the sequence length is known:
    // the row holds max_ctx entries (the descriptor reads zeros past them)
    // and positions at or past L are masked below, so the loads need not
    // wait for the length lookup.  All of them are unconditional and in
    // flight together.  The launch guarantees NT * EPT >= part_len.
    auto pos_of = [&](int k) { return k * NT + tid; };
    const rsrc_t srs = make_rsrc(sc, (uint32_t)(max_ctx - p0) * 4u);
    uint32_t keyreg[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k)
        keyreg[k] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(srs, (uint32_t)pos_of(k) * 4u, 0u, 0);
    const int L = min(max(cache_len(map, b, max_ctx) - p0, 0), part_len);
    auto valid = [&](int k) { return pos_of(k) < L; };
    int32_t *out = idx + ((size_t)bg * gridDim.y + blockIdx.y) * M;
    if (L <= M) {
        for (int i = tid; i < M; i += NT) out[i] = i < L ? p0 + i : -1;
        return;
    }
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, tmax = 0u;
    bool active = false;  // this thread holds a key
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        keyreg[k] = order_key(__uint_as_float(keyreg[k]));
        if (valid(k)) {
            kmin = min(kmin, keyreg[k]);
            kmax = max(kmax, keyreg[k]);
            active = true;
        }
    }
    tmax = kmax;  // this thread's largest key

    // ---- shortcut: a threshold from the threads' maxima ----------------------
    // The M-th largest of the threads' maxima is at or below the M-th largest
    // key (the maxima are keys of distinct positions), so every key of the
    // top M lies at or above any T with at least M maxima >= T.  One
    // histogram pass over the maxima gives such a T (the lower edge of the
    // bin where the count from the top reaches M); the keys >= T -- about M
    // plus the threads holding two or more of the top M -- are packed in
    // position order (per (round k, wave) counts, one block scan over that
    // k-major grid, ballot ranks within a wave), and one wave selects their M
    // largest exactly (ties to the lower position).  When more than CAP keys
    // pass T the exact passes below run instead.
    static_assert(EPT * NW <= NT, "one scan entry per thread");
    __shared__ uint32_t fkey[CAP], fpos[CAP];
    __shared__ uint32_t scan_tmp[NW + 1];
    __shared__ uint32_t kbase[EPT * NW];
    const bool shortcut = 2 * M <= CAP;
    if (shortcut) {
        const uint32_t mlo = wave_min_u32(active ? tmax : 0xFFFFFFFFu);
        const uint32_t mhi = wave_max_u32(tmax);
        if (lane == 0) {
            red[wave] = mlo;
            red[NW + wave] = mhi;
        }
        for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
        __syncthreads();
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            lo = min(lo, red[w]);
            hi = max(hi, red[NW + w]);
        }
        const uint32_t span = hi >= lo ? hi - lo : 0u;
        const int width = span == 0 ? 0 : 32 - __builtin_clz(span);
        const int shift = width > 11 ? width - 11 : 0;
        if (active) atomicAdd(&hist[(tmax - lo) >> shift], 1u);
        __syncthreads();
        if (wave == 0) {
            // lane l owns bins 2016 - 32*l .. 2047 - 32*l, walked downwards
            const uint32_t *hl = hist + 2016 - 32 * lane;
            uint32_t hsum = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const u32x4 v = reinterpret_cast<const u32x4 *>(hl)[q];
                hsum += v[0] + v[1] + v[2] + v[3];
            }
            const uint32_t incl = wave_inclusive_scan(hsum);
            const uint32_t before = incl - hsum;
            if (before < (uint32_t)M && incl >= (uint32_t)M) {
                uint32_t run = before;
                int fe = 0;
                bool got = false;
#pragma unroll
                for (int q = 7; q >= 0; --q) {
                    const u32x4 v = reinterpret_cast<const u32x4 *>(hl)[q];
#pragma unroll
                    for (int e = 3; e >= 0; --e) {
                        const bool hit = !got && run + v[e] >= (uint32_t)M;
                        fe = hit ? 4 * q + e : fe;
                        got = got || hit;
                        run += v[e];
                    }
                }
                red[2 * NW] = lo + ((uint32_t)(2016 - 32 * lane + fe) << shift);
            }
            // fewer than M threads hold keys: no bin reaches M
            const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
            if (lane == 0) red[2 * NW + 1] = total >= (uint32_t)M ? 1u : 0u;
        }
        __syncthreads();
        const uint32_t T = red[2 * NW];
        const bool have_T = red[2 * NW + 1] != 0u;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const uint32_t c = (uint32_t)__popcll(__ballot(valid(k) && keyreg[k] >= T));
            if (lane == 0) kbase[k * NW + wave] = c;
        }
        __syncthreads();
        uint32_t C;
        const uint32_t mine = tid < EPT * NW ? kbase[tid] : 0u;
        const uint32_t ex = block_exclusive_scan<NT>(mine, scan_tmp, &C);
        if (tid < EPT * NW) kbase[tid] = ex;
        __syncthreads();
        if (have_T && C >= (uint32_t)M && C <= (uint32_t)CAP) {
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                const bool sel = valid(k) && keyreg[k] >= T;
                const uint64_t bm = __ballot(sel);
                if (sel) {
                    const uint32_t p = kbase[k * NW + wave] + mbcnt64(bm);
                    fkey[p] = keyreg[k];
                    fpos[p] = (uint32_t)pos_of(k);
                }
            }
            __syncthreads();
            if (wave != 0) return;
            constexpr int NE = CAP / 64;
            uint32_t kr[NE];
#pragma unroll
            for (int e = 0; e < NE; ++e) kr[e] = e * 64 + lane < (int)C ? fkey[e * 64 + lane] : 0u;
            uint32_t theta, take_eq;
            // every packed key lies in [T, hi]
            const uint32_t span_c = hi - T;
            wave_kth_u32<NE>(kr, (int)C, (uint32_t)M, hist, T, span_c == 0 ? 0 : 32 - __builtin_clz(span_c),
                             theta, take_eq);
            uint32_t base = 0, eq_seen = 0;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const bool in = e * 64 + lane < (int)C;
                const bool gt = in && kr[e] > theta;
                const bool eq = in && kr[e] == theta;
                const uint64_t em = __ballot(eq);
                const uint32_t er = eq_seen + mbcnt64(em);
                eq_seen += (uint32_t)__popcll(em);
                const bool keep = gt || (eq && er < take_eq);
                const uint64_t km = __ballot(keep);
                const uint32_t pos = base + mbcnt64(km);
                base += (uint32_t)__popcll(km);
                if (keep && pos < (uint32_t)M) out[pos] = p0 + (int32_t)fpos[e * 64 + lane];
            }
            return;
        }
    }

    for (int w = tid; w < NWORD; w += NT) {
        bitmap[w] = 0u;
        eqmap[w] = 0u;
    }
    if (tid == 0) found[3] = 0u;  // boundary candidates appended
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    if (lane == 0) {
        red[wave] = kmin;
        red[NW + wave] = kmax;
    }
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        lo = min(lo, red[w]);
        hi = max(hi, red[NW + w]);
    }
    const uint32_t span = hi - lo;
    int width = span == 0 ? 0 : 32 - __builtin_clz(span);  // bits of key - lo
    uint32_t need = (uint32_t)M;
    uint64_t bin_hi;     // keys >= bin_hi are selected outright
    uint32_t bin_lo;     // keys in [bin_lo, bin_hi) are the boundary candidates
    uint32_t cnt_b = 0;  // how many there are
    bool tied = false;   // boundary bin is one key value
    for (;;) {
        const int shift = width > 11 ? width - 11 : 0;
        for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
        __syncthreads();
        const uint64_t hi_excl = (uint64_t)lo + ((uint64_t)1 << width);
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const uint32_t u = keyreg[k];
            if (valid(k) && u >= lo && (uint64_t)u < hi_excl) atomicAdd(&hist[(u - lo) >> shift], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l owns bins 2016 - 32*l .. 2047 - 32*l, walked downwards
            const uint32_t *hl = hist + 2016 - 32 * lane;
            uint32_t hsum = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const u32x4 v = reinterpret_cast<const u32x4 *>(hl)[q];
                hsum += v[0] + v[1] + v[2] + v[3];
            }
            const uint32_t before = wave_inclusive_scan(hsum) - hsum;
            if (before < need && before + hsum >= need) {
                uint32_t run = before, frem = 0, fcnt = 0;
                int fe = 0;
#pragma unroll
                for (int q = 7; q >= 0; --q) {
                    const u32x4 v = reinterpret_cast<const u32x4 *>(hl)[q];
#pragma unroll
                    for (int e = 3; e >= 0; --e) {
                        const bool hit = run < need && run + v[e] >= need;
                        fe = hit ? 4 * q + e : fe;
                        frem = hit ? need - run : frem;
                        fcnt = hit ? v[e] : fcnt;
                        run += v[e];
                    }
                }
                found[0] = 2016 - 32 * lane + fe;
                found[1] = frem;
                found[2] = fcnt;
            }
        }
        __syncthreads();
        const uint32_t bin = found[0], rem = found[1], cnt_bin = found[2];
        const uint32_t blo = lo + (bin << shift);
        if (rem == cnt_bin) {  // the whole bin is taken: keys >= blo are exactly the top M
            bin_hi = blo;
            bin_lo = blo;
            cnt_b = 0;
            break;
        }
        if (cnt_bin <= 64 || shift == 0) {
            bin_lo = blo;
            bin_hi = (uint64_t)blo + ((uint64_t)1 << shift);
            cnt_b = cnt_bin;
            need = rem;
            tied = shift == 0;
            break;
        }
        lo = blo;
        width = shift;
        need = rem;
        __syncthreads();  // found[] is rewritten by the next pass
    }
    // ---- mark the keys above the boundary bin; collect the boundary keys ----
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int s = pos_of(k);
        const uint32_t u = keyreg[k];
        if (valid(k) && (uint64_t)u >= bin_hi) atomicOr(&bitmap[s >> 5], 1u << (s & 31));
        if (cnt_b > 0 && valid(k) && u >= bin_lo && (uint64_t)u < bin_hi) {
            if (tied) {
                atomicOr(&eqmap[s >> 5], 1u << (s & 31));
            } else {
                const uint32_t slot = atomicAdd(&found[3], 1u);
                if (slot < 64u) {
                    cand_key[slot] = u;
                    cand_pos[slot] = (uint32_t)s;
                }
            }
        }
    }
    __syncthreads();
    if (wave != 0) return;
    if (cnt_b > 0 && !tied) {
        // exact rank among the boundary keys: higher key first, lower position on ties
        const uint32_t C = min(cnt_b, 64u);
        const bool mine = (uint32_t)lane < C;
        const uint32_t ku = mine ? cand_key[lane] : 0u, pu = mine ? cand_pos[lane] : 0xFFFFFFFFu;
        uint32_t rank = 0;
        for (uint32_t j = 0; j < C; ++j) {
            const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)ku, (int)j);
            const uint32_t pj = (uint32_t)__builtin_amdgcn_readlane((int)pu, (int)j);
            rank += (kj > ku || (kj == ku && pj < pu)) ? 1u : 0u;
        }
        if (mine && rank < need) atomicOr(&bitmap[pu >> 5], 1u << (pu & 31));
        wave_lds_sync();
    }
    // ---- ordered write-out: lane l walks bitmap words [WPL*l, WPL*l + WPL);
    // a position's slot is (selected before it) + min(tied before it, need) ----
    uint32_t gcnt = 0, ecnt = 0;
#pragma unroll
    for (int e = 0; e < WPL; ++e) {
        const int w = WPL * lane + e;
        gcnt += w < NWORD ? (uint32_t)__builtin_popcount(bitmap[w]) : 0u;
        ecnt += w < NWORD ? (uint32_t)__builtin_popcount(eqmap[w]) : 0u;
    }
    uint32_t gpos = wave_inclusive_scan(gcnt) - gcnt;
    uint32_t epos = wave_inclusive_scan(ecnt) - ecnt;
    const uint32_t take = tied ? need : 0u;
#pragma unroll
    for (int e = 0; e < WPL; ++e) {
        const int w = WPL * lane + e;
        const uint32_t gw = w < NWORD ? bitmap[w] : 0u, ew = w < NWORD ? eqmap[w] : 0u;
        uint32_t bits = gw | ew;
        while (bits) {
            const int bit = __builtin_ctz(bits);
            bits &= bits - 1u;
            const int s = 32 * w + bit;
            if ((gw >> bit) & 1u) {
                const uint32_t pos = gpos + min(epos, take);
                if (pos < (uint32_t)M) out[pos] = p0 + s;
                ++gpos;
            } else {
                if (epos < take) {
                    const uint32_t pos = gpos + epos;
                    if (pos < (uint32_t)M) out[pos] = p0 + s;
                }
                ++epos;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Merge of the two parts' sets of one (sequence, group): the 2M candidates
// (positions ascending within each part, the parts in order, -1 padded) are
// ranked by the 64-bit key (score order key, complemented position), the
// M-th largest found by eight 8-bit radix passes of a 256-bin histogram, and
// the kept ones written in candidate order, which is position order.
template <int NT, int E>
__global__ __launch_bounds__(NT) void decode_merge_kernel(const float *scores, const int32_t *cand, int M,
                                                          int max_ctx, int32_t *idx) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wtmp[NT / 64 + 1];
    __shared__ uint32_t found[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bg = blockIdx.x, C = 2 * M;
    const int32_t *cb = cand + (size_t)bg * C;
    const float *sc = scores + (size_t)bg * max_ctx;
    int32_t pos[E];
    uint64_t key[E];  // 0 for no candidate; a candidate's key is at least 2^32
    uint32_t own = 0;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int i = k * NT + tid;
        pos[k] = i < C ? cb[i] : -1;
    }
#pragma unroll
    for (int k = 0; k < E; ++k) {
        key[k] = pos[k] >= 0 ? ((uint64_t)order_key(sc[pos[k]]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos[k])
                             : 0ull;
        own += pos[k] >= 0 ? 1u : 0u;
    }
    uint32_t nval;
    block_exclusive_scan<NT>(own, wtmp, &nval);
    uint64_t theta = 1ull;  // every candidate is kept when there are at most M
    if (nval > (uint32_t)M) {
        uint64_t prefix = 0ull;  // the bits of theta above the current digit
        uint32_t need = (uint32_t)M;
#pragma unroll 1
        for (int sh = 56; sh >= 0; sh -= 8) {
            for (int i = tid; i < 256; i += NT) hist[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const bool live = key[k] != 0ull && (sh == 56 || (key[k] >> (sh + 8)) == (prefix >> (sh + 8)));
                if (live) atomicAdd(&hist[(key[k] >> sh) & 255u], 1u);
            }
            __syncthreads();
            if (wave == 0) {
                // lane l owns bins 4 l .. 4 l + 3; the count from the top reaches need in one of them
                const u32x4 h = *reinterpret_cast<const u32x4 *>(hist + 4 * lane);
                const uint32_t incl = wave_inclusive_scan(h[0] + h[1] + h[2] + h[3]);
                const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
                uint32_t run = total - incl;
#pragma unroll
                for (int bb = 3; bb >= 0; --bb) {
                    if (run < need && run + h[bb] >= need) {
                        found[0] = 4 * lane + bb;
                        found[1] = need - run;
                    }
                    run += h[bb];
                }
            }
            __syncthreads();
            prefix |= (uint64_t)found[0] << sh;
            need = found[1];
            __syncthreads();
        }
        theta = prefix;  // the M-th largest key: exactly M keys are >= it
    }
    int32_t *out = idx + (size_t)bg * M;
    uint32_t base = 0;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const bool kept = key[k] != 0ull && key[k] >= theta;
        uint32_t tot;
        const uint32_t at = block_exclusive_scan<NT>(kept ? 1u : 0u, wtmp, &tot);
        if (kept) out[base + at] = pos[k];
        base += tot;
    }
    for (int i = (int)base + tid; i < M; i += NT) out[i] = -1;
}

template <typename T, int D, int DI, int HIPAD>
hipError_t launch_ss(const DecodeScoreArgs &a, bool with_state, hipStream_t s) {
    // state groups: column slices of every head's state (else the select
    // launch runs them)
    const int n_state = with_state ? a.B * a.Hq * (D / 32) : 0;
    const int n_score = a.B * a.tiles_per_seq;
    launch_kernel((decode_score_state_kernel<T, D, DI, HIPAD>), dim3(n_state + n_score),
                       dim3(256), 0, s, a, n_state);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_ss(const DecodeScoreArgs &a, int d, int dI, bool with_state, hipStream_t s) {
    const bool h8 = a.HI > 4;
#define LISA_SS(D_, DI_)                                                                                \
    if (d == D_ && dI == DI_)                                                                            \
        return h8 ? launch_ss<T, D_, DI_, 8>(a, with_state, s) : launch_ss<T, D_, DI_, 4>(a, with_state, s);
    LISA_SS(64, 32) LISA_SS(64, 64) LISA_SS(128, 32) LISA_SS(128, 64)
#undef LISA_SS
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_score_state(const DecodeScoreArgs &a, int dtype, int d, int dI, bool with_state,
                                     hipStream_t s) {
    return dtype == 1 ? dispatch_ss<uint16_t>(a, d, dI, with_state, s) : dispatch_ss<float>(a, d, dI, with_state, s);
}

hipError_t launch_decode_select(const float *scores, const CacheMap &cu, int B, int G, int M,
                                int max_ctx, int32_t *idx, int32_t *cand, const DecodeScoreArgs *st, int dtype,
                                int d, hipStream_t s) {
    const dim3 grid(B * G);
    const int n_state = st ? B * st->Hq * (d / 32) : 0;
    const int first = 0;                // the select launch runs every state group
    const int nsw = (n_state + 3) / 4;  // state work-groups
    const DecodeScoreArgs sa = st ? *st : DecodeScoreArgs{};
    const dim3 sgrid((unsigned)(B * G + nsw));
    // above 33,792 positions: two parts of 32,768 (keys in registers), then a merge
    if (max_ctx > 33 * 1024) {
        if (!cand || max_ctx > 2 * 32768 || M > 2048) return hipErrorInvalidValue;
        launch_kernel((decode_topm_kernel<1024, 32, 1024>), dim3(B * G + nsw, 2), dim3(1024), 0, s, scores, cu, G,
                      M, max_ctx, 32768, cand, B * G, sa, first, n_state, dtype, d);
        launch_kernel((decode_merge_kernel<1024, 4>), grid, dim3(1024), 0, s, scores, (const int32_t *)cand, M,
                      max_ctx, idx);
        return hipGetLastError();
    }
#define LISA_TOPM(NT_, E, CAP_)                                                                    \
    if (max_ctx <= (E) * (NT_)) {                                                                  \
        launch_kernel((decode_topm_kernel<NT_, E, CAP_>), sgrid, dim3(NT_), 0, s, scores, cu, G, \
                      M, max_ctx, max_ctx, idx, B * G, sa, first, n_state, dtype, d);              \
        return hipGetLastError();                                                                  \
    }
    // keys per thread stay in registers: 1024 threads (128 VGPRs) up to 33,792
    // positions (longer contexts take the two-part path above)
    LISA_TOPM(1024, 8, 1024) LISA_TOPM(1024, 17, 1024) LISA_TOPM(1024, 33, 1024)
#undef LISA_TOPM
    return hipErrorInvalidValue;  // longer contexts are rejected by the API layer
}

}  // namespace lisa
