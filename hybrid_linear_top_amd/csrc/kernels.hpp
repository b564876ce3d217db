// Launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lisa {

// ---- kernel launches ----------------------------------------------------------
// Stage timing (lisa_stage_timing) attaches its events to the dispatches
// themselves: while a stage is timed on this thread, the stage's first launch
// carries the start event and every launch the stop event
// (hipExtLaunchKernelGGL), so the pair brackets the kernels' own execution,
// from the first one's start to the last one's end, not two marker packets
// around them.  Otherwise launches are plain.
struct DispatchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
    int launches = 0;
};
DispatchEvents &dispatch_events();  // this thread's (defined with the entry points)

template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                          Args... args) {
    DispatchEvents &de = dispatch_events();
    if (de.stop) {
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, de.launches == 0 ? de.start : nullptr, de.stop, 0u,
                              static_cast<KArgs>(args)...);
        ++de.launches;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shmem, s, static_cast<KArgs>(args)...);
    }
}

// ---- decode ---------------------------------------------------------------
// Where position s of sequence b lives in a decode cache.  Packed caches
// (table == nullptr): row cu[b] + s, with L_b = cu[b+1] - cu[b].  Paged
// caches: row table[b][s >> log2_block] * block + (s & (block - 1)) of the
// page pool, with L_b = lengths[b].
struct CacheMap {
    const int64_t *cu;
    const int32_t *table;    // [B, max_blocks] page ids, or nullptr
    const int32_t *lengths;  // [B] (paged only)
    int log2_block, max_blocks;
};
__device__ __forceinline__ int cache_len(const CacheMap &m, int b, int max_ctx) {
    const int64_t L = m.table ? (int64_t)m.lengths[b] : m.cu[b + 1] - m.cu[b];
    return (int)(L < 0 ? 0 : (L > max_ctx ? max_ctx : L));
}
// row of position s given the sequence's first packed row (row0, packed) or
// its page-table row (tb, paged)
__device__ __forceinline__ int64_t cache_row(const CacheMap &m, int64_t row0, const int32_t *tb, int s) {
    if (!m.table) return row0 + s;
    return ((int64_t)tb[s >> m.log2_block] << m.log2_block) + (s & ((1 << m.log2_block) - 1));
}

struct DecodeScoreArgs {
    const void *q;            // [B,Hq,d]
    const void *k_cache;      // [sumL,G,d]
    const void *v_cache;      // [sumL,G,d]
    const void *q_idx;        // [B,G,HI,dI]
    const void *k_idx_cache;  // [sumL,G,dI]
    const void *w_idx;        // [B,G,HI]
    const int64_t *cu;        // [B+1] device
    CacheMap map;
    int64_t pool_rows;        // paged caches: rows in the page pool
    float *state;             // [B,Hq,d,d] in/out
    float *olin;              // [B,Hq,d] workspace
    float *scores;            // [B,G,max_ctx] workspace
    int B, Hq, G, HI, max_ctx;
    int tiles_per_seq;        // ceil(max_ctx / kDecodeTile)
};
constexpr int kDecodeTile = 128;  // tokens per score work-group

// with_state: the score launch runs the linear-attention state step (no
// select launch follows); else the select launch runs it, beside the selects
hipError_t launch_decode_score_state(const DecodeScoreArgs &a, int dtype, int d, int dI, bool with_state,
                                     hipStream_t s);
// cand: workspace of B * G * 2 * M int32 (decode_cand_bytes), used above
// 33,792 positions (two parts, then a merge); may be null below.  st: when
// not null, the launch also runs the state step of st (dtype, head dim d).
hipError_t launch_decode_select(const float *scores, const CacheMap &map, int B, int G, int M,
                                int max_ctx, int32_t *idx, int32_t *cand, const DecodeScoreArgs *st, int dtype,
                                int d, hipStream_t s);
inline size_t decode_cand_bytes(int B, int G, int M, int max_ctx) {
    return max_ctx > 33 * 1024 ? (size_t)B * G * 2 * M * 4 : 0;
}

// ---- sparse attention + gate (prefill and decode) -------------------------
struct SparseArgs {
    const void *q;        // prefill [B,n,Hq,d]; decode [B,Hq,d]
    const void *k;        // prefill [B,past+n,G,d];  decode cache [sumL,G,d]
    const void *v;
    const int64_t *cu;    // decode only
    CacheMap map;         // decode only
    int64_t pool_rows;    // paged decode: rows in the page pool (bounds the gathers)
    const int32_t *idx;   // [units, M]  (units = B*n*G or B*G)
    const void *lin;      // o_lin: prefill = out buffer (dtype); decode = fp32 workspace
    const void *gate;     // prefill [B,n,Hq]; decode [B,Hq]
    void *out;            // prefill [B,n,Hq,d]; decode [B,Hq,d]
    int B, n, Hq, G, r, M, max_ctx;
    int past;             // prefill: query t (0-based among the n) sits at position past + t
    int window;           // 1: the set of a query at position t is max(0, t-M+1)..t (idx unused)
    float scale_log2;     // softmax scale * log2(e)
    int units;
    int split_lo;         // set by the launch (bf16 prefill)
};
hipError_t launch_sparse_gate(const SparseArgs &a, int dtype, int d, bool decode, hipStream_t s);

// ---- prefill: chunked linear attention -----------------------------------
struct LinearArgs {
    const void *q, *k, *v;       // [B,n,Hq,d]; k, v [B,kv_rows,G,d], rows kv_off.. are the n tokens
    const float *state_in;       // [B,Hq,d,d] or null
    float *state_out;            // [B,Hq,d,d] or null
    float *dS;                   // [B,G,nC,d,d] fp32: per-chunk K^T V, stored transposed [j][i]
    void *P;                     // [B,Hp,nC,d,d] dtype: exclusive prefix states, transposed
    void *out;                   // [B,n,Hq,d]: receives o_lin
    int B, n, Hq, G, r, nC;
    int kv_rows, kv_off;
    int per_head;                // 1 if state_in != null (prefix states per query head)
    int state_t;                 // chunk output only: P holds the prefixes untransposed
                                 // (those of the transposed recurrence), read transposed
};
hipError_t launch_linear_chunk_state(const LinearArgs &a, int dtype, int d, hipStream_t s);
hipError_t launch_linear_prefix_scan(const LinearArgs &a, int dtype, int d, hipStream_t s);
hipError_t launch_linear_chunk_output(const LinearArgs &a, int dtype, int d, hipStream_t s);

// ---- prefill: indexer + streaming top-M ------------------------------------
struct IndexerArgs {
    const void *q_idx;   // [B,n,G,HI,dI]
    const void *k_idx;   // [B,past+n,G,dI]
    const void *w_idx;   // [B,n,G,HI]
    void *k_packed;      // workspace: k_idx re-laid out per key tile (indexer_packed_bytes)
    void *cand;          // workspace: per-query candidate buffers, (score, key) pairs (indexer_cand_bytes)
    int32_t *idx;        // [B,n,G,M]: key positions in 0..past+t
    int B, n, G, HI, M;
    int past;            // query t (0-based among the n) sits at position past + t
};
size_t indexer_packed_bytes(int B, int nk, int G, int dI, int dtype);
size_t indexer_cand_bytes(int B, int n, int G, int M);
hipError_t launch_indexer_pack(const IndexerArgs &a, int dtype, int dI, hipStream_t s);
hipError_t launch_indexer_prefill(const IndexerArgs &a, int dtype, int dI, hipStream_t s);

// ---- prefill backward ----------------------------------------------------------
struct BwdPrepArgs {
    const void *q, *k, *v, *z, *dout;   // q, z, dout per head [B,n,Hq,(d)]; k, v [B,n,G,d]
    void *Grev, *qrev, *vrep, *krep;    // [B,n,Hq,d] in the layer dtype
    int B, n, Hq, G, d;
};
struct BwdCombineArgs {
    const void *z;                      // gate logits [B,n,Hq]
    const void *dq_lin, *o_k, *o_v;     // [B,n,Hq,d] layer dtype: S_t d_out (not yet scaled
                                        // by 1 - gamma); o_k, o_v in reversed time
    float *dq;                          // [B,n,Hq,d]
    float *dk, *dv;                     // [B,n,G,d]
    int B, n, Hq, G, d;
};
struct SparseBwdArgs {
    const void *q, *k, *v, *z, *dout;         // layer dtype
    const void *rlin;                         // [B,n,Hq,d] S_t d_out (q . rlin = d_out . o_lin)
    const int32_t *idx;                       // [B,n,G,M] the forward's sets
    float *dq, *dk, *dv, *dgate;              // dq += ; dk, dv atomically += ; dgate =
    float *coef;                              // bf16 path: [B,n,G,M,r,2] (scale ds, gamma p) per slot and head
    uint32_t *sorted;                         // bf16 path: per block of positions, its sorted entries
    int B, n, Hq, G, r, M;
    float scale;
};
size_t sparse_bwd_lds_bytes(int r, int M, int d);
// positions per block of the key-side pass (0: the shape does not fit)
int sparse_bwd_key_block(int r, int M, int d);
// workspace of the key side's sorted entries
size_t sparse_bwd_sorted_bytes(int B, int n, int G, int M);
hipError_t launch_bwd_prep(const BwdPrepArgs &a, int dtype, hipStream_t s);
hipError_t launch_transpose_states(const float *src, float *dst, int64_t nmat, int d, hipStream_t s);
hipError_t launch_bwd_combine(const BwdCombineArgs &a, int dtype, hipStream_t s);
hipError_t launch_sparse_bwd(const SparseBwdArgs &a, int dtype, int d, hipStream_t s);
// bf16, in this order: part 0 the query side (dq, dgate, coefficients),
// part 1 the key side's sort, part 2 its walk (dk, dv)
hipError_t launch_sparse_bwd_split(const SparseBwdArgs &a, int d, int part, hipStream_t s);

}  // namespace lisa
