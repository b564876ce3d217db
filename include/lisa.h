/*
 * lisa.h -- C ABI of the MI355X (gfx950) LISA layer forward pass.
 *
 * LISA (Linear-Indexed Sparse Attention, arXiv 2607.19358) replaces a
 * layer's self-attention by two branches that run in parallel and a gate
 * that fuses them (arxivdaily page for 2607.19358, English abstract):
 *   - a Lightning Indexer scores every visible token and keeps the top-M of
 *     the full context for a sparse softmax self-attention; the indexer uses
 *     query/key projections and a ReLU'd dot product (gptget.net analysis of
 *     2607.19358, method-details section); M = 256 in the paper's runs (same
 *     page, experiment-design section);
 *   - a linear-attention branch with the identity feature map and a state
 *     matrix S_t updated once per token (gptget.net, method-details);
 *   - a gate mixes the two outputs (arxivdaily abstract; the zhuanzhiai page,
 *     abstract, says the gate is learned).
 * The library is the attention core after the projections: the caller owns
 * the learned projections and passes their outputs.
 *
 * Definitions used (the pages give prose only; these are the readings):
 *   groups    G = num_kv_heads; query head h belongs to group
 *             g(h) = floor(h * G / num_q_heads) (contiguous blocks of r =
 *             num_q_heads / G heads).  One indexer per group.
 *   indexer   I[t,s] = sum_j w[t,g,j] * max(0, q_idx[t,g,j,:] . k_idx[s,g,:])
 *             for candidates s = 0..t (the current token included); the key
 *             k_idx is shared by the idx_heads indexer heads.
 *   top-M     the min(M, t+1) candidates first in the order (higher I, then
 *             lower s); -0.0 equals +0.0.  Written ascending, padded with -1.
 *   sparse    o_sp[t,h] = sum_{s in set} softmax_s(scale * q[t,h].k[s,g]) v[s,g],
 *             scale = softmax_scale > 0 ? softmax_scale : 1/sqrt(head_dim).
 *   linear    S_t = S_{t-1} + k[t,g] v[t,g]^T (S_{-1} = state_in or 0; one
 *             fp32 d x d state per query head, row index = key dim);
 *             o_lin[t,h] = q[t,h]^T S_t  (no normaliser, no decay).
 *   gate      gamma = 1 / (1 + exp(-gate[t,h])); out = gamma*o_sp + (1-gamma)*o_lin.
 *
 * Conventions for every entry point:
 *   - All tensors are dense, row-major, contiguous device buffers owned by
 *     the caller, 16-byte aligned.  Activations (q, k, v, q_idx, k_idx,
 *     w_idx, gate, out) use dims->dtype (LISA_BF16 = bf16 bit patterns, or
 *     LISA_F32); states are always fp32; indices int32.
 *   - Work is enqueued on `stream` and the call returns at once; there is no
 *     device synchronisation inside.  Calls on different streams are
 *     independent if their workspaces and outputs are distinct.
 *   - Arguments are validated before anything is enqueued.  On error nothing
 *     is enqueued and lisa_last_error() (thread-local) describes it.
 *   - Non-finite inputs are undefined behaviour (no fault, unspecified
 *     values).  The library allocates nothing; the workspace comes from the
 *     caller and must be at least the size the *_workspace_bytes query gives.
 *   - With LISA_LOG=1 in the environment (read once per process), every call
 *     that passed its checks prints one line to stderr naming the entry point
 *     and its shapes, before it enqueues anything.
 *
 * Supported shapes: head_dim in {64, 128}; idx_dim in {32, 64};
 * 1 <= idx_heads <= 8; num_q_heads % num_kv_heads == 0 with r <= 16;
 * chunk in {0, 64} (0 means 64); prefill: 1 <= top_m <= 512, n <= 32768;
 * decode: 1 <= top_m <= 2048, max_ctx <= 65536.  Also refused
 * (LISA_ERR_UNSUPPORTED), because kernels address a sequence's rows through
 * buffer descriptors with a 32-bit byte extent and count a launch's threads
 * in 32 bits: one sequence's K/V rows plus one (positions + 1, times
 * num_kv_heads x head_dim x element size; in decode max_ctx positions, or the
 * page pool's rows) above 4 GiB - 1, a position's K/V row of all groups of
 * 16 MiB or more (row offsets are 24-bit products), the indexer-key rows
 * above 4 GiB - 1, 2^22 or more
 * (sequence, position, group) units in one call, and in the backward
 * num_q_heads x top_m above 2^21 (a 256-position block of per-slot
 * coefficients).
 * Refusals and their reasons:
 *   - chunk 16 or 32: the linear branch's result does not depend on the
 *     chunk length (it only regroups the same sums), and the kernels are
 *     tiled for 64-row MFMA blocks, so only 64 is taken;
 *   - prefill top_m above 512: the fused indexer's final select holds a
 *     query's 2 top_m + 128 best candidates in registers across the wave
 *     (18 per lane at top_m = 512), and its workspace keeps 4 top_m + 256
 *     candidates per query; larger top_m are served by the decode step (up
 *     to 2048) and by the window variant (up to 2048), whose selects work
 *     differently.
 */
#ifndef LISA_H
#define LISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *lisa_stream_t; /* a hipStream_t; NULL = default stream */

typedef enum {
    LISA_OK = 0,
    LISA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, bad count */
    LISA_ERR_UNSUPPORTED = 2,      /* a shape outside the supported set above */
    LISA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
    LISA_ERR_HIP = 4               /* a HIP launch failed; message has the HIP error */
} lisa_status;

enum { LISA_F32 = 0, LISA_BF16 = 1 };

typedef struct {
    int32_t num_q_heads;   /* Hq */
    int32_t num_kv_heads;  /* Hkv = G, also the number of indexers */
    int32_t head_dim;      /* d = d_k = d_v */
    int32_t idx_heads;     /* H_I, indexer heads per group */
    int32_t idx_dim;       /* d_I */
    int32_t top_m;         /* M */
    int32_t chunk;         /* linear-attention chunk length in prefill (0 or 64) */
    float softmax_scale;   /* <= 0: 1/sqrt(head_dim) */
    int32_t dtype;         /* LISA_F32 or LISA_BF16 */
} lisa_dims;

/* Workspace needed by lisa_prefill for batch B and length n (any top_m up to
 * 2048, so the query also serves lisa_prefill_window). */
lisa_status lisa_prefill_workspace_bytes(const lisa_dims *dims, int32_t B, int32_t n,
                                         size_t *bytes);

/* Workspace needed by lisa_prefill_continue for n new tokens after `past`
 * cached ones (the indexer keeps a re-laid-out copy of all past + n indexer
 * keys).  past == 0 gives lisa_prefill_workspace_bytes. */
lisa_status lisa_prefill_continue_workspace_bytes(const lisa_dims *dims, int32_t B, int32_t past,
                                                  int32_t n, size_t *bytes);

/*
 * Whole-prompt forward pass of one LISA layer (all four parts above).
 *   q      [B, n, Hq, d]          k, v  [B, n, Hkv, d]
 *   q_idx  [B, n, G, H_I, d_I]    k_idx [B, n, G, d_I]    w_idx [B, n, G, H_I]
 *   gate   [B, n, Hq]  (logits z; gamma = sigmoid(z))
 *   state_in  [B, Hq, d, d] fp32 or NULL (zero initial state)
 *   out    [B, n, Hq, d]  (written)
 *   state_out [B, Hq, d, d] fp32 or NULL: S after the last token
 *   topm_out  [B, n, G, M] int32 or NULL: the selected sets
 * n == 0 or B == 0 is a valid no-op.
 */
lisa_status lisa_prefill(const lisa_dims *dims, int32_t B, int32_t n, const void *q,
                         const void *k, const void *v, const void *q_idx, const void *k_idx,
                         const void *w_idx, const void *gate, const float *state_in, void *out,
                         float *state_out, int32_t *topm_out, void *workspace,
                         size_t workspace_bytes, lisa_stream_t stream);

/*
 * Continued prefill: n more prompt tokens of each sequence against the cache
 * of its first `past` tokens -- the step between a prompt that was already
 * processed and token-by-token generation.  Per position the result is the
 * layer defined above: query row t (0-based) is position past + t, its
 * candidates are positions 0..past+t, and the linear branch continues from
 * S_{past-1}.  So `out` equals rows past..past+n-1 of one lisa_prefill over
 * all past + n tokens.
 *   q      [B, n, Hq, d]   q_idx [B, n, G, H_I, d_I]   w_idx [B, n, G, H_I]
 *   gate   [B, n, Hq]
 *   k_cache, v_cache [B, past + n, Hkv, d]; k_idx_cache [B, past + n, G, d_I]:
 *          every position, the n new tokens included (rows past..).
 *   state_in  [B, Hq, d, d] fp32 or NULL: S after the first `past` tokens
 *          (NULL = zero, e.g. past == 0).
 *   out    [B, n, Hq, d]; state_out [B, Hq, d, d] fp32 or NULL: S after the
 *          last token; topm_out [B, n, G, M] int32 or NULL: positions in
 *          0..past+t, ascending, -1 padded.
 * The workspace is lisa_prefill_continue_workspace_bytes(dims, B, past, n).
 * past + n <= 32768; n == 0 or B == 0 is a valid no-op; past == 0 is
 * lisa_prefill.
 */
lisa_status lisa_prefill_continue(const lisa_dims *dims, int32_t B, int32_t past, int32_t n,
                                  const void *q, const void *k_cache, const void *v_cache,
                                  const void *q_idx, const void *k_idx_cache, const void *w_idx,
                                  const void *gate, const float *state_in, void *out,
                                  float *state_out, int32_t *topm_out, void *workspace,
                                  size_t workspace_bytes, lisa_stream_t stream);

/*
 * Sliding-window variant (the model before the indexer is introduced: in
 * the first training stage the linear branch is paired with a static
 * sliding-window attention, which the indexer later replaces -- arxivdaily
 * page for 2607.19358, English abstract).  Readings: the window is the same
 * budget M = dims->top_m (1..2048 here), the set of position t is
 * max(0, t-M+1)..t, and the gate and linear branch are as above.  Arguments
 * as lisa_prefill_continue without the indexer inputs and topm_out (the
 * indexer fields of dims are ignored); same workspace query.
 */
lisa_status lisa_prefill_window(const lisa_dims *dims, int32_t B, int32_t past, int32_t n,
                                const void *q, const void *k_cache, const void *v_cache,
                                const void *gate, const float *state_in, void *out,
                                float *state_out, void *workspace, size_t workspace_bytes,
                                lisa_stream_t stream);

/*
 * Backward pass of lisa_prefill: the gradients of
 *     L = <d_out, out> + <d_state_out, state_out>
 * with respect to q, k, v, the gate logits and state_in, obtained from the
 * layer's definition (gptget.net analysis of arXiv 2607.19358,
 * method-details section) by the chain rule, with the selected sets held at
 * the forward's.  A top-M set is a piecewise-constant function of q_idx,
 * k_idx and w_idx, so those inputs get no gradient and are not taken.
 *   q, k, v, gate, state_in   as given to lisa_prefill (state_in may be NULL)
 *   topm         [B, n, G, M] int32: the forward's topm_out for these inputs
 *                (entries outside 0..t are skipped; sets that are not
 *                ascending give the same result, only more slowly)
 *   d_out        [B, n, Hq, d] in the layer dtype
 *   d_state_out  [B, Hq, d, d] fp32 or NULL (zero)
 *   dq  [B, n, Hq, d]; dk, dv [B, n, Hkv, d]; dgate [B, n, Hq]; all fp32,
 *       written (dk and dv are accumulated with atomics, so their last bits
 *       may differ from run to run)
 *   d_state_in  [B, Hq, d, d] fp32 or NULL
 * Up to 16 query heads per group; for fp32, top_m * heads-per-group is
 * bounded by the kernel's LDS (UNSUPPORTED beyond).  The workspace is
 * lisa_prefill_backward_workspace_bytes(dims, B, n): seven activation-sized
 * buffers and the chunk states of the linear passes, plus (bf16) 8 * top_m
 * bytes per position and query head for the sparse branch's per-slot
 * coefficients.
 */
lisa_status lisa_prefill_backward_workspace_bytes(const lisa_dims *dims, int32_t B, int32_t n,
                                                  size_t *bytes);
lisa_status lisa_prefill_backward(const lisa_dims *dims, int32_t B, int32_t n, const void *q,
                                  const void *k, const void *v, const void *gate,
                                  const float *state_in, const int32_t *topm, const void *d_out,
                                  const float *d_state_out, float *dq, float *dk, float *dv,
                                  float *dgate, float *d_state_in, void *workspace,
                                  size_t workspace_bytes, lisa_stream_t stream);

/* Workspace needed by lisa_decode_step for B sequences of at most max_ctx
 * visible tokens each.  The indexer scores are kept per sequence in rows of
 * max_ctx entries ([B, G, max_ctx] fp32), so the size depends on B and
 * max_ctx only: the total context length of a ragged batch is not needed. */
lisa_status lisa_decode_workspace_bytes(const lisa_dims *dims, int32_t B, int32_t max_ctx,
                                        size_t *bytes);

/*
 * One generated token per sequence against packed token-major caches.
 *   cu_ctx  [B+1] int64, DEVICE memory: sequence b owns cache rows
 *           [cu_ctx[b], cu_ctx[b+1]); L_b = cu_ctx[b+1]-cu_ctx[b] >= 1 visible
 *           tokens.  The caller has already appended the new token's k, v and
 *           k_idx as the last row, so the new token is position t = L_b - 1.
 *   max_ctx host int32 >= every L_b (sizes the workspace; rows beyond it are
 *           ignored, which gives unspecified results but never reads out of
 *           bounds).
 *   q [B, Hq, d]; k_cache, v_cache [sum L, Hkv, d]; q_idx [B, G, H_I, d_I];
 *   k_idx_cache [sum L, G, d_I]; w_idx [B, G, H_I]; gate [B, Hq];
 *   state [B, Hq, d, d] fp32, in/out: S_{t-1} on entry, S_t on return.
 *   out [B, Hq, d]; topm_out [B, G, M] int32 or NULL.
 * B == 0 is a valid no-op.
 */
lisa_status lisa_decode_step(const lisa_dims *dims, int32_t B, const int64_t *cu_ctx,
                             int32_t max_ctx, const void *q, const void *k_cache,
                             const void *v_cache, const void *q_idx, const void *k_idx_cache,
                             const void *w_idx, const void *gate, float *state, void *out,
                             int32_t *topm_out, void *workspace, size_t workspace_bytes,
                             lisa_stream_t stream);

/*
 * lisa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The step's scratch (indexer scores,
 * o_lin, and the sets when topm_out is NULL) lives in a static device array
 * of the library, 32 MiB per GPU, held until the process ends; nothing is
 * allocated or freed.  A step needing more than that
 * (lisa_decode_workspace_bytes(dims, B, max_ctx) > 32 MiB, e.g. B * G *
 * max_ctx above about 8 M) returns LISA_ERR_UNSUPPORTED.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (concurrent
 * streams or threads) race and must be serialized by the caller.  The first
 * call on each device looks the array's device address up (a HIP call made
 * after argument validation).  Other arguments as lisa_decode_step.
 */
lisa_status lisa_decode_step_noalloc(const lisa_dims *dims, int32_t B, const int64_t *cu_ctx,
                                     int32_t max_ctx, const void *q, const void *k_cache,
                                     const void *v_cache, const void *q_idx, const void *k_idx_cache,
                                     const void *w_idx, const void *gate, float *state, void *out,
                                     int32_t *topm_out, lisa_stream_t stream);

/*
 * lisa_decode_step on paged (block-table) caches, the layout serving systems
 * keep KV caches in (the pages say nothing about cache layouts; the result
 * is the same decode step).  The three caches are page pools of
 * num_pages * block_size rows: k_pages, v_pages [rows, Hkv, d];
 * k_idx_pages [rows, G, d_I].  Position s of sequence b is row
 *   block_table[b * max_blocks + s / block_size] * block_size + s % block_size.
 *   lengths      [B] int32, DEVICE: L_b >= 1 visible tokens, the new token's
 *                k, v, k_idx already written at position L_b - 1.
 *   block_table  [B, max_blocks] int32, DEVICE: page ids in [0, num_pages)
 *                for every block holding a position below L_b (others are
 *                not read); ids out of range are undefined behaviour.
 *   block_size   a power of two in [1, 4096]; max_blocks * block_size >= max_ctx.
 *   The K/V pool of one cache is at most 2 GiB.
 * Other arguments and the workspace query as lisa_decode_step.
 */
lisa_status lisa_decode_step_paged(const lisa_dims *dims, int32_t B, const int32_t *lengths,
                                   const int32_t *block_table, int32_t block_size,
                                   int32_t max_blocks, int32_t num_pages, int32_t max_ctx,
                                   const void *q, const void *k_pages, const void *v_pages,
                                   const void *q_idx, const void *k_idx_pages, const void *w_idx,
                                   const void *gate, float *state, void *out, int32_t *topm_out,
                                   void *workspace, size_t workspace_bytes, lisa_stream_t stream);

/*
 * One generated token per sequence with the sliding-window set
 * max(0, t-M+1)..t (see lisa_prefill_window); arguments as lisa_decode_step
 * without the indexer inputs and topm_out; same workspace query.
 */
lisa_status lisa_decode_step_window(const lisa_dims *dims, int32_t B, const int64_t *cu_ctx,
                                    int32_t max_ctx, const void *q, const void *k_cache,
                                    const void *v_cache, const void *gate, float *state, void *out,
                                    void *workspace, size_t workspace_bytes,
                                    lisa_stream_t stream);

/*
 * Per-kernel timing, for benchmarking only.  While enabled (process-wide),
 * each stage of an entry point is timed by a pair of HIP events attached to
 * its kernel dispatches on the caller's stream (hipExtLaunchKernel): from the
 * start of the stage's first kernel to the end of its last, so the figures
 * are the kernels' own execution times.  This adds host work per launch, so
 * whole-call timings should be taken with it disabled.  Stages, in order:
 * linear_chunk_state, linear_prefix_scan, linear_chunk_output, indexer_pack,
 * indexer_topm, sparse_gate_prefill, decode_score_state, decode_select,
 * sparse_gate_decode, then the backward's bwd_operands, bwd_linear,
 * bwd_combine, bwd_sparse, bwd_sparse_query, bwd_sparse_sort, bwd_sparse_keys.
 */
lisa_status lisa_stage_timing(int32_t enable);

/*
 * Waits for the recorded events, adds their elapsed times to per-stage
 * totals and copies out up to max_stages entries: static stage names (the
 * library owns the strings), launch counts and total milliseconds since the
 * last reset.  Any output pointer may be NULL.  *n_stages receives the number
 * of stages.  reset != 0 clears the totals after copying.
 */
lisa_status lisa_stage_timing_read(int32_t max_stages, const char **names, int64_t *launches,
                                   double *total_ms, int32_t *n_stages, int32_t reset);

/*
 * Roofline calibration, for benchmarking only (not part of the layer).
 * kind LISA_PROBE_COPY: a plain streaming copy of `bytes` (a multiple of 16,
 * 16-byte aligned buffers) from src to dst; *work = 2 * bytes moved.
 * kind LISA_PROBE_READ: a read-only stream over `bytes` of src (dst is a
 * sink of at least 8 MiB that is never written in practice); *work = bytes.
 * kind LISA_PROBE_MFMA: `iters` rounds of eight independent bf16
 * 16x16x32 MFMAs per wave on register operands, 8 waves per SIMD; dst is a
 * sink of at least 2 MiB that is never written in practice; *work = the
 * flops issued.
 * kind LISA_PROBE_GATHER: 65536 waves, each `iters` batches of 16 loads of
 * random 256-byte rows (16 lanes a row) of the table src of `bytes` (a power
 * of two rows of 256 bytes, 16-byte aligned); dst is a sink of at least
 * 1 KiB that is never written in practice; *work = the bytes gathered.
 * Enqueued on `stream`; the caller times it with events.
 * Returns LISA_ERR_INVALID_ARGUMENT for a bad kind or buffer (nothing is
 * enqueued then); the error message is not set.
 */
enum { LISA_PROBE_COPY = 0, LISA_PROBE_MFMA = 1, LISA_PROBE_READ = 2, LISA_PROBE_GATHER = 3 };
lisa_status lisa_peak_probe(int32_t kind, const void *src, void *dst, size_t bytes, int32_t iters,
                            double *work, lisa_stream_t stream);

/* Message for the last failing call on this thread ("" if none). */
const char *lisa_last_error(void);

/* Build description: target architecture and library version. */
const char *lisa_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* LISA_H */
