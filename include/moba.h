/*
 * libmoba — MoBA (Mixture of Block Attention) for AMD Instinct MI355X (gfx950):
 * the causal prefill forward pass, its backward pass, the decode step, pooling
 * variants with dynamic k, and packed (varlen) batches.
 *
 * The method (Moonshot AI's MoBA as described by the pomoai MoBA overview,
 * "核心原理" steps 1-3, and by the 智东西 report, section 二):
 *   - the N-token context is cut into n = N / block_size blocks of
 *     block_size contiguous tokens;
 *   - every query t in block j = t / block_size scores each past block i < j by
 *     the dot product of q_t with the block's mean key (no parameters, no scale);
 *   - it keeps its own block j (causally masked inside the block) plus the
 *     topk - 1 best-scoring past blocks; a future block is never chosen;
 *   - it attends, softmax(q k^T / sqrt(D)) v, over the union of those blocks
 *     only; per-block partial outputs are merged by log-sum-exp weighting.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   One sequence (batch 1; the *_varlen calls pack several), H query heads and
 *   H key/value heads.
 *   q, k, v, out : device pointers, row-major [N][H][D] (token, head, dim),
 *                  bf16 for the plain entry points and fp32 for the *_f32 twins.
 *   lse          : device pointer, fp32 [H][N], natural log of the softmax
 *                  denominator sum_s exp(q_t . k_s / sqrt(D)) over the attended keys.
 *   sel          : device pointer, int32 [H][N][topk], chosen blocks of every
 *                  (head, query) in ascending order, padded with -1 when the
 *                  query has fewer than topk eligible blocks (j + 1 < topk).
 *   kbar         : device pointer, fp32 [H][n][D], block mean keys.
 *   topk         : blocks per query including the forced current block;
 *                  topk >= n selects every past block (full causal attention;
 *                  the bf16 prefill and backward then run a dense causal path).
 *   stream       : HIP stream the work is enqueued on (0 = the null stream).
 *   Selection ties (equal fp32 scores) go to the lower block index.
 *
 * Ownership and synchronisation: the caller owns every pointer argument. The
 * library never frees or retains them. Temporary device workspace is taken
 * from a library-owned stream-ordered memory pool on `stream` and returned to
 * it on the same stream. Every call returns once its kernels are enqueued; it
 * performs no host synchronisation. Device faults surface at the caller's next
 * synchronisation, as for any HIP launch.
 *
 * Errors: arguments are checked before any HIP call or enqueue, and on an
 * argument error nothing is written.
 *   MOBA_ERR_INVALID_ARG   null pointer, N < 1, H < 1, topk < 1,
 *                          block_size < 1, or block_size not dividing N.
 *   MOBA_ERR_UNSUPPORTED   D not 64 or 128, block_size not a multiple of 64,
 *                          a pointer not 16-byte aligned, more than
 *                          MOBA_MAX_BLOCKS blocks, topk in (MOBA_MAX_TOPK, n),
 *                          N >= 2^28, or a device that is not gfx950; also a
 *                          call that takes pool workspace on a stream under
 *                          graph capture (nothing is enqueued: the pool
 *                          allocation is not recorded into graphs).
 *   MOBA_ERR_HIP           a HIP runtime call or launch failed; the HIP error
 *                          code is kept per thread (moba_last_hip_error).
 *   MOBA_ERR_OUT_OF_MEMORY the workspace could not be allocated.
 *
 * Reentrancy: calls on different streams may run concurrently; the only
 * process-wide state is a per-device cache of device properties and memory
 * pools, created once. Results are bitwise deterministic (no floating-point
 * atomics).
 */
#ifndef MOBA_H
#define MOBA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOBA_MAX_TOPK 32      /* largest ranked topk when topk < n */
#define MOBA_MAX_BLOCKS 4096  /* largest n = N / block_size */

typedef enum {
  MOBA_OK = 0,
  MOBA_ERR_INVALID_ARG = 1,
  MOBA_ERR_UNSUPPORTED = 2,
  MOBA_ERR_HIP = 3,
  MOBA_ERR_OUT_OF_MEMORY = 4
} moba_status;

/*
 * Block mean keys: kbar[h][i][:] = (1/block_size) * sum of k[t][h][:] over the
 * block_size tokens t of block i, rounded once to fp32 (the sum is formed in
 * fp64 in a fixed order, so the result is the correctly rounded mean whenever
 * that sum is exact). Mean pooling of each block's keys is the gate's
 * "representative vector" (wzjinhao.cn MoBA article, section 3, score_pooling
 * = mean; 0539edu.com NSA/MoBA explainer, section 1).
 * k: bf16 [N][H][D]; kbar: fp32 [H][n][D].
 */
int moba_block_mean_keys(const void* k, float* kbar, int64_t N, int32_t H, int32_t D,
                         int32_t block_size, hipStream_t stream);
int moba_block_mean_keys_f32(const float* k, float* kbar, int64_t N, int32_t H, int32_t D,
                             int32_t block_size, hipStream_t stream);

/*
 * Gate and causal top-k only: writes sel (see conventions). The gate score of
 * past block i for query t is the fp32 dot product <q_t, kbar_i> with kbar the
 * fp32 block mean; future blocks are never scored and the current block is
 * always chosen (wzjinhao.cn MoBA article, section 3, causal_mask and
 * current_block_force; 智东西 report, section 二, gating and causality).
 * q, k: bf16 [N][H][D] (fp32 for the _f32 twin); sel: int32 [H][N][topk].
 */
int moba_gate_topk(const void* q, const void* k, int32_t* sel, int64_t N, int32_t H, int32_t D,
                   int32_t block_size, int32_t topk, hipStream_t stream);
int moba_gate_topk_f32(const float* q, const float* k, int32_t* sel, int64_t N, int32_t H,
                       int32_t D, int32_t block_size, int32_t topk, hipStream_t stream);

/*
 * Query lists only: the pooling, gate and regrouping stages of
 * moba_prefill_fwd, with the regrouped queries handed back. Attention runs
 * block by block over the queries that chose each block (智东西 report,
 * section 二, implementation steps 1-2: queries reordered by their block
 * assignment); a query's own block is not listed, since its queries are that
 * block's own tokens.
 *   sel  : int32 [H][N][topk], written as by moba_gate_topk.
 *   offs : int32 [H * n + 1]. List (h, b) is qidx[offs[h*n + b] ..
 *          offs[h*n + b + 1]); offs[H * n] = P, the total number of
 *          (query, past block) pairs.
 *   qidx : int32 [qidx_len]; entry = query position t of a query with
 *          b in sel(t) and b < t / block_size; each list ascending, lists in
 *          (h, b) order. P = H * sum over blocks j of block_size *
 *          min(topk - 1, j) (a closed form the caller sizes qidx with);
 *          qidx_len < P is MOBA_ERR_INVALID_ARG, entries past P are not written.
 * bf16 q, k only. P >= 2^31 is MOBA_ERR_UNSUPPORTED. offs and qidx need 16-byte
 * alignment like every other pointer. The lists are integer work in fixed
 * orders: for a given sel they are bitwise reproducible.
 */
int moba_block_query_lists(const void* q, const void* k, int32_t* sel, int32_t* offs, int32_t* qidx,
                           int64_t qidx_len, int64_t N, int32_t H, int32_t D, int32_t block_size, int32_t topk,
                           hipStream_t stream);

/*
 * Block pooling variants. The gate scores each past block through one
 * representative key; the pages pool by the mean (wzjinhao.cn MoBA article,
 * section 3, score_pooling = mean) and suggest trying max or weighted pooling
 * instead (the same article, closing section):
 *   MOBA_POOL_MEAN      mean of the block's keys (the default everywhere);
 *   MOBA_POOL_MAX       per-dimension maximum over the block's keys;
 *   MOBA_POOL_WEIGHTED  sum of w[h][t] * k[t][h][:] over the block divided by
 *                       the sum of the weights; `weights` fp32 [H][N],
 *                       non-negative; a block whose weights are all zero pools
 *                       to the zero vector.
 * The pooled key is rounded once to fp32 (max is exact; mean and weighted are
 * summed in fp64). `weights` is read in the weighted mode only (NULL there is
 * MOBA_ERR_INVALID_ARG; it needs 4-byte alignment); an unknown mode is
 * MOBA_ERR_INVALID_ARG.
 */
#define MOBA_POOL_MEAN 0
#define MOBA_POOL_MAX 1
#define MOBA_POOL_WEIGHTED 2

/* Pooled block keys: kbar fp32 [H][n][D] from bf16 k [N][H][D]. */
int moba_block_pool_keys(const void* k, const float* weights, float* kbar, int64_t N, int32_t H, int32_t D,
                         int32_t block_size, int32_t pooling, hipStream_t stream);

/* moba_gate_topk, moba_prefill_fwd and moba_prefill_bwd (bf16) with the gate's
 * block keys pooled as `pooling` says. */
int moba_gate_topk_pooled(const void* q, const void* k, const float* weights, int32_t* sel, int64_t N, int32_t H,
                          int32_t D, int32_t block_size, int32_t topk, int32_t pooling, hipStream_t stream);
int moba_prefill_fwd_pooled(const void* q, const void* k, const void* v, const float* weights, void* out, float* lse,
                            int64_t N, int32_t H, int32_t D, int32_t block_size, int32_t topk, int32_t pooling,
                            hipStream_t stream);
int moba_prefill_bwd_pooled(const void* q, const void* k, const void* v, const float* weights, const void* out,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv, int64_t N, int32_t H,
                            int32_t D, int32_t block_size, int32_t topk, int32_t pooling, hipStream_t stream);

/*
 * Packed (varlen) batches: num_seqs independent sequences concatenated along
 * the token axis, the FlashAttention-style packing the pages build on (智东西
 * report, section 二, implementation steps: varlen attention over reordered
 * queries). cu_seqlens is a HOST array of num_seqs + 1 token offsets (0, then
 * non-decreasing; T = cu_seqlens[num_seqs] tokens in all), read during the call;
 * every sequence length must be a multiple of block_size (empty sequences are
 * allowed). Blocks never straddle sequences, and a query's gate only sees the
 * past blocks of its own sequence: each sequence gets exactly what a separate
 * call on it would give. q, k, v, out, dout, dq, dk, dv: bf16 [T][H][D]; lse:
 * fp32 [H][T]; sel: int32 [H][T][topk] with global block indices. At most 512
 * sequences (MOBA_ERR_UNSUPPORTED above); a bad cu_seqlens is
 * MOBA_ERR_INVALID_ARG. These calls never take the dense path.
 */
int moba_gate_topk_varlen(const void* q, const void* k, int32_t* sel, const int64_t* cu_seqlens, int32_t num_seqs,
                          int32_t H, int32_t D, int32_t block_size, int32_t topk, hipStream_t stream);
int moba_prefill_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                            const int64_t* cu_seqlens, int32_t num_seqs, int32_t H, int32_t D, int32_t block_size,
                            int32_t topk, hipStream_t stream);
int moba_prefill_bwd_varlen(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, void* dq, void* dk, void* dv, const int64_t* cu_seqlens,
                            int32_t num_seqs, int32_t H, int32_t D, int32_t block_size, int32_t topk,
                            hipStream_t stream);

/*
 * Dynamic k (host only, no GPU work): the top_k that keeps a late query's
 * sparsity 1 - block_size * k / N at `sparsity` for a context of N tokens,
 * k = nearest integer to (1 - sparsity) * N / block_size (ties to even),
 * clamped to 1 .. N / block_size. The wzjinhao.cn MoBA article lets k grow with
 * the context (closing section); its section 3 table pairs each context length
 * with (block_size, top_k) at about constant sparsity, which this reproduces.
 * Returns k >= 1, or -MOBA_ERR_INVALID_ARG when N < 1, block_size < 1, N is
 * not a multiple of block_size, or sparsity is outside [0, 1).
 */
int32_t moba_topk_for_sparsity(int64_t N, int32_t block_size, double sparsity);

/*
 * Full MoBA causal prefill (when topk >= n every block is kept and the call
 * runs as causal attention over the whole sequence: no gate, lists or
 * partials): out[t][h][:] = softmax over the attended keys of
 * q_t . k_s / sqrt(D), applied to v, where the attended keys are every key of
 * the chosen past blocks and the keys of the own block up to t itself; lse as
 * in the conventions. Implements the five steps of the 智东西 report, section
 * 二 (assign blocks, regroup queries by block, block attention, scatter back,
 * online-softmax combination) with the attention formula of the 0539edu.com
 * explainer, section 1.
 * q, k, v, out: bf16 [N][H][D] (fp32 for the _f32 twin); lse: fp32 [H][N].
 */
int moba_prefill_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t N, int32_t H, int32_t D, int32_t block_size, int32_t topk,
                     hipStream_t stream);
int moba_prefill_fwd_f32(const float* q, const float* k, const float* v, float* out, float* lse,
                         int64_t N, int32_t H, int32_t D, int32_t block_size, int32_t topk,
                         hipStream_t stream);

/*
 * Backward of the bf16 prefill: dq, dk, dv = the gradients of out (for the
 * upstream gradient dout) with respect to q, k and v. The pages train and
 * continually pretrain with MoBA (智东西 report, section 三); the top-k gate is
 * piecewise constant and carries no gradient, so the same selection as the
 * forward call (recomputed here from q and k) is held fixed and the gradients
 * are those of the masked softmax attention over the attended keys. lse carries
 * no upstream gradient. out and lse are those moba_prefill_fwd returned for the
 * same q, k, v, block_size and topk.
 * q, k, v, out, dout, dq, dk, dv: bf16 [N][H][D]; lse: fp32 [H][N] (natural
 * log). Same shape limits and error behaviour as moba_prefill_fwd; dq, dk, dv
 * are written in full (keys no query attends get zero gradients).
 */
int moba_prefill_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int64_t N, int32_t H, int32_t D,
                     int32_t block_size, int32_t topk, hipStream_t stream);

/*
 * moba_prefill_fwd with stage timing: identical work and results, and, when
 * `events` is not NULL, events[0..MOBA_STAGE_EVENTS-1] (created by the caller
 * with hipEventCreate) are recorded on `stream` at the stage boundaries:
 *   0 before the block mean-pool, 1 before the gate/top-k, 2 before the query
 *   lists, 3 before the past-block attention, 4 before the own-block
 *   attention (which also performs the LSE merge when every query keeps at
 *   most 16 past blocks on the bf16 path), 5 before the separate merge (an
 *   empty stage when it was fused), 6 after it. The fp32 path runs the whole
 *   block attention in the past-block stage (the own-block stage is empty).
 * hipEventElapsedTime between neighbours gives each stage's device time.
 * Individual entries may be NULL: that boundary is then not recorded (each
 * recorded event costs the stream a few microseconds).
 */
#define MOBA_STAGE_EVENTS 7
int moba_prefill_fwd_timed(const void* q, const void* k, const void* v, void* out, float* lse,
                           int64_t N, int32_t H, int32_t D, int32_t block_size, int32_t topk,
                           hipStream_t stream, hipEvent_t* events);

/*
 * MoBA decode step (bf16): the newest token of a K/V cache attends its gated
 * blocks. After the prefill, generation adds one token at a time; the
 * wzjinhao.cn MoBA article (section 3) runs that step as full attention or
 * gated like a prefill row. The token's key and value must already be the
 * last rows of the cache, so the token sits at position t = N - 1, in block
 * j = floor(t / B); N need not be a multiple of B (the own block may be
 * partial). Its gate scores the fp32 means of the complete past blocks
 * 0 .. j-1 exactly like moba_gate_topk scores a prefill row (no scale,
 * ranking by score then lower block index), keeps the topk - 1 best and its
 * own block; topk > j keeps every block (full attention over the cache).
 *   q: bf16 [H][D], the new token's query.   k, v: bf16 [N][H][D] cache.
 *   kbar: fp32 [H][kbar_blocks][D] block means of the cache's complete blocks
 *         as moba_block_mean_keys writes them (at least j blocks per head,
 *         kbar_blocks >= j); NULL makes the call compute them from k (one
 *         pass over the first j*B rows).
 *   out: bf16 [H][D].   lse: fp32 [H], natural log of the softmax
 *         denominator.   sel: NULL, or int32 [H][topk] receiving the kept
 *         blocks in ascending order, -1 padded.
 * Errors: MOBA_ERR_INVALID_ARG for null q/k/v/out/lse, N, H, block_size or
 * topk < 1, kbar_blocks < j with kbar given; MOBA_ERR_UNSUPPORTED for D not
 * 64/128, topk in (MOBA_MAX_TOPK, j], sel with topk > MOBA_MAX_BLOCKS,
 * pointers not 16-byte aligned, not gfx950. Nothing is enqueued on error.
 * Enqueues on `stream` and returns; the workspace comes from the same
 * stream-ordered pool as the prefill.
 */
int moba_decode_fwd(const void* q, const void* k, const void* v, const float* kbar, int32_t kbar_blocks,
                    void* out, float* lse, int32_t* sel, int64_t N, int32_t H, int32_t D,
                    int32_t block_size, int32_t topk, hipStream_t stream);

/*
 * moba_decode_fwd without any device allocation, for callers that cannot
 * allocate: code under HIP graph capture, tight generation loops, harnesses
 * that forbid hipMalloc. Same arguments, results and error behaviour as
 * moba_decode_fwd (bit for bit), but its workspace is a fixed library array of
 * MOBA_NOALLOC_SCRATCH_BYTES per GPU (held from the first call on that GPU
 * until the process ends) instead of the stream-ordered pool; the call itself
 * allocates and frees nothing. A step whose workspace would exceed that size
 * (roughly H * units * (D + 2) * 4 bytes of partials plus H * j * (D + 2) * 4
 * bytes of block means and scores when kbar is NULL; the one-launch gated step
 * needs none) returns MOBA_ERR_UNSUPPORTED and enqueues nothing. All calls on
 * one GPU share the array and it keeps the last call's contents (every byte a
 * call reads it has written first): calls that may overlap on one GPU (other
 * streams, or other threads without ordering) race and must be serialised by
 * the caller; calls ordered on one stream are safe. Under capture it records
 * kernel nodes only (no memory nodes); replaying such a graph is not exercised
 * by this library's tests.
 */
#define MOBA_NOALLOC_SCRATCH_BYTES (64u << 20)
int moba_decode_fwd_noalloc(const void* q, const void* k, const void* v, const float* kbar, int32_t kbar_blocks,
                            void* out, float* lse, int32_t* sel, int64_t N, int32_t H, int32_t D,
                            int32_t block_size, int32_t topk, hipStream_t stream);

/*
 * Debug aid for the workspace (the lists, partial outputs and counters the
 * stages hand to each other, e.g. the regrouped query lists of the 智东西
 * report, section 二, implementation step 2). With `on` non-zero, every later
 * call that takes workspace memory first fills all of it with 0xFF bytes (NaN
 * in fp32 and bf16, -1 in int32) by a fill kernel on its stream, so that a
 * stage reading workspace it did not write first shows up as non-finite or
 * different output. Process-wide switch, off by default; it changes no
 * result of a correct call. Returns the previous setting.
 */
int moba_debug_poison_workspace(int on);

/* Static, NUL-terminated name of a status code ("MOBA_OK", ...). */
const char* moba_status_string(int status);

/* hipError_t behind the calling thread's last MOBA_ERR_HIP (0 if none). */
int moba_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOBA_H */
