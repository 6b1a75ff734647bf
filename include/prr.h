/*
 * prr.h - C ABI of libprr.so, the MI355X (gfx950) hot path of PRR: predict, reuse and repair for
 * dynamic sparse attention during long-context decoding.
 *
 * Citations:
 *   [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context LLM
 *           Decoding" (full paper text)
 *   [blog]  "PRR: Predict, Reuse, and Repair - Accelerating Dynamic Sparse Attention for Long-Context
 *           LLM Decoding" (xllm-io paper review; equation numbers (1)-(6))
 *
 * Conventions shared by every entry point
 *   - Every pointer named "device" is GPU memory owned by the caller; the library allocates nothing and
 *     keeps no mutable global state (apart from the per-thread arming of prr_time_next_kernel and the
 *     checking mode's result word).  Host structs are read only during the call.
 *   - Work is enqueued on `stream` and runs asynchronously in stream order.  Nothing is copied to the
 *     host: set sizes stay on the device.
 *   - Problems the host can see (null pointers, sizes, unsupported shapes, a short workspace) return a
 *     status BEFORE anything is enqueued.  A failed launch returns PRR_EHIP.
 *   - Device-side preconditions are the caller's contract: block indices in range and unique within a
 *     set, M disjoint from P, finite inputs, page-table entries in [0, num_pages).  Out-of-range block
 *     and page indices are clamped (never read out of bounds) but give unspecified results.
 *   - Checking mode: with PRR_CHECK=1 in the environment (read once per process), prr_spec_attn,
 *     prr_repair, prr_select, prr_select_spec and prr_select_spec_predict first check every input
 *     set on the stream (count within [0, cap], entries within [0, ceil(seq_len / block)), no repeats),
 *     wait for the result and return PRR_EINVAL, with nothing else enqueued, if one fails.  The mode
 *     synchronises with the host and keeps its result in one device word of the library, so calls in it
 *     must not overlap; it is for debugging.
 *   - Block sets are int32 lists per (sequence, kv head): idx[b][kvh][0 .. count[b][kvh]), any order on
 *     input; sets produced by the library are unique and ascending.
 *   - Query head h of a sequence uses kv head h / G with G = num_q_heads / num_kv_heads (contiguous
 *     grouping); the block set of a kv head is shared by its G query heads ([paper] A.1).
 */
#ifndef PRR_H
#define PRR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum prr_status {
    PRR_OK = 0,
    PRR_EINVAL = 1,       /* null pointer, negative or inconsistent size */
    PRR_EUNSUPPORTED = 2, /* valid but not implemented: head_dim, page size, group size, dtype, N */
    PRR_EWORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_bytes query */
    PRR_EHIP = 4          /* a HIP launch or runtime call failed */
} prr_status;

/* Cache element types.  PRR_FP8: k and v hold 8-bit E4M3 codes (the OCP 8-bit floating-point format,
 * FN variant: bias 7, subnormals, no infinities; the NaN codes 0x7F / 0xFF must not occur), one byte per
 * element; queries and min/max metadata are bf16 (every finite E4M3 value is a bf16 value, so keys and
 * values enter the bf16 products exactly).  Low-bit KV is the pages' future work ([paper] Limitations). */
typedef enum prr_dtype { PRR_F32 = 0, PRR_BF16 = 1, PRR_FP8 = 2 } prr_dtype;

/* How selection scores a block ([paper] §2.1: each block is compressed to a representative scored
 * against the query):
 *   PRR_SCORE_QUEST  Quest's bound over the channel-wise min/max keys ([paper] A.1; metadata of
 *                    prr_build_meta);
 *   PRR_SCORE_MEAN   the block's mean key ("e.g., mean"): sum_i qbar_i mean_{p,i} (metadata of
 *                    prr_build_mean_meta). */
typedef enum prr_score_mode { PRR_SCORE_QUEST = 0, PRR_SCORE_MEAN = 1 } prr_score_mode;

/* Paged KV cache.  Page size must be 16 tokens.  One (page, kv head) tile is contiguous:
 *   k: [num_pages][num_kv_heads][page_size][head_dim]  (token-major tile)
 *   v: [num_pages][num_kv_heads][head_dim][page_size]  (channel-major tile)
 * page_table[b][j] is the physical page holding tokens [16 j, 16 j + 16) of sequence b; seq_len[b] is
 * the number of valid tokens.  head_dim must be 64 or 128.  q (where an entry point takes it) has the
 * same dtype as k and v (bf16 for an fp8 cache), layout [batch][num_q_heads][head_dim]. */
typedef struct prr_kv_cache {
    const void *k;              /* device */
    const void *v;              /* device */
    const int32_t *page_table;  /* device, [batch][max_pages] */
    const int32_t *seq_len;     /* device, [batch] */
    int32_t batch;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t num_pages;
    int32_t max_pages;
    prr_dtype dtype;
} prr_kv_cache;

/* A block set per (sequence, kv head): idx [batch][num_kv_heads][cap], count [batch][num_kv_heads].
 *
 * pages (device, may be NULL): the set's page work list, the flat (unit, page) items the attention
 * passes walk ([paper] §4.3: the repair kernel reads the missed tiles; the survey's M work list), laid out
 * [batch][num_kv_heads][cap * (block / page_size)] for the block size of the calls that write and read it.
 * Slot e * (block / page_size) + s of a unit holds the physical page (through the cache's page table) of
 * page s of block idx[e], for e < count, or -1 where that page held no token when the list was written.
 * Writers: prr_select, prr_select_spec(_predict) and prr_layer_step write M's list with M; prr_predict and a
 * carried predictor write P_next's with P_next; A's list is not written.  Readers: the speculative pass
 * (prr_spec_attn(_noalloc), prr_select_spec(_predict), prr_layer_step) reads P's list, repair (prr_repair,
 * prr_layer_step) reads M's: the K/V tile loads then start in the round trip that reads the set, instead
 * of waiting for a page-table lookup.  A -1 slot whose page holds tokens by the time of the read is looked
 * up in the page table then.  A list stays valid while every page that held a token when it was written
 * keeps its physical page (an append-only paged cache: a page is mapped when its first token is written
 * and keeps its mapping); results are the same with and without a list.  A NULL list: the readers look
 * every page up. */
typedef struct prr_block_set {
    int32_t *idx;    /* device */
    int32_t *count;  /* device */
    int32_t cap;
    int32_t *pages;  /* device, may be NULL: the page work list above */
} prr_block_set;

/* Partial attention state per query head ([paper] §4.3, the speculative kernel's extra outputs):
 *   acc[b][h][:] = sum_j e^{s_j - m} v_j   (unnormalised output; O = acc / l)
 *   l[b][h]      = sum_j e^{s_j - m}       (softmax denominator)
 *   m[b][h]      = max_j s_j               (running maximum, natural-log units)
 * with s_j = scale * (q . k_j) over the tokens of the blocks folded in so far.  The empty state is
 * acc = 0, l = 0, m = -inf.  All fp32, device. */
typedef struct prr_attn_state {
    float *acc;  /* [batch][num_q_heads][head_dim] */
    float *l;    /* [batch][num_q_heads] */
    float *m;    /* [batch][num_q_heads] */
} prr_attn_state;

/* ---- sizes ---------------------------------------------------------------------------------- */

/* Blocks per sequence that the page table can address: max_pages * page_size / block. */
int32_t prr_max_blocks(const prr_kv_cache *kv, int32_t block);

/* Row length (elements) of the metadata array: prr_max_blocks rounded up to a multiple of 8. */
int32_t prr_meta_stride(const prr_kv_cache *kv, int32_t block);

/* Bytes of block metadata: batch * num_kv_heads * head_dim * 2 * prr_meta_stride * sizeof(elem). */
size_t prr_meta_bytes(const prr_kv_cache *kv, int32_t block);

/* Workspace bytes needed by prr_spec_attn / prr_repair / prr_select_spec for sets of capacity `cap`
 * (blocks): arrival counters (per (sequence, kv head) unit) and one partial attention state per chunk. */
size_t prr_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block, int32_t cap);

/* Zero a workspace on `stream` with a fill kernel (no memset node).  An attention workspace must be
 * zero before its first use; every attention call leaves it ready for the next one.  Calls that run
 * concurrently need distinct workspaces. */
prr_status prr_workspace_clear(void *ws, size_t ws_bytes, hipStream_t stream);

/* ---- entry points --------------------------------------------------------------------------- */

/* Block metadata for Quest selection ([paper] A.1: channel-wise min and max keys m_p, M_p of every
 * block, stored per kv head).  meta layout: [batch][num_kv_heads][head_dim][2][stride] in the cache
 * dtype (bf16 for an fp8 cache: exact), row 0 = min, row 1 = max, column p = block p (stride = prr_meta_stride).  Blocks at or beyond
 * ceil(seq_len / block) are not written.  A partial last block uses its valid tokens only.
 * block must be a positive multiple of page_size.  Reads all of K once; not part of the per-step path. */
prr_status prr_build_meta(const prr_kv_cache *kv, int32_t block, void *meta, hipStream_t stream);

/* Bytes of mean-pooled block metadata: batch * num_kv_heads * head_dim * prr_meta_stride * 4. */
size_t prr_mean_meta_bytes(const prr_kv_cache *kv, int32_t block);

/* Mean-pooled block metadata ([paper] §2.1: a block compressed to its mean key).  meta layout:
 * [batch][num_kv_heads][head_dim][stride] fp32, column p = block p: the channel-wise mean of the block's
 * valid tokens, summed in float64 in token order, divided by their count, rounded once to float32.
 * Blocks at or beyond ceil(seq_len / block) are not written. */
prr_status prr_build_mean_meta(const prr_kv_cache *kv, int32_t block, float *meta, hipStream_t stream);

/* Decode-loop append (one token per sequence and step; [paper] §4.1: blocks are born as decoding grows
 * the context, and [paper] A.1: the metadata of the block being filled must cover its tokens).  For every
 * sequence b with t = seq_len[b] < max_pages * page_size: writes k_new[b][h] to the K cache and
 * v_new[b][h] to the V cache at position t (physical page page_table[b][t / page_size], slot t mod
 * page_size; the V tile is channel-major), updates the metadata of block t / block (row 0 = channel-wise
 * min, row 1 = max; the block's first token sets both, later tokens take the running min/max, which equals
 * a rebuild by prr_build_meta over the block's valid tokens; with mode PRR_SCORE_MEAN, meta holds block
 * means and the block's mean is recomputed as prr_build_mean_meta does), then sets seq_len[b] = t + 1.  A sequence
 * whose cache is full (or whose page-table entry is out of range) is left untouched.
 * k_new, v_new: [batch][num_kv_heads][head_dim] in the cache dtype (E4M3 codes for fp8), device.  seq_len must be kv->seq_len
 * (written in place); kv->k and kv->v are written.  meta as for prr_build_meta. */
prr_status prr_append(const prr_kv_cache *kv, int32_t block, const void *k_new, const void *v_new, void *meta,
                      prr_score_mode mode, int32_t *seq_len, hipStream_t stream);

/* Quest selection, GQA-extended ([paper] A.1; [paper] §1, §2.1 top-K selection; [paper] §3 M = A \ P).
 *   scores[b][kvh][p] (fp64, row length prr_max_blocks) = sum_{i=0}^{d-1} max(qbar_i mn_{p,i},
 *       qbar_i mx_{p,i}), qbar = (1/G) sum_g q[b][kvh G + g], summed in channel order from +0.0 in
 *       float64 with no fused multiply-add, for p < N_b = ceil(seq_len[b] / block);
 *   A = the min(topk, N_b) highest scores (ties to the smaller block index), ascending;
 *   M = A \ P (ascending) when P is given.
 * With mode PRR_SCORE_MEAN, meta holds block means (prr_build_mean_meta) and scores[b][kvh][p] =
 * sum_i qbar_i mean_{p,i}, with the same qbar, order and precision.
 * P may be NULL (then M must be NULL).  A->cap and M->cap must be >= topk.  q: [batch][num_q_heads]
 * [head_dim], device, dtype of the cache (bf16 for fp8).
 * Row length: prr_max_blocks(kv, block) up to 131072 blocks (2M tokens at block 16).  Without a
 * workspace (ws NULL) one workgroup per (b, kvh) ranks the row, up to 32768 blocks.  With ws
 * (prr_select_workspace_bytes(kv, mode, block, topk) of caller memory, zeroed once like an attention
 * workspace; every call leaves it ready for the next), rows of more than 8192 blocks are ranked in three
 * part-parallel stages: each scoring workgroup keeps its blocks' local top-K, groups of parts keep theirs,
 * then one ranking per (b, kvh).  The result is the same exact top-K either way.  Rows above 32768 blocks
 * need ws (PRR_EWORKSPACE without it); a non-NULL ws smaller than the query gives PRR_EWORKSPACE.  The
 * query is 0 for rows of up to 8192 blocks and for shapes with more candidates than the stages rank
 * (large topk at long rows; those give PRR_EUNSUPPORTED above 32768 blocks). */
size_t prr_select_workspace_bytes(const prr_kv_cache *kv, prr_score_mode mode, int32_t block, int32_t topk);

prr_status prr_select(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, const void *meta,
                      prr_score_mode mode, int32_t block, int32_t topk, const prr_block_set *P, double *scores,
                      prr_block_set *A, prr_block_set *M, void *ws, size_t ws_bytes, hipStream_t stream);

/* Selection and the speculative pass over P together (the overlap of [paper] §1, Figure 1 flow, and §3:
 * speculation over P runs concurrently with selection; the two only read P).  Computes what
 *     prr_select(q, num_q_heads, kv, meta, block, topk, P, scores, A, M, ...) and
 *     prr_spec_attn(q, num_q_heads, kv, block, P, scale, out, ws, ws_bytes)
 * compute, as one grid whose workgroups do either part (bf16 caches; fp32 caches run the two calls in
 * turn), followed by the top-K on the same stream.  scores, A and M are the same bit for bit.  The state
 * is too while the scoring workgroups (ceil(N_max / 512) per (sequence, kv head); ceil(N_max / 1024) for
 * min/max scoring of rows of 32768 blocks and more that rank in three stages, and of rows of more than
 * 2048 blocks whose 512-block parts would number more than 256 in all) number at most the
 * GPU's compute units; with more of them the speculative pass is cut into fewer, longer chunks so that the
 * whole grid is resident at once, and the state then differs from prr_spec_attn's by rounding only (the
 * order of the sums changes).  P and M must be non-NULL; A->cap and M->cap >= topk; rows as for
 * prr_select (up to 131072 blocks; rows above 32768 blocks, and any row whose candidate slots exceed
 * what one ranking holds, rank in three stages: inside the grid while its scoring workgroups number at
 * most twice the compute units, else in launches after it).  ws: prr_select_spec_workspace_bytes(kv, num_q_heads, block, topk, P->cap): the attention
 * workspace of prr_spec_attn plus room for top-K candidates and a work counter (zeroed once like an
 * attention workspace; every call leaves it ready for the next). */
size_t prr_select_spec_workspace_bytes(const prr_kv_cache *kv, int32_t num_q_heads, int32_t block, int32_t topk,
                                       int32_t cap);

prr_status prr_select_spec(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, const void *meta,
                           prr_score_mode mode, int32_t block, int32_t topk, const prr_block_set *P,
                           double *scores, prr_block_set *A, prr_block_set *M, float scale, prr_attn_state *out,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/* EMA level/trend predictor, one decode step ([paper] §4.1; [blog] Eqs. (2)-(3)).
 * For every (b, kvh) with N_b = ceil(seq_len[b] / block) blocks and live[b][kvh] blocks that already
 * carry state: blocks p < live get
 *     trend = beta (IS - level) + (1 - beta) trend;  level = alpha IS + (1 - alpha) level
 * (both with the previous level); blocks live <= p < N_b start at level = IS, trend = 0.  Then
 * live = N_b and P_next = the `budget` blocks with the largest level + gamma trend (ties to the smaller
 * index), ascending.  All arithmetic fp64 in the order written, no fused multiply-add.
 * scores, level, trend: [batch][num_kv_heads][max_blocks] fp64, device; live [batch][num_kv_heads]
 * int32 (zero for a fresh sequence).  P_next->cap >= budget.  max_blocks <= 131072; rows above 32768
 * blocks need ws (PRR_EWORKSPACE without it; PRR_EUNSUPPORTED for budgets with no part-parallel plan).
 * ws (may be NULL): prr_predict_workspace_bytes of caller memory, zeroed once like an attention workspace
 * (every call leaves it ready for the next).  With it, rows of more than 2048 blocks are updated by
 * 512-block parts in parallel and P_next is ranked from the parts' local top-|P| candidates (exact, as
 * in the two-stage top-K; with more than 4096 candidate slots, groups of parts keep their top-|P| in
 * between); without it one workgroup per (b, kvh) does the whole row.  Same results either way.  A
 * non-NULL ws smaller than the query gives PRR_EWORKSPACE.  The query is 0 where no workspace is used:
 * rows of up to 2048 blocks, and budgets with no part-parallel plan (above 512 at 32768 blocks); it is not
 * monotone in the budget, so a workspace for several budgets takes the largest of their queries. */
size_t prr_predict_workspace_bytes(int32_t batch, int32_t num_kv_heads, int32_t max_blocks, int32_t budget);

/* kv (may be NULL unless P_next->pages is set): the cache whose page table P_next's page list maps
 * through (same batch, num_kv_heads and block; its seq_len should be `seq_len`). */
prr_status prr_predict(const double *scores, const int32_t *seq_len, int32_t batch,
                       int32_t num_kv_heads, int32_t block, int32_t max_blocks, double alpha,
                       double beta, double gamma, int32_t budget, double *level, double *trend,
                       int32_t *live, prr_block_set *P_next, const prr_kv_cache *kv, void *ws, size_t ws_bytes,
                       hipStream_t stream);

/* The arguments of prr_predict, for prr_select_spec_predict. */
typedef struct prr_predict_args {
    const double *scores;
    const int32_t *seq_len;
    int32_t batch;
    int32_t num_kv_heads;
    int32_t block;
    int32_t max_blocks;
    double alpha, beta, gamma;
    int32_t budget;
    double *level;
    double *trend;
    int32_t *live;
    prr_block_set *P_next;
    void *ws;          /* as prr_predict's (may be NULL) */
    size_t ws_bytes;
    const prr_kv_cache *kv;   /* as prr_predict's (may be NULL unless P_next->pages is set) */
} prr_predict_args;

/* prr_select_spec, plus (pred non-NULL) the predictor step prr_predict would run on *pred, typically
 * the previous layer's: in a stack of layers the predictor of one layer needs only that layer's scores
 * and is off the critical path ([paper] §1 and the Figure 1 flow; [paper] §4.1), so its workgroups join
 * this launch and use the slots selection leaves while the speculative pass runs (rows of up to 2048
 * blocks; longer rows get their own launch after this one, on the same stream).  Results equal
 * prr_select_spec(...) followed by prr_predict(*pred).  The predictor's buffers must not overlap any
 * buffer of the selection or speculative pass (PRR_EINVAL for the same scores, set or state pointers).
 * pred NULL: exactly prr_select_spec. */
prr_status prr_select_spec_predict(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, const void *meta,
                                   prr_score_mode mode, int32_t block, int32_t topk, const prr_block_set *P,
                                   double *scores, prr_block_set *A, prr_block_set *M, float scale,
                                   prr_attn_state *out, void *ws, size_t ws_bytes, const prr_predict_args *pred,
                                   hipStream_t stream);

/* The whole layer step of the method ([paper] §1 and the Figure 1 flow, §3, §4.3; [blog] Eq. (6)): selection of
 * A (with M = A \ P), the speculative pass over P and the repair of its state with M, with the results of
 *     prr_select_spec_predict(q, ..., P, scores, A, M, scale, state, ws, pred)
 *     prr_repair(q, ..., M, scale, state, out)
 * scores, A and M bit for bit; state (fp32, written, not read) = the attention state over P u M, and out
 * (nullable, [batch][num_q_heads][head_dim] fp32) = acc / l, within float32 rounding of those two calls
 * (the partial states merge in another grouping).  With a bf16 or fp8 cache and a top-K that finishes inside
 * the launch (rows of up to 4096 candidate slots, 512-block parts times min(K, 512); longer ones when the
 * launch's scoring workgroups, ceil(N_max / 512) per (sequence, kv head) or ceil(N_max / 1024) as for
 * prr_select_spec, number at most twice the GPU's compute units), it is one launch: the repair of a (sequence, kv head) starts as soon as its M is
 * known, while other units still stream their speculative tiles, and the speculative and repair partial
 * states merge once.  Otherwise it runs the two calls' launches.  Arguments as for prr_select_spec_predict (pred may be
 * NULL).  ws: prr_layer_step_workspace_bytes(kv, num_q_heads, block, topk, P->cap, M->cap), zeroed once
 * like an attention workspace; every call leaves it ready for the next.  In the one-launch form a repair
 * workgroup waits for its unit's M with a bounded wait; the 32-bit word at the start of the workspace's
 * final 256 bytes is a status word that such a workgroup sets to non-zero if it ever gives up (after about
 * a second: that state then lacks the unit's repair).  Workgroups are dispatched in index order, selection
 * first, so it stays zero; the library never clears it. */
size_t prr_layer_step_workspace_bytes(const prr_kv_cache *kv, int32_t num_q_heads, int32_t block, int32_t topk,
                                      int32_t p_cap, int32_t m_cap);

prr_status prr_layer_step(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, const void *meta,
                          prr_score_mode mode, int32_t block, int32_t topk, const prr_block_set *P, double *scores,
                          prr_block_set *A, prr_block_set *M, float scale, prr_attn_state *state, float *out,
                          void *ws, size_t ws_bytes, const prr_predict_args *pred, hipStream_t stream);

/* Speculative block-sparse decode attention over P ([paper] §3 and §4.3, the instrumented speculative
 * kernel that also stores the softmax denominator and running maximum; [paper] §1).  Writes the
 * unnormalised state of every query head over the tokens of its kv head's blocks in P (tokens at or
 * beyond seq_len are masked).  An empty P writes the empty state.  scale is the softmax scale
 * (1/sqrt(head_dim) for standard attention).  ws: prr_attn_workspace_bytes(..., P->cap). */
prr_status prr_spec_attn(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, int32_t block,
                         const prr_block_set *P, float scale, prr_attn_state *out, void *ws,
                         size_t ws_bytes, hipStream_t stream);

/* prr_spec_attn without a workspace argument, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the arrival counters and
 * partial states live in a buffer of PRR_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends (the GPU of `stream`, the current one for the null stream).  The call
 * allocates nothing; it clears the counters with a fill kernel, then runs prr_spec_attn's kernel, with the
 * same results.  Sets whose prr_attn_workspace_bytes(..., P->cap) exceeds the buffer give PRR_EWORKSPACE
 * (nothing enqueued).  Every call on one GPU shares that GPU's buffer: calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race and give wrong results. */
#define PRR_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
prr_status prr_spec_attn_noalloc(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, int32_t block,
                                 const prr_block_set *P, float scale, prr_attn_state *out, hipStream_t stream);

/* Incremental repair ([paper] §4.3, repair via online softmax; [blog] Eq. (6)): folds the tokens of the
 * missed blocks M into `state` in place with the online-softmax recurrence
 *     m' = max(m, m~),  l' = e^{m - m'} l + e^{m~ - m'} l~,  acc' = e^{m - m'} acc + e^{m~ - m'} acc~
 * where (acc~, l~, m~) is the attention of the missed tokens.  Reads the state and the missed K/V once
 * and writes the state once.  An empty M leaves the state bit-for-bit unchanged.  When `out`
 * ([batch][num_q_heads][head_dim] fp32, device) is non-NULL the normalised output acc'/l' is also
 * written (0 where l' = 0).  ws: prr_attn_workspace_bytes(..., M->cap). */
prr_status prr_repair(const void *q, int32_t num_q_heads, const prr_kv_cache *kv, int32_t block,
                      const prr_block_set *M, float scale, prr_attn_state *state, float *out,
                      void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes needed by prr_calibrate for `rows` x `blocks` scores and `n_candidates` candidates. */
size_t prr_calibrate_workspace_bytes(int32_t rows, int32_t blocks, int32_t n_candidates);

/* Online predictor calibration ([paper] §4.2, prefill trajectory and grid search; [blog] Eqs. (4)-(5)).
 * scores [rows][blocks] (fp32, device) is the prefill score matrix: row phi holds the block scores at
 * prefill token phi.  grid [n_candidates][3] (fp64, device) lists candidates (alpha, beta, gamma).  For
 * each candidate the EMA level/trend predictor runs over the rows: row 0 sets level = IS_0, trend = 0;
 * each later row phi is predicted (level + gamma trend), the `topk` highest predictions P_phi are
 * compared with the `topk` highest true scores A_phi of the row (ties to the smaller block index) by
 *     h_phi = sum_{b in P_phi n A_phi} IS_{phi,b} / sum_{b in A_phi} IS_{phi,b}   (0 when A_phi is empty),
 * and the row is absorbed with the update of prr_predict (float64, same operation order, no fused
 * multiply-add).  H[c] = mean of h_phi over phi = 1 .. rows-1 (0 when rows = 1), written to H
 * [n_candidates] (fp64, device); *best (int32, device) = the first candidate with the largest H.
 * Predicted and true sets are exact; H follows float64 rounding of a fixed reduction order.
 * blocks <= 4096, n_candidates <= 4096.  ws: prr_calibrate_workspace_bytes (no initialisation needed). */
prr_status prr_calibrate(const float *scores, int32_t rows, int32_t blocks, int32_t topk, const double *grid,
                         int32_t n_candidates, double *H, int32_t *best, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* Critical-path-aware speculation budget ([paper] §4.4, A.6; Eq. 1: |P| <= delta |A|).  Host code:
 * every pointer is HOST memory, nothing touches the GPU, and both calls are pure functions of their
 * arguments (thread-safe).  The caller profiles once, per configuration, the selection latency and the
 * speculative-attention latency (any one time unit) over a grid of context lengths and budget ratios:
 *   ctx      [n_ctx]             context lengths in tokens, strictly ascending, > 0
 *   t_select [n_ctx]             selection latency at each length
 *   deltas   [n_delta]           budget ratios, strictly ascending, >= 0
 *   t_spec   [n_delta][n_ctx]    speculative-attention latency with |P| = delta K at each length
 * 1 <= n_ctx, n_delta <= PRR_BUDGET_MAX_POINTS; 0 <= degree <= min(PRR_BUDGET_MAX_DEGREE, n_ctx - 1);
 * every value finite.  Violations return PRR_EINVAL and write nothing.
 *
 * prr_budget_fit: ordinary least-squares polynomials of `degree` in x = T / ctx[n_ctx - 1], one for the
 * selection latency and one per delta (the pages estimate lengths outside the grid by polynomial
 * regression).  coef [1 + n_delta][degree + 1]: row 0 selection, row 1 + j delta j; coef[r][k]
 * multiplies x^k.  Solved by Householder QR in float64.
 *
 * prr_budget_choose: the estimates at `context` tokens (> 0): the table row itself when `context` equals
 * a profiled length, else the polynomials of prr_budget_fit (coef from the same table and degree).
 * *choice = the largest j with est_spec[j] <= est_select (the largest delta whose speculative pass ends
 * no later than selection), or -1 when there is none.  est [1 + n_delta] (nullable) receives est_select then
 * est_spec[0 .. n_delta).  *budget_blocks (nullable; then topk is not read) = |P| in blocks for a top-K of
 * `topk` (>= 0) blocks: the largest set Eq. (1), |P| <= delta |A|, admits, floor(delta topk) (float64, with a
 * relative slack of 1e-9 for products that round just below an integer), at the chosen delta, or at the
 * smallest profiled delta when none fits (speculating over fewer blocks leaves more to repair, which is on
 * the critical path too). */
#define PRR_BUDGET_MAX_POINTS 64
#define PRR_BUDGET_MAX_DEGREE 4
prr_status prr_budget_fit(const double *ctx, int32_t n_ctx, const double *t_select, const double *deltas,
                          int32_t n_delta, const double *t_spec, int32_t degree, double *coef);
prr_status prr_budget_choose(const double *ctx, int32_t n_ctx, const double *t_select, const double *deltas,
                             int32_t n_delta, const double *t_spec, int32_t degree, const double *coef,
                             double context, int32_t *choice, double *est, int32_t topk, int32_t *budget_blocks);

/* ---- kernel timing (measurement) ------------------------------------------------------------ */

/* Arms two HIP events (created by the caller with timing enabled, e.g. hipEventCreate; either may be
 * NULL) for the next prr_* call on the calling thread that enqueues GPU work.  That call launches its
 * kernels through hipExtLaunchKernel with these events: `start` takes the start time of its first
 * kernel and `stop` the end time of its last, so hipEventElapsedTime(start, stop) is the GPU time of the
 * call's kernels (for a one-kernel call, that kernel's duration), without the cost of separate event
 * records around them.  The next such call consumes the arming whether or not it launches (a call that
 * fails its argument checks records nothing); the checking mode's set checks are never timed.  Results
 * do not depend on it.  Per thread; always PRR_OK. */
prr_status prr_time_next_kernel(hipEvent_t start, hipEvent_t stop);

/* Human-readable name of a status code (static string). */
const char *prr_strerror(prr_status status);

#ifdef __cplusplus
}
#endif

#endif /* PRR_H */
