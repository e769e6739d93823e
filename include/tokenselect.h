/*
 * tokenselect.h - C ABI of the MI355X (gfx950) decode-step hot path of
 * TokenSelect-style dynamic token-level KV-cache selection.
 *
 * Per layer and per request a decode step
 *   0. checks the Selection Cache (cosine of the concatenated query against the
 *      query stored at the last reselection),
 *   1. scores the current query against every cached key of its KV head
 *      (paged pool, GQA: query head h reads KV head h / (H / H_kv)),
 *   2. normalises each head's scores by a softmax over all N cached tokens,
 *   3. sums the normalised scores over the H query heads (head soft vote),
 *   4. keeps the top_k positions of the vote, united with the n_local most
 *      recent positions,
 *   5. runs scaled-dot-product attention over only those positions.
 *
 * Sources: "TokenSelect: Efficient Long-Context Inference and Length
 * Extrapolation for LLMs via Dynamic Token-Level KV Cache Selection"
 * (deepnotes page): selective sparse attention formalisation (SDPA over the
 * selected keys plus the current one), head soft vote equation, Selection Cache
 * (appendix Algorithm 1), Paged Dot Product Kernel (appendix Algorithm 2).
 * Blog review of the same paper: section 3 (Fig. 4 data flow: only indices move,
 * the paged KV stays in place), section 3.2 (Algorithm 1), section 4.2 (budget of
 * selected plus local tokens).
 *
 * Conventions shared by every entry point
 *   - Array arguments are DEVICE pointers unless stated; the structs are host
 *     memory read during the call only. The library keeps no pointer after a
 *     call returns and allocates no memory: the caller owns every buffer,
 *     including the workspace.
 *   - Work is enqueued on `stream` in order; no call synchronises the host with
 *     the device. Calls are reentrant; calls that share a workspace must be
 *     ordered on one stream.
 *   - Host-side validation runs before any launch. On failure nothing is
 *     launched and a non-zero ts_status is returned; tokenselect_last_error()
 *     gives a message (thread-local). A failed launch returns TS_ERR_DEVICE.
 *   - Device-side contract (not checked by the steps; tokenselect_validate checks
 *     it on request): every block-table entry a request
 *     reaches (pages [0, ceil(N_r / page_size))) is a valid pool page;
 *     0 <= N_r <= block_table_stride * page_size; sum of N_r <=
 *     shape.max_total_tokens; every selected index lies in [0, N_r). A request
 *     with N_r = 0 selects nothing (sel_count 0) and its attention output is 0.
 *
 * Layouts
 *   q          [batch][H][d]                      element type `dtype`
 *   k_pool     [num_pages][H_kv][page_size][d]    element type `dtype`
 *   v_pool     same as k_pool
 *   block_table int32 [batch][block_table_stride]: logical page p of request r
 *              is pool page block_table[r * stride + p]; token i of request r
 *              is slot i % page_size of logical page i / page_size.
 *   seq_lens   int32 [batch]: N_r, cached tokens including the current one.
 *   Ragged token axis: request r owns positions [off_r, off_r + N_r) with
 *   off_r = N_0 + ... + N_{r-1} (computed on the device from seq_lens).
 *   logits     fp32: request r, query head h = g * G + j (G = H / H_kv), token i at
 *              off_r * H + (g * N_r + i) * G + j, i.e. [H_kv][N_r][G] per request.
 *   head_stats fp32 [batch][H][2]: (M_h, Z_h) = (max_i z, sum_i exp(z - M_h)).
 *   vote       fp32 log2 of the head soft vote, log2 v_i: request r, token i at
 *              off_r + i (finite where the linear vote would underflow fp32).
 *   sel_idx    int32 [batch][top_k]: the TopK positions of request r, ascending,
 *              in the first sel_count[r] = min(top_k, N_r) entries (the top-p
 *              budget instead when ts_select.top_p > 0).
 *   out        [batch][H][d] element type `dtype` (bf16 results are rounded to
 *              nearest even from fp32 accumulators).
 */
#ifndef TOKENSELECT_H
#define TOKENSELECT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TS_OK = 0,
  TS_ERR_INVALID_ARG = 1,   /* null pointer, inconsistent sizes, negative values */
  TS_ERR_UNSUPPORTED = 2,   /* valid but not built: head_dim != 128, page_size != 16, G > 8 ... */
  TS_ERR_WORKSPACE = 3,     /* ws_bytes smaller than tokenselect_workspace_size() */
  TS_ERR_DEVICE = 4         /* a HIP launch failed; the HIP error text is in last_error */
} ts_status;

typedef enum { TS_F32 = 0, TS_BF16 = 1 } ts_dtype;

/* Problem shape (host struct). */
typedef struct {
  int32_t num_q_heads;        /* H, >= 1                                         */
  int32_t num_kv_heads;       /* H_kv, >= 1, H % H_kv == 0, H / H_kv <= 8         */
  int32_t head_dim;           /* d; the library supports 128                    */
  int32_t page_size;          /* tokens per page; the library supports 16       */
  int32_t batch;              /* requests, 1 ... 1024                           */
  int32_t block_table_stride; /* int32 entries per block-table row, >= 1        */
  int64_t max_total_tokens;   /* upper bound of sum_r N_r (sizes grids/workspace) */
  int32_t dtype;              /* ts_dtype of q, K/V pools and out               */
} ts_shape;

/* Selection parameters (host struct). */
typedef struct {
  int32_t top_k;              /* k >= 1: TopK budget of the head soft vote       */
  int32_t n_local;            /* L >= 0: most recent positions always attended;
                                 the decode window is [N_r - max(L, 1), N_r), so
                                 the current token is attended even with L = 0  */
  float score_scale;          /* multiplies <q, k> before the selection softmax;
                                 1.0 is the printed vote equation (raw logits)  */
  float attn_scale;           /* SDPA scale, normally 1/sqrt(d)                  */
  double cos_threshold;       /* theta: reuse the cached selection iff cos >= theta */
  double top_p;               /* 0: fixed TopK budget. 0 < p <= 1: dynamic top-p budget,
                                 the fewest largest votes holding at least p of the
                                 vote mass, capped at top_k (RTPurbo post, dynamic
                                 token selection and its histogram top-p kernel;
                                 UniPrefill page, minimal set holding 99% of the
                                 importance). Vote masses are taken as the integers
                                 rint(v * 2^40), so the budget is exact and
                                 deterministic; sel_count[r] receives it. */
} ts_select;

/* Selection Cache state, caller-owned device buffers kept across steps
   (deepnotes appendix Algorithm 1: C_Q, C_T and the first-query flag). */
typedef struct {
  void* cached_q;             /* [batch][H * d], element type dtype: C_Q         */
  int32_t* cached_idx;        /* [batch][top_k]: C_T, the TopK of the last miss  */
  int32_t* cached_count;      /* [batch]: entries of cached_idx in use           */
  int32_t* valid;             /* [batch]: 0 = no cached query (forces a miss);
                                 the caller zeroes it to reset a request         */
} ts_cache;

/* Bytes of workspace every entry point below needs for `shape` and `sel`
   (the decode step's need, which covers the others). Returns 0 if the shape or
   the selection parameters are invalid. */
size_t tokenselect_workspace_size(const ts_shape* shape, const ts_select* sel);

/* Steps 1-2. Paged dot product z[h][i] = score_scale * <q_h, K_{h/G}[i]> for every
   cached token i < N_r of every request (deepnotes appendix Algorithm 2), and the
   per-head softmax statistics (M_h, Z_h) over all N_r tokens (head soft vote
   equation). `logits` holds max_total_tokens * H floats, `head_stats`
   batch * H * 2 floats, or is NULL: then only the logits are computed (one kernel;
   the statistics of step 2 are not folded). */
ts_status tokenselect_score(const ts_shape* shape, const ts_select* sel,
                            const void* q, const void* k_pool,
                            const int32_t* block_table, const int32_t* seq_lens,
                            float* logits, float* head_stats,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Steps 3-4 (TopK part). Head soft vote v_i = sum_h exp(z[h][i] - M_h) / Z_h
   (deepnotes head soft vote equation), computed as lv_i = log2 v_i by a
   log-sum-exp over the heads, and TopK over all N_r positions: the k largest
   votes (largest lv), ties to the lower position, written ascending to
   sel_idx[r][0 .. sel_count[r]) with sel_count[r] = min(top_k, N_r) (with top_p > 0:
   the top-p budget, at most min(top_k, N_r)). `vote`
   (max_total_tokens floats) receives lv and may be NULL; then lv stays in the
   workspace. The local window is not written: step 5 adds it. */
ts_status tokenselect_vote_topk(const ts_shape* shape, const ts_select* sel,
                                const float* logits, const float* head_stats,
                                const int32_t* seq_lens, float* vote,
                                int32_t* sel_idx, int32_t* sel_count,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* Step 5. Attention of every query head over S_r = TopK_r united with
   [max(0, N_r - max(n_local, 1)), N_r), without duplicates: out[r][h] = sum_{i in S_r}
   softmax_i(attn_scale * <q_h, K_{h/G}[i]>) V_{h/G}[i] (deepnotes selective
   sparse attention formalisation: the selected keys plus the current one, so the
   current token N_r - 1 is in S_r even with n_local = 0). The first sel_count[r]
   entries of row r must be strictly ascending (a repeated entry would be attended
   twice); entries outside [0, N_r) are ignored. tokenselect_validate_selection checks
   this on request. A request with N_r = 0 has an empty S_r and gets out[r] = 0; its
   block-table row is not read. */
ts_status tokenselect_sparse_attn(const ts_shape* shape, const ts_select* sel,
                                  const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  const int32_t* sel_idx, const int32_t* sel_count,
                                  void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Steps 0-5 for one decode step of every request, with no host synchronisation.
   Per request: hit = valid && |Q| > 0 && |C_Q| > 0 && cos(Q, C_Q) >= theta, with
   Q the H*d query elements and the cosine accumulated in fp64 (deepnotes appendix
   Algorithm 1). On a miss steps 1-4 run, C_Q <- Q, C_T <- TopK, valid <- 1;
   on a hit C_T is reused. Step 5 always runs with the current N_r window.
   hit[r] (device int32 [batch]) receives 1 for a reuse, 0 for a reselection. */
ts_status tokenselect_decode_step(const ts_shape* shape, const ts_select* sel,
                                  const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  const ts_cache* cache, int32_t* hit, void* out,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of the static device scratch behind tokenselect_decode_step_noalloc (64 MiB):
   enough for tokenselect_workspace_size() of e.g. 32 query heads over ~480K cached
   tokens in total. */
#define TS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* tokenselect_decode_step without a workspace argument, for callers that cannot
   allocate device memory (code under HIP graph capture, tight serving loops,
   harnesses that forbid hipMalloc). Same arguments, results and errors as
   tokenselect_decode_step; the workspace is a static device array of
   TS_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the
   process ends (its address is looked up on the first call on a device). The call
   allocates nothing. A shape whose tokenselect_workspace_size() exceeds
   TS_NOALLOC_SCRATCH_BYTES is rejected with TS_ERR_WORKSPACE before any launch.
   Every call on one GPU uses that GPU's one scratch array: calls that may overlap
   on one device (several streams, several host threads) race and must be ordered
   by the caller; the scratch keeps no state from one call to the next that a later
   call relies on. */
ts_status tokenselect_decode_step_noalloc(const ts_shape* shape, const ts_select* sel,
                                          const void* q, const void* k_pool, const void* v_pool,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          const ts_cache* cache, int32_t* hit, void* out,
                                          hipStream_t stream);

/* ---------------------------------------------------------------- chunk-wise prefill
   A prefill chunk of request r is its c_r newest tokens: their K/V are already in
   the pool at positions [P_r, P_r + c_r) with P_r = N_r - c_r (seq_lens[r] = N_r
   counts the chunk). The chunk selects once from the mean of its c_r queries over
   the past positions [0, P_r), and chunk query j attends
     S_j = TopK_r  united with  [max(0, P_r - n_local), P_r + j]
   (the window of n_local positions before the chunk plus the chunk's causal part).
   Sources: deepnotes page, selection frequency of the prefill stage (the c x d
   query block of a chunk is averaged and the mean goes through the selection
   function) and the selective sparse attention formalisation; blog review section
   3.2 (chunk-wise selection in prefill: the chunk shares one selection).
   Layouts (in addition to the decode ones):
     q_chunk    [batch][max_chunk][H][d] element type dtype; rows j >= c_r unused
     chunk_lens int32 [batch] device: c_r, 1 <= c_r <= min(max_chunk, N_r)
     out        [batch][max_chunk][H][d] element type dtype; rows j >= c_r untouched
     sel_idx    int32 [batch][top_k]: TopK over the past, ascending, sel_count[r] =
                min(top_k, P_r) entries (0 for a first chunk, P_r = 0)
   Out-of-contract chunk lengths are clamped on the device (no access leaves the
   request's pages; results are then unspecified). The decode entry points' rules on
   pointers, streams, ownership and errors apply. */

/* Workspace bytes of the prefill entry points for chunks of up to max_chunk
   tokens (1 <= max_chunk <= shape->max_total_tokens: both are capacities, and a
   chunk's tokens are among the batch's); 0 if the arguments are invalid. */
size_t tokenselect_prefill_workspace_size(const ts_shape* shape, const ts_select* sel,
                                          int32_t max_chunk);

/* Selection of a chunk: qbar_h = (1/c_r) sum_j q_chunk[r][j][h] (fp64 sum, rounded
   once to fp32), then steps 1-4 of the decode path with qbar over [0, P_r): logits
   z = score_scale * <qbar_h, K>, per-head (M_h, Z_h), log2 head soft vote and TopK.
   logits, head_stats and vote are optional outputs in the decode layouts with
   N_r replaced by P_r (NULL keeps them in the workspace). */
ts_status tokenselect_prefill_select(const ts_shape* shape, const ts_select* sel, int32_t max_chunk,
                                     const void* q_chunk, const int32_t* chunk_lens,
                                     const void* k_pool, const int32_t* block_table,
                                     const int32_t* seq_lens, float* logits, float* head_stats,
                                     float* vote, int32_t* sel_idx, int32_t* sel_count, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* Chunk attention: out[r][j][h] = sum_{i in S_j} softmax_i(attn_scale * <q_h, K_{h/G}[i]>)
   V_{h/G}[i] for every chunk query j < c_r, given TopK_r in sel_idx / sel_count
   (ascending, entries in [0, P_r)). Runs on the matrix cores (bf16: products in
   bf16 with fp32 accumulation, probabilities rounded to bf16 for the value product;
   fp32: fp32 throughout). */
ts_status tokenselect_chunk_attn(const ts_shape* shape, const ts_select* sel, int32_t max_chunk,
                                 const void* q_chunk, const int32_t* chunk_lens,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* sel_idx, const int32_t* sel_count, void* out,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* One prefill chunk: tokenselect_prefill_select (TopK into sel_idx / sel_count)
   followed by tokenselect_chunk_attn, with no host synchronisation. */
ts_status tokenselect_prefill_chunk(const ts_shape* shape, const ts_select* sel, int32_t max_chunk,
                                    const void* q_chunk, const int32_t* chunk_lens,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    int32_t* sel_idx, int32_t* sel_count, void* out, void* ws,
                                    size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- selection-function ablations
   Alternatives to the head soft vote, over the decode logits and head statistics
   of tokenselect_score (deepnotes page, selection-function design and the token-level
   motivation, Fig. 2b; blog review section 2). Each writes a TopK in the decode
   sel_idx / sel_count layout (ascending, ties to the lower position):
     TS_SELECT_SOFT_VOTE  the head soft vote (same result as tokenselect_vote_topk);
     TS_SELECT_NAIVE_TOPK a position scores its largest raw logit over the H heads;
     TS_SELECT_HARD_VOTE  every head takes its own TopK(top_k) of its logits, a position
                          scores the number of heads that picked it, then TopK of the
                          counts; needs batch * H <= 1024;
     TS_SELECT_BLOCK      blocks of `block` positions score the sum of their tokens'
                          votes, as log2 sum 2^lv (fp64 in position order, rounded once
                          to fp32); the max(1, top_k / block) best blocks are expanded
                          to their positions (sel_count counts them; a request's last
                          block may be short).
   `score` (optional, may be NULL) receives what the final TopK ran on: log2 votes,
   max logits, or head counts ([sum N_r] floats), or block scores ([sum ceil(N_r / block)]).
   top_p must be 0. */
typedef enum {
  TS_SELECT_SOFT_VOTE = 0,
  TS_SELECT_NAIVE_TOPK = 1,
  TS_SELECT_HARD_VOTE = 2,
  TS_SELECT_BLOCK = 3
} ts_select_fn;

/* Workspace bytes of tokenselect_select_ablation; 0 if the arguments are invalid. */
size_t tokenselect_ablation_workspace_size(const ts_shape* shape, const ts_select* sel, int32_t fn,
                                           int32_t block);

ts_status tokenselect_select_ablation(const ts_shape* shape, const ts_select* sel, int32_t fn,
                                      int32_t block, const float* logits, const float* head_stats,
                                      const int32_t* seq_lens, float* score, int32_t* sel_idx,
                                      int32_t* sel_count, void* ws, size_t ws_bytes,
                                      hipStream_t stream);

/* Check of the device-side contract above, for callers that want it before a step
   (the other entry points trust these inputs): for every request r, 0 <= N_r <=
   block_table_stride * page_size, and every block-table entry it reaches (pages
   [0, min(ceil(N_r / page_size), block_table_stride))) lies in [0, num_pool_pages).
   Entries are only read, never followed. `report` (device uint64[4], caller-owned,
   8-byte aligned) receives: [0] the number of violations, [1] the smallest key
   (r << 32) | p over them, p the page index or 0xffffffff for a length violation
   (all ones if there is none), [2] the number of length violations, [3] the sum of
   the non-negative N_r (compare it with max_total_tokens). Only batch,
   block_table_stride and page_size of `shape` are used. Asynchronous on `stream`:
   read the report after synchronising. */
ts_status tokenselect_validate(const ts_shape* shape, const int32_t* block_table,
                               const int32_t* seq_lens, int64_t num_pool_pages, uint64_t* report,
                               hipStream_t stream);

/* Check of a selection handed to tokenselect_sparse_attn (or kept as Selection
   Cache state), for callers that build or keep selections themselves: for every
   request r, 0 <= sel_count[r] <= min(top_k, max(N_r, 0)) and the first sel_count[r]
   entries of sel_idx[r] lie in [0, N_r) and are strictly ascending. `report` (device
   uint64[4], caller-owned, 8-byte aligned) receives: [0] the number of violations,
   [1] the smallest key (r << 32) | e over them, e the entry index or 0xffffffff for a
   count violation (all ones if there is none), [2] the number of count violations,
   [3] the sum of the in-range counts. Only batch of `shape` and top_k of `sel` are
   used. Asynchronous on `stream`: read the report after synchronising. */
ts_status tokenselect_validate_selection(const ts_shape* shape, const ts_select* sel,
                                         const int32_t* seq_lens, const int32_t* sel_idx,
                                         const int32_t* sel_count, uint64_t* report,
                                         hipStream_t stream);

/* Static text for a status code. */
const char* tokenselect_status_string(ts_status status);

/* Message of the last failed call on this thread ("" if none). */
const char* tokenselect_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TOKENSELECT_H */
