/*
 * dsa.h — content-aware top-k block-sparse attention for AMD MI355X (gfx950).
 *
 * C ABI of libdsa.so.  Every entry point takes plain device pointers and
 * sizes, enqueues its kernels on the given HIP stream (a hipStream_t passed
 * as void*; NULL = the default stream) and returns without waiting.
 *
 * Pages cited (by subject, address and section):
 *   [DMA] Dynamic Mask Attention retelling, lsdiaocha.cn/2025/0807/3170092.shtml
 *   [SA]  sparse-attention explainer, studyai.ink/2025/08/30 ("什么是稀疏注意力")
 *   [NSA] Native Sparse Attention summary, news.news/tag/稀疏注意力
 *   [SF]  The Sparse Frontier retelling, techwalker.com/2025/0429/3165971.shtml
 *
 * Conventions shared by every call
 *   - Tensors are passed as bare pointers to dense row-major buffers whose
 *     shapes are given in brackets; there are no strides.  Dense layouts
 *     keep every block of keys (every page) one contiguous run ([NSA] §04:
 *     selected blocks must be read contiguously), which the kernels' block
 *     staging relies on; a caller holding strided views makes them dense
 *     first.  The sizes passed are validated; the buffers' extents are the
 *     caller's contract (the Python binding checks every tensor's shape).
 *     bf16 tensors hold IEEE bfloat16 bits.
 *   - dtype is DSA_F32 or DSA_BF16 and applies to q, k, v and outputs of the
 *     same role; scores, log-sum-exp and gate logits are always float32;
 *     index and count tensors are int32.
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     device memory, keeps no pointer after a call returns and holds no
 *     global mutable state besides a thread-local error message.  Scratch
 *     memory comes only through an explicit workspace argument whose size
 *     the matching *_workspace_size() call returns.
 *   - Errors: a call returns DSA_OK (0) or a negative status.  On
 *     DSA_E_ARG, DSA_E_UNSUPPORTED or DSA_E_WORKSPACE nothing is enqueued and
 *     no output is touched; dsa_last_error() names the offending argument.
 *     DSA_E_HIP reports a failed launch with the HIP error text.
 *   - Device pointers must be 16-byte aligned.
 *   - Results are deterministic: fixed reduction orders, no floating-point
 *     atomics; two identical calls produce identical bits.
 *   - Supported: head dim D in {64, 128}; block / page sizes that are
 *     multiples of 32 (up to 256); bf16 for every call, float32 for the
 *     scoring, selection and prefill calls as well.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_VERSION 101   /* 101: dsa_nsa_select_window_combine */

enum dsa_status {
  DSA_OK = 0,
  DSA_E_ARG = -1,          /* null pointer, bad size, misaligned pointer, bad k/window */
  DSA_E_UNSUPPORTED = -2,  /* dtype / head dim / block size with no compiled kernel */
  DSA_E_WORKSPACE = -3,    /* workspace missing or smaller than *_workspace_size() */
  DSA_E_HIP = -4           /* kernel launch failed (text in dsa_last_error) */
};

enum dsa_dtype { DSA_F32 = 0, DSA_BF16 = 1 };

enum dsa_score_kind {
  DSA_SCORE_POOLED = 0,      /* prefill: mean-pooled query block . mean-pooled key block */
  DSA_SCORE_PAGE_BOUND = 1,  /* decode: per-page min/max key bound */
  DSA_SCORE_POOLED_HEAD = 2  /* prefill, one score per query head (no group sum) */
};

int dsa_version(void);
const char* dsa_status_string(int status);
/* Message of the last failed call on this thread ("" if none). */
const char* dsa_last_error(void);

/*
 * Block / page importance scores ([DMA] §四-§五: a per-position importance
 * score from content, causal mask, then top-k; [SF] §二 page-level decode).
 *
 * kind = DSA_SCORE_POOLED ([SA] "策略" block granularity):
 *   q [B,Hq,n,D], k_or_kmin = K [B,Hkv,n,D] (n = sequence length), kmax = NULL,
 *   block = rows per block, nb = ceil(n/block).
 *   scores [B,Hkv,nb,nb] float32: scores[b,g,i,j] = sum over the Hq/Hkv query
 *   heads h of group g of mean(Q[b,h,block i]) . mean(K[b,g,block j]) for
 *   j <= i, -inf for j > i.  Means, dots and the head sum are accumulated
 *   in float64 and rounded once to float32.  Needs a workspace of
 *   dsa_block_scores_workspace_size() bytes.
 *
 * kind = DSA_SCORE_POOLED_HEAD: as DSA_SCORE_POOLED with every query head
 *   its own selection unit ([DMA] §四: every head gets its own mask):
 *   scores [B,Hq,nb,nb], scores[b,h,i,j] = mean(Q[b,h,block i]) .
 *   mean(K[b,h/(Hq/Hkv),block j]).  Needs a (larger) workspace of
 *   dsa_block_scores_workspace_size() bytes.
 *
 * kind = DSA_SCORE_PAGE_BOUND:
 *   q [B,Hq,D], k_or_kmin = kmin [B,Hkv,n,D], kmax [B,Hkv,n,D] (n = pages),
 *   block ignored.  scores [B,Hkv,n] float32: sum over the group's heads h
 *   and over d of max(q[b,h,d]*kmin[..,d], q[b,h,d]*kmax[..,d]), the
 *   largest q.k any key inside the page's min/max box can reach, accumulated
 *   in float64.  No workspace (pass NULL, 0).
 */
size_t dsa_block_scores_workspace_size(int kind, int B, int Hq, int Hkv, int n, int D, int block);
int dsa_block_scores(int kind, int dtype, const void* q, const void* k_or_kmin, const void* kmax,
                     int B, int Hq, int Hkv, int n, int D, int block,
                     void* workspace, size_t workspace_bytes, float* scores, void* stream);

/*
 * Top-k selection plus local window ([DMA] §五: keep the k highest-weight
 * history positions after the causal mask, all others become -inf).
 *
 * scores [rows, n_q, n_k] float32 (rows = B*Hkv).  For causal != 0, row i
 * of each score matrix draws its top-k from key blocks 0 .. i-n_local and
 * always keeps the window i-n_local+1 .. i (clipped at 0); n_q <= n_k.
 * For causal == 0 the candidates are 0 .. n_k-1-n_local and the window is the
 * last n_local blocks.  Ranking: higher score first, equal scores by lower
 * index, NaN after every number.
 * idx [rows, n_q, k+n_local] int32: the chosen blocks ascending, padded with
 * -1; count [rows, n_q] int32: number of valid entries.
 * Limits: 0 <= k, 0 <= n_local, n_k <= 8192.
 */
int dsa_topk_select(const float* scores, int rows, int n_q, int n_k, int k, int n_local,
                    int causal, int32_t* idx, int32_t* count, void* stream);

/*
 * Exact softmax attention over the selected key blocks only ([DMA] §四-§五:
 * masked positions are skipped, never multiplied; the result equals the
 * masked dense computation).
 *
 * q, out [B,Hq,S,D]; k, v [B,Hkv,S,D]; query head h uses KV head
 * h / (Hq/Hkv).  scale multiplies q.k (normally 1/sqrt(D)).
 * Index mode (idx != NULL): idx [B,Hkv,ceil(S/block),idx_width] ascending
 *   block lists (-1 padded) and count [B,Hkv,ceil(S/block)], as written by
 *   dsa_topk_select; row t of query block i sees keys s <= t of the listed
 *   key blocks.  window must be 0.
 * Window mode (idx == NULL, count == NULL, window > 0): row t sees keys
 *   max(0, t-window+1) .. t ([NSA] §03 sliding branch).
 * lse [B,Hq,S] float32 (may be NULL): natural-log sum of exp of the scaled
 * logits of each row (-inf for a row that sees no key, whose output is 0).
 * Internal math: bf16 products with float32 accumulation (float32 for
 * DSA_F32); out is rounded to dtype.
 */
int dsa_sparse_attn_prefill(int dtype, const void* q, const void* k, const void* v,
                            int B, int Hq, int Hkv, int S, int D,
                            const int32_t* idx, const int32_t* count, int idx_width, int block,
                            int window, float scale, void* out, float* lse, void* stream);

/*
 * dsa_sparse_attn_prefill in index mode with two extensions.
 *  - Selection unit: sel_heads consecutive query heads share one index list
 *    ([DMA] §四 gives every head its own mask; sel_heads = Hq/Hkv is the
 *    per-KV-group sharing of dsa_sparse_attn_prefill, sel_heads = 1 gives
 *    per-query-head lists).  idx [B,Hq/sel_heads,ceil(S/block),idx_width],
 *    count [B,Hq/sel_heads,ceil(S/block)]; query head h uses the lists of
 *    unit h / sel_heads and the K/V of its KV head.
 *  - key_bias [B,Hkv,S] float32 or NULL: an additive term of every key's
 *    logit, scale q.k + key_bias[b,g,s] ([DMA] §五: a kept position's mask
 *    value is its dynamic weight; dsa_dma_weights computes them).  Supported
 *    for DSA_F32, and for bf16 with D = 128, blocks a multiple of 64 and
 *    sel_heads * block >= 256; otherwise DSA_E_UNSUPPORTED.
 * Everything else as dsa_sparse_attn_prefill (lse includes the bias).
 * Errors: DSA_E_ARG unless sel_heads divides Hq/Hkv.
 */
int dsa_sparse_attn_prefill_ex(int dtype, const void* q, const void* k, const void* v,
                               int B, int Hq, int Hkv, int S, int D,
                               const int32_t* idx, const int32_t* count, int idx_width,
                               int block, int sel_heads, const float* key_bias, float scale,
                               void* out, float* lse, void* stream);

/*
 * Value-driven dynamic weights ([DMA] §四-§五: a weight per history position
 * from the value content, delta = exp(tau(v Delta) x A), tau non-negative).
 * v [B,Hkv,S,D] (dtype), proj [Hkv,D] float32 (Delta, one projection per KV
 * head), gain [Hkv] float32 (A).  Writes weights [B,Hkv,S] float32:
 *   weights[b,g,s] = exp(gain[g] * softplus(v[b,g,s,:] . proj[g,:])),
 * softplus(x) = log(1 + e^x), float32 arithmetic.  If block_scores is not
 * NULL, also writes block_scores [B,Hkv,nb,nb] (nb = ceil(S/block)): for
 * j <= i the largest weight of key block j, -inf above the diagonal — the
 * input dsa_topk_select expects for causal block selection.
 */
int dsa_dma_weights(int dtype, const void* v, int B, int Hkv, int S, int D, const float* proj,
                    const float* gain, int block, float* weights, float* block_scores,
                    void* stream);

/*
 * Gradients of dsa_sparse_attn_prefill in index mode ([DMA] §四-§五: the
 * masked computation stays differentiable; a position the mask removes gets
 * exactly zero gradient, the kept positions the ordinary softmax gradient).
 * The index lists are constants of the backward: selection is a discrete
 * choice and passes no gradient.
 *
 * q, out, dout, dq [B,Hq,S,D]; k, v, dk, dv [B,Hkv,S,D]; idx, count,
 * idx_width, block and scale exactly as given to the forward; out and lse
 * [B,Hq,S] are the forward's results for these inputs.  With P the
 * forward's softmax weights (recomputed from lse), dP = dout . v and
 * Dt = dout . out per row:
 *   dS = P (dP - Dt),  dq = scale dS k,  dk = scale dS^T q,  dv = P^T dout,
 * summed over every row of the group's query heads that sees the key.
 * Keys that no row sees get zero.  Every output element is written.
 * Internal math: bf16 products (P and dS rounded to bf16) with float32
 * accumulation; sums run in a fixed order, so results are reproducible.
 * Needs a workspace of dsa_sparse_attn_prefill_backward_workspace_size()
 * bytes (row terms and the inverted block lists); its contents on entry do
 * not matter.  bf16 only; idx rows strictly ascending within count.
 */
size_t dsa_sparse_attn_prefill_backward_workspace_size(int B, int Hq, int Hkv, int S, int D,
                                                       int block);
int dsa_sparse_attn_prefill_backward(int dtype, const void* q, const void* k, const void* v,
                                     const void* out, const float* lse, const void* dout,
                                     int B, int Hq, int Hkv, int S, int D,
                                     const int32_t* idx, const int32_t* count, int idx_width,
                                     int block, float scale, void* workspace,
                                     size_t workspace_bytes, void* dq, void* dk, void* dv,
                                     void* stream);

/*
 * Per-page key summaries for decode ([DMA] §三 per-block cache summaries;
 * [SF] §四 page granularity): kmin/kmax [B,Hkv,L/page,D] = element-wise
 * minimum / maximum of K [B,Hkv,L,D] over each page (exact).  L % page == 0.
 */
int dsa_page_minmax(int dtype, const void* k, int B, int Hkv, int L, int D, int page,
                    void* kmin, void* kmax, void* stream);

/*
 * Single-query decode attention over the selected pages of a full KV cache
 * ([SF] §二-§四: the cache is kept whole, only selected pages are read).
 *
 * q, out [B,Hq,D]; k_cache, v_cache [B,Hkv,L,D]; idx [B,Hkv,idx_width]
 * page lists (ascending, -1 padded), count [B,Hkv]; page = tokens per page.
 * The query follows all L cached tokens, so every token of a selected page
 * is visible.  Pages are split over workgroups whose partial results
 * (max, sum, weighted values) are merged in a fixed order.  bf16 only;
 * L % page == 0, page in {32, 64, 128, 256, 512}, Hq/Hkv in {1,2,4,8}.
 */
size_t dsa_sparse_attn_decode_workspace_size(int B, int Hq, int Hkv, int idx_width, int page,
                                             int D);
int dsa_sparse_attn_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
                           int B, int Hq, int Hkv, int L, int D,
                           const int32_t* idx, const int32_t* count, int idx_width, int page,
                           float scale, void* workspace, size_t workspace_bytes,
                           void* out, void* stream);

/*
 * dsa_sparse_attn_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, kernels and results, with the partial
 * results kept in a scratch array of DSA_DECODE_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends (its
 * address is looked up on a device's first call).  Nothing is allocated or
 * freed by the call.  A decode whose partial results exceed the scratch
 * (more than dsa_sparse_attn_decode_workspace_size() would ask for) returns
 * DSA_E_WORKSPACE.  Every partial result read in a call is written earlier
 * in the same call, so the scratch needs no clearing; but all calls on one
 * GPU share it, so calls that overlap in time on one GPU (different streams
 * or threads) race and must be serialised by the caller.
 */
#define DSA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
int dsa_sparse_attn_decode_noalloc(int dtype, const void* q, const void* k_cache,
                                   const void* v_cache, int B, int Hq, int Hkv, int L, int D,
                                   const int32_t* idx, const int32_t* count, int idx_width,
                                   int page, float scale, void* out, void* stream);

/*
 * Paged KV cache for serving ([SF] §二-§四: the whole cache is kept and a
 * decode step reads only the pages it selects; here the cache of a whole
 * batch lives in one pool of pages).
 *
 * Layout: k_pool, v_pool [n_pool, Hkv, page, D] bf16; kmin, kmax
 * [n_pool, Hkv, D] bf16 (per pool page, the element-wise min / max of the
 * keys written to it so far); page_table [B, max_pages] int32: logical page
 * p of sequence b (tokens p*page .. p*page+page-1) is pool page
 * page_table[b*max_pages + p]; seq_len [B] int32: tokens of sequence b.
 * Pool pages are owned by the caller; two sequences must not share one.
 *
 * dsa_paged_append: writes token seq_len[b] of every sequence (k_new, v_new
 * [B,Hkv,D]) into its page, folds its key into the page's kmin/kmax (the
 * page's first token sets them) and increments seq_len[b].  A sequence whose
 * page slot (>= max_pages) or pool id (outside [0, n_pool)) is out of range
 * is left unchanged.
 *
 * dsa_paged_page_scores: scores [B,Hkv,max_pages] float32, the page bound of
 * dsa_block_scores(DSA_SCORE_PAGE_BOUND) for logical pages below
 * ceil(seq_len[b]/page) (read through the page table, float64 sums), -inf
 * for the rest.  Feed it to dsa_topk_select (causal = 0, n_local = 0).
 *
 * dsa_paged_decode: as dsa_sparse_attn_decode over the pool: idx
 * [B,Hkv,idx_width] logical pages, count [B,Hkv]; only tokens below
 * seq_len[b] are attended, selected pages past the length hold nothing.
 * Workspace: dsa_sparse_attn_decode_workspace_size(B, Hq, Hkv, idx_width,
 * page, D) bytes.  bf16 only; page in {32,64,128,256,512}, Hq/Hkv in
 * {1,2,4,8}.
 */
int dsa_paged_append(int dtype, const void* k_new, const void* v_new, int B, int Hkv, int D,
                     int page, int max_pages, const int32_t* page_table, int32_t* seq_len,
                     int n_pool, void* k_pool, void* v_pool, void* kmin, void* kmax,
                     void* stream);
int dsa_paged_page_scores(int dtype, const void* q, const void* kmin, const void* kmax, int B,
                          int Hq, int Hkv, int D, int page, int max_pages,
                          const int32_t* page_table, const int32_t* seq_len, int n_pool,
                          float* scores, void* stream);
int dsa_paged_decode(int dtype, const void* q, const void* k_pool, const void* v_pool, int B,
                     int Hq, int Hkv, int D, int page, int max_pages, const int32_t* page_table,
                     const int32_t* seq_len, int n_pool, const int32_t* idx, const int32_t* count,
                     int idx_width, float scale, void* workspace, size_t workspace_bytes,
                     void* out, void* stream);

/*
 * Compressed keys / values for the coarse branch ([NSA] §03 "compressed
 * attention": a quick scan of summaries of the history).
 * ck, cv [B,Hkv,n_cmp,D] with n_cmp = (S-len)/stride + 1:
 * ck[c] = mean(K[c*stride .. c*stride+len-1]): float64 sum, divided by len
 * and rounded once to bf16 (nearest, ties to even), so a summary is the
 * exactly rounded mean of its keys (of its values for cv).
 */
int dsa_nsa_compress(int dtype, const void* k, const void* v, int B, int Hkv, int S, int D,
                     int len, int stride, void* ck, void* cv, void* stream);

/*
 * Compressed-branch attention and the block scores that drive selection
 * ([NSA] §03).  q, out [B,Hq,S,D]; ck, cv [B,Hkv,n_cmp,D].
 * Row t sees summary c iff c*stride + len - 1 <= t; a row that sees none
 * gets out = 0 and lse = -inf.  lse [B,Hq,S] float32 is required.
 * block_scores [B,Hkv,nb,nb] float32 (nb = ceil(S/sel_block)), may be NULL:
 * for query block i and key block j, the branch probability mass of the
 * summaries overlapping block j, each split in proportion to its overlap
 * with the block, summed over the block's rows and the group's heads and
 * divided by rows x heads (values in [0,1]; 0 for j > i).
 * Limits: n_cmp <= 8192 (else DSA_E_UNSUPPORTED).
 */
int dsa_nsa_cmp_attn(int dtype, const void* q, const void* ck, const void* cv,
                     int B, int Hq, int Hkv, int S, int D, int len, int stride, int sel_block,
                     float scale, void* out, float* lse, float* block_scores, void* stream);

/*
 * Per-token selection for the selected branch ([NSA] §03 at the granularity
 * of the original method: each query token ranks the key blocks for its own
 * KV group from its compressed-branch attention, and every query head of
 * the group then attends to that token's blocks).
 *
 * dsa_nsa_cmp_token_scores: scores [B,Hkv,S,nb] float32 (nb =
 * ceil(S/sel_block)); for token t and key block j, the compressed-branch
 * probability of the summaries overlapping block j, each split in
 * proportion to its overlap, averaged over the group's query heads (a row
 * that sees a summary sums to 1; blocks after t's own block get 0).  q
 * [B,Hq,S,D] and ck [B,Hkv,n_cmp,D] bf16 as given to dsa_nsa_cmp_attn, lse
 * [B,Hq,S] the log-sum-exp it wrote.  Limits: Hq/Hkv <= 16;
 * (sel_block + len - 2) / stride <= 31 (a block overlaps at most 32
 * summaries); else DSA_E_UNSUPPORTED.
 *
 * dsa_topk_select_tokens: as dsa_topk_select with causal candidates per
 * token: row t of each S-row score matrix [rows, S, n_k] draws its top-k
 * from blocks 0 .. t/block - n_local and keeps the window
 * t/block - n_local + 1 .. t/block.  idx [rows, S, k+n_local], count
 * [rows, S].  Needs ceil(S/block) <= n_k <= 8192.
 *
 * dsa_sparse_attn_tokens: out [B,Hq,S,D] bf16: row t of every query head of
 * group g attends to the keys s <= t of the key blocks (block tokens each)
 * listed in idx [B,Hkv,S,idx_width] (ascending, -1 padded) with count
 * [B,Hkv,S]; lse [B,Hq,S] float32 may be NULL (as dsa_sparse_attn_prefill).
 * Lists hold distinct blocks (as dsa_topk_select_tokens writes them); keys
 * of a listed block outside [0, t] are masked.  Limits: bf16, D = 128,
 * Hq/Hkv <= 16, block = 64, idx_width <= 64 (else DSA_E_UNSUPPORTED).
 */
int dsa_nsa_cmp_token_scores(int dtype, const void* q, const void* ck, const float* lse, int B,
                             int Hq, int Hkv, int S, int D, int len, int stride, int sel_block,
                             float scale, float* scores, void* stream);
int dsa_topk_select_tokens(const float* scores, int rows, int S, int n_k, int k, int n_local,
                           int block, int32_t* idx, int32_t* count, void* stream);
int dsa_sparse_attn_tokens(int dtype, const void* q, const void* k, const void* v, int B, int Hq,
                           int Hkv, int S, int D, const int32_t* idx, const int32_t* count,
                           int idx_width, int block, float scale, void* out, float* lse,
                           void* stream);

/*
 * Gated combine of the three branches ([NSA] §03: each token and head
 * weighs the compressed, selected and sliding outputs):
 * out[b,h,t] = sigmoid(z0)*o_cmp + sigmoid(z1)*o_sel + sigmoid(z2)*o_win with
 * z = gate_logits[b,t,h,0..2] ([B,S,Hq,3] float32).  o_*, out [B,Hq,S,D].
 */
int dsa_nsa_combine(int dtype, const void* o_cmp, const void* o_sel, const void* o_win,
                    const float* gate_logits, int B, int Hq, int S, int D, void* out,
                    void* stream);

/*
 * The sliding branch and the gated combine in one call ([NSA] §03): the
 * window attention of dsa_sparse_attn_prefill (window mode, 64-token query
 * blocks) whose epilogue forms out = sigmoid(z0)*o_cmp + sigmoid(z1)*o_sel +
 * sigmoid(z2)*o_win from its own float32 result, so o_win never goes through
 * memory.  Same layouts as dsa_nsa_combine; q, k, v as dsa_sparse_attn_prefill.
 * Rounded once to bf16 (the two-call path rounds o_win first).  Limits: bf16,
 * D = 128, Hq/Hkv >= 4, window <= 8000 (else DSA_E_UNSUPPORTED).
 */
int dsa_nsa_window_combine(int dtype, const void* q, const void* k, const void* v, int B, int Hq,
                           int Hkv, int S, int D, int window, float scale, const void* o_cmp,
                           const void* o_sel, const float* gate_logits, void* out,
                           void* stream);

/*
 * The selected and sliding branches and the gated combine in one call
 * ([NSA] §03: the three branches share each token's queries; [NSA] §04:
 * work is arranged around the query rows that stay on chip).  Each 64k-token
 * query block of each KV group holds its query rows once: its rows attend to
 * the blocks listed in idx/count (as dsa_sparse_attn_prefill in index mode,
 * block = sel_block), that output is rounded to bf16, then the same rows
 * attend to the token window t-window+1 .. t (as window mode), and
 * out = sigmoid(z0)*o_cmp + sigmoid(z1)*o_sel + sigmoid(z2)*o_win is formed in
 * float32 from the window result and rounded once.  With sel_block = 64
 * equal, bit for bit, to dsa_sparse_attn_prefill (index mode) into o_sel
 * followed by dsa_nsa_window_combine; neither o_sel nor o_win goes through
 * memory.
 * q [B,Hq,S,D], k, v [B,Hkv,S,D], idx [B,Hkv,nb,idx_width] (ascending, -1
 * padded, nb = ceil(S/sel_block)), count [B,Hkv,nb] int32, o_cmp and out
 * [B,Hq,S,D], gate_logits [B,S,Hq,3] float32; all device buffers owned by the
 * caller; no workspace.  Limits: bf16, D = 128, sel_block a multiple of 64,
 * Hq/Hkv * sel_block >= 256, idx_width * sel_block/64 + (window +
 * sel_block)/64 + 2 <= 128 (else DSA_E_UNSUPPORTED).
 */
int dsa_nsa_select_window_combine(int dtype, const void* q, const void* k, const void* v, int B,
                                  int Hq, int Hkv, int S, int D, const int32_t* idx,
                                  const int32_t* count, int idx_width, int sel_block, int window,
                                  float scale, const void* o_cmp, const float* gate_logits,
                                  void* out, void* stream);

/*
 * Measurement helper, not a step of the method: reads src [bytes] (device,
 * 16-byte aligned, bytes a positive multiple of 16) once with 16-byte
 * streaming loads, each workgroup taking whole 16 KiB runs (four loads in
 * flight per lane), and writes sink[w] = XOR of the 32-bit
 * words workgroup w read, for w < dsa_read_stream_sink_words() (the other
 * sink words are untouched).  The XOR of all sink words is the XOR of every
 * word of src.  Its rate is the achievable HBM read bandwidth that the
 * memory-bound decode calls ([SF] §四: read only the selected pages) are
 * compared with.  Errors: DSA_E_ARG (pointers, size), DSA_E_WORKSPACE (sink
 * too small).
 */
size_t dsa_read_stream_sink_words(void);
int dsa_read_stream(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
