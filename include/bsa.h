/*
 * bsa.h -- C ABI of libbsa: query-aware block-sparse attention over a chunked,
 * paged GQA KV cache, hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * The method (cited by page title and section):
 *  [P1] "Sparse Attention for Web Agents -- Offline Replay Records",
 *       section "The comparison": chunk the KV cache, score every chunk against
 *       the current query, keep the top-scoring chunks and attend only to them;
 *       chunking is fixed 16-token pages (Quest, BlockSparse) or variable
 *       16-256-token chunks (TSA); scoring is the per-dimension min/max
 *       envelope (TSA, Quest) or the key centroid (BlockSparse); the budget is
 *       page_size x top_k attended tokens.
 *  [P2] "webarena" dataset README, section "Method configurations at a glance":
 *       ratio budget max(topk_val + bos + eos, int(cached_block_len * ratio))
 *       with forced first (bos) / last (eos) pages, topk_val = 1.
 *  [P3] "Technische Samenvatting: Onzekerheidsgestuurde Selectie voor
 *       Blok-schaarse Aandacht", section "Methodologie" steps 1-5: block
 *       scoring, per-query-tile selection (tile score = max over the tile's
 *       rows), the cut-off margin sigma, head averaging with a per-layer
 *       quantile trigger, and expansion of triggered tiles to rho*k blocks with
 *       sentinel padding so every tile has the same dispatch shape.
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE memory unless marked [host].  Structs passed by
 *    pointer are read on the host during the call and may be freed after it.
 *  - Every call validates its arguments on the host BEFORE any HIP call and
 *    returns BSA_OK (0) or a negative BSA_ERR_* code; bsa_last_error() then
 *    gives a thread-local description.  No exception crosses the ABI.
 *  - Work is only enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream); no call synchronises.  Kernel faults surface at the caller's next
 *    synchronisation.  Buffers must stay alive until the enqueued work ends.
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    retains device memory; scratch comes in through `workspace`, sized by the
 *    matching *_workspace_bytes() function.  Input values must be finite (not
 *    checked).  Calls on distinct streams may run concurrently.
 *  - All results are deterministic: no floating-point atomics are used.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define BSA_OK 0
#define BSA_ERR_INVALID_ARG (-1)   /* a pointer, size or combination is invalid */
#define BSA_ERR_UNSUPPORTED (-2)   /* valid but not implemented (dtype, head_dim, group size, ...) */
#define BSA_ERR_WORKSPACE (-3)     /* workspace NULL or smaller than required */
#define BSA_ERR_LAUNCH (-4)        /* the HIP runtime rejected a kernel launch */

/* element types of K, V, Q and of the min/max metadata */
#define BSA_F32 0
#define BSA_BF16 1

/* chunk scoring ([P1] method table) */
#define BSA_ENVELOPE 0   /* sum_d max(q_d*kmin_d, q_d*kmax_d): Quest / TSA */
#define BSA_CENTROID 1   /* q . mean(chunk keys): BlockSparse */

/* which metadata bsa_build_chunk_meta writes (bit mask) */
#define BSA_META_ENVELOPE 1u
#define BSA_META_CENTROID 2u

/* selection budgets */
#define BSA_BUDGET_TOPK 0     /* keep top_k chunks ([P1] budget = page_size x top_k) */
#define BSA_BUDGET_TOKENS 1   /* longest score-order prefix whose total length <= tokens */
#define BSA_BUDGET_RATIO 2    /* [P2] ratio budget with forced bos / eos pages */

/*
 * A paged KV cache.  Element (physical page p, KV head h, slot o, dim d) of K
 * (or V) is at k[p*stride_page + h*stride_head + o*stride_token + d] (strides in
 * elements).  The default paged layout [n_pages][H_kv][page_size][D] has
 * strides (H_kv*P*D, P*D, D): each (page, head) is one contiguous run.  A
 * token-major cache [T][H_kv][D] cut into blocks of P tokens has strides
 * (P*H_kv*D, D, H_kv*D).  Logical page j of sequence b is physical page
 * block_table[b*max_pages + j]; block_table == NULL means b*max_pages + j.
 * seq_lens [batch] holds each sequence's cached token count (device).
 * Requirements: head_dim 64 or 128; page_size a power of two in [1, 256]
 * (16 for the fastest decode path); k, v 16-byte aligned and every stride a
 * multiple of 16 bytes / element size.
 */
typedef struct {
    const void *k;
    const void *v;
    int64_t stride_page, stride_head, stride_token;
    const int32_t *block_table;
    const int32_t *seq_lens;
    int32_t batch, num_kv_heads, head_dim, page_size, max_pages, dtype;
} bsa_kv;

/*
 * Variable chunking ([P1] TSA row: chunks aligned to document structure).
 * chunk_starts [batch][max_chunks+1] token offsets (chunk c of sequence b is
 * [starts[c], starts[c+1]) , increasing, starts[0] = 0, last = seq_len);
 * num_chunks [batch].  Pass NULL (or a struct with chunk_starts NULL) for
 * fixed pages: chunk c is page c, [c*P, min(c*P+P, L)), and max_chunks is
 * kv->max_pages.
 */
typedef struct {
    const int32_t *chunk_starts;
    const int32_t *num_chunks;
    int32_t max_chunks;
} bsa_chunks;

/* Per-chunk metadata, each [batch][H_kv][max_chunks][D]: kmin / kmax in the
 * cache's element type (exact), centroid in float32; each array 16-byte
 * aligned (read and written as 16-byte vectors).  A pointer may be NULL if
 * the corresponding BSA_META_* bit / score kind is not used. */
typedef struct {
    void *kmin;
    void *kmax;
    float *centroid;
} bsa_meta;

/* Selection budget ([P1] "The comparison"; [P2] "Method configurations"). */
typedef struct {
    int32_t mode;      /* BSA_BUDGET_* */
    int32_t top_k;     /* TOPK: chunks kept per (sequence, KV head) */
    int64_t tokens;    /* TOKENS: attended-token budget */
    int32_t bos, eos;  /* RATIO: force page 0 / the last page */
    double ratio;      /* RATIO: topk_ratio */
} bsa_budget;

/*
 * Step 1 ([P1] method table; [P3] step 1): per (sequence, KV head, chunk,
 * dim), over the chunk's valid tokens: kmin = min K, kmax = max K,
 * centroid = sum K / count (float32, tokens summed in order).  Chunks past a
 * sequence's count are left untouched.  `which` = BSA_META_* bits.
 * Layout: see bsa_meta.  Errors: INVALID_ARG (NULL pointer for a requested
 * output, bad sizes), UNSUPPORTED (dtype, head_dim, page_size).
 */
int bsa_build_chunk_meta(const bsa_kv *kv, const bsa_chunks *chunks /* nullable */, const bsa_meta *meta,
                         uint32_t which, void *stream);

/*
 * Step 1 after tokens were appended (the decode loop): recomputes, per
 * (sequence, KV head), the chunks whose tokens include positions
 * >= from_len[b] -- the chunk holding token from_len[b] and the following
 * ones, at most max_touched of them -- with the rules and results of
 * bsa_build_chunk_meta (bit-identical to a full rebuild of those chunks).
 * from_len == NULL refreshes only each sequence's last chunk (one token
 * appended since the previous call); a sequence with from_len[b] >=
 * seq_lens[b] is left alone.  kv->seq_lens (and chunks, for variable chunks)
 * must already describe the grown sequences.  max_touched in
 * [1, max_chunks]; for fixed pages appending a tokens touches at most
 * ceil(a / page_size) + 1 chunks.
 * Errors: as bsa_build_chunk_meta, INVALID_ARG (max_touched).
 */
int bsa_update_chunk_meta(const bsa_kv *kv, const bsa_chunks *chunks, const bsa_meta *meta, uint32_t which,
                          const int32_t *from_len, int32_t max_touched, void *stream);

/*
 * Step 2: chunk scores.  score_kind BSA_ENVELOPE or BSA_CENTROID ([P1]).
 * Scores are raw dot products (no 1/sqrt(d)); for selection per KV head the
 * scores of a GQA group's query heads are combined by their maximum.
 *  - Decode (rows_per_query == 1): q [batch][H_q][D] (kv dtype, num_rows ==
 *    batch); scores [batch][H_kv][max_chunks] float32, -inf past a sequence's
 *    last chunk.
 *  - Query tiles (rows_per_query == R > 1, [P3] step 2): kv->batch == 1,
 *    token-major keys in blocks of kv->page_size tokens, q [num_rows][H_q][D]
 *    bf16; tile t holds rows [t*R, t*R+R); its score for block b is the max
 *    over the tile's rows and the group's heads.  With causal != 0 a tile only
 *    sees blocks starting at or before its last row (requires R ==
 *    page_size); other blocks get -inf.  scores [ceil(num_rows/R)][H_kv]
 *    [max_chunks].  Computed on the matrix cores: the envelope as
 *    [q+ | q-] x [kmax ; kmin], the centroid as q x [c_hi ; c_lo] with the
 *    float32 centroid split into two bfloat16 terms (relative error ~2^-17).
 * Errors: INVALID_ARG, UNSUPPORTED (group size > 16, head_dim, dtype).
 */
int bsa_score_chunks(const void *q, int32_t num_q_heads, int32_t num_rows, int32_t rows_per_query,
                     const bsa_kv *kv, const bsa_chunks *chunks /* nullable */, const bsa_meta *meta,
                     int32_t score_kind, int32_t causal, float *scores, void *stream);

/*
 * Step 3 (decode): per (sequence, KV head) selection from scores
 * [batch][H_kv][max_chunks] under `budget` [host]. Candidates are ordered by
 * score descending, lower chunk index first among equal scores.
 *  TOPK:   the first min(top_k, n) chunks ([P1]).
 *  RATIO:  K = min(n, max(1+bos+eos, floor(n*ratio))) with n the number of
 *          cached pages; page 0 (bos) and page n-1 (eos) are always kept and
 *          count inside K ([P2]).
 *  TOKENS: the longest prefix of the order whose total token count <= tokens
 *          (every chunk when the sequence fits).
 * Output: sel_idx [batch][H_kv][max_sel] chunk ids ascending, -1 after the
 * last; sel_count [batch][H_kv].  max_sel must hold the largest possible
 * count (TOPK: min(top_k, max_chunks); RATIO: the formula at max_chunks;
 * TOKENS: min(tokens, max_chunks)).  max_chunks <= 16384.
 * Errors: INVALID_ARG (budget values, max_sel too small), UNSUPPORTED.
 */
/*
 * The largest number of chunks a row of max_chunks candidates can keep under
 * `budget` [host]: the size max_sel must have for bsa_select_topk and
 * bsa_select_attn_decode.  TOPK: min(top_k, max_chunks) ([P1] budget =
 * page_size x top_k).  TOKENS: min(tokens, max_chunks) (every kept chunk holds
 * at least one token).  RATIO ([P2] "Method configurations at a glance"):
 * min(max_chunks, max(1 + bos + eos, floor(max_chunks * ratio))).
 * Returns the count (>= 1), or a negative BSA_ERR_* code for an invalid budget
 * or max_chunks < 1 (bsa_last_error() describes it).  Host only; no HIP call.
 */
int32_t bsa_select_max_count(const bsa_budget *budget /* [host] */, int32_t max_chunks);
int bsa_select_topk(const float *scores, const bsa_kv *kv, const bsa_chunks *chunks /* nullable */,
                    const bsa_budget *budget /* [host] */, int32_t *sel_idx, int32_t *sel_count, int32_t max_sel,
                    void *stream);

/*
 * Steps 2-5 of the uncertainty router ([P3] "Methodologie").
 * tile_scores [num_tiles][H_kv][num_blocks] (e.g. from bsa_score_chunks with
 * rows_per_query > 1).  Tile t sees n_t = min(t+1, num_blocks) blocks when
 * causal (tile rows == block size), else num_blocks.  Per (tile, KV head),
 * blocks are ordered by score (descending, lower index first) and
 *   sigma = (s_(k-1) - s_(k)) / (s_(0) - s_(k))          (0-indexed, sorted)
 * with sigma = 0 when s_(0) == s_(k) and sigma = 1 (tile not eligible) when
 * n_t <= k.  sigma_bar[t] = mean over KV heads.  The threshold is the
 * `quantile` quantile (linear interpolation between order statistics) of
 * sigma_bar over eligible tiles (NaN when no tile is eligible), or
 * fixed_threshold when it is not NaN;
 * triggered[t] = eligible && sigma_bar[t] < threshold.  kv_idx[t][h] holds
 * the first k blocks of the order (min(rho*k, n_t) when triggered),
 * ascending, padded with -1 to rho*k entries.
 * Outputs: kv_idx [num_tiles][H_kv][rho*k], sigma [num_tiles][H_kv],
 * sigma_bar [num_tiles], triggered [num_tiles] (0/1), threshold [1].
 * Selection and expansion are one code path in two launches: per (tile, KV
 * head) the top max(rho*k, k+1) blocks and sigma, written as the top k then
 * the next rho*k - k blocks; then the threshold and triggers, and each row
 * finished (cut after k, or the two runs merged into ascending order).
 * Limits: max(rho*k, k+1) <= 256, num_blocks <= 8192, num_tiles <= 8192.
 * The router needs no scratch: bsa_router_workspace_bytes() returns 0 and
 * workspace may be NULL (kept in the signature for callers that pass one).
 * Errors: INVALID_ARG, UNSUPPORTED (limits).
 */
size_t bsa_router_workspace_bytes(int32_t num_tiles, int32_t num_kv_heads, int32_t k, int32_t rho);
int bsa_select_topk_router(const float *tile_scores, int32_t num_tiles, int32_t num_kv_heads, int32_t num_blocks,
                           int32_t causal, int32_t k, int32_t rho, float quantile, float fixed_threshold,
                           int32_t *kv_idx, float *sigma, float *sigma_bar, uint8_t *triggered, float *threshold,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Step 4 (decode, [P1] "attend only to those"): softmax(q K^T * scale) V over
 * the tokens of the selected chunks only, for every query head; query head j
 * reads KV head j / (H_q / H_kv).  Split-K: each (sequence, KV head) range of
 * selected chunks is cut into num_splits parts (0 = automatic); each part
 * runs an online softmax for the whole GQA group and the parts are merged.
 * sel_idx [batch][H_kv][max_sel] / sel_count [batch][H_kv] as produced by
 * bsa_select_topk; sel_idx == NULL attends to every chunk (dense baseline).
 * q [batch][H_q][D] (kv dtype); out [batch][H_q][D] float32; q, out and
 * workspace 16-byte aligned.
 * Group size H_q/H_kv <= 16.  workspace >= bsa_decode_workspace_bytes(...)
 * (0 bytes when the resolved split count is 1 and the balanced schedule below
 * does not apply): the partials, merged by a second kernel on the same
 * stream.  Splits are capped at 64.  Calls that share a workspace must not
 * overlap.  sel_count entries are clamped to [0, max_sel] by every schedule
 * (the first max_sel entries are attended).  With more than one split, out
 * may be NULL: the merge is skipped and the workspace holds the partials
 * (layout at bsa_decode_merge).  A row with nothing to attend to (an empty
 * sequence, a count of 0) comes out NaN: the softmax over an empty set.
 * Balanced schedule: with num_splits == 0, out != NULL, a selection, fixed
 * pages (chunks NULL or chunks->chunk_starts NULL), 16-token pages, 16 <= batch x H_kv <= 4096 and batch x H_kv x max_sel
 * >= 49152, the kept pages of all rows are laid end to end and cut into 256
 * equal shares, one workgroup each, instead of a fixed split count per row
 * (rows of unequal length then keep every compute unit busy to the end).
 * Its partials live in the workspace in an internal layout and are merged
 * by the library; bsa_decode_workspace_bytes(kv, H_q, max_sel, 0) covers
 * both schedules (and the kept lists bsa_select_attn_decode may keep there).
 * The results differ from a split grid's in rounding only.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, LAUNCH.
 */
int32_t bsa_decode_num_splits(const bsa_kv *kv, int32_t num_q_heads, int32_t max_items, int32_t num_splits);
size_t bsa_decode_workspace_bytes(const bsa_kv *kv, int32_t num_q_heads, int32_t max_items, int32_t num_splits);
int bsa_sparse_attn_decode(const void *q, int32_t num_q_heads, const bsa_kv *kv, const bsa_chunks *chunks,
                           const int32_t *sel_idx, const int32_t *sel_count, int32_t max_sel, float softmax_scale,
                           int32_t num_splits, float *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The split merge of step 4 on its own, for partials left in the workspace by
 * bsa_sparse_attn_decode / bsa_select_attn_decode with out == NULL.  The
 * workspace holds o [batch][H_q][num_splits][head_dim] float32 (unnormalised
 * per-split outputs) followed by (m, l) [batch][H_q][num_splits][2] float32
 * (per-split running max of the base-2 scaled logits and softmax sum);
 *   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
 * num_splits in [2, 64]; head_dim 64 or 128.  out [batch][H_q][head_dim];
 * out and workspace 16-byte aligned.
 * Errors: INVALID_ARG, UNSUPPORTED, LAUNCH.
 */
int bsa_decode_merge(const void *workspace, int32_t batch, int32_t num_q_heads, int32_t head_dim,
                     int32_t num_splits, float *out, void *stream);

/*
 * Steps 3 + 4 fused (decode, [P1] "The comparison": keep the top chunks under
 * the budget, attend only to them; [P2] ratio budget): the selection of
 * bsa_select_topk and the attention of bsa_sparse_attn_decode in one launch
 * (plus the split merge), for fixed 16-token pages without a chunk list.
 * scores [batch][H_kv][max_pages] from bsa_score_chunks.  The kept set is the
 * one bsa_select_topk returns for the same scores and budget, and out is
 * bit-identical to bsa_sparse_attn_decode on that set with the same split
 * count (for num_splits = 0, with max_sel equal to the largest possible
 * selection K there).  With num_splits = 0 and out given on a batch where the
 * balanced schedule applies (see bsa_sparse_attn_decode, with K for max_sel),
 * this call runs the selection kernel of bsa_select_topk and then the
 * balanced attention instead of the fused kernel, and for max_pages > 8192 it
 * runs that selection kernel and then bsa_sparse_attn_decode's split-grid
 * attention (the fused kernel selects rows of at most 8192 pages); in both
 * cases the kept lists stay in the workspace unless sel_idx is given.  sel_idx / sel_count (both or neither) optionally receive the kept
 * list as bsa_select_topk writes it (max_sel >= the largest possible
 * selection K).  Splits resolve as bsa_decode_num_splits(kv, H_q, K,
 * num_splits), num_splits in [0, 64], and each split keeps at most 2048
 * pages; workspace >= bsa_decode_workspace_bytes(kv, H_q, K, num_splits).
 * max_pages <= 16384; group size <= 16.  Calls sharing a workspace must not
 * overlap.  out may be NULL with more than one split, as for
 * bsa_sparse_attn_decode; q, out and workspace 16-byte aligned.
 * Errors: INVALID_ARG, UNSUPPORTED (page size, limits), WORKSPACE, LAUNCH.
 */
int bsa_select_attn_decode(const void *q, int32_t num_q_heads, const bsa_kv *kv, const float *scores,
                           const bsa_budget *budget, float softmax_scale, int32_t num_splits, float *out,
                           int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * One whole decode step in one call ([P1] "The comparison": score every
 * chunk against the query, keep the top chunks under the budget, attend only
 * to them; [P2] ratio budget), for fixed 16-token pages: the chunk scores of
 * bsa_score_chunks (score_kind BSA_ENVELOPE or BSA_CENTROID, meta as built
 * by bsa_build_chunk_meta), then exactly what bsa_select_attn_decode does
 * with out given (the fused selection + attention and the split merge, or
 * on batches where the balanced schedule applies the selection kernel and
 * the balanced attention).  out [batch][H_q][D] float32 is required and is
 * bit-identical to bsa_score_chunks + bsa_select_attn_decode with the same
 * num_splits (0 = automatic).  scores (nullable) receives the chunk scores
 * [batch][H_kv][max_pages] as bsa_score_chunks writes them (else they stay
 * in the workspace); sel_idx / sel_count (both or neither) receive the kept
 * list as in bsa_select_attn_decode.  workspace (16-byte aligned, >=
 * bsa_decode_step_workspace_bytes(kv, H_q, budget, num_splits) bytes) holds
 * the split partials and the scores; it needs no initial contents, and
 * calls sharing it must not overlap.  q, out 16-byte aligned; group size
 * <= 16; max_pages <= 16384.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, LAUNCH.
 */
size_t bsa_decode_step_workspace_bytes(const bsa_kv *kv, int32_t num_q_heads, const bsa_budget *budget /* [host] */,
                                       int32_t num_splits);
int bsa_decode_step(const void *q, int32_t num_q_heads, const bsa_kv *kv, const bsa_meta *meta, int32_t score_kind,
                    const bsa_budget *budget /* [host] */, float softmax_scale, int32_t num_splits, float *out,
                    float *scores, int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * bsa_select_attn_decode for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments, kernels and bits,
 * with the scratch taken from a static device array of
 * BSA_STATIC_SCRATCH_BYTES in the library (one per GPU, held until the
 * process ends).  The call makes no allocation.  It runs on the CURRENT
 * device (the one `stream` belongs to); the first call on a device looks up
 * that device's copy of the array.  Calls on one GPU share its array and
 * race if they overlap (in time, on any streams): serialise them.  No
 * kernel of this call needs the array cleared.  out must be given (partials
 * left in the array would be out of the caller's reach).  A call whose
 * scratch need (bsa_decode_workspace_bytes for its plan) exceeds
 * BSA_STATIC_SCRATCH_BYTES is refused with BSA_ERR_UNSUPPORTED before any
 * HIP call.
 * Errors: as bsa_select_attn_decode, INVALID_ARG (out NULL), UNSUPPORTED
 * (scratch too small).
 */
#define BSA_STATIC_SCRATCH_BYTES (16u << 20)
int bsa_select_attn_decode_static(const void *q, int32_t num_q_heads, const bsa_kv *kv, const float *scores,
                                  const bsa_budget *budget, float softmax_scale, int32_t num_splits, float *out,
                                  int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, void *stream);

/*
 * Step 5 attention ([P3] step 5): causal prefill over query tiles of
 * tile_rows rows.  Row r of tile t, query head j, attends to the keys of the
 * non-sentinel blocks in kv_idx[t][j / (H_q/H_kv)] (idx_stride entries per
 * (tile, KV head), ascending, -1 padded) whose position is <= r;
 * kv_idx == NULL attends to every block up to the diagonal (dense causal
 * baseline).  A (tile, KV head) list ends at its first entry that is
 * negative or past the tile; a row with no block to attend to comes out NaN
 * (the softmax over an empty set).  kv: batch 1, token-major bf16 [num_rows][H_kv][D] with
 * page_size == tile_rows == 64 and block_table NULL.  q [num_rows][H_q][D]
 * bf16; out [num_rows][H_q][D] float32.  Matrix-core kernel (bf16 Q.K^T,
 * fp16 P.V, fp32 accumulation; V must lie in the fp16 range: a finite value
 * beyond it, |v| > 65504, becomes infinite in the fp16 copy, and every row
 * that attends to its block comes out non-finite in that KV head's query
 * heads, never finite and wrong).  Group size
 * <= 8, head_dim 128, idx_stride <= 1024, stride_token < 2^24 elements.
 * workspace (16-byte aligned, >=
 * bsa_tile_prefill_workspace_bytes(kv, num_rows)) receives an fp16 copy of V
 * made by the call itself; calls sharing a workspace must not overlap.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, LAUNCH.
 */
size_t bsa_tile_prefill_workspace_bytes(const bsa_kv *kv, int32_t num_rows);
int bsa_sparse_attn_tile_prefill(const void *q, int32_t num_q_heads, int32_t num_rows, const bsa_kv *kv,
                                 int32_t tile_rows, const int32_t *kv_idx, int32_t idx_stride, float softmax_scale,
                                 float *out, void *workspace, size_t workspace_bytes, void *stream);

/* Text for a status code, and the thread-local detail of the last failure. */
const char *bsa_status_string(int32_t status);
const char *bsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BSA_H */
