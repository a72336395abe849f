// api.cpp -- the C ABI of libbsa: host-side validation, launch geometry and
// workspace sizing.  Every entry point checks its arguments before touching
// HIP, so argument errors are reported without a device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "bsa_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return BSA_OK;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int x) {
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}

size_t elem_size(int dtype) { return dtype == BSA_BF16 ? 2 : 4; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every call that reads the cache.
int check_kv(const bsa_kv *kv, bool need_v, bsa::KvView *view) {
    if (!kv) return fail(BSA_ERR_INVALID_ARG, "kv is NULL");
    if (!kv->k) return fail(BSA_ERR_INVALID_ARG, "kv->k is NULL");
    if (need_v && !kv->v) return fail(BSA_ERR_INVALID_ARG, "kv->v is NULL");
    if (!kv->seq_lens) return fail(BSA_ERR_INVALID_ARG, "kv->seq_lens is NULL");
    if (kv->batch < 1 || kv->num_kv_heads < 1 || kv->max_pages < 1)
        return fail(BSA_ERR_INVALID_ARG, "batch (%d), num_kv_heads (%d) and max_pages (%d) must be >= 1", kv->batch,
                    kv->num_kv_heads, kv->max_pages);
    if (kv->dtype != BSA_F32 && kv->dtype != BSA_BF16)
        return fail(BSA_ERR_UNSUPPORTED, "dtype %d is not BSA_F32 or BSA_BF16", kv->dtype);
    if (kv->head_dim != 64 && kv->head_dim != 128)
        return fail(BSA_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", kv->head_dim);
    if (!is_pow2(kv->page_size) || kv->page_size > 256)
        return fail(BSA_ERR_UNSUPPORTED, "page_size %d is not a power of two in [1, 256]", kv->page_size);
    const int64_t unit = 16 / (int64_t)elem_size(kv->dtype);
    if (kv->stride_page <= 0 || kv->stride_head <= 0 || kv->stride_token <= 0 || kv->stride_page % unit ||
        kv->stride_head % unit || kv->stride_token % unit)
        return fail(BSA_ERR_INVALID_ARG, "strides must be positive multiples of %lld elements (16 bytes)",
                    (long long)unit);
    if (!aligned16(kv->k) || (kv->v && !aligned16(kv->v)))
        return fail(BSA_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
    if (view) {
        *view = bsa::KvView{kv->k, kv->v, kv->stride_page, kv->stride_head, kv->stride_token, kv->block_table,
                            kv->seq_lens, kv->batch, kv->num_kv_heads, kv->head_dim, kv->page_size,
                            log2i(kv->page_size), kv->max_pages, kv->dtype};
    }
    return BSA_OK;
}

int check_chunks(const bsa_kv *kv, const bsa_chunks *ch, bsa::ChunkView *view) {
    if (ch && ch->chunk_starts) {
        if (!ch->num_chunks) return fail(BSA_ERR_INVALID_ARG, "chunks->num_chunks is NULL");
        if (ch->max_chunks < 1) return fail(BSA_ERR_INVALID_ARG, "chunks->max_chunks must be >= 1");
        *view = bsa::ChunkView{ch->chunk_starts, ch->num_chunks, ch->max_chunks};
    } else {
        *view = bsa::ChunkView{nullptr, nullptr, kv->max_pages};
    }
    return BSA_OK;
}

int check_heads(const bsa_kv *kv, int32_t num_q_heads, int max_group) {
    if (num_q_heads < 1 || num_q_heads % kv->num_kv_heads)
        return fail(BSA_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
                    kv->num_kv_heads);
    if (num_q_heads / kv->num_kv_heads > max_group)
        return fail(BSA_ERR_UNSUPPORTED, "GQA group size %d exceeds %d", num_q_heads / kv->num_kv_heads, max_group);
    return BSA_OK;
}

int launched(hipError_t e) {
    if (e != hipSuccess) return fail(BSA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// The largest number of chunks a row of max_chunks can keep under *budget.
int budget_need(const bsa_budget *budget, int max_chunks, int64_t *need) {
    switch (budget->mode) {
    case BSA_BUDGET_TOPK:
        if (budget->top_k < 1) return fail(BSA_ERR_INVALID_ARG, "top_k must be >= 1");
        *need = budget->top_k < max_chunks ? budget->top_k : max_chunks;
        return BSA_OK;
    case BSA_BUDGET_TOKENS:
        if (budget->tokens < 1) return fail(BSA_ERR_INVALID_ARG, "tokens must be >= 1");
        *need = budget->tokens < max_chunks ? budget->tokens : max_chunks;
        return BSA_OK;
    case BSA_BUDGET_RATIO: {
        if (!(budget->ratio > 0.0 && budget->ratio <= 1.0))
            return fail(BSA_ERR_INVALID_ARG, "ratio must be in (0, 1]");
        if ((budget->bos != 0 && budget->bos != 1) || (budget->eos != 0 && budget->eos != 1))
            return fail(BSA_ERR_INVALID_ARG, "bos and eos must be 0 or 1");
        int64_t K = (int64_t)std::floor((double)max_chunks * budget->ratio);
        const int64_t forced = 1 + budget->bos + budget->eos;
        if (K < forced) K = forced;
        *need = K < max_chunks ? K : max_chunks;
        return BSA_OK;
    }
    default:
        return fail(BSA_ERR_INVALID_ARG, "budget mode %d is not a BSA_BUDGET_* value", budget->mode);
    }
}

constexpr int kMaxSelectChunks = 16384;   // candidates per row: 1024 threads x 16 in the selection kernel
constexpr int kMaxFusedChunks = 8192;     // rows the fused kernel selects itself (512 threads x 16)
constexpr int kMaxRouterBlocks = 8192;
constexpr int kMaxRouterTiles = 8192;

constexpr int kMaxItemsPerSplit = 2048;  // the fused selection keeps one split's pages in LDS

int resolve_splits(const bsa_kv *kv, int32_t max_items, int32_t num_splits) {
    if (num_splits > 0) return num_splits;
    const int bh = kv->batch * kv->num_kv_heads;
    // ~256 workgroups, one per compute unit: the fused kernel repeats the
    // selection in every split, so few, long splits pay off as long as every
    // compute unit gets one (measured decode steps at 16 x 32K tokens, 4 KV
    // heads: 4 splits 50.2 us, 3 splits 51.0 us, 8 splits slower; 8 KV heads:
    // 2 splits 88.6 us, 3 splits 94.6 us; one sequence: 32 splits, the cap
    // below, best of 8 to 64)
    int s = (256 + bh - 1) / bh;
    const int cap = (max_items + 7) / 8;                // at least ~8 items per workgroup
    if (s > cap) s = cap;
    const int floor_s = (max_items + kMaxItemsPerSplit - 1) / kMaxItemsPerSplit;
    if (s < floor_s) s = floor_s;
    if (s < 1) s = 1;
    if (s > 64) s = 64;
    return s;
}

// The balanced schedule (one share of the rows' kept pages per compute unit)
// replaces the split grid for automatic splits on batches of 16-token pages
// when the library merges itself: at least 16 rows (batch x H_kv) and room
// for long shares (rows x max items >= 192 x 256 pages).  It costs two
// dependent memory round trips that the split grid does not pay (the counts
// before the first page numbers, and before the merge's partials), about
// 3 us measured on 16 equal rows, and saves the idle tail of unequal rows
// (9-11 % at 16 x U[8K, 32K] tokens, ratios 1/4 to 1/2), so smaller steps keep
// the split grid.
bool balanced_applies(const bsa_kv *kv, int32_t max_items, int32_t num_splits) {
    if (num_splits != 0 || !kv || kv->page_size != 16 || max_items < 1) return false;
    const int64_t rows = (int64_t)kv->batch * kv->num_kv_heads;
    return rows >= 16 && rows <= bsa::kBalMaxRows && rows * max_items >= 192 * bsa::kBalWgs;
}

size_t balanced_workspace_bytes(const bsa_kv *kv, int32_t num_q_heads) {
    const int64_t rows = (int64_t)kv->batch * kv->num_kv_heads;
    const size_t n = (size_t)(rows + bsa::kBalWgs) * (num_q_heads / kv->num_kv_heads) * (kv->head_dim + 2) * sizeof(float);
    return (n + 15) & ~(size_t)15;
}

// The split grid's partial outputs and (max, sum) pairs: none with one split.
size_t partials_bytes(const bsa_kv *kv, int32_t num_q_heads, int splits) {
    return splits <= 1 ? 0 : (size_t)kv->batch * num_q_heads * splits * (kv->head_dim + 2) * sizeof(float);
}

// The fused entry point on the balanced schedule keeps the kept lists (max
// items and a count per row) after the partials when the caller takes none.
size_t balanced_list_bytes(const bsa_kv *kv, int32_t max_items) {
    const int64_t rows = (int64_t)kv->batch * kv->num_kv_heads;
    return (size_t)rows * (max_items + 1) * sizeof(int32_t);
}

}  // namespace

extern "C" {

const char *bsa_status_string(int32_t status) {
    switch (status) {
    case BSA_OK: return "BSA_OK";
    case BSA_ERR_INVALID_ARG: return "BSA_ERR_INVALID_ARG";
    case BSA_ERR_UNSUPPORTED: return "BSA_ERR_UNSUPPORTED";
    case BSA_ERR_WORKSPACE: return "BSA_ERR_WORKSPACE";
    case BSA_ERR_LAUNCH: return "BSA_ERR_LAUNCH";
    default: return "BSA_ERR_UNKNOWN";
    }
}

const char *bsa_last_error(void) { return g_err; }

static int check_meta_args(const bsa_kv *kv, const bsa_chunks *chunks, const bsa_meta *meta, uint32_t which,
                           bsa::KvView *v, bsa::ChunkView *c) {
    int rc = check_kv(kv, false, v);
    if (rc) return rc;
    if ((rc = check_chunks(kv, chunks, c))) return rc;
    if (!meta) return fail(BSA_ERR_INVALID_ARG, "meta is NULL");
    if (which == 0 || (which & ~(BSA_META_ENVELOPE | BSA_META_CENTROID)))
        return fail(BSA_ERR_INVALID_ARG, "which must be a non-empty combination of BSA_META_* bits");
    if ((which & BSA_META_ENVELOPE) && (!meta->kmin || !meta->kmax))
        return fail(BSA_ERR_INVALID_ARG, "meta->kmin / kmax is NULL");
    if ((which & BSA_META_CENTROID) && !meta->centroid) return fail(BSA_ERR_INVALID_ARG, "meta->centroid is NULL");
    if (!aligned16(meta->kmin) || !aligned16(meta->kmax) || !aligned16(meta->centroid))
        return fail(BSA_ERR_INVALID_ARG, "meta arrays must be 16-byte aligned");
    return BSA_OK;
}

int bsa_build_chunk_meta(const bsa_kv *kv, const bsa_chunks *chunks, const bsa_meta *meta, uint32_t which,
                         void *stream) {
    bsa::KvView v;
    bsa::ChunkView c;
    int rc = check_meta_args(kv, chunks, meta, which, &v, &c);
    if (rc) return rc;
    return launched(bsa::launch_chunk_meta(v, c, meta->kmin, meta->kmax, meta->centroid, which, nullptr, 0,
                                           (hipStream_t)stream));
}

int bsa_update_chunk_meta(const bsa_kv *kv, const bsa_chunks *chunks, const bsa_meta *meta, uint32_t which,
                          const int32_t *from_len, int32_t max_touched, void *stream) {
    bsa::KvView v;
    bsa::ChunkView c;
    int rc = check_meta_args(kv, chunks, meta, which, &v, &c);
    if (rc) return rc;
    if (max_touched < 1 || max_touched > c.max_chunks)
        return fail(BSA_ERR_INVALID_ARG, "max_touched %d must be in [1, max_chunks %d]", max_touched, c.max_chunks);
    return launched(bsa::launch_chunk_meta(v, c, meta->kmin, meta->kmax, meta->centroid, which, from_len,
                                           max_touched, (hipStream_t)stream));
}

int bsa_score_chunks(const void *q, int32_t num_q_heads, int32_t num_rows, int32_t rows_per_query, const bsa_kv *kv,
                     const bsa_chunks *chunks, const bsa_meta *meta, int32_t score_kind, int32_t causal,
                     float *scores, void *stream) {
    bsa::KvView v;
    bsa::ChunkView c;
    int rc = check_kv(kv, false, &v);
    if (rc) return rc;
    if ((rc = check_chunks(kv, chunks, &c))) return rc;
    if (!q || !scores || !meta) return fail(BSA_ERR_INVALID_ARG, "q, scores and meta must be non-NULL");
    if (!aligned16(q)) return fail(BSA_ERR_INVALID_ARG, "q must be 16-byte aligned");
    if (score_kind != BSA_ENVELOPE && score_kind != BSA_CENTROID)
        return fail(BSA_ERR_INVALID_ARG, "score_kind %d is not BSA_ENVELOPE or BSA_CENTROID", score_kind);
    if (score_kind == BSA_ENVELOPE && (!meta->kmin || !meta->kmax))
        return fail(BSA_ERR_INVALID_ARG, "envelope scoring needs meta->kmin and meta->kmax");
    if (score_kind == BSA_CENTROID && !meta->centroid)
        return fail(BSA_ERR_INVALID_ARG, "centroid scoring needs meta->centroid");
    if (!aligned16(meta->kmin) || !aligned16(meta->kmax) || !aligned16(meta->centroid))
        return fail(BSA_ERR_INVALID_ARG, "meta arrays must be 16-byte aligned");
    if (rows_per_query < 1) return fail(BSA_ERR_INVALID_ARG, "rows_per_query must be >= 1");
    if (rows_per_query == 1) {
        if ((rc = check_heads(kv, num_q_heads, 16))) return rc;
        if (num_rows != kv->batch)
            return fail(BSA_ERR_INVALID_ARG, "decode scoring needs num_rows (%d) == batch (%d)", num_rows, kv->batch);
        return launched(bsa::launch_score_decode(q, num_q_heads, v, c, meta->kmin, meta->kmax, meta->centroid,
                                                 score_kind, scores, (hipStream_t)stream));
    }
    if ((rc = check_heads(kv, num_q_heads, 8))) return rc;
    if (kv->dtype != BSA_BF16 || kv->head_dim != 128)
        return fail(BSA_ERR_UNSUPPORTED, "tile scoring supports bf16 with head_dim 128");
    if (rows_per_query != 64) return fail(BSA_ERR_UNSUPPORTED, "tile scoring supports 64-row tiles");
    if (kv->batch != 1) return fail(BSA_ERR_INVALID_ARG, "tile scoring needs batch == 1");
    if (chunks && chunks->chunk_starts) return fail(BSA_ERR_UNSUPPORTED, "tile scoring uses fixed key blocks");
    if (causal && kv->page_size != rows_per_query)
        return fail(BSA_ERR_UNSUPPORTED, "causal tile scoring needs block size == rows_per_query");
    if (num_rows < 1) return fail(BSA_ERR_INVALID_ARG, "num_rows must be >= 1");
    return launched(bsa::launch_score_tiles(q, num_q_heads, num_rows, rows_per_query, v, kv->max_pages, meta->kmin,
                                            meta->kmax, meta->centroid, score_kind, causal, scores,
                                            (hipStream_t)stream));
}

int32_t bsa_select_max_count(const bsa_budget *budget, int32_t max_chunks) {
    if (!budget) return fail(BSA_ERR_INVALID_ARG, "budget is NULL");
    if (max_chunks < 1) return fail(BSA_ERR_INVALID_ARG, "max_chunks must be >= 1");
    int64_t need;
    if (int rc = budget_need(budget, max_chunks, &need)) return rc;
    ok();
    return (int32_t)need;
}

int bsa_select_topk(const float *scores, const bsa_kv *kv, const bsa_chunks *chunks, const bsa_budget *budget,
                    int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, void *stream) {
    bsa::KvView v;
    bsa::ChunkView c;
    int rc = check_kv(kv, false, &v);
    if (rc) return rc;
    if ((rc = check_chunks(kv, chunks, &c))) return rc;
    if (!scores || !budget || !sel_idx || !sel_count)
        return fail(BSA_ERR_INVALID_ARG, "scores, budget, sel_idx and sel_count must be non-NULL");
    if (c.max_chunks > kMaxSelectChunks)
        return fail(BSA_ERR_UNSUPPORTED, "max_chunks %d exceeds %d", c.max_chunks, kMaxSelectChunks);
    if (max_sel < 1) return fail(BSA_ERR_INVALID_ARG, "max_sel must be >= 1");
    int64_t need;
    if ((rc = budget_need(budget, c.max_chunks, &need))) return rc;
    if (max_sel < need)
        return fail(BSA_ERR_INVALID_ARG, "max_sel %d is smaller than the largest possible selection %lld", max_sel,
                    (long long)need);
    return launched(bsa::launch_select(scores, v, c, *budget, sel_idx, sel_count, max_sel, (hipStream_t)stream));
}

size_t bsa_router_workspace_bytes(int32_t num_tiles, int32_t num_kv_heads, int32_t k, int32_t rho) {
    (void)num_tiles, (void)num_kv_heads, (void)k, (void)rho;
    return 0;  // the router writes its lists straight into kv_idx
}

int bsa_select_topk_router(const float *tile_scores, int32_t num_tiles, int32_t num_kv_heads, int32_t num_blocks,
                           int32_t causal, int32_t k, int32_t rho, float quantile, float fixed_threshold,
                           int32_t *kv_idx, float *sigma, float *sigma_bar, uint8_t *triggered, float *threshold,
                           void *workspace, size_t workspace_bytes, void *stream) {
    if (!tile_scores || !kv_idx || !sigma || !sigma_bar || !triggered || !threshold)
        return fail(BSA_ERR_INVALID_ARG, "tile_scores and every output pointer must be non-NULL");
    if (num_tiles < 1 || num_kv_heads < 1 || num_blocks < 1 || k < 1 || rho < 1)
        return fail(BSA_ERR_INVALID_ARG, "num_tiles, num_kv_heads, num_blocks, k and rho must be >= 1");
    const int want = (rho * k > k + 1) ? rho * k : k + 1;
    if (want > 256) return fail(BSA_ERR_UNSUPPORTED, "max(rho*k, k+1) = %d exceeds 256", want);
    if (num_blocks > kMaxRouterBlocks) return fail(BSA_ERR_UNSUPPORTED, "num_blocks %d exceeds %d", num_blocks,
                                                   kMaxRouterBlocks);
    if (num_tiles > kMaxRouterTiles)
        return fail(BSA_ERR_UNSUPPORTED, "num_tiles %d exceeds %d", num_tiles, kMaxRouterTiles);
    if (std::isnan(fixed_threshold) && !(quantile >= 0.f && quantile <= 1.f))
        return fail(BSA_ERR_INVALID_ARG, "quantile must be in [0, 1]");
    (void)workspace, (void)workspace_bytes;
    return launched(bsa::launch_router(tile_scores, num_tiles, num_kv_heads, num_blocks, causal, k, rho, quantile,
                                       fixed_threshold, kv_idx, sigma, sigma_bar, triggered, threshold, workspace,
                                       (hipStream_t)stream));
}

int32_t bsa_decode_num_splits(const bsa_kv *kv, int32_t num_q_heads, int32_t max_items, int32_t num_splits) {
    (void)num_q_heads;
    if (!kv || kv->batch < 1 || kv->num_kv_heads < 1 || max_items < 1) return 1;
    return resolve_splits(kv, max_items, num_splits);
}

size_t bsa_decode_workspace_bytes(const bsa_kv *kv, int32_t num_q_heads, int32_t max_items, int32_t num_splits) {
    const int s = bsa_decode_num_splits(kv, num_q_heads, max_items, num_splits);
    if (!kv || num_q_heads < 1 || kv->num_kv_heads < 1) return 0;
    size_t n = partials_bytes(kv, num_q_heads, s);
    if (balanced_applies(kv, max_items, num_splits))
        n = std::max(n, balanced_workspace_bytes(kv, num_q_heads) + balanced_list_bytes(kv, max_items));
    // the fused call on rows longer than its kernel selects keeps the kept
    // lists after the partials
    if (kv->page_size == 16 && kv->max_pages > kMaxFusedChunks)
        n = std::max(n, ((n + 15) & ~(size_t)15) + balanced_list_bytes(kv, max_items));
    return n;
}

// Decode outputs and split partials are written as 16-byte vectors.
static int check_out_ws(const float *out, const void *workspace) {
    if (out && !aligned16(out)) return fail(BSA_ERR_INVALID_ARG, "out must be 16-byte aligned");
    if (workspace && !aligned16(workspace)) return fail(BSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return BSA_OK;
}

int bsa_sparse_attn_decode(const void *q, int32_t num_q_heads, const bsa_kv *kv, const bsa_chunks *chunks,
                           const int32_t *sel_idx, const int32_t *sel_count, int32_t max_sel, float softmax_scale,
                           int32_t num_splits, float *out, void *workspace, size_t workspace_bytes, void *stream) {
    bsa::KvView v;
    bsa::ChunkView c;
    int rc = check_kv(kv, true, &v);
    if (rc) return rc;
    if ((rc = check_chunks(kv, chunks, &c))) return rc;
    if ((rc = check_heads(kv, num_q_heads, 16))) return rc;
    if (!q) return fail(BSA_ERR_INVALID_ARG, "q must be non-NULL");
    if (!aligned16(q)) return fail(BSA_ERR_INVALID_ARG, "q must be 16-byte aligned");
    if (sel_idx && (!sel_count || max_sel < 1))
        return fail(BSA_ERR_INVALID_ARG, "sel_idx needs sel_count and max_sel >= 1");
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
        return fail(BSA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
    if (num_splits < 0) return fail(BSA_ERR_INVALID_ARG, "num_splits must be >= 0");
    const int items = sel_idx ? max_sel : c.max_chunks;
    if (out && sel_idx && !c.starts && balanced_applies(kv, items, num_splits)) {
        const size_t need = balanced_workspace_bytes(kv, num_q_heads);
        if (!workspace || workspace_bytes < need)
            return fail(BSA_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", need, workspace_bytes);
        if ((rc = check_out_ws(out, workspace))) return rc;
        return launched(bsa::launch_decode_balanced(q, num_q_heads, v, sel_idx, sel_count, max_sel, softmax_scale,
                                                    out, workspace, (hipStream_t)stream));
    }
    const int splits = resolve_splits(kv, items, num_splits);
    if (!out && splits == 1)
        return fail(BSA_ERR_INVALID_ARG, "out may be NULL only with more than one split (partials stay in the "
                                         "workspace)");
    const size_t need = bsa_decode_workspace_bytes(kv, num_q_heads, items, splits);
    if (need && (!workspace || workspace_bytes < need))
        return fail(BSA_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if ((rc = check_out_ws(out, need ? workspace : nullptr))) return rc;
    return launched(bsa::launch_decode(q, num_q_heads, v, c, sel_idx, sel_count, max_sel, softmax_scale, splits, out,
                                       workspace, (hipStream_t)stream));
}

static size_t al16(size_t n) { return (n + 15) & ~(size_t)15; }

// The fused decode call's host side: every argument check and the launch
// plan, without a HIP call, so the no-allocation variant can size its scratch
// before touching the device.
struct FusedPlan {
    bsa::KvView v;
    int64_t need;       // the largest possible selection K
    bool balanced;      // selection kernel + balanced attention instead of the fused kernel
    bool two_pass;      // selection kernel + split-grid attention (rows longer than the fused kernel selects)
    int splits;         // the fused kernel's split count
    size_t ws_need;     // workspace bytes the launch uses
};

static int plan_select_attn_decode(const void *q, int32_t num_q_heads, const bsa_kv *kv, const bsa_budget *budget,
                                   float softmax_scale, int32_t num_splits, float *out, int32_t *sel_idx,
                                   int32_t *sel_count, int32_t max_sel, FusedPlan *p) {
    int rc = check_kv(kv, true, &p->v);
    if (rc) return rc;
    if ((rc = check_heads(kv, num_q_heads, 16))) return rc;
    if (!q || !budget) return fail(BSA_ERR_INVALID_ARG, "q and budget must be non-NULL");
    if (!aligned16(q)) return fail(BSA_ERR_INVALID_ARG, "q must be 16-byte aligned");
    if (kv->page_size != 16) return fail(BSA_ERR_UNSUPPORTED, "fused selection needs 16-token pages");
    if (kv->max_pages > kMaxSelectChunks)
        return fail(BSA_ERR_UNSUPPORTED, "max_pages %d exceeds %d", kv->max_pages, kMaxSelectChunks);
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
        return fail(BSA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
    if (num_splits < 0 || num_splits > 64) return fail(BSA_ERR_INVALID_ARG, "num_splits must be in [0, 64]");
    if ((rc = budget_need(budget, kv->max_pages, &p->need))) return rc;
    if ((sel_idx == nullptr) != (sel_count == nullptr))
        return fail(BSA_ERR_INVALID_ARG, "sel_idx and sel_count are both given or both NULL");
    if (sel_idx && max_sel < p->need)
        return fail(BSA_ERR_INVALID_ARG, "max_sel %d is smaller than the largest possible selection %lld", max_sel,
                    (long long)p->need);
    if (out && !aligned16(out)) return fail(BSA_ERR_INVALID_ARG, "out must be 16-byte aligned");
    p->balanced = out && balanced_applies(kv, (int)p->need, num_splits);
    p->two_pass = false;
    if (p->balanced) {
        p->splits = 0;
        p->ws_need = balanced_workspace_bytes(kv, num_q_heads) + (sel_idx ? 0 : balanced_list_bytes(kv, (int)p->need));
        return BSA_OK;
    }
    p->splits = resolve_splits(kv, (int)p->need, num_splits);
    if (kv->max_pages > kMaxFusedChunks) {
        // rows longer than the fused kernel selects: the selection kernel,
        // then the split-grid attention (the same kernels and bits as the two
        // calls); the partials, then the kept lists when the caller takes none
        if (!out && p->splits == 1)
            return fail(BSA_ERR_INVALID_ARG, "out may be NULL only with more than one split (partials stay in the "
                                             "workspace)");
        p->two_pass = true;
        p->ws_need = al16(partials_bytes(kv, num_q_heads, p->splits)) + (sel_idx ? 0 : balanced_list_bytes(kv, (int)p->need));
        return BSA_OK;
    }
    if ((p->need + p->splits - 1) / p->splits > kMaxItemsPerSplit)
        return fail(BSA_ERR_INVALID_ARG, "%d splits keep more than %d pages each; use more splits", p->splits,
                    kMaxItemsPerSplit);
    if (!out && p->splits == 1)
        return fail(BSA_ERR_INVALID_ARG, "out may be NULL only with more than one split (partials stay in the "
                                         "workspace)");
    p->ws_need = bsa_decode_workspace_bytes(kv, num_q_heads, (int)p->need, p->splits);
    return BSA_OK;
}

// Enqueues a planned fused decode call; the workspace (16-byte aligned, at
// least p.ws_need bytes when p.ws_need > 0) has been checked by the caller.
static int launch_select_attn_decode(const FusedPlan &p, const void *q, int32_t num_q_heads, const bsa_kv *kv,
                                     const float *scores, const bsa_budget *budget, float softmax_scale, float *out,
                                     int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, void *workspace,
                                     void *stream) {
    if (p.balanced) {
        // a large batch: the selection kernel, then the attention on the
        // balanced schedule (the same kernels and bits as the two calls)
        const size_t part = balanced_workspace_bytes(kv, num_q_heads);
        const int64_t rows = (int64_t)kv->batch * kv->num_kv_heads;
        int32_t *si = sel_idx, *sc = sel_count;
        int32_t ms = max_sel;
        if (!si) {
            si = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + part);
            sc = si + rows * p.need;
            ms = (int32_t)p.need;
        }
        bsa::ChunkView c;
        check_chunks(kv, nullptr, &c);
        hipError_t e = bsa::launch_select(scores, p.v, c, *budget, si, sc, ms, (hipStream_t)stream);
        if (e == hipSuccess)
            e = bsa::launch_decode_balanced(q, num_q_heads, p.v, si, sc, ms, softmax_scale, out, workspace,
                                            (hipStream_t)stream);
        return launched(e);
    }
    if (p.two_pass) {
        const size_t part = al16(partials_bytes(kv, num_q_heads, p.splits));
        const int64_t rows = (int64_t)kv->batch * kv->num_kv_heads;
        int32_t *si = sel_idx, *sc = sel_count;
        int32_t ms = max_sel;
        if (!si) {
            si = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + part);
            sc = si + rows * p.need;
            ms = (int32_t)p.need;
        }
        bsa::ChunkView c;
        check_chunks(kv, nullptr, &c);
        hipError_t e = bsa::launch_select(scores, p.v, c, *budget, si, sc, ms, (hipStream_t)stream);
        if (e == hipSuccess)
            e = bsa::launch_decode(q, num_q_heads, p.v, c, si, sc, ms, softmax_scale, p.splits, out,
                                   part ? workspace : nullptr, (hipStream_t)stream);
        return launched(e);
    }
    return launched(bsa::launch_select_decode(q, num_q_heads, p.v, scores, *budget, sel_idx, sel_count,
                                              sel_idx ? max_sel : 0, softmax_scale, p.splits, out,
                                              p.ws_need ? workspace : nullptr, (hipStream_t)stream));
}

int bsa_select_attn_decode(const void *q, int32_t num_q_heads, const bsa_kv *kv, const float *scores,
                           const bsa_budget *budget, float softmax_scale, int32_t num_splits, float *out,
                           int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, void *workspace,
                           size_t workspace_bytes, void *stream) {
    FusedPlan p;
    if (!scores) return fail(BSA_ERR_INVALID_ARG, "scores must be non-NULL");
    int rc = plan_select_attn_decode(q, num_q_heads, kv, budget, softmax_scale, num_splits, out, sel_idx, sel_count,
                                     max_sel, &p);
    if (rc) return rc;
    if (p.ws_need && (!workspace || workspace_bytes < p.ws_need))
        return fail(BSA_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", p.ws_need, workspace_bytes);
    if (p.ws_need && !aligned16(workspace)) return fail(BSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return launch_select_attn_decode(p, q, num_q_heads, kv, scores, budget, softmax_scale, out, sel_idx, sel_count,
                                     max_sel, workspace, stream);
}

// ---- one decode step: scoring, then selection + attention + merge ------------

struct StepPlan {
    FusedPlan f;
    bsa::ChunkView c;
    size_t scores_off, total;
};

static int plan_decode_step(const void *q, int32_t num_q_heads, const bsa_kv *kv, const bsa_meta *meta,
                            int32_t score_kind, const bsa_budget *budget, float softmax_scale, int32_t num_splits,
                            float *out, int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, StepPlan *p) {
    if (!out) return fail(BSA_ERR_INVALID_ARG, "out must be non-NULL");
    int rc = plan_select_attn_decode(q, num_q_heads, kv, budget, softmax_scale, num_splits, out, sel_idx, sel_count,
                                     max_sel, &p->f);
    if (rc) return rc;
    check_chunks(kv, nullptr, &p->c);
    if (!meta) return fail(BSA_ERR_INVALID_ARG, "meta is NULL");
    if (score_kind != BSA_ENVELOPE && score_kind != BSA_CENTROID)
        return fail(BSA_ERR_INVALID_ARG, "score_kind %d is not BSA_ENVELOPE or BSA_CENTROID", score_kind);
    if (score_kind == BSA_ENVELOPE && (!meta->kmin || !meta->kmax))
        return fail(BSA_ERR_INVALID_ARG, "envelope scoring needs meta->kmin and meta->kmax");
    if (score_kind == BSA_CENTROID && !meta->centroid)
        return fail(BSA_ERR_INVALID_ARG, "centroid scoring needs meta->centroid");
    if (!aligned16(meta->kmin) || !aligned16(meta->kmax) || !aligned16(meta->centroid))
        return fail(BSA_ERR_INVALID_ARG, "meta arrays must be 16-byte aligned");
    const size_t rows = (size_t)kv->batch * kv->num_kv_heads;
    p->scores_off = al16(p->f.ws_need);
    p->total = p->scores_off + al16(rows * kv->max_pages * sizeof(float));
    return BSA_OK;
}

size_t bsa_decode_step_workspace_bytes(const bsa_kv *kv, int32_t num_q_heads, const bsa_budget *budget,
                                       int32_t num_splits) {
    if (!kv || !budget || kv->batch < 1 || kv->num_kv_heads < 1 || kv->max_pages < 1 || num_q_heads < 1) return 0;
    int64_t need;
    if (budget_need(budget, kv->max_pages, &need)) return 0;
    const bool bal = balanced_applies(kv, (int)need, num_splits);
    size_t ws = bal ? balanced_workspace_bytes(kv, num_q_heads) + balanced_list_bytes(kv, (int)need)
                    : bsa_decode_workspace_bytes(kv, num_q_heads, (int)need, resolve_splits(kv, (int)need, num_splits));
    const size_t rows = (size_t)kv->batch * kv->num_kv_heads;
    return al16(ws) + al16(rows * kv->max_pages * sizeof(float));
}

int bsa_decode_step(const void *q, int32_t num_q_heads, const bsa_kv *kv, const bsa_meta *meta, int32_t score_kind,
                    const bsa_budget *budget, float softmax_scale, int32_t num_splits, float *out, float *scores,
                    int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, void *workspace, size_t workspace_bytes,
                    void *stream) {
    StepPlan p;
    int rc = plan_decode_step(q, num_q_heads, kv, meta, score_kind, budget, softmax_scale, num_splits, out, sel_idx,
                              sel_count, max_sel, &p);
    if (rc) return rc;
    if (!workspace || workspace_bytes < p.total)
        return fail(BSA_ERR_WORKSPACE, "decode step workspace needs %zu bytes, got %zu", p.total, workspace_bytes);
    if (!aligned16(workspace)) return fail(BSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    float *sc = scores ? scores : reinterpret_cast<float *>(static_cast<char *>(workspace) + p.scores_off);
    hipError_t e = bsa::launch_score_decode(q, num_q_heads, p.f.v, p.c, meta->kmin, meta->kmax, meta->centroid,
                                            score_kind, sc, (hipStream_t)stream);
    if (e != hipSuccess) return launched(e);
    return launch_select_attn_decode(p.f, q, num_q_heads, kv, sc, budget, softmax_scale, out, sel_idx, sel_count,
                                     max_sel, workspace, stream);
}

// ---- the no-allocation fused decode entry point -------------------------------
// Device scratch for bsa_select_attn_decode_static: one copy of this array per
// GPU, loaded with the library's code object and held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address); it takes each device's address once, from
// hipGetSymbolAddress, and uses that pointer.
static __device__ __align__(256) unsigned char scratch[BSA_STATIC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void *g_scratch_ptr[64] = {};

// The scratch address on the current device, taken on the first call there.
static int scratch_on_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(BSA_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(BSA_ERR_UNSUPPORTED, "device %d: at most 64 devices", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(BSA_ERR_LAUNCH, "hipGetSymbolAddress of the static scratch failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return BSA_OK;
}

int bsa_select_attn_decode_static(const void *q, int32_t num_q_heads, const bsa_kv *kv, const float *scores,
                                  const bsa_budget *budget, float softmax_scale, int32_t num_splits, float *out,
                                  int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, void *stream) {
    if (!out) return fail(BSA_ERR_INVALID_ARG, "out must be non-NULL (partials in the static scratch are not "
                                               "reachable by the caller)");
    FusedPlan p;
    if (!scores) return fail(BSA_ERR_INVALID_ARG, "scores must be non-NULL");
    int rc = plan_select_attn_decode(q, num_q_heads, kv, budget, softmax_scale, num_splits, out, sel_idx, sel_count,
                                     max_sel, &p);
    if (rc) return rc;
    if (p.ws_need > (size_t)BSA_STATIC_SCRATCH_BYTES)
        return fail(BSA_ERR_UNSUPPORTED,
                    "this call needs %zu bytes of scratch; the static scratch holds %zu (use bsa_select_attn_decode "
                    "with a workspace)",
                    p.ws_need, (size_t)BSA_STATIC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (p.ws_need && (rc = scratch_on_current_device(&ws))) return rc;
    return launch_select_attn_decode(p, q, num_q_heads, kv, scores, budget, softmax_scale, out, sel_idx, sel_count,
                                     max_sel, ws, stream);
}

int bsa_decode_merge(const void *workspace, int32_t batch, int32_t num_q_heads, int32_t head_dim,
                     int32_t num_splits, float *out, void *stream) {
    if (!workspace || !out) return fail(BSA_ERR_INVALID_ARG, "workspace and out must be non-NULL");
    if (batch < 1 || num_q_heads < 1) return fail(BSA_ERR_INVALID_ARG, "batch and num_q_heads must be >= 1");
    if (head_dim != 64 && head_dim != 128) return fail(BSA_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", head_dim);
    if (num_splits < 2 || num_splits > 64) return fail(BSA_ERR_INVALID_ARG, "num_splits must be in [2, 64]");
    if (int rc = check_out_ws(out, workspace)) return rc;
    const float *part_o = (const float *)workspace;
    const float *part_ml = part_o + (size_t)batch * num_q_heads * num_splits * head_dim;
    return launched(bsa::launch_decode_merge(num_splits, part_o, part_ml, out, num_q_heads, batch, head_dim,
                                             (hipStream_t)stream));
}

size_t bsa_tile_prefill_workspace_bytes(const bsa_kv *kv, int32_t num_rows) {
    if (!kv || num_rows < 1 || kv->num_kv_heads < 1 || kv->head_dim < 1) return 0;
    return (size_t)num_rows * kv->num_kv_heads * kv->head_dim * 2;  // V in fp16, [rows][H_kv][D]
}

int bsa_sparse_attn_tile_prefill(const void *q, int32_t num_q_heads, int32_t num_rows, const bsa_kv *kv,
                                 int32_t tile_rows, const int32_t *kv_idx, int32_t idx_stride, float softmax_scale,
                                 float *out, void *workspace, size_t workspace_bytes, void *stream) {
    bsa::KvView v;
    int rc = check_kv(kv, true, &v);
    if (rc) return rc;
    if ((rc = check_heads(kv, num_q_heads, 8))) return rc;
    if (!q || !out) return fail(BSA_ERR_INVALID_ARG, "q and out must be non-NULL");
    if (!aligned16(q)) return fail(BSA_ERR_INVALID_ARG, "q must be 16-byte aligned");
    if (kv->dtype != BSA_BF16 || kv->head_dim != 128)
        return fail(BSA_ERR_UNSUPPORTED, "tile prefill supports bf16 with head_dim 128");
    if (kv->batch != 1 || kv->block_table)
        return fail(BSA_ERR_UNSUPPORTED, "tile prefill needs batch 1 and a token-major cache (block_table NULL)");
    if (tile_rows != 64 || kv->page_size != 64)
        return fail(BSA_ERR_UNSUPPORTED, "tile prefill supports 64-row tiles over 64-token blocks");
    if (kv->stride_page != 64 * kv->stride_token)
        return fail(BSA_ERR_UNSUPPORTED, "tile prefill needs a token-major cache (stride_page == 64 * stride_token)");
    if (kv->stride_token >= (int64_t(1) << 24))  // 64 rows of 2-byte elements stay within 32-bit offsets
        return fail(BSA_ERR_UNSUPPORTED, "tile prefill needs stride_token < 2^24 elements");
    if (num_rows < 1) return fail(BSA_ERR_INVALID_ARG, "num_rows must be >= 1");
    if (kv_idx && idx_stride < 1) return fail(BSA_ERR_INVALID_ARG, "idx_stride must be >= 1");
    if (kv_idx && idx_stride > 1024) return fail(BSA_ERR_UNSUPPORTED, "idx_stride %d exceeds 1024", idx_stride);
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
        return fail(BSA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
    const size_t need = bsa_tile_prefill_workspace_bytes(kv, num_rows);
    if (!workspace || workspace_bytes < need)
        return fail(BSA_ERR_WORKSPACE, "tile prefill workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned16(workspace)) return fail(BSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return launched(bsa::launch_tile_prefill(q, num_q_heads, num_rows, v, tile_rows, kv_idx, idx_stride,
                                             softmax_scale, out, workspace, (hipStream_t)stream));
}

}  // extern "C"
