/*
 * bsa_oracle.c -- plain fp64 CPU oracle for query-aware block-sparse attention
 * over a chunked GQA KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the HIP library.
 *
 * Everything is double precision, written as plain loops in the order the
 * method's steps are stated, with no blocking, fusion or reordering.  The
 * library sort (qsort) is the only primitive used as a step.  OpenMP only
 * distributes independent (sequence, KV head) / (tile, KV head) / row units.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "Sparse Attention for Web Agents -- Offline Replay Records",
 *       section "The comparison" (method table; budget = page_size x top_k).
 *  [P2] "webarena" dataset README, section "Method configurations at a glance"
 *       (ratio budget with forced bos/eos pages).
 *  [P3] "Technische Samenvatting: Onzekerheidsgestuurde Selectie voor
 *       Blok-schaarse Aandacht", section "Methodologie" steps 1-5 (block
 *       scoring, per-tile selection, the cut-off margin sigma, head averaging
 *       with a per-layer quantile trigger, sentinel-padded expansion).
 *
 * Readings taken where the pages are silent are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Paged KV cache as the oracle sees it.                                     */
/* Element (physical page p, KV head h, slot o, dim d) of K or V lives at     */
/* base[p*stride_page + h*stride_head + o*stride_token + d].                  */
/* Logical page j of sequence b is physical page block_table[b*max_pages+j]   */
/* (block_table == NULL means physical page b*max_pages + j).                 */
/* ------------------------------------------------------------------------ */
typedef struct {
    const double *k;
    const double *v;
    int64_t stride_page, stride_head, stride_token;
    const int32_t *block_table;
    const int32_t *seq_lens;
    int32_t batch, num_kv_heads, head_dim, page_size, max_pages;
} orc_cache;

enum { ORC_ENVELOPE = 0, ORC_CENTROID = 1 };
enum { ORC_TOPK = 0, ORC_TOKENS = 1, ORC_RATIO = 2 };

static const double *token_row(const orc_cache *c, const double *base, int b, int h, int t)
{
    int page = t / c->page_size;
    int slot = t % c->page_size;
    int64_t phys = c->block_table ? c->block_table[(int64_t)b * c->max_pages + page]
                                  : (int64_t)b * c->max_pages + page;
    return base + phys * c->stride_page + (int64_t)h * c->stride_head + (int64_t)slot * c->stride_token;
}

/* Number of chunks of sequence b: fixed pages cover [0, L) in page_size steps
 * (the last page may be partial); variable chunks are given explicitly. */
static int chunk_count(const orc_cache *c, const int32_t *num_chunks, const int32_t *chunk_starts, int b)
{
    if (chunk_starts) return num_chunks[b];
    return (c->seq_lens[b] + c->page_size - 1) / c->page_size;
}

/* Token interval [s, e) of chunk ch of sequence b.  Fixed pages: [P*ch,
 * min(P*ch+P, L)).  Variable chunks: [start_ch, start_{ch+1}). */
static void chunk_interval(const orc_cache *c, const int32_t *chunk_starts, int max_chunks, int b, int ch,
                           int *s, int *e)
{
    if (chunk_starts) {
        *s = chunk_starts[(int64_t)b * (max_chunks + 1) + ch];
        *e = chunk_starts[(int64_t)b * (max_chunks + 1) + ch + 1];
    } else {
        int L = c->seq_lens[b];
        *s = ch * c->page_size;
        *e = *s + c->page_size < L ? *s + c->page_size : L;
    }
}

/* ------------------------------------------------------------------------ */
/* Step 1: per-chunk metadata ([P1] method table: envelope = per-dimension    */
/* min/max of the chunk's keys, centroid = mean of the chunk's keys; [P3]     */
/* step 1).  Over the chunk's valid tokens only; the centroid divides by the  */
/* number of valid tokens.  Outputs are [batch][H_kv][max_chunks][D].          */
/* ------------------------------------------------------------------------ */
void orc_chunk_meta(const orc_cache *c, const int32_t *chunk_starts, const int32_t *num_chunks,
                    int32_t max_chunks, double *kmin, double *kmax, double *cen)
{
    const int D = c->head_dim;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < c->batch; ++b)
        for (int h = 0; h < c->num_kv_heads; ++h) {
            int n = chunk_count(c, num_chunks, chunk_starts, b);
            for (int ch = 0; ch < n; ++ch) {
                int s, e;
                chunk_interval(c, chunk_starts, max_chunks, b, ch, &s, &e);
                int64_t o = (((int64_t)b * c->num_kv_heads + h) * max_chunks + ch) * D;
                for (int d = 0; d < D; ++d) {
                    double lo = INFINITY, hi = -INFINITY, sum = 0.0;
                    for (int t = s; t < e; ++t) {
                        double x = token_row(c, c->k, b, h, t)[d];
                        if (x < lo) lo = x;
                        if (x > hi) hi = x;
                        sum += x;
                    }
                    kmin[o + d] = lo;
                    kmax[o + d] = hi;
                    cen[o + d] = sum / (double)(e - s);
                }
            }
        }
}

/* One query head against one chunk's metadata.
 * Envelope ([P1] "per-dimension min/max upper bound"): sum over d of
 * max(q_d*kmin_d, q_d*kmax_d).  Centroid ([P1] "mean of chunk keys"): q . cen.
 * *denom receives sum_d |term_d|, the conditioning denominator of the sum. */
static double chunk_score(const double *q, const double *kmin, const double *kmax, const double *cen, int D,
                          int kind, double *denom)
{
    double s = 0.0, a = 0.0;
    for (int d = 0; d < D; ++d) {
        double term;
        if (kind == ORC_ENVELOPE) {
            double x = q[d] * kmin[d], y = q[d] * kmax[d];
            term = x > y ? x : y;
        } else {
            term = q[d] * cen[d];
        }
        s += term;
        a += fabs(term);
    }
    *denom = a;
    return s;
}

/* ------------------------------------------------------------------------ */
/* Step 2 (decode): score every chunk against the current query.  Selection  */
/* is per KV head, so the per-query-head scores of a GQA group are combined  */
/* by their maximum (the same max rule [P3] step 2 uses over a tile's rows).  */
/* Raw dot products, no 1/sqrt(d): a positive scale changes no ranking.       */
/* head_scores [B][H_q][max_chunks] (may be NULL), scores and denom           */
/* [B][H_kv][max_chunks]; denom is the largest per-head denominator.          */
/* ------------------------------------------------------------------------ */
void orc_score_decode(const double *q, int32_t num_q_heads, const orc_cache *c, const int32_t *chunk_starts,
                      const int32_t *num_chunks, int32_t max_chunks, const double *kmin, const double *kmax,
                      const double *cen, int32_t kind, double *head_scores, double *scores, double *denom)
{
    const int D = c->head_dim, Hkv = c->num_kv_heads, g = num_q_heads / Hkv;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < c->batch; ++b)
        for (int h = 0; h < Hkv; ++h) {
            int n = chunk_count(c, num_chunks, chunk_starts, b);
            for (int ch = 0; ch < n; ++ch) {
                int64_t mo = (((int64_t)b * Hkv + h) * max_chunks + ch) * D;
                double best = -INFINITY, best_den = 0.0;
                for (int jj = 0; jj < g; ++jj) {
                    int j = h * g + jj;
                    double den;
                    double s = chunk_score(q + ((int64_t)b * num_q_heads + j) * D, kmin + mo, kmax + mo, cen + mo, D,
                                           kind, &den);
                    if (head_scores) head_scores[((int64_t)b * num_q_heads + j) * max_chunks + ch] = s;
                    if (s > best) best = s;
                    if (den > best_den) best_den = den;
                }
                int64_t so = ((int64_t)b * Hkv + h) * max_chunks + ch;
                scores[so] = best;
                if (denom) denom[so] = best_den;
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Candidate order shared by every selection rule: score descending, and the  */
/* lower chunk index first among equal scores (the pages do not say how ties */
/* break; the lower index is the plainest deterministic choice).              */
/* ------------------------------------------------------------------------ */
typedef struct { double s; int32_t i; } cand;

static int cand_cmp(const void *pa, const void *pb)
{
    const cand *a = (const cand *)pa, *b = (const cand *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->i > b->i) - (a->i < b->i);
}

static int int_cmp(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* ------------------------------------------------------------------------ */
/* Step 3 (decode): per-KV-head top-k under a budget.                         */
/*  ORC_TOPK   ([P1] "Budget = page_size x top_k"): keep the first min(k, n)  */
/*             chunks of the order.                                          */
/*  ORC_RATIO  ([P2] "New directory" budget): K = min(n, max(1+bos+eos,       */
/*             floor(n*ratio))) with n the number of cached pages; page 0 is  */
/*             forced when bos, the last page when eos; the forced pages     */
/*             count inside K and the rest are filled in order.              */
/*  ORC_TOKENS (variable chunks filled "until the token budget is filled"):  */
/*             the longest prefix of the order whose total length <= budget  */
/*             (everything when the whole context fits).                     */
/* Output: kept ids ascending in sel_idx [B][H_kv][max_sel], count in         */
/* sel_count [B][H_kv].  Returns -1 if a count exceeds max_sel, else 0.      */
/* chunk_len [B][max_chunks] is needed for ORC_TOKENS only.                   */
/* ------------------------------------------------------------------------ */
int orc_select(const double *scores, int32_t batch, int32_t num_kv_heads, int32_t max_chunks,
               const int32_t *n_chunks, const int32_t *chunk_len, int32_t mode, int32_t top_k, int64_t tokens,
               double ratio, int32_t bos, int32_t eos, int32_t *sel_idx, int32_t *sel_count, int32_t max_sel)
{
    int err = 0;
    #pragma omp parallel for collapse(2) schedule(dynamic) reduction(| : err)
    for (int b = 0; b < batch; ++b)
        for (int h = 0; h < num_kv_heads; ++h) {
            int n = n_chunks[b];
            const double *row = scores + ((int64_t)b * num_kv_heads + h) * max_chunks;
            cand *order = (cand *)malloc(sizeof(cand) * (n > 0 ? n : 1));
            int32_t *keep = (int32_t *)malloc(sizeof(int32_t) * (n > 0 ? n : 1));
            char *taken = (char *)calloc(n > 0 ? n : 1, 1);
            for (int i = 0; i < n; ++i) { order[i].s = row[i]; order[i].i = i; }
            qsort(order, n, sizeof(cand), cand_cmp);
            int m = 0;
            if (mode == ORC_TOPK) {
                int K = top_k < n ? top_k : n;
                for (int i = 0; i < K; ++i) keep[m++] = order[i].i;
            } else if (mode == ORC_RATIO) {
                int forced_min = 1 + (bos ? 1 : 0) + (eos ? 1 : 0);
                int K = (int)floor((double)n * ratio);
                if (K < forced_min) K = forced_min;
                if (K > n) K = n;
                if (n > 0 && bos && !taken[0]) { taken[0] = 1; keep[m++] = 0; }
                if (n > 0 && eos && !taken[n - 1]) { taken[n - 1] = 1; keep[m++] = n - 1; }
                for (int i = 0; i < n && m < K; ++i)
                    if (!taken[order[i].i]) { taken[order[i].i] = 1; keep[m++] = order[i].i; }
            } else { /* ORC_TOKENS */
                const int32_t *len = chunk_len + (int64_t)b * max_chunks;
                int64_t total = 0;
                for (int i = 0; i < n; ++i) {
                    if (total + len[order[i].i] > tokens) break;
                    total += len[order[i].i];
                    keep[m++] = order[i].i;
                }
            }
            qsort(keep, m, sizeof(int32_t), int_cmp);
            if (m > max_sel) {
                err |= 1;
                m = max_sel;
            }
            int32_t *dst = sel_idx + ((int64_t)b * num_kv_heads + h) * max_sel;
            for (int i = 0; i < max_sel; ++i) dst[i] = i < m ? keep[i] : -1;
            sel_count[(int64_t)b * num_kv_heads + h] = m;
            free(order);
            free(keep);
            free(taken);
        }
    return err ? -1 : 0;
}

/* Softmax attention of one query row over an explicit token list, two-pass in
 * double: logits l_t = scale * q.k_t, weights exp(l_t - max l), output
 * sum_t w_t v_t / sum_t w_t.  rows_k / rows_v hold the token rows. */
static void attend(const double *q, const double *const *rows_k, const double *const *rows_v, int n, int D,
                   double scale, double *logit, double *out)
{
    double mx = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += q[d] * rows_k[t][d];
        logit[t] = s * scale;
        if (logit[t] > mx) mx = logit[t];
    }
    double den = 0.0;
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    for (int t = 0; t < n; ++t) {
        double w = exp(logit[t] - mx);
        den += w;
        for (int d = 0; d < D; ++d) out[d] += w * rows_v[t][d];
    }
    for (int d = 0; d < D; ++d) out[d] /= den;
}

/* ------------------------------------------------------------------------ */
/* Step 4 (decode): attend only to the selected chunks ([P1] "attend only to  */
/* those").  Query head j of sequence b reads KV head j / (H_q/H_kv); the     */
/* single decode query sees every cached token of its selected chunks.      */
/* sel_idx == NULL means dense attention over all L tokens.                   */
/* out [B][H_q][D].                                                          */
/* ------------------------------------------------------------------------ */
void orc_decode_attn(const double *q, int32_t num_q_heads, const orc_cache *c, const int32_t *chunk_starts,
                     const int32_t *num_chunks, int32_t max_chunks, const int32_t *sel_idx,
                     const int32_t *sel_count, int32_t max_sel, double scale, double *out)
{
    const int D = c->head_dim, Hkv = c->num_kv_heads, g = num_q_heads / Hkv;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < c->batch; ++b)
        for (int j = 0; j < num_q_heads; ++j) {
            int h = j / g, L = c->seq_lens[b];
            const double **rk = (const double **)malloc(sizeof(double *) * (L > 0 ? L : 1));
            const double **rv = (const double **)malloc(sizeof(double *) * (L > 0 ? L : 1));
            double *logit = (double *)malloc(sizeof(double) * (L > 0 ? L : 1));
            int n = 0;
            if (!sel_idx) {
                for (int t = 0; t < L; ++t) {
                    rk[n] = token_row(c, c->k, b, h, t);
                    rv[n] = token_row(c, c->v, b, h, t);
                    ++n;
                }
            } else {
                int cnt = sel_count[(int64_t)b * Hkv + h];
                const int32_t *ids = sel_idx + ((int64_t)b * Hkv + h) * max_sel;
                for (int i = 0; i < cnt; ++i) {
                    int s, e;
                    chunk_interval(c, chunk_starts, max_chunks, b, ids[i], &s, &e);
                    for (int t = s; t < e; ++t) {
                        rk[n] = token_row(c, c->k, b, h, t);
                        rv[n] = token_row(c, c->v, b, h, t);
                        ++n;
                    }
                }
            }
            attend(q + ((int64_t)b * num_q_heads + j) * D, rk, rv, n, D, scale, logit,
                   out + ((int64_t)b * num_q_heads + j) * D);
            free(rk);
            free(rv);
            free(logit);
        }
}

/* Number of key blocks a query tile can see.  Causal: every block that starts
 * at or before the tile's last row; the diagonal block is visible and competes
 * in the top-k like any other (its keys after a row are masked only in the
 * attention step). */
static int tile_visible(int t, int T, int tile_rows, int block_size, int n_blocks, int causal)
{
    if (!causal) return n_blocks;
    int last = (t + 1) * tile_rows - 1;
    if (last > T - 1) last = T - 1;
    int v = last / block_size + 1;
    return v < n_blocks ? v : n_blocks;
}

/* ------------------------------------------------------------------------ */
/* Step 2 (prefill, [P3] step 2): the score of block bk for tile t and KV     */
/* head h is the maximum, over the tile's rows and the GQA group's query      */
/* heads, of the block score of step 1.  Q [T][H_q][D] token-major; metadata */
/* [H_kv][n_blocks][D].  Tiles listed in tiles[0..n_list) (NULL = all);      */
/* out / denom [n_list][H_kv][n_blocks]; blocks a tile cannot see get -inf.  */
/* ------------------------------------------------------------------------ */
void orc_tile_scores(const double *Q, int32_t T, int32_t num_q_heads, int32_t num_kv_heads, int32_t D,
                     const double *kmin, const double *kmax, const double *cen, int32_t n_blocks,
                     int32_t tile_rows, int32_t block_size, int32_t causal, int32_t kind, const int32_t *tiles,
                     int32_t n_list, double *out, double *denom)
{
    const int g = num_q_heads / num_kv_heads;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int it = 0; it < n_list; ++it)
        for (int h = 0; h < num_kv_heads; ++h) {
            int t = tiles ? tiles[it] : it;
            int vis = tile_visible(t, T, tile_rows, block_size, n_blocks, causal);
            int r0 = t * tile_rows, r1 = r0 + tile_rows < T ? r0 + tile_rows : T;
            for (int bk = 0; bk < n_blocks; ++bk) {
                int64_t o = ((int64_t)it * num_kv_heads + h) * n_blocks + bk;
                if (bk >= vis) {
                    out[o] = -INFINITY;
                    if (denom) denom[o] = 0.0;
                    continue;
                }
                int64_t mo = ((int64_t)h * n_blocks + bk) * D;
                double best = -INFINITY, best_den = 0.0;
                for (int r = r0; r < r1; ++r)
                    for (int jj = 0; jj < g; ++jj) {
                        double den;
                        double s = chunk_score(Q + ((int64_t)r * num_q_heads + h * g + jj) * D, kmin + mo, kmax + mo,
                                               cen + mo, D, kind, &den);
                        if (s > best) best = s;
                        if (den > best_den) best_den = den;
                    }
                out[o] = best;
                if (denom) denom[o] = best_den;
            }
        }
}

/* Empirical quantile with linear interpolation between order statistics
 * (Hyndman-Fan definition 7): position (m-1)*p in the ascending sample. */
static int dbl_cmp(const void *pa, const void *pb)
{
    double a = *(const double *)pa, b = *(const double *)pb;
    return (a > b) - (a < b);
}

double orc_quantile(const double *x, int32_t m, double p)
{
    if (m <= 0) return NAN;
    double *s = (double *)malloc(sizeof(double) * m);
    memcpy(s, x, sizeof(double) * m);
    qsort(s, m, sizeof(double), dbl_cmp);
    double pos = (m - 1) * p;
    int lo = (int)floor(pos);
    double frac = pos - lo;
    double r = lo + 1 < m ? s[lo] + frac * (s[lo + 1] - s[lo]) : s[lo];
    free(s);
    return r;
}

/* ------------------------------------------------------------------------ */
/* Steps 2-5 of the uncertainty router ([P3] "Methodologie").                 */
/*  For each (tile t, KV head h) over its n visible blocks, order the blocks  */
/*  by score (descending, lower index first).                                */
/*  Step 3: sigma = (s_(k-1) - s_(k)) / (s_(0) - s_(k)) with s_(0) the        */
/*  largest score, 0-indexed.  When s_(0) == s_(k) the top k+1 tie and the    */
/*  cut is maximally ambiguous: sigma = 0.  A tile with n <= k has no cut:    */
/*  sigma = 1, it is not eligible and never triggers.                        */
/*  Step 4: sigma_bar_t = mean over the KV heads; the threshold tau is the    */
/*  `quantile` quantile of sigma_bar over the eligible tiles (or fixed_tau    */
/*  when use_fixed); tile t triggers when eligible and sigma_bar_t < tau.    */
/*  Step 5: kv_idx[t][h] = the first k blocks of the order (first            */
/*  min(rho*k, n) when triggered), ascending, then -1 sentinels up to rho*k.  */
/* ts [n_tiles][H_kv][n_blocks]; n_visible [n_tiles];                         */
/* kv_idx [n_tiles][H_kv][rho*k]; sigma [n_tiles][H_kv]; sigma_bar,           */
/* eligible, triggered [n_tiles]; *tau.                                       */
/* ------------------------------------------------------------------------ */
void orc_router(const double *ts, int32_t n_tiles, int32_t num_kv_heads, int32_t n_blocks,
                const int32_t *n_visible, int32_t k, int32_t rho, double quantile, int32_t use_fixed,
                double fixed_tau, int32_t *kv_idx, double *sigma, double *sigma_bar, uint8_t *eligible,
                uint8_t *triggered, double *tau)
{
    const int width = rho * k;
    /* score order of every (tile, head), truncated to rho*k entries */
    int32_t *top = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_tiles * num_kv_heads * width);

    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int t = 0; t < n_tiles; ++t)
        for (int h = 0; h < num_kv_heads; ++h) {
            int n = n_visible[t];
            const double *row = ts + ((int64_t)t * num_kv_heads + h) * n_blocks;
            cand *order = (cand *)malloc(sizeof(cand) * (n > 0 ? n : 1));
            for (int i = 0; i < n; ++i) { order[i].s = row[i]; order[i].i = i; }
            qsort(order, n, sizeof(cand), cand_cmp);
            double sg;
            if (n <= k) {
                sg = 1.0;
            } else {
                double s0 = order[0].s, sk1 = order[k - 1].s, sk = order[k].s;
                sg = (s0 == sk) ? 0.0 : (sk1 - sk) / (s0 - sk);
            }
            sigma[(int64_t)t * num_kv_heads + h] = sg;
            int32_t *dst = top + ((int64_t)t * num_kv_heads + h) * width;
            for (int i = 0; i < width; ++i) dst[i] = i < n ? order[i].i : -1;
            free(order);
        }

    double *elig_vals = (double *)malloc(sizeof(double) * (n_tiles > 0 ? n_tiles : 1));
    int m = 0;
    for (int t = 0; t < n_tiles; ++t) {
        double acc = 0.0;
        for (int h = 0; h < num_kv_heads; ++h) acc += sigma[(int64_t)t * num_kv_heads + h];
        sigma_bar[t] = acc / num_kv_heads;
        eligible[t] = n_visible[t] > k;
        if (eligible[t]) elig_vals[m++] = sigma_bar[t];
    }
    *tau = use_fixed ? fixed_tau : orc_quantile(elig_vals, m, quantile);
    free(elig_vals);

    for (int t = 0; t < n_tiles; ++t) triggered[t] = eligible[t] && (sigma_bar[t] < *tau);

    #pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < n_tiles; ++t)
        for (int h = 0; h < num_kv_heads; ++h) {
            int n = n_visible[t];
            int keep = triggered[t] ? width : k;
            if (keep > n) keep = n;
            int32_t *dst = kv_idx + ((int64_t)t * num_kv_heads + h) * width;
            const int32_t *src = top + ((int64_t)t * num_kv_heads + h) * width;
            for (int i = 0; i < keep; ++i) dst[i] = src[i];
            qsort(dst, keep, sizeof(int32_t), int_cmp);
            for (int i = keep; i < width; ++i) dst[i] = -1;
        }
    free(top);
}

/* ------------------------------------------------------------------------ */
/* Step 5 attention (prefill, [P3] step 5): row r of tile t, query head j,    */
/* attends causally (key position <= r) to the keys of the non-sentinel       */
/* blocks listed in kv_idx[t][j / g].  kv_idx == NULL: dense causal.          */
/* Q [T][H_q][D], K/V [T][H_kv][D] token-major.  Rows listed in rows[];       */
/* out [n_rows][H_q][D].                                                     */
/* ------------------------------------------------------------------------ */
void orc_tile_attn(const double *Q, const double *K, const double *V, int32_t T, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t D, int32_t block_size, int32_t tile_rows, const int32_t *kv_idx,
                   int32_t idx_stride, double scale, const int32_t *rows, int32_t n_rows, double *out)
{
    const int g = num_q_heads / num_kv_heads;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int ir = 0; ir < n_rows; ++ir)
        for (int j = 0; j < num_q_heads; ++j) {
            int r = rows[ir], h = j / g, t = r / tile_rows;
            const double **rk = (const double **)malloc(sizeof(double *) * (r + 1));
            const double **rv = (const double **)malloc(sizeof(double *) * (r + 1));
            double *logit = (double *)malloc(sizeof(double) * (r + 1));
            int n = 0;
            if (!kv_idx) {
                for (int p = 0; p <= r; ++p) {
                    rk[n] = K + ((int64_t)p * num_kv_heads + h) * D;
                    rv[n] = V + ((int64_t)p * num_kv_heads + h) * D;
                    ++n;
                }
            } else {
                const int32_t *ids = kv_idx + ((int64_t)t * num_kv_heads + h) * idx_stride;
                for (int i = 0; i < idx_stride; ++i) {
                    if (ids[i] < 0) continue;
                    for (int p = ids[i] * block_size; p < (ids[i] + 1) * block_size && p < T; ++p) {
                        if (p > r) break;
                        rk[n] = K + ((int64_t)p * num_kv_heads + h) * D;
                        rv[n] = V + ((int64_t)p * num_kv_heads + h) * D;
                        ++n;
                    }
                }
            }
            attend(Q + ((int64_t)r * num_q_heads + j) * D, rk, rv, n, D, scale, logit,
                   out + ((int64_t)ir * num_q_heads + j) * D);
            free(rk);
            free(rv);
            free(logit);
        }
}
