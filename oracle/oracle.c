/*
 * oracle.c -- plain, slow, fp64 CPU reference for block-sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library; it is built with gcc.
 *
 * Sources (cited by page title and section; no listing is reproduced):
 *  [G]  "Sparse Attention" glossary entry (Ultralytics; German, Turkish,
 *       Vietnamese and Spanish editions carry the same content).
 *       - section on common sparsity patterns: sliding window over previous
 *         tokens, strided tokens, global tokens, random links (BigBird),
 *         attention sinks; content-based DeepSeek Sparse Attention, whose
 *         indexer scores every earlier token and keeps the 2,048 best.
 *       - section on turning a pattern into savings: the local_plus_sinks
 *         mask function (causal AND (q-kv <= window OR kv < sinks)), the
 *         split of the mask into 128 x 128 blocks and the sparsity figure
 *         defined as the share of blocks holding no allowed pair.
 *  [B]  "Sparse transformers: how to cut the O(n^2) of attention" blog
 *       (1gpt.online), section on how it looks in code: dense scores
 *       q.k^T / sqrt(d), disallowed pairs set to -inf, softmax, times V;
 *       section on the main sparsity templates (strided, fixed, sliding
 *       window, global tokens) and on combining them.
 *
 * What is computed (the plain definitions; nothing is blocked or fused):
 *  - orc_allowed: the per-pair predicate, a union of the pattern terms,
 *    intersected with causality when requested ([G] patterns, [B] templates).
 *  - orc_block_lists: for every (query block, key block) cell, the number of
 *    allowed pairs inside the clipped tile; live = count > 0, full = count ==
 *    tile size, partial otherwise; live key blocks listed in ascending order
 *    ([G] block split and sparsity definition).
 *  - orc_attn_rows: for each requested (batch*head, query) row, fp64 scores
 *    over every allowed key, m = max, LSE = m + ln(sum exp(s - m)),
 *    O = sum exp(s - LSE) v  ([B] masked attention: masking with -inf and a
 *    softmax is the same as a softmax restricted to the allowed keys).
 *    A row with no allowed key gives O = 0, LSE = -inf.
 *  - orc_attn_gather_rows: the same softmax restricted to an explicit key
 *    list (the per-query top-k set of [G] DeepSeek Sparse Attention).
 *  - orc_indexer_scores: indexer score of query t and key s <= t as a
 *    float32 sequential fused-multiply-add chain over the indexer dimension
 *    (the pages give no formula; this fixed order is the reading adopted),
 *    plus the fp64 value of the same dot product.
 *  - orc_topk_rows: the k candidates that come first in the total order
 *    (score descending, index ascending; a NaN score above every number),
 *    emitted in ascending index order.
 *  - orc_select_blocks: content-selected key blocks per (batch*head, query
 *    block), the "selection of the most relevant blocks" of [G]'s common
 *    sparsity patterns (Native Sparse Attention), read as: the block's own
 *    (diagonal) key blocks, plus the n_select causally reachable key blocks
 *    of highest score <mean query of the block, mean key of the block>
 *    (ties to the lower block), means taken over the block size in fp64.
 *  - orc_attn_sel_rows: attention of each row over the keys of its query
 *    block's selected key blocks, causally ([B] masked attention with the
 *    mask given by the selected blocks).
 *  - orc_attn_bwd: the gradient of the masked attention ([B]'s scores, -inf
 *    fill, softmax, times V -- [G] notes NSA is trained end to end) with
 *    respect to Q, K and V for an upstream gradient dO, by the chain rule on
 *    the definition: P = softmax over the allowed keys, dV = P^T dO,
 *    dP = dO V^T, dS = P * (dP - rowsum(P * dP)), dQ = scale dS K,
 *    dK = scale dS^T Q.
 *
 * Inputs are raw bfloat16 bit patterns (uint16); each is widened exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t causal;
    int64_t q_offset;
    int64_t window_left;   /* < 0: local term off */
    int64_t window_right;
    int64_t sinks;
    int64_t stride;        /* <= 0: strided term off */
    int64_t stride_phase;
    int64_t global_tokens;
    int64_t unit;          /* <= 0: unit-level terms off */
    int64_t unit_window;   /* < 0: unit band off */
    const int32_t *rand_units; /* host table [rand_rows, n_rand], -1 = empty */
    int64_t n_rand;
    int64_t rand_rows;
} orc_pattern;

static double bf16_to_f64(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Is the pair (query position q, key position kv) allowed?  q and kv are
 * absolute positions (q already includes the pattern's offset). */
int orc_allowed(const orc_pattern *p, int64_t q, int64_t kv)
{
    if (p->causal && kv > q)
        return 0;
    if (p->window_left >= 0 && q - kv <= p->window_left && kv - q <= p->window_right)
        return 1;
    if (kv < p->sinks)
        return 1;
    if (p->stride > 0 && q >= kv && (q - kv) % p->stride == p->stride_phase)
        return 1;
    if (q < p->global_tokens || kv < p->global_tokens)
        return 1;
    if (p->unit > 0) {
        int64_t qu = q / p->unit, ku = kv / p->unit;
        int64_t du = qu > ku ? qu - ku : ku - qu;
        if (p->unit_window >= 0 && du <= p->unit_window)
            return 1;
        if (p->rand_units && p->n_rand > 0 && qu < p->rand_rows) {
            for (int64_t r = 0; r < p->n_rand; ++r)
                if (p->rand_units[qu * p->n_rand + r] == ku)
                    return 1;
        }
    }
    return 0;
}

/* Block lists by brute force over every pair of every cell.
 * kv_count [nqb], kv_index [nqb, nkb] (ascending, -1 padded),
 * kv_partial [nqb, nkb] aligned with kv_index (1 = partial, 0 = full or pad),
 * live_pairs = total allowed pairs, cell_counts [nqb, nkb] optional. */
void orc_block_lists(const orc_pattern *p, int64_t n_q, int64_t n_kv, int32_t bq, int32_t bk,
                     int32_t *kv_count, int32_t *kv_index, uint8_t *kv_partial,
                     int64_t *live_pairs, int64_t *cell_counts)
{
    int64_t nqb = (n_q + bq - 1) / bq, nkb = (n_kv + bk - 1) / bk;
    int64_t total = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : total)
    for (int64_t i = 0; i < nqb; ++i) {
        int64_t q0 = i * bq, q1 = q0 + bq < n_q ? q0 + bq : n_q;
        int32_t n_live = 0;
        for (int64_t j = 0; j < nkb; ++j) {
            int64_t k0 = j * bk, k1 = k0 + bk < n_kv ? k0 + bk : n_kv;
            int64_t c = 0;
            for (int64_t q = q0; q < q1; ++q)
                for (int64_t kv = k0; kv < k1; ++kv)
                    c += orc_allowed(p, q + p->q_offset, kv);
            if (cell_counts)
                cell_counts[i * nkb + j] = c;
            total += c;
            if (c > 0) {
                kv_index[i * nkb + n_live] = (int32_t)j;
                kv_partial[i * nkb + n_live] = (uint8_t)(c != (q1 - q0) * (k1 - k0));
                ++n_live;
            }
        }
        kv_count[i] = n_live;
        for (int64_t e = n_live; e < nkb; ++e) {
            kv_index[i * nkb + e] = -1;
            kv_partial[i * nkb + e] = 0;
        }
    }
    *live_pairs = total;
}

/* Softmax-weighted sum over an explicit key list, fp64 throughout. */
static void attend_list(const uint16_t *qrow, const uint16_t *kbase, const uint16_t *vbase,
                        int32_t d, double scale, const int64_t *keys, int64_t nk,
                        double *s_buf, double *o, double *lse)
{
    for (int32_t c = 0; c < d; ++c)
        o[c] = 0.0;
    if (nk == 0) {
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int64_t e = 0; e < nk; ++e) {
        const uint16_t *krow = kbase + keys[e] * (int64_t)d;
        double acc = 0.0;
        for (int32_t c = 0; c < d; ++c)
            acc += bf16_to_f64(qrow[c]) * bf16_to_f64(krow[c]);
        s_buf[e] = acc * scale;
        if (s_buf[e] > m)
            m = s_buf[e];
    }
    double sum = 0.0;
    for (int64_t e = 0; e < nk; ++e)
        sum += exp(s_buf[e] - m);
    double L = m + log(sum);
    for (int64_t e = 0; e < nk; ++e) {
        double w = exp(s_buf[e] - L);
        const uint16_t *vrow = vbase + keys[e] * (int64_t)d;
        for (int32_t c = 0; c < d; ++c)
            o[c] += w * bf16_to_f64(vrow[c]);
    }
    *lse = L;
}

/* rows[r] = (b*H + h) * n_q + query_row; tensors contiguous [B, H, N, d]. */
void orc_attn_rows(const orc_pattern *p, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   int64_t n_q, int64_t n_kv, int32_t d, double scale, const int64_t *rows,
                   int64_t n_rows, double *o, double *lse, int64_t *n_allowed)
{
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_kv > 0 ? n_kv : 1));
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(n_kv > 0 ? n_kv : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t bh = rows[r] / n_q, qi = rows[r] % n_q;
            int64_t qpos = qi + p->q_offset;
            int64_t nk = 0;
            for (int64_t kv = 0; kv < n_kv; ++kv)
                if (orc_allowed(p, qpos, kv))
                    keys[nk++] = kv;
            if (n_allowed)
                n_allowed[r] = nk;
            attend_list(q + (bh * n_q + qi) * (int64_t)d, k + bh * n_kv * (int64_t)d,
                        v + bh * n_kv * (int64_t)d, d, scale, keys, nk, s_buf, o + r * (int64_t)d,
                        lse + r);
        }
        free(keys);
        free(s_buf);
    }
}

/* Gather attention: idx [n_q, topk] (per query row; -1 entries are padding),
 * shared by every (b, h) when idx_bh_stride == 0, else offset by bh * stride. */
void orc_attn_gather_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t n_q,
                          int64_t n_kv, int32_t d, double scale, const int32_t *idx, int32_t topk,
                          int64_t idx_bh_stride, const int64_t *rows, int64_t n_rows, double *o,
                          double *lse)
{
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(topk > 0 ? topk : 1));
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(topk > 0 ? topk : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t bh = rows[r] / n_q, qi = rows[r] % n_q;
            const int32_t *list = idx + bh * idx_bh_stride + qi * (int64_t)topk;
            int64_t nk = 0;
            for (int32_t e = 0; e < topk; ++e)
                if (list[e] >= 0 && list[e] < n_kv)
                    keys[nk++] = list[e];
            attend_list(q + (bh * n_q + qi) * (int64_t)d, k + bh * n_kv * (int64_t)d,
                        v + bh * n_kv * (int64_t)d, d, scale, keys, nk, s_buf, o + r * (int64_t)d,
                        lse + r);
        }
        free(keys);
        free(s_buf);
    }
}

/* Indexer scores for query rows `rows` (row r has position q_offset + r) and
 * every key s < n_kv: candidates s <= t get the fp32 FMA chain value, the
 * others -inf.  exact (optional) gets the fp64 dot product. */
void orc_indexer_scores(const uint16_t *qi, const uint16_t *ki, int64_t n_kv, int32_t d,
                        int64_t q_offset, const int64_t *rows, int64_t n_rows, float *sigma,
                        double *exact)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t t = rows[r] + q_offset;
        const uint16_t *qr = qi + rows[r] * (int64_t)d;
        for (int64_t s = 0; s < n_kv; ++s) {
            float *out = sigma + r * n_kv + s;
            if (s > t) {
                *out = -INFINITY;
                if (exact)
                    exact[r * n_kv + s] = -INFINITY;
                continue;
            }
            const uint16_t *kr = ki + s * (int64_t)d;
            float acc = 0.0f;
            double ex = 0.0;
            for (int32_t c = 0; c < d; ++c) {
                acc = fmaf(bf16_to_f32(qr[c]), bf16_to_f32(kr[c]), acc);
                ex += bf16_to_f64(qr[c]) * bf16_to_f64(kr[c]);
            }
            *out = acc;
            if (exact)
                exact[r * n_kv + s] = ex;
        }
    }
}

typedef struct {
    float key;
    int32_t idx;
} orc_scored;

/* Total order: larger score first, then smaller index first.  -0.0 and +0.0
 * are equal scores.  The pages rank by score only; to make the order total on
 * every float input, a NaN score (of either sign) ranks above every number
 * and NaNs are equal scores (so among NaNs the smaller index comes first). */
static int cmp_scored(const void *a, const void *b)
{
    const orc_scored *x = (const orc_scored *)a, *y = (const orc_scored *)b;
    int xn = isnan(x->key), yn = isnan(y->key);
    if (xn != yn)
        return xn ? -1 : 1;
    if (!xn) {
        if (x->key > y->key)
            return -1;
        if (x->key < y->key)
            return 1;
    }
    return (x->idx > y->idx) - (x->idx < y->idx);
}

static int cmp_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Top-k per row: candidates are the first n_cand[r] entries of sigma row r.
 * Output idx [n_rows, k]: the selected indices ascending, -1 padded. */
void orc_topk_rows(const float *sigma, const int64_t *n_cand, int64_t n_rows, int64_t n_kv,
                   int32_t k, int32_t *idx)
{
#pragma omp parallel
    {
        orc_scored *buf = (orc_scored *)malloc(sizeof(orc_scored) * (size_t)(n_kv > 0 ? n_kv : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t nc = n_cand[r] < n_kv ? n_cand[r] : n_kv;
            for (int64_t s = 0; s < nc; ++s) {
                buf[s].key = sigma[r * n_kv + s];
                buf[s].idx = (int32_t)s;
            }
            qsort(buf, (size_t)nc, sizeof(orc_scored), cmp_scored);
            int64_t take = nc < k ? nc : k;
            int32_t *out = idx + r * (int64_t)k;
            for (int64_t e = 0; e < take; ++e)
                out[e] = buf[e].idx;
            qsort(out, (size_t)take, sizeof(int32_t), cmp_i32);
            for (int64_t e = take; e < k; ++e)
                out[e] = -1;
        }
        free(buf);
    }
}

/* Content-selected key blocks.  q [BH, n_q, d], k [BH, n_kv, d] contiguous
 * bf16 bits; query row r has position q_offset + r.  For every (bh, query
 * block i) with rows [i*bq, min((i+1)*bq, n_q)) and positions [p0, p1]:
 *   qm[c] = (sum over the block's rows, in row order, of q[r][c]) / bq
 *   km_j[c] = (sum over key block j's rows of k[s][c]) / bk
 * (rows past the end count as zero; bq, bk are powers of two, so the
 * division is exact), both in fp64;
 *   score(i, j) = qm . km_j, an fp64 fused multiply-add chain over c;
 *   reachable: j*bk <= p1 (some key of the block is causally visible);
 *   own: the key blocks holding positions p0 .. p1;
 *   selected = own  +  the n_sel reachable, not-own blocks first in the
 *   order (score descending, block ascending).
 * Output per (bh, i): kv_count, kv_index (ascending, -1 padded), kv_partial
 * (1 when some pair of the clipped tile is not causal), and live_pairs = the
 * causal pairs over all selected tiles. */
void orc_select_blocks(const uint16_t *q, const uint16_t *k, int64_t BH, int64_t n_q, int64_t n_kv, int32_t d,
                       int64_t q_offset, int32_t bq, int32_t bk, int32_t n_sel, int32_t *kv_count,
                       int32_t *kv_index, uint8_t *kv_partial, int64_t *live_pairs)
{
    int64_t nqb = (n_q + bq - 1) / bq, nkb = (n_kv + bk - 1) / bk;
    int64_t total = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : total)
    for (int64_t item = 0; item < BH * nqb; ++item) {
        int64_t bh = item / nqb, i = item % nqb;
        int64_t r0 = i * bq, r1 = r0 + bq < n_q ? r0 + bq : n_q;
        int64_t p0 = q_offset + r0, p1 = q_offset + r1 - 1;
        double *qm = (double *)malloc(sizeof(double) * (size_t)d);
        double *km = (double *)malloc(sizeof(double) * (size_t)d);
        double *score = (double *)malloc(sizeof(double) * (size_t)(nkb > 0 ? nkb : 1));
        unsigned char *sel = (unsigned char *)calloc((size_t)(nkb > 0 ? nkb : 1), 1);
        for (int32_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t r = r0; r < r1; ++r)
                acc += bf16_to_f64(q[(bh * n_q + r) * d + c]);
            qm[c] = acc / bq;
        }
        for (int64_t j = 0; j < nkb; ++j) {
            int64_t s0 = j * bk, s1 = s0 + bk < n_kv ? s0 + bk : n_kv;
            for (int32_t c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int64_t s = s0; s < s1; ++s)
                    acc += bf16_to_f64(k[(bh * n_kv + s) * d + c]);
                km[c] = acc / bk;
            }
            double dot = 0.0;
            for (int32_t c = 0; c < d; ++c)
                dot = fma(qm[c], km[c], dot);
            score[j] = dot;
            int own = s0 <= p1 && s1 - 1 >= p0;
            if (own)
                sel[j] = 1;
        }
        /* n_sel times: the best reachable block not taken yet */
        for (int32_t t = 0; t < n_sel; ++t) {
            int64_t best = -1;
            for (int64_t j = 0; j < nkb; ++j) {
                if (sel[j] || j * bk > p1)
                    continue;
                if (best < 0 || score[j] > score[best])
                    best = j;
            }
            if (best < 0)
                break;
            sel[best] = 2;
        }
        int32_t n_live = 0;
        for (int64_t j = 0; j < nkb; ++j) {
            if (!sel[j])
                continue;
            int64_t s0 = j * bk, s1 = s0 + bk < n_kv ? s0 + bk : n_kv;
            int64_t cnt = 0;
            for (int64_t qp = p0; qp <= p1; ++qp)
                for (int64_t s = s0; s < s1; ++s)
                    cnt += s <= qp;
            total += cnt;
            kv_index[item * nkb + n_live] = (int32_t)j;
            kv_partial[item * nkb + n_live] = (uint8_t)(cnt != (p1 - p0 + 1) * (s1 - s0));
            ++n_live;
        }
        kv_count[item] = n_live;
        for (int64_t e = n_live; e < nkb; ++e) {
            kv_index[item * nkb + e] = -1;
            kv_partial[item * nkb + e] = 0;
        }
        free(qm);
        free(km);
        free(score);
        free(sel);
    }
    *live_pairs = total;
}

/* Attention of rows over content-selected blocks: row (bh, r) attends to the
 * keys s <= q_offset + r whose block s / bk is listed for (bh, r / bq) in
 * kv_count / kv_index ([BH, nqb] / [BH, nqb, nkb], as orc_select_blocks
 * writes them).  rows[] as in orc_attn_rows. */
void orc_attn_sel_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t n_q, int64_t n_kv,
                       int32_t d, double scale, int64_t q_offset, int32_t bq, int32_t bk, const int32_t *kv_count,
                       const int32_t *kv_index, const int64_t *rows, int64_t n_rows, double *o, double *lse)
{
    int64_t nqb = (n_q + bq - 1) / bq, nkb = (n_kv + bk - 1) / bk;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_kv > 0 ? n_kv : 1));
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(n_kv > 0 ? n_kv : 1));
        unsigned char *in = (unsigned char *)malloc((size_t)(nkb > 0 ? nkb : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t bh = rows[r] / n_q, qi = rows[r] % n_q;
            int64_t item = bh * nqb + qi / bq;
            memset(in, 0, (size_t)(nkb > 0 ? nkb : 1));
            for (int32_t e = 0; e < kv_count[item]; ++e) {
                int32_t j = kv_index[item * nkb + e];
                if (j >= 0 && j < nkb)
                    in[j] = 1;
            }
            int64_t nk = 0;
            for (int64_t s = 0; s < n_kv; ++s)
                if (s <= q_offset + qi && in[s / bk])
                    keys[nk++] = s;
            attend_list(q + (bh * n_q + qi) * (int64_t)d, k + bh * n_kv * (int64_t)d,
                        v + bh * n_kv * (int64_t)d, d, scale, keys, nk, s_buf, o + r * (int64_t)d, lse + r);
        }
        free(keys);
        free(s_buf);
        free(in);
    }
}

/* Gradients of the masked attention of the (b*H + h) slices listed in bh[]
 * (all their rows), fp64.  q, dout [BH, n_q, d], k, v [BH, n_kv, d] bf16
 * bits; dq [n_bh, n_q, d], dk, dv [n_bh, n_kv, d] in the order of bh[].
 * Pass 1, per query row: the allowed keys, P = exp(s - LSE), dq.
 * Pass 2, per key row: the queries that may see it, dk and dv. */
void orc_attn_bwd(const orc_pattern *p, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const uint16_t *dout, int64_t n_q, int64_t n_kv, int32_t d, double scale, const int64_t *bh,
                  int64_t n_bh, double *dq, double *dk, double *dv)
{
    double *lse = (double *)malloc(sizeof(double) * (size_t)(n_bh * n_q > 0 ? n_bh * n_q : 1));
    double *dsum = (double *)malloc(sizeof(double) * (size_t)(n_bh * n_q > 0 ? n_bh * n_q : 1));
    /* pass 1: per query row */
#pragma omp parallel
    {
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(n_kv > 0 ? n_kv : 1));
        double *dp_buf = (double *)malloc(sizeof(double) * (size_t)(n_kv > 0 ? n_kv : 1));
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_kv > 0 ? n_kv : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n_bh * n_q; ++r) {
            int64_t t = r / n_q, qi = r % n_q, g = bh[t];
            const uint16_t *qrow = q + (g * n_q + qi) * d, *grow = dout + (g * n_q + qi) * d;
            const uint16_t *kb = k + g * n_kv * d, *vb = v + g * n_kv * d;
            int64_t nk = 0;
            for (int64_t kv = 0; kv < n_kv; ++kv)
                if (orc_allowed(p, qi + p->q_offset, kv))
                    keys[nk++] = kv;
            double *dqr = dq + r * d;
            for (int32_t c = 0; c < d; ++c)
                dqr[c] = 0.0;
            if (nk == 0) {
                lse[r] = -INFINITY;
                dsum[r] = 0.0;
                continue;
            }
            double m = -INFINITY;
            for (int64_t e = 0; e < nk; ++e) {
                double acc = 0.0, acc2 = 0.0;
                for (int32_t c = 0; c < d; ++c) {
                    acc += bf16_to_f64(qrow[c]) * bf16_to_f64(kb[keys[e] * d + c]);
                    acc2 += bf16_to_f64(grow[c]) * bf16_to_f64(vb[keys[e] * d + c]);
                }
                s_buf[e] = acc * scale;
                dp_buf[e] = acc2;
                if (s_buf[e] > m)
                    m = s_buf[e];
            }
            double sum = 0.0;
            for (int64_t e = 0; e < nk; ++e)
                sum += exp(s_buf[e] - m);
            double L = m + log(sum), D = 0.0;
            for (int64_t e = 0; e < nk; ++e)
                D += exp(s_buf[e] - L) * dp_buf[e];
            lse[r] = L;
            dsum[r] = D;
            for (int64_t e = 0; e < nk; ++e) {
                double ds = exp(s_buf[e] - L) * (dp_buf[e] - D);
                for (int32_t c = 0; c < d; ++c)
                    dqr[c] += scale * ds * bf16_to_f64(kb[keys[e] * d + c]);
            }
        }
        free(s_buf);
        free(dp_buf);
        free(keys);
    }
    /* pass 2: per key row */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < n_bh * n_kv; ++r) {
        int64_t t = r / n_kv, kv = r % n_kv, g = bh[t];
        const uint16_t *krow = k + (g * n_kv + kv) * d, *vrow = v + (g * n_kv + kv) * d;
        double *dkr = dk + r * d, *dvr = dv + r * d;
        for (int32_t c = 0; c < d; ++c) {
            dkr[c] = 0.0;
            dvr[c] = 0.0;
        }
        for (int64_t qi = 0; qi < n_q; ++qi) {
            if (!orc_allowed(p, qi + p->q_offset, kv))
                continue;
            const uint16_t *qrow = q + (g * n_q + qi) * d, *grow = dout + (g * n_q + qi) * d;
            double acc = 0.0, acc2 = 0.0;
            for (int32_t c = 0; c < d; ++c) {
                acc += bf16_to_f64(qrow[c]) * bf16_to_f64(krow[c]);
                acc2 += bf16_to_f64(grow[c]) * bf16_to_f64(vrow[c]);
            }
            double P = exp(acc * scale - lse[t * n_q + qi]);
            double ds = P * (acc2 - dsum[t * n_q + qi]);
            for (int32_t c = 0; c < d; ++c) {
                dvr[c] += P * bf16_to_f64(grow[c]);
                dkr[c] += scale * ds * bf16_to_f64(qrow[c]);
            }
        }
    }
    free(lse);
    free(dsum);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
