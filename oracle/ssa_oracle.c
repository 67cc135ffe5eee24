/*
 * CPU oracle for streaming sparse attention (SSA).
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow, obviously correct
 * reference that the GPU kernels are checked against. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it. The
 * product library never links, loads or calls it, and this file shares no
 * code with the HIP kernels.
 *
 * What it computes follows "Efficient Context Scaling with LongCat ZigZag
 * Attention" as digested on the 163.com page (section 01, part (1) "LongCat
 * ZigZag Attention", calibration paragraph and the SSA output paragraph after
 * it; part (2), the paragraph on the deployed configuration):
 *   - in SSA each query token attends only to some sink blocks and some local
 *     blocks;
 *   - the selected, blocked keys K* and values V* are defined by the number
 *     of sink blocks s, the number of local blocks l and the block size b;
 *   - the deployed setting is b = 128, s = 1, l = 7: a 1,024-token window.
 * The SSA output equation itself did not survive on the page. The readings
 * taken where the page is silent:
 *   - blocks are b consecutive token positions aligned at position 0;
 *   - the sink blocks are the first s blocks of the sequence;
 *   - the local blocks are the l most recent blocks, the query's own block
 *     included (only then do s + l = 8 blocks of 128 make the 1,024-token
 *     window);
 *   - a key in both sets counts once; the mask is causal (key j <= query i);
 *   - the output is scaled-dot-product softmax attention over the selected
 *     keys, with an explicit softmax scale; the log-sum-exp is natural-log.
 * So, for query position i with query block qb = i / b, key j is attended iff
 *     j <= i  and  ( j / b < s  or  j / b > qb - l ).
 * "full" mode drops the block rule and keeps only j <= i: plain causal
 * attention, the dense comparator the pages measure SSA against.
 *
 * Arithmetic: inputs (float32, or bfloat16 bit patterns, both exact in double)
 * are widened to double; dot products, exp and sums run in double with the C
 * library's exp/log. There is no tiling, no online rescaling and no split.
 *
 * Decode: the newest token sits at position L - 1 of a context of L tokens
 * whose keys and values (the new token's included) are already in a paged
 * cache; token t lives in page page_table[t / P] at slot t % P.
 *
 * Backward: the pages train with SSA in place (the digest's section 01,
 * part (1), the training paragraph after the SSA output, and part (2), the
 * mid-training and post-training of the sparsified model), so the
 * gradients of q, k and v are those of the same operator, by the chain rule
 * through the masked softmax; oracle_ssa_backward writes them out per row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ELEM_F32 = 0, ELEM_BF16 = 1 };

/* Read element idx of an array of float32 or of bfloat16 bit patterns. */
static double elem_at(const void *base, int elem, int64_t idx)
{
    if (elem == ELEM_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* List the attended keys of query position i in increasing order. SSA's
 * block rule: walk the blocks 0..qb (qb = i / b, the query's own block) and
 * keep a block when it is a sink block (one of the first s) or a local block
 * (one of the l blocks ending at qb); inside a kept block take the causal
 * keys j <= i. In full mode every block is kept. Returns the count. */
static int64_t attended_keys(int64_t i, int64_t b, int64_t s, int64_t l,
                             int full, int64_t *out)
{
    int64_t n = 0;
    int64_t qb = i / b;
    for (int64_t c = 0; c <= qb; ++c) {
        int is_sink = c < s;
        int is_local = c > qb - l;
        if (!full && !is_sink && !is_local)
            continue;
        for (int64_t j = c * b; j < (c + 1) * b && j <= i; ++j)
            out[n++] = j;
    }
    return n;
}

/* Softmax attention of one query over n explicitly given key/value rows:
 *   score_j = scale * <q, k_j>,  w_j = exp(score_j - m) / sum exp(score - m),
 *   out = sum_j w_j v_j,  lse = m + log(sum exp(score - m)).
 * krow[j] / vrow[j] are element offsets of key and value row j. */
static void attend_rows(int elem, const double *qd, int d_qk, int d_v,
                        const void *kb, const int64_t *krow, const void *vb,
                        const int64_t *vrow, int64_t n, double scale,
                        double *score, double *out, double *lse_out,
                        double *w_out, const int64_t *keypos)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int d = 0; d < d_qk; ++d)
            acc += qd[d] * elem_at(kb, elem, krow[j] + d);
        score[j] = scale * acc;
        if (score[j] > m)
            m = score[j];
    }
    double denom = 0.0;
    for (int64_t j = 0; j < n; ++j)
        denom += exp(score[j] - m);
    for (int d = 0; d < d_v; ++d)
        out[d] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double w = exp(score[j] - m) / denom;
        if (w_out)
            w_out[keypos[j]] = w;
        for (int d = 0; d < d_v; ++d)
            out[d] += w * elem_at(vb, elem, vrow[j] + d);
    }
    if (lse_out)
        *lse_out = m + log(denom);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Prefill: every query row of a whole sequence.
 *   q [B, N, Hq, d_qk], k [B, N, Hkv, d_qk], v [B, N, Hkv, d_v], addressed by
 *   element strides (batch, token, head) with unit stride along the head dim.
 *   Query head h reads kv head h / (Hq / Hkv).
 *   rows: the query positions to evaluate (NULL: all N, n_rows ignored).
 *   o   [B, R, Hq, d_v]  (R = number of rows evaluated), written;
 *   lse [B, Hq, R] or NULL;
 *   w   [B, Hq, R, N] dense attention weights or NULL (tiny inputs only).
 * Returns 0, or -1 on a bad argument. */
int oracle_ssa_prefill(int elem, const void *q, const void *k, const void *v,
                       const int64_t *q_str, const int64_t *k_str,
                       const int64_t *v_str, int B, int N, int Hq, int Hkv,
                       int d_qk, int d_v, int block, int sink, int local,
                       int full, double scale, const int64_t *rows,
                       int64_t n_rows, double *o, double *lse, double *w)
{
    if (B < 0 || N < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d_qk <= 0 ||
        d_v <= 0 || block < 1 || (!full && (sink < 0 || local < 1)))
        return -1;
    int64_t R = rows ? n_rows : N;
    for (int64_t r = 0; r < R; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= N))
            return -1;
    if (w)
        memset(w, 0, sizeof(double) * (size_t)B * Hq * R * N);
    int64_t group = Hq / Hkv;
    int64_t total = (int64_t)B * Hq * R;

#pragma omp parallel
    {
        int64_t *keys = malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
        int64_t *krow = malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
        int64_t *vrow = malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
        double *score = malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *qd = malloc(sizeof(double) * (size_t)d_qk);
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < total; ++t) {
            int64_t r = t % R;
            int64_t h = (t / R) % Hq;
            int64_t bb = t / (R * Hq);
            int64_t i = rows ? rows[r] : r;
            int64_t g = h / group;
            int64_t qoff = bb * q_str[0] + i * q_str[1] + h * q_str[2];
            for (int d = 0; d < d_qk; ++d)
                qd[d] = elem_at(q, elem, qoff + d);
            int64_t n = attended_keys(i, block, sink, local, full, keys);
            for (int64_t j = 0; j < n; ++j) {
                krow[j] = bb * k_str[0] + keys[j] * k_str[1] + g * k_str[2];
                vrow[j] = bb * v_str[0] + keys[j] * v_str[1] + g * v_str[2];
            }
            double *out = o + ((bb * R + r) * Hq + h) * d_v;
            double *lse_out = lse ? lse + (bb * Hq + h) * R + r : NULL;
            double *w_out = w ? w + ((bb * Hq + h) * R + r) * N : NULL;
            attend_rows(elem, qd, d_qk, d_v, k, krow, v, vrow, n, scale,
                        score, out, lse_out, w_out, keys);
        }
        free(keys);
        free(krow);
        free(vrow);
        free(score);
        free(qd);
    }
    return 0;
}

/* Decode against a paged cache: one new query per sequence.
 *   q [B, Hq, d_qk] contiguous.
 *   k_cache / v_cache: element strides (page, slot, head), unit stride along
 *     the head dim; v_cache may be k_cache (a latent row whose first d_v
 *     entries are the value).
 *   page_table [B, max_pages] physical page ids; ctx_lens [B] context lengths
 *     L (the new token included). Query position is L - 1.
 *   o [B, Hq, d_v]; lse [B, Hq] or NULL. A sequence with L <= 0 gets a zero
 *   output and lse = -inf.
 * Returns 0, or -1 on a bad argument (page id out of range included). */
int oracle_decode_paged(int elem, const void *q, const void *k_cache,
                        const void *v_cache, const int64_t *k_str,
                        const int64_t *v_str, int64_t num_pages,
                        const int32_t *page_table, int64_t max_pages,
                        const int32_t *ctx_lens, int page_size, int B, int Hq,
                        int Hkv, int d_qk, int d_v, int block, int sink,
                        int local, int full, double scale, double *o,
                        double *lse)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d_qk <= 0 || d_v <= 0 ||
        page_size < 1 || block < 1 || (!full && (sink < 0 || local < 1)))
        return -1;
    int64_t maxL = 0;
    for (int bb = 0; bb < B; ++bb) {
        int64_t L = ctx_lens[bb];
        if (L > max_pages * page_size)
            return -1;
        if (L > maxL)
            maxL = L;
        for (int64_t t = 0; t < L; t += page_size) {
            int32_t p = page_table[bb * max_pages + t / page_size];
            if (p < 0 || p >= num_pages)
                return -1;
        }
    }
    int64_t group = Hq / Hkv;
    int64_t total = (int64_t)B * Hq;
    int64_t cap = maxL > 0 ? maxL : 1;

#pragma omp parallel
    {
        int64_t *keys = malloc(sizeof(int64_t) * (size_t)cap);
        int64_t *krow = malloc(sizeof(int64_t) * (size_t)cap);
        int64_t *vrow = malloc(sizeof(int64_t) * (size_t)cap);
        double *score = malloc(sizeof(double) * (size_t)cap);
        double *qd = malloc(sizeof(double) * (size_t)d_qk);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < total; ++t) {
            int64_t h = t % Hq, bb = t / Hq, g = h / group;
            int64_t L = ctx_lens[bb];
            double *out = o + (bb * Hq + h) * d_v;
            if (L <= 0) {
                for (int d = 0; d < d_v; ++d)
                    out[d] = 0.0;
                if (lse)
                    lse[bb * Hq + h] = -INFINITY;
                continue;
            }
            for (int d = 0; d < d_qk; ++d)
                qd[d] = elem_at(q, elem, (bb * Hq + h) * d_qk + d);
            int64_t n = attended_keys(L - 1, block, sink, local, full, keys);
            for (int64_t j = 0; j < n; ++j) {
                int64_t tok = keys[j];
                int64_t page = page_table[bb * max_pages + tok / page_size];
                int64_t slot = tok % page_size;
                krow[j] = page * k_str[0] + slot * k_str[1] + g * k_str[2];
                vrow[j] = page * v_str[0] + slot * v_str[1] + g * v_str[2];
            }
            attend_rows(elem, qd, d_qk, d_v, k_cache, krow, v_cache, vrow, n,
                        scale, score, out, lse ? lse + bb * Hq + h : NULL,
                        NULL, keys);
        }
        free(keys);
        free(krow);
        free(vrow);
        free(score);
        free(qd);
    }
    return 0;
}

/* Backward of the prefill operator: the gradients of q, k and v for an
 * upstream gradient dout = dL/do. The pages train with SSA in place
 * (mid-training and post-training run on the sparse layers), so the operator
 * is differentiated as written, with no approximation. For query row i with
 * attended keys A(i) and weights w_j (recomputed here in double):
 *   g_j   = <dout_i, v_j>                      (dL/dw_j)
 *   ds_j  = w_j * (g_j - sum_{j' in A(i)} w_j' g_j')   (softmax Jacobian)
 *   dq_i  = scale * sum_j ds_j k_j
 *   dk_j += scale * ds_j q_i
 *   dv_j += w_j dout_i
 * A kv head collects these from every query head of its group.
 *   q, k, v, dout: as for oracle_ssa_prefill; dout [B, N, Hq, d_v] with
 *   element strides do_str (batch, token, head).
 *   rows: the query positions whose terms are taken (NULL: all N); dk and dv
 *   then hold those rows' share only, which makes sampled checks of large
 *   shapes cheap.
 *   dq [B, R, Hq, d_qk], dk [B, N, Hkv, d_qk], dv [B, N, Hkv, d_v]: contiguous
 *   doubles, overwritten.
 * Work is split over (batch, kv head): one thread owns the dk/dv rows it adds
 * to, and adds in a fixed order. Returns 0, or -1 on a bad argument. */
int oracle_ssa_backward(int elem, const void *q, const void *k, const void *v,
                        const void *dout, const int64_t *q_str,
                        const int64_t *k_str, const int64_t *v_str,
                        const int64_t *do_str, int B, int N, int Hq, int Hkv,
                        int d_qk, int d_v, int block, int sink, int local,
                        int full, double scale, const int64_t *rows,
                        int64_t n_rows, double *dq, double *dk, double *dv)
{
    if (B < 0 || N < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d_qk <= 0 ||
        d_v <= 0 || block < 1 || (!full && (sink < 0 || local < 1)))
        return -1;
    int64_t R = rows ? n_rows : N;
    for (int64_t r = 0; r < R; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= N))
            return -1;
    memset(dq, 0, sizeof(double) * (size_t)B * R * Hq * d_qk);
    memset(dk, 0, sizeof(double) * (size_t)B * N * Hkv * d_qk);
    memset(dv, 0, sizeof(double) * (size_t)B * N * Hkv * d_v);
    int64_t group = Hq / Hkv;
    int64_t tasks = (int64_t)B * Hkv;
    size_t cap = (size_t)(N > 0 ? N : 1);

#pragma omp parallel
    {
        int64_t *keys = malloc(sizeof(int64_t) * cap);
        double *score = malloc(sizeof(double) * cap);
        double *w = malloc(sizeof(double) * cap);
        double *gw = malloc(sizeof(double) * cap);
        double *qd = malloc(sizeof(double) * (size_t)d_qk);
        double *dod = malloc(sizeof(double) * (size_t)d_v);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < tasks; ++t) {
            int64_t g = t % Hkv, bb = t / Hkv;
            for (int64_t h = g * group; h < (g + 1) * group; ++h) {
                for (int64_t r = 0; r < R; ++r) {
                    int64_t i = rows ? rows[r] : r;
                    int64_t qoff = bb * q_str[0] + i * q_str[1] + h * q_str[2];
                    int64_t dooff = bb * do_str[0] + i * do_str[1] + h * do_str[2];
                    for (int d = 0; d < d_qk; ++d)
                        qd[d] = elem_at(q, elem, qoff + d);
                    for (int d = 0; d < d_v; ++d)
                        dod[d] = elem_at(dout, elem, dooff + d);
                    int64_t n = attended_keys(i, block, sink, local, full, keys);

                    /* Forward weights of row i. */
                    double m = -INFINITY;
                    for (int64_t a = 0; a < n; ++a) {
                        int64_t koff = bb * k_str[0] + keys[a] * k_str[1] + g * k_str[2];
                        double acc = 0.0;
                        for (int d = 0; d < d_qk; ++d)
                            acc += qd[d] * elem_at(k, elem, koff + d);
                        score[a] = scale * acc;
                        if (score[a] > m)
                            m = score[a];
                    }
                    double denom = 0.0;
                    for (int64_t a = 0; a < n; ++a)
                        denom += exp(score[a] - m);
                    for (int64_t a = 0; a < n; ++a)
                        w[a] = exp(score[a] - m) / denom;

                    /* dL/dw_j and the weighted mean it is measured from. */
                    double mean = 0.0;
                    for (int64_t a = 0; a < n; ++a) {
                        int64_t voff = bb * v_str[0] + keys[a] * v_str[1] + g * v_str[2];
                        double acc = 0.0;
                        for (int d = 0; d < d_v; ++d)
                            acc += dod[d] * elem_at(v, elem, voff + d);
                        gw[a] = acc;
                        mean += w[a] * acc;
                    }

                    double *dqi = dq + ((bb * R + r) * Hq + h) * d_qk;
                    for (int64_t a = 0; a < n; ++a) {
                        int64_t j = keys[a];
                        double ds = w[a] * (gw[a] - mean);
                        int64_t koff = bb * k_str[0] + j * k_str[1] + g * k_str[2];
                        double *dkj = dk + ((bb * N + j) * Hkv + g) * d_qk;
                        double *dvj = dv + ((bb * N + j) * Hkv + g) * d_v;
                        for (int d = 0; d < d_qk; ++d) {
                            dqi[d] += scale * ds * elem_at(k, elem, koff + d);
                            dkj[d] += scale * ds * qd[d];
                        }
                        for (int d = 0; d < d_v; ++d)
                            dvj[d] += w[a] * dod[d];
                    }
                }
            }
        }
        free(keys);
        free(score);
        free(w);
        free(gw);
        free(qd);
        free(dod);
    }
    return 0;
}
