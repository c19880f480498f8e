/*
 * sgqa_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU oracle for the Sparse GQA full-attention layer of
 * StepFun's Step 5 Preview.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the HIP library never does, and
 * this file shares no source with it.
 *
 * What the layer computes, and where the pages say so:
 *   - ai4snews "Step 5 Preview bets on depth over width", Interpretation,
 *     second paragraph: the indexer entries of neighbouring history positions
 *     are compressed into block representations with block size 8, which cuts
 *     indexer and top-k selection cost 8x.
 *   - ai.info "StepFun Details Step 5 Preview's 92-Block Agent Design",
 *     section "Sparse GQA targets million-token context": Sparse GQA picks
 *     relevant historical blocks instead of the whole history; tokens are
 *     grouped into blocks of eight; top-k is 4096 tokens with those blocks.
 *   - same page, section "Why StepFun chose 92 transformer blocks": the full
 *     attention path is Gated Grouped-Query Attention.
 *   - phantomic12 "Step 5 Preview" catalogue entry, config.json and
 *     ATTENTION SPLIT parts: 64 query heads, 4 attention groups (4 KV heads),
 *     head_dim 192; sparse_config topk 512, proxy_dim 256 on the
 *     full-attention layers.
 *
 * Readings taken where the pages are silent:
 *   block representation = mean of the block's proxy keys over the tokens
 *   present; score = plain dot product of the query's proxy with a block
 *   representation; candidates = complete past blocks j < floor(t/B); k counts
 *   blocks including the query's own block, which is always kept; ties go to
 *   the lower block index; output in ascending block order padded with -1;
 *   head h uses KV head floor(h / (Hq/Hkv)); softmax scale 1/sqrt(d) (passed
 *   in); a token attends to positions s <= t only; the gate is one logit per
 *   (token, head) applied as a logistic sigmoid after normalisation.
 *
 * Every floating-point step runs in double.  bf16 inputs are widened exactly.
 * Nothing here is blocked, fused or reordered beyond the definitions above.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double widen_bf16(uint16_t h)
{
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Threads an OpenMP region of this library uses (reported beside the oracle's timings). */
int32_t orc_num_threads(void)
{
    int32_t n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = (int32_t)omp_get_num_threads();
    }
    return n;
}

/* Number of index blocks for a sequence of L tokens: ceil(L / B). */
int64_t orc_num_blocks(int64_t L, int32_t B)
{
    return (L + B - 1) / B;
}

/* Number of candidate (complete, past) blocks of a query at position t. */
int64_t orc_num_candidates(int64_t t, int32_t B)
{
    return t / B;
}

/*
 * Block compression (ai4snews Interpretation, para. 2; ai.info "Sparse GQA
 * targets million-token context"): kb[j] is the mean of kp over the tokens
 * of block j that exist, i.e. positions jB .. min(jB+B, L) - 1.
 *   kp : [L][P] bf16      kb : [ceil(L/B)][P] double
 */
void orc_index_build(const uint16_t *kp, int64_t L, int32_t P, int32_t B, double *kb)
{
    const int64_t nblk = orc_num_blocks(L, B);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nblk; ++j) {
        const int64_t first = j * B;
        int64_t n = L - first;
        if (n > B)
            n = B;
        for (int32_t p = 0; p < P; ++p) {
            double sum = 0.0;
            for (int64_t s = first; s < first + n; ++s)
                sum += widen_bf16(kp[s * P + p]);
            kb[j * P + p] = sum / (double)n;
        }
    }
}

/*
 * Index maintenance straight from the keys.  The pages fix only the proxy
 * width (phantomic12 config.json, sparse_config: proxy_dim 256) and that the
 * indexer works on block representations of size 8 (ai4snews Interpretation,
 * para. 2).  Reading: a token's proxy key is a linear projection of its
 * concatenated KV-head keys, kp[s] = K[s] . W.  The projection is linear, so
 * the block mean of the proxy keys is the projection of the block's mean key:
 *   kb[j][p] = sum_i wt[p][i] * m_j[i],  m_j[i] = (1/n_j) sum_{s in block j} K[s][i]
 * with n_j = min(B, L - jB) (only the tokens present) and i over the
 * width = Hkv*d coordinates of the concatenated key.
 *   K : [L][width] bf16 (a [L][Hkv][d] cache)   wt : [P][width] bf16 (W transposed)
 *   kb : [ceil(L/B)][P] double
 */
void orc_index_build_from_keys(const uint16_t *K, int64_t L, int32_t width, const uint16_t *wt,
                               int32_t P, int32_t B, double *kb)
{
    const int64_t nblk = orc_num_blocks(L, B);
#pragma omp parallel
    {
        double *m = (double *)malloc(sizeof(double) * (size_t)width);
#pragma omp for schedule(static)
        for (int64_t j = 0; j < nblk; ++j) {
            const int64_t first = j * B;
            int64_t n = L - first;
            if (n > B)
                n = B;
            for (int32_t i = 0; i < width; ++i) {
                double sum = 0.0;
                for (int64_t s = first; s < first + n; ++s)
                    sum += widen_bf16(K[s * width + i]);
                m[i] = sum / (double)n;
            }
            for (int32_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int32_t i = 0; i < width; ++i)
                    acc += widen_bf16(wt[(int64_t)p * width + i]) * m[i];
                kb[j * P + p] = acc;
            }
        }
        free(m);
    }
}

/*
 * Indexer scores (phantomic12 config.json / sparse_config: proxy_dim 256):
 * for each query row r at position t[r], score[r][j] = sum_p qp[r][p]*kb[j][p]
 * for every candidate block j < floor(t[r]/B).  Entries past the candidate
 * count are left untouched.
 *   qp : [nrows][P] bf16; kb : [nblk][P] double; out : [nrows][out_stride]
 */
void orc_scores(const uint16_t *qp, int64_t nrows, const int64_t *t, int32_t B, int32_t P,
                const double *kb, double *out, int64_t out_stride)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t c = orc_num_candidates(t[r], B);
        const uint16_t *q = qp + r * P;
        for (int64_t j = 0; j < c; ++j) {
            double acc = 0.0;
            for (int32_t p = 0; p < P; ++p)
                acc += widen_bf16(q[p]) * kb[j * P + p];
            out[r * out_stride + j] = acc;
        }
    }
}

typedef struct {
    double score;
    int64_t block;
} scored_block;

/* Order: higher score first; equal scores -> lower block index first. */
static int by_score_desc_then_index(const void *a, const void *b)
{
    const scored_block *x = (const scored_block *)a;
    const scored_block *y = (const scored_block *)b;
    if (x->score > y->score)
        return -1;
    if (x->score < y->score)
        return 1;
    if (x->block < y->block)
        return -1;
    if (x->block > y->block)
        return 1;
    return 0;
}

static int by_int32_asc(const void *a, const void *b)
{
    const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/*
 * Causal top-k by explicit sort (ai.info "Sparse GQA targets million-token
 * context": relevant historical blocks are selected; phantomic12 sparse_config
 * topk 512).  For the query at t with own block c = floor(t/B):
 *   if c <= k-1 every block 0..c is kept;
 *   else the candidates 0..c-1 are sorted by (score desc, index asc), the
 *   first k-1 are kept, and c is added.
 * The row is written in ascending block order, padded with -1 up to k.
 *   scores : [nrows][stride] double (entries j < c used)   idx : [nrows][k]
 */
void orc_topk(const double *scores, int64_t nrows, int64_t stride, const int64_t *t,
              int32_t B, int32_t k, int32_t *idx)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t c = orc_num_candidates(t[r], B);
        int32_t *row = idx + r * (int64_t)k;
        int32_t count = 0;
        if (c <= (int64_t)k - 1) {
            for (int64_t j = 0; j <= c; ++j)
                row[count++] = (int32_t)j;
        } else {
            scored_block *cand = (scored_block *)malloc((size_t)c * sizeof(scored_block));
            for (int64_t j = 0; j < c; ++j) {
                cand[j].score = scores[r * stride + j];
                cand[j].block = j;
            }
            qsort(cand, (size_t)c, sizeof(scored_block), by_score_desc_then_index);
            for (int32_t i = 0; i < k - 1; ++i)
                row[count++] = (int32_t)cand[i].block;
            free(cand);
            row[count++] = (int32_t)c;
            qsort(row, (size_t)count, sizeof(int32_t), by_int32_asc);
        }
        for (int32_t i = count; i < k; ++i)
            row[i] = -1;
    }
}

/*
 * Tokens a query at t attends to: every position of every selected block,
 * restricted to positions <= t (the own block may extend past t).  -1 entries
 * are padding.  Writes the positions in ascending order; returns the count.
 */
int64_t orc_token_set(const int32_t *sel, int32_t k, int32_t B, int64_t t, int64_t *tokens)
{
    int64_t n = 0;
    for (int32_t i = 0; i < k; ++i) {
        if (sel[i] < 0)
            continue;
        for (int32_t o = 0; o < B; ++o) {
            const int64_t s = (int64_t)sel[i] * B + o;
            if (s <= t)
                tokens[n++] = s;
        }
    }
    return n;
}

static double logistic(double x)
{
    return 1.0 / (1.0 + exp(-x));
}

/*
 * Gated grouped-query attention of one query token over an explicit list of
 * n key/value rows (ai.info "Why StepFun chose 92 transformer blocks": Gated
 * Grouped-Query Attention; phantomic12 config.json: 64 heads, 4 groups,
 * head_dim 192).  For head h with group g = floor(h / (Hq/Hkv)):
 *   z_s  = scale * sum_i q[h][i] * K[s][g][i]
 *   a    = sum_s softmax(z)_s * V[s][g][:]
 *   out  = a * sigmoid(gate[h]);   lse = log sum_s exp(z_s)
 *   q : [Hq][d] bf16; krows, vrows : [n][Hkv][d] double; gate : [Hq] bf16;
 *   out : [Hq][d]
 */
void orc_attend_f64(const uint16_t *q, const double *krows, const double *vrows, int64_t n,
                    const uint16_t *gate, int32_t Hq, int32_t Hkv, int32_t d, double scale,
                    double *out, double *lse)
{
    const int32_t heads_per_group = Hq / Hkv;
    double *z = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int32_t h = 0; h < Hq; ++h) {
        const int32_t g = h / heads_per_group;
        double m = -INFINITY;
        for (int64_t s = 0; s < n; ++s) {
            double dot = 0.0;
            for (int32_t i = 0; i < d; ++i)
                dot += widen_bf16(q[h * d + i]) * krows[(s * Hkv + g) * d + i];
            z[s] = scale * dot;
            if (z[s] > m)
                m = z[s];
        }
        double Z = 0.0;
        for (int64_t s = 0; s < n; ++s) {
            z[s] = exp(z[s] - m);
            Z += z[s];
        }
        const double gate_factor = logistic(widen_bf16(gate[h]));
        for (int32_t i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int64_t s = 0; s < n; ++s)
                acc += z[s] * vrows[(s * Hkv + g) * d + i];
            out[h * d + i] = (acc / Z) * gate_factor;
        }
        if (lse)
            lse[h] = m + log(Z);
    }
    free(z);
}

/* The same over bf16 rows: widened exactly, then orc_attend_f64. */
void orc_attend(const uint16_t *q, const uint16_t *krows, const uint16_t *vrows, int64_t n,
                const uint16_t *gate, int32_t Hq, int32_t Hkv, int32_t d, double scale,
                double *out, double *lse)
{
    const size_t cnt = (size_t)(n > 0 ? n : 1) * (size_t)Hkv * (size_t)d;
    double *kd = (double *)malloc(cnt * sizeof(double));
    double *vd = (double *)malloc(cnt * sizeof(double));
    for (size_t e = 0; e < (size_t)n * (size_t)Hkv * (size_t)d; ++e) {
        kd[e] = widen_bf16(krows[e]);
        vd[e] = widen_bf16(vrows[e]);
    }
    orc_attend_f64(q, kd, vd, n, gate, Hq, Hkv, d, scale, out, lse);
    free(kd);
    free(vd);
}

/*
 * Sparse attention for a batch of query rows with the whole K/V cache on the
 * host: for each row r, build its token set from idx[r] and attend.
 *   q : [nrows][Hq][d]; t : [nrows]; K, V : [L][Hkv][d]; G : [nrows][Hq];
 *   idx : [nrows][k]; out : [nrows][Hq][d]; lse : [nrows][Hq] (nullable)
 * Returns 0, or -1 if a selected token lies outside [0, L).
 */
int orc_sparse_attention(const uint16_t *q, const int64_t *t, int64_t nrows,
                         const uint16_t *K, const uint16_t *V, int64_t L,
                         const uint16_t *G, const int32_t *idx, int32_t k, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t d, double scale,
                         double *out, double *lse)
{
    int bad = 0;
    const int64_t row = (int64_t)Hkv * d;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t *tok = (int64_t *)malloc((size_t)k * B * sizeof(int64_t));
        const int64_t n = orc_token_set(idx + r * (int64_t)k, k, B, t[r], tok);
        uint16_t *kr = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * row * sizeof(uint16_t));
        uint16_t *vr = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * row * sizeof(uint16_t));
        for (int64_t i = 0; i < n; ++i) {
            if (tok[i] < 0 || tok[i] >= L) {
                bad = 1;
                tok[i] = 0;
            }
            memcpy(kr + i * row, K + tok[i] * row, (size_t)row * sizeof(uint16_t));
            memcpy(vr + i * row, V + tok[i] * row, (size_t)row * sizeof(uint16_t));
        }
        orc_attend(q + r * (int64_t)Hq * d, kr, vr, n, G + r * (int64_t)Hq, Hq, Hkv, d, scale,
                   out + r * (int64_t)Hq * d, lse ? lse + r * (int64_t)Hq : NULL);
        free(kr);
        free(vr);
        free(tok);
    }
    return bad ? -1 : 0;
}

/*
 * Gated sliding-window attention, the sibling layer type (ai.info "Why StepFun
 * chose 92 transformer blocks": the efficient layers use Gated Sliding Window
 * Attention; phantomic12 config.json: sliding_window 512).  Reading: the window
 * is the W most recent positions, the query's own included, so a query at t
 * attends to max(0, t-W+1) .. t.  Writes the positions and returns the count.
 */
int64_t orc_window_token_set(int64_t t, int64_t W, int64_t *tokens)
{
    int64_t first = t - W + 1;
    if (first < 0)
        first = 0;
    int64_t n = 0;
    for (int64_t s = first; s <= t; ++s)
        tokens[n++] = s;
    return n;
}

/*
 * Window attention for a batch of query rows with the cache on the host; same
 * arithmetic as orc_attend.  Shapes as orc_sparse_attention, no selection.
 */
int orc_window_attention(const uint16_t *q, const int64_t *t, int64_t nrows, const uint16_t *K,
                         const uint16_t *V, int64_t L, const uint16_t *G, int64_t W, int32_t Hq,
                         int32_t Hkv, int32_t d, double scale, double *out, double *lse)
{
    int bad = 0;
    const int64_t row = (int64_t)Hkv * d;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t cap = W < t[r] + 1 ? W : t[r] + 1;
        int64_t *tok = (int64_t *)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(int64_t));
        const int64_t n = orc_window_token_set(t[r], W, tok);
        uint16_t *kr = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * row * sizeof(uint16_t));
        uint16_t *vr = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * row * sizeof(uint16_t));
        for (int64_t i = 0; i < n; ++i) {
            if (tok[i] < 0 || tok[i] >= L) {
                bad = 1;
                tok[i] = 0;
            }
            memcpy(kr + i * row, K + tok[i] * row, (size_t)row * sizeof(uint16_t));
            memcpy(vr + i * row, V + tok[i] * row, (size_t)row * sizeof(uint16_t));
        }
        orc_attend(q + r * (int64_t)Hq * d, kr, vr, n, G + r * (int64_t)Hq, Hq, Hkv, d, scale,
                   out + r * (int64_t)Hq * d, lse ? lse + r * (int64_t)Hq : NULL);
        free(kr);
        free(vr);
        free(tok);
    }
    return bad ? -1 : 0;
}

/*
 * Backward of the gated sparse attention with the selection held fixed.  The
 * pages say full attention is the bottleneck in training as well as in
 * inference (ai.info "Sparse GQA targets million-token context"); they state no
 * training recipe for the indexer, so the selection is an input here.  For one
 * query, given g_out[h][:] = dL/dout[h][:] and the forward of orc_attend_f64
 * (z_s = scale * q_h . k_s, P_s = softmax(z)_s, a_h = sum_s P_s v_s,
 * out_h = sigmoid(G_h) a_h), the chain rule gives, for head h of group g:
 *   dG_h   = (g_out_h . a_h) * sigmoid(G_h) * (1 - sigmoid(G_h))
 *   da_h   = sigmoid(G_h) g_out_h
 *   dP_s   = da_h . v_s,   dz_s = P_s (dP_s - sum_r P_r dP_r)
 *   dq_h   = scale * sum_s dz_s k_s
 *   dk_s  += scale * dz_s q_h,   dv_s += P_s da_h       (summed over the heads of g)
 * The forward is recomputed here; dkrows / dvrows [n][Hkv][d] are accumulated
 * into (the caller zeroes them), dq [Hq][d] and dgate [Hq] are written.
 */
void orc_attend_backward(const uint16_t *q, const uint16_t *krows, const uint16_t *vrows,
                         int64_t n, const uint16_t *gate, const uint16_t *gout, int32_t Hq,
                         int32_t Hkv, int32_t d, double scale, double *dq, double *dkrows,
                         double *dvrows, double *dgate)
{
    const int32_t heads_per_group = Hq / Hkv;
    double *P = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double *dP = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double *a = (double *)malloc((size_t)d * sizeof(double));
    for (int32_t h = 0; h < Hq; ++h) {
        const int32_t g = h / heads_per_group;
        double m = -INFINITY;
        for (int64_t s = 0; s < n; ++s) {
            double dot = 0.0;
            for (int32_t i = 0; i < d; ++i)
                dot += widen_bf16(q[h * d + i]) * widen_bf16(krows[(s * Hkv + g) * d + i]);
            P[s] = scale * dot;
            if (P[s] > m)
                m = P[s];
        }
        double Z = 0.0;
        for (int64_t s = 0; s < n; ++s) {
            P[s] = exp(P[s] - m);
            Z += P[s];
        }
        for (int64_t s = 0; s < n; ++s)
            P[s] /= Z;
        for (int32_t i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int64_t s = 0; s < n; ++s)
                acc += P[s] * widen_bf16(vrows[(s * Hkv + g) * d + i]);
            a[i] = acc;
        }
        const double sg = logistic(widen_bf16(gate[h]));
        double go_a = 0.0;
        for (int32_t i = 0; i < d; ++i)
            go_a += widen_bf16(gout[h * d + i]) * a[i];
        dgate[h] = go_a * sg * (1.0 - sg);
        double Dsum = 0.0;
        for (int64_t s = 0; s < n; ++s) {
            double acc = 0.0;
            for (int32_t i = 0; i < d; ++i)
                acc += sg * widen_bf16(gout[h * d + i]) * widen_bf16(vrows[(s * Hkv + g) * d + i]);
            dP[s] = acc;
            Dsum += P[s] * acc;
        }
        for (int32_t i = 0; i < d; ++i)
            dq[h * d + i] = 0.0;
        for (int64_t s = 0; s < n; ++s) {
            const double dz = P[s] * (dP[s] - Dsum);
            for (int32_t i = 0; i < d; ++i) {
                dq[h * d + i] += scale * dz * widen_bf16(krows[(s * Hkv + g) * d + i]);
                dkrows[(s * Hkv + g) * d + i] += scale * dz * widen_bf16(q[h * d + i]);
                dvrows[(s * Hkv + g) * d + i] += P[s] * sg * widen_bf16(gout[h * d + i]);
            }
        }
    }
    free(P);
    free(dP);
    free(a);
}

/*
 * The backward for query rows at positions t over selections idx (as
 * orc_sparse_attention): dq [nrows][Hq][d] and dgate [nrows][Hq] per row, and
 * dK / dV [L][Hkv][d] summed over every row that attends to a token (zeroed
 * here).  Rows run in parallel with private dK / dV sums added at the end.
 */
int orc_sparse_attention_backward(const uint16_t *q, const int64_t *t, int64_t nrows,
                                  const uint16_t *K, const uint16_t *V, int64_t L,
                                  const uint16_t *G, const int32_t *idx, int32_t k, int32_t B,
                                  int32_t Hq, int32_t Hkv, int32_t d, double scale,
                                  const uint16_t *gout, double *dq, double *dK, double *dV,
                                  double *dgate)
{
    int bad = 0;
    const int64_t row = (int64_t)Hkv * d;
    memset(dK, 0, (size_t)L * row * sizeof(double));
    memset(dV, 0, (size_t)L * row * sizeof(double));
#pragma omp parallel reduction(| : bad)
    {
        double *pk = (double *)calloc((size_t)L * row, sizeof(double));
        double *pv = (double *)calloc((size_t)L * row, sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t *tok = (int64_t *)malloc((size_t)k * B * sizeof(int64_t));
            const int64_t n = orc_token_set(idx + r * (int64_t)k, k, B, t[r], tok);
            const size_t cnt = (size_t)(n > 0 ? n : 1) * row;
            uint16_t *kr = (uint16_t *)malloc(cnt * sizeof(uint16_t));
            uint16_t *vr = (uint16_t *)malloc(cnt * sizeof(uint16_t));
            double *dkr = (double *)calloc(cnt, sizeof(double));
            double *dvr = (double *)calloc(cnt, sizeof(double));
            for (int64_t i = 0; i < n; ++i) {
                if (tok[i] < 0 || tok[i] >= L) {
                    bad = 1;
                    tok[i] = 0;
                }
                memcpy(kr + i * row, K + tok[i] * row, (size_t)row * sizeof(uint16_t));
                memcpy(vr + i * row, V + tok[i] * row, (size_t)row * sizeof(uint16_t));
            }
            orc_attend_backward(q + r * (int64_t)Hq * d, kr, vr, n, G + r * (int64_t)Hq,
                                gout + r * (int64_t)Hq * d, Hq, Hkv, d, scale,
                                dq + r * (int64_t)Hq * d, dkr, dvr, dgate + r * (int64_t)Hq);
            for (int64_t i = 0; i < n; ++i)
                for (int64_t e = 0; e < row; ++e) {
                    pk[tok[i] * row + e] += dkr[i * row + e];
                    pv[tok[i] * row + e] += dvr[i * row + e];
                }
            free(kr);
            free(vr);
            free(dkr);
            free(dvr);
            free(tok);
        }
#pragma omp critical
        {
            for (int64_t e = 0; e < L * row; ++e) {
                dK[e] += pk[e];
                dV[e] += pv[e];
            }
        }
        free(pk);
        free(pv);
    }
    return bad ? -1 : 0;
}

/*
 * FP8 storage of cached rows (decode path).  The pages give FP8 only for the
 * released checkpoint: e4m3 with scaling blocks of 128 (phantomic12 entry,
 * "quant_method fp8, e4m3, block size 128"; ai4snews "Open Weights" para. on
 * FP8 vs BF16).  Reading: a cached row (one token's K or V row of one KV head,
 * d values, or one index row, P values) is stored as e4m3 codes with one fp32
 * scale per row.
 *
 * OCP 8-bit E4M3: sign bit, 4 exponent bits (bias 7), 3 fraction bits;
 * exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; no
 * infinities; the largest finite magnitude is 448.
 */
double orc_e4m3_decode(uint8_t c)
{
    const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    const double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -v : v;
}

/* Nearest e4m3 value of y, ties to the even code, magnitudes >= 448 saturate. */
uint8_t orc_e4m3_encode(float y)
{
    const uint8_t sgn = signbit(y) ? 0x80 : 0x00;
    const double a = fabs((double)y);
    if (a >= 448.0)
        return (uint8_t)(sgn | 0x7E);
    int ex;
    frexp(a, &ex);          /* a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1 */
    int E = ex - 1;
    if (a == 0.0 || E < -6)
        E = -6;             /* subnormal range: spacing 2^-9 */
    const double r = nearbyint(ldexp(a, 3 - E));  /* value / spacing, ties to even */
    if (r == 0.0)
        return sgn;
    if (E == -6 && r < 8.0)
        return (uint8_t)(sgn | (uint8_t)r);       /* subnormal code m */
    int Ev = E, mant = (int)r - 8;
    if (r == 16.0) {        /* rounded up into the next binade */
        Ev = E + 1;
        mant = 0;
    }
    return (uint8_t)(sgn | (uint8_t)(((Ev + 7) << 3) | mant));
}

/*
 * Row quantisation, every step in fp32 so that the integer codes are decided
 * in the kernel's precision: amax = max |x|, scale = amax / 448 (1 for a zero
 * row), code = e4m3(x / scale).
 *   x : [rows][cols] bf16   codes : [rows][cols]   scales : [rows] float
 */
void orc_quantize_rows(const uint16_t *x, int64_t rows, int32_t cols, uint8_t *codes,
                       float *scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float amax = 0.0f;
        for (int32_t i = 0; i < cols; ++i) {
            const float v = fabsf((float)widen_bf16(x[r * cols + i]));
            if (v > amax)
                amax = v;
        }
        float scale = amax / 448.0f;
        if (!(scale > 0.0f))
            scale = 1.0f;
        scales[r] = scale;
        for (int32_t i = 0; i < cols; ++i)
            codes[r * cols + i] = orc_e4m3_encode((float)widen_bf16(x[r * cols + i]) / scale);
    }
}

/* Dequantised rows: e4m3 value times the row's scale, in double. */
void orc_dequant_rows(const uint8_t *codes, const float *scales, int64_t rows, int32_t cols,
                      double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t i = 0; i < cols; ++i)
            out[r * cols + i] = orc_e4m3_decode(codes[r * cols + i]) * (double)scales[r];
}
