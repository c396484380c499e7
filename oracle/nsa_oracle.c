/*
 * nsa_oracle.c -- plain, slow CPU reference of Native Sparse Attention (NSA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The HIP library
 * shares no code, header, table or constant with it.
 *
 * Arithmetic is IEEE double throughout.  Loops are scalar and follow the
 * order in which the pages describe the method; the only parallelism is an
 * OpenMP loop over independent items (compressed blocks; (batch, query
 * position, KV group) rows), which leaves every sum in source order.
 *
 * Sources (web pages, cited by title and section):
 *  [deepdaiv]  deepdaiv newsletter on DeepSeek's Native Sparse Attention
 *              (deepdaiv.stibee.com/p/82): the paragraphs on token compression,
 *              token selection and the sliding window (the three branches that
 *              see the same input).
 *  [valuable12] "AI 모델의 '긴 문장 처리' 한계 돌파, 딥시크의 새 어텐션 기술 화제"
 *              (valuable12.com), section II (NSA structure: l=32, d=16, l'=64,
 *              n=16 including 1 initial and 2 local blocks, w=512) and section
 *              III.3 (decode reads 5,632 tokens instead of 65,536 at 64k).
 *  [allinfo]   DSA explainer (allinfo.ai.kr), section "쉽게 이해하기": the
 *              softmax denominator runs over the selected set only.
 *  [ctol]      ctol-kr.com news article on NSA, "주요 내용" and "하드웨어 인식
 *              설계": group-centric loading of GQA heads with a shared KV fetch.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * repository's design notes):
 *  - compression: one linear map of the flattened, position-embedded block,
 *    W[c][tau*dim + e] applied to (x[i*d + tau][e] + PE[tau][e]); no bias,
 *    no activation; one (W, PE) pair for K and one for V shared by all KV
 *    heads; only complete blocks: N_cmp = floor((T - l)/d) + 1 for T >= l.
 *  - compressed causality: block i is visible to position t iff i*d + l - 1 <= t.
 *  - softmax scale 1/sqrt(d_k) in all three branches.
 *  - importance: the compressed branch's softmax probabilities summed over the
 *    G query heads of a KV group, mapped to selection blocks by token overlap:
 *    w(i, j) = |[i*d, i*d+l) intersect [j*l', (j+1)*l')| / d.
 *  - selection: forced blocks {0, j_cur-1, j_cur} (j_cur = floor(t/l')), then
 *    the highest-scoring remaining blocks (ties: lower j) up to n in total;
 *    if no more than n candidates exist, all are taken.  Ascending, -1 padded.
 *  - selected branch: one softmax over the union of the selected blocks'
 *    tokens with tau <= t; window branch: tokens [max(0, t-w+1), t].
 *  - gates: g_c = sigmoid(W_g[h][c] . q_h + b_g[h][c]) for c in (cmp, slc, win);
 *    o = g_cmp*o_cmp + g_slc*o_slc + g_win*o_win.
 *  - an empty visible set (t < l - 1) gives o_cmp = 0 and zero scores.
 *  - decode: the query is the last cached token, t = seq_len - 1.
 *  - backward ([deepdaiv]: the sparsity is learned in training, so the three
 *    branches, the compression map and the gates are differentiated): the
 *    block selection is piecewise constant and held fixed; the bf16 rounding
 *    of the compressed K/V (bf16 configurations) is passed straight through.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <fenv.h>
#include <omp.h>

typedef struct {
    int B, T, Hkv, G, dk, dv; /* H_q = Hkv*G; query head h belongs to KV group h/G */
    int l, d, lsel, n, w;     /* block length, stride, selection block, count, window */
    double scale;             /* softmax scale */
} orc_cfg;

/* Number of complete compression blocks of a length-T sequence. */
int orc_n_cmp(int T, int l, int d)
{
    if (T < l) return 0;
    return (T - l) / d + 1;
}

/* Round a double to the nearest bfloat16 value (8 significant bits), ties to
 * even.  The compressed K/V of the bf16 configurations are stored in bf16, so
 * the oracle rounds them at that point too. */
double orc_round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    double m = frexp(x, &e);               /* x = m * 2^e, 0.5 <= |m| < 1 */
    double r = nearbyint(ldexp(m, 8));     /* default mode: nearest, ties even */
    return ldexp(r, e - 8);
}

/* Token compression ([deepdaiv], token compression paragraph; [valuable12] II:
 * blocks of l tokens at stride d).
 *   x   [B][H][T][dim]     keys or values
 *   W   [dim][l*dim]       linear map, input index tau*dim + e
 *   PE  [l][dim]           intra-block position embedding
 *   out [B][H][n_out][dim] with n_out >= N_cmp; entries past N_cmp are zeroed */
void orc_compress(int B, int H, int T, int dim, int l, int d, int n_out, int round_bf16,
                  const double *x, const double *W, const double *PE, double *out)
{
    int ncmp = orc_n_cmp(T, l, d);
    /* every (b, h, i) summary is independent of the others */
#pragma omp parallel for collapse(3) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++)
            for (int i = 0; i < n_out; i++) {
                const double *xs = x + ((size_t)b * H + h) * (size_t)T * dim;
                double *os = out + ((size_t)b * H + h) * (size_t)n_out * dim;
                for (int c = 0; c < dim; c++) {
                    double acc = 0.0;
                    if (i < ncmp) {
                        for (int tau = 0; tau < l; tau++)
                            for (int e = 0; e < dim; e++)
                                acc += W[(size_t)c * l * dim + (size_t)tau * dim + e] *
                                       (xs[(size_t)(i * d + tau) * dim + e] + PE[(size_t)tau * dim + e]);
                        if (round_bf16) acc = orc_round_bf16(acc);
                    }
                    os[(size_t)i * dim + c] = acc;
                }
        }
}

/* Compression by a small two-layer network ([deepdaiv], token-compression
 * paragraph: a small neural network with an intra-block position encoding
 * summarises each block; the pages give no layer count, width or activation,
 * so this reading takes two layers, hidden width = dim, ReLU, no biases):
 *   a   = W1 vec(x_i + PE), exactly as orc_compress with W = W1, rounded to
 *         bf16 when round_bf16 (the hidden layer is stored like a summary)
 *   h   = max(a, 0)
 *   out = W2 h, rounded to bf16 when round_bf16
 *   W1 [dim][l*dim], PE [l][dim], W2 [dim][dim] (out[c] = sum_j W2[c][j] h[j]);
 *   entries past N_cmp are zero. */
void orc_compress_mlp(int B, int H, int T, int dim, int l, int d, int n_out, int round_bf16, const double *x,
                      const double *W1, const double *PE, const double *W2, double *out)
{
    orc_compress(B, H, T, dim, l, d, n_out, round_bf16, x, W1, PE, out);
    int ncmp = orc_n_cmp(T, l, d);
#pragma omp parallel for collapse(3) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++)
            for (int i = 0; i < n_out; i++) {
                double *row = out + (((size_t)b * H + h) * (size_t)n_out + i) * dim;
                if (i >= ncmp) continue;
                double *hid = (double *)malloc(sizeof(double) * (size_t)dim);
                for (int j = 0; j < dim; j++) hid[j] = row[j] > 0.0 ? row[j] : 0.0;
                for (int c = 0; c < dim; c++) {
                    double acc = 0.0;
                    for (int j = 0; j < dim; j++) acc += W2[(size_t)c * dim + j] * hid[j];
                    row[c] = round_bf16 ? orc_round_bf16(acc) : acc;
                }
                free(hid);
            }
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Softmax attention of one query vector over an explicit list of key rows.
 *   keys[r] = row index into K/V (row stride dk / dv); out[dv] = sum p_r V[r]
 *   returns the log-sum-exp of the scaled logits (or -INFINITY if empty). */
static double attend_list(const double *qh, const double *K, const double *V, int dk, int dv,
                          double scale, const int *rows, int nrows, double *out, double *p_out)
{
    for (int c = 0; c < dv; c++) out[c] = 0.0;
    if (nrows == 0) return -INFINITY;
    double *s = (double *)malloc(sizeof(double) * (size_t)nrows);
    double mx = -INFINITY;
    for (int r = 0; r < nrows; r++) {
        const double *kr = K + (size_t)rows[r] * dk;
        double dot = 0.0;
        for (int e = 0; e < dk; e++) dot += qh[e] * kr[e];
        s[r] = scale * dot;
        if (s[r] > mx) mx = s[r];
    }
    double sum = 0.0;
    for (int r = 0; r < nrows; r++) {
        s[r] = exp(s[r] - mx);
        sum += s[r];
    }
    for (int r = 0; r < nrows; r++) {
        double p = s[r] / sum;
        if (p_out) p_out[r] = p;
        const double *vr = V + (size_t)rows[r] * dv;
        for (int c = 0; c < dv; c++) out[c] += p * vr[c];
    }
    free(s);
    return mx + log(sum);
}

/* Overlap weight between compression block i and selection block j:
 * number of shared tokens divided by the stride d. */
static double overlap_weight(const orc_cfg *c, int i, int j)
{
    long a0 = (long)i * c->d, a1 = a0 + c->l;
    long b0 = (long)j * c->lsel, b1 = b0 + c->lsel;
    long lo = a0 > b0 ? a0 : b0, hi = a1 < b1 ? a1 : b1;
    return hi > lo ? (double)(hi - lo) / c->d : 0.0;
}

typedef struct { double s; int j; } cand_t;

/* Higher score first; on exact equality, lower block index first. */
static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int int_cmp(const void *pa, const void *pb)
{
    int a = *(const int *)pa, b = *(const int *)pb;
    return (a > b) - (a < b);
}

/* Block selection for one (position, KV group) row ([deepdaiv], token
 * selection paragraph; [valuable12] II: n blocks including the initial block
 * and 2 local blocks).  S[0..j_cur] are the importance scores.  Writes n
 * ascending indices, -1 padded; returns the number selected. */
static int select_blocks(const orc_cfg *c, int t, const double *S, int *idx)
{
    int jcur = t / c->lsel;
    int *sel = (int *)malloc(sizeof(int) * (size_t)(jcur + 1));
    char *forced = (char *)calloc((size_t)jcur + 1, 1);
    int nsel = 0;
    int fcand[3] = {0, jcur - 1, jcur};
    for (int f = 0; f < 3; f++) {
        int j = fcand[f];
        if (j >= 0 && j <= jcur && !forced[j]) {
            forced[j] = 1;
            sel[nsel++] = j;
        }
    }
    int nrest = jcur + 1 - nsel;
    int k = c->n - nsel;
    cand_t *rest = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nrest > 0 ? nrest : 1));
    int r = 0;
    for (int j = 0; j <= jcur; j++)
        if (!forced[j]) { rest[r].s = S[j]; rest[r].j = j; r++; }
    if (nrest <= k) {
        for (int q = 0; q < nrest; q++) sel[nsel++] = rest[q].j;
    } else {
        qsort(rest, (size_t)nrest, sizeof(cand_t), cand_cmp);
        for (int q = 0; q < k; q++) sel[nsel++] = rest[q].j;
    }
    qsort(sel, (size_t)nsel, sizeof(int), int_cmp);
    for (int q = 0; q < c->n; q++) idx[q] = q < nsel ? sel[q] : -1;
    free(rest);
    free(forced);
    free(sel);
    return nsel;
}

/* One (position t, KV group) row of the NSA forward pass.
 *   q      [G][dk]      the G query heads of the group at position t
 *   kc, vc [>=N_cmp(t)][dk|dv]  compressed keys / values of the group
 *   k, v   [>=t+1][dk|dv]       raw keys / values of the group
 *   wg     [G][3][dk], bg [G][3]  gate weights of these heads
 *   idx_in [n] or NULL: if given, these blocks are used instead of selecting
 *   o      [G][dv]
 *   idx_out[n], scores[nb] (nb >= j_cur+1; entries past j_cur = -inf) or NULL,
 *   branches [3][G][dv] (o_cmp, o_slc, o_win) or NULL, gates [G][3] or NULL,
 *   lse [3][G] or NULL: each branch's log-sum-exp of its logits scale q.K
 *   over its own key set (-inf if the set is empty), branches in the order
 *   of `branches` */
void orc_row(const orc_cfg *c, int t, const double *q, const double *kc, const double *vc,
             const double *k, const double *v, const double *wg, const double *bg,
             const int *idx_in, double *o, int *idx_out, double *scores, int nb,
             double *branches, double *gates, double *lse)
{
    const int G = c->G, dk = c->dk, dv = c->dv;
    const int jcur = t / c->lsel;
    /* compressed blocks visible at t: i*d + l - 1 <= t */
    int nvis = (t - (c->l - 1) >= 0) ? (t - (c->l - 1)) / c->d + 1 : 0;
    double *S = (double *)calloc((size_t)jcur + 1, sizeof(double));
    double *ocmp = (double *)calloc((size_t)G * dv, sizeof(double));
    double *oslc = (double *)calloc((size_t)G * dv, sizeof(double));
    double *owin = (double *)calloc((size_t)G * dv, sizeof(double));
    double *p = (double *)malloc(sizeof(double) * (size_t)(nvis > 0 ? nvis : 1));
    double *P = (double *)calloc((size_t)(nvis > 0 ? nvis : 1), sizeof(double));
    int *rows = (int *)malloc(sizeof(int) * (size_t)(t + 1 > nvis ? t + 1 : nvis + 1));

    /* Compressed branch and its per-group importance. */
    for (int i = 0; i < nvis; i++) rows[i] = i;
    for (int h = 0; h < G; h++) {
        double L = attend_list(q + (size_t)h * dk, kc, vc, dk, dv, c->scale, rows, nvis,
                               ocmp + (size_t)h * dv, p);
        if (lse) lse[h] = L;
        for (int i = 0; i < nvis; i++) P[i] += p[i];
    }
    for (int i = 0; i < nvis; i++) {
        /* block i spans tokens [i*d, i*d+l); it can touch at most the blocks
         * holding its first and last token */
        int j0 = (i * c->d) / c->lsel, j1 = (i * c->d + c->l - 1) / c->lsel;
        for (int j = j0; j <= j1; j++) S[j] += overlap_weight(c, i, j) * P[i];
    }
    if (scores)
        for (int j = 0; j < nb; j++) scores[j] = j <= jcur ? S[j] : -INFINITY;

    /* Selection. */
    int idx[64];
    int nsel;
    if (idx_in) {
        nsel = 0;
        for (int q2 = 0; q2 < c->n; q2++) {
            idx[q2] = idx_in[q2];
            if (idx_in[q2] >= 0) nsel++;
        }
    } else {
        nsel = select_blocks(c, t, S, idx);
    }
    if (idx_out)
        for (int q2 = 0; q2 < c->n; q2++) idx_out[q2] = idx[q2];

    /* Selected branch: one softmax over the union of the selected blocks'
     * tokens that are causal ([allinfo]: denominator over the selected set). */
    int nr = 0;
    {
        int *sorted = (int *)malloc(sizeof(int) * (size_t)(c->n));
        int m = 0;
        for (int q2 = 0; q2 < c->n; q2++)
            if (idx[q2] >= 0) sorted[m++] = idx[q2];
        qsort(sorted, (size_t)m, sizeof(int), int_cmp);
        for (int q2 = 0; q2 < m; q2++) {
            if (q2 > 0 && sorted[q2] == sorted[q2 - 1]) continue; /* a set, not a list */
            for (int tau = sorted[q2] * c->lsel; tau < (sorted[q2] + 1) * c->lsel; tau++)
                if (tau <= t) rows[nr++] = tau;
        }
        free(sorted);
    }
    for (int h = 0; h < G; h++) {
        double L = attend_list(q + (size_t)h * dk, k, v, dk, dv, c->scale, rows, nr, oslc + (size_t)h * dv, NULL);
        if (lse) lse[G + h] = L;
    }

    /* Sliding window: [max(0, t-w+1), t]. */
    int lo = t - c->w + 1 > 0 ? t - c->w + 1 : 0;
    nr = 0;
    for (int tau = lo; tau <= t; tau++) rows[nr++] = tau;
    for (int h = 0; h < G; h++) {
        double L = attend_list(q + (size_t)h * dk, k, v, dk, dv, c->scale, rows, nr, owin + (size_t)h * dv, NULL);
        if (lse) lse[2 * G + h] = L;
    }

    /* Gated combination. */
    for (int h = 0; h < G; h++) {
        double g3[3];
        for (int cc = 0; cc < 3; cc++) {
            double z = bg[h * 3 + cc];
            const double *wr = wg + ((size_t)h * 3 + cc) * dk;
            for (int e = 0; e < dk; e++) z += wr[e] * q[(size_t)h * dk + e];
            g3[cc] = sigmoid(z);
            if (gates) gates[h * 3 + cc] = g3[cc];
        }
        for (int cc = 0; cc < dv; cc++)
            o[(size_t)h * dv + cc] = g3[0] * ocmp[(size_t)h * dv + cc] +
                                     g3[1] * oslc[(size_t)h * dv + cc] +
                                     g3[2] * owin[(size_t)h * dv + cc];
    }
    if (branches) {
        memcpy(branches, ocmp, sizeof(double) * (size_t)G * dv);
        memcpy(branches + (size_t)G * dv, oslc, sizeof(double) * (size_t)G * dv);
        memcpy(branches + (size_t)2 * G * dv, owin, sizeof(double) * (size_t)G * dv);
    }
    (void)nsel;
    free(rows); free(P); free(p); free(owin); free(oslc); free(ocmp); free(S);
}

/* Prefill forward over a list of rows.
 *   q        [R][Hq][dk]   query rows (row r is position t_list[r] of batch b_list[r])
 *   kc, vc   [B][Hkv][npad][dk|dv]
 *   k, v     [B][Hkv][T][dk|dv]
 *   wg [Hq][3][dk], bg [Hq][3]
 *   idx_in   [R][Hkv][n] or NULL
 *   o        [R][Hq][dv];  idx_out [R][Hkv][n];  scores [R][Hkv][nb] or NULL;
 *   branches [R][3][Hq][dv] or NULL; lse [R][3][Hq] (per branch, as orc_row) or NULL */
void orc_forward_rows(const orc_cfg *c, int R, const int *b_list, const int *t_list,
                      const double *q, const double *kc, const double *vc, int npad,
                      const double *k, const double *v, const double *wg, const double *bg,
                      const int *idx_in, double *o, int *idx_out, double *scores, int nb,
                      double *branches, double *lse)
{
    const int Hkv = c->Hkv, G = c->G, Hq = Hkv * G, dk = c->dk, dv = c->dv, n = c->n, T = c->T;
    long total = (long)R * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (long job = 0; job < total; job++) {
        int r = (int)(job / Hkv), g = (int)(job % Hkv);
        int b = b_list[r], t = t_list[r];
        const double *qr = q + ((size_t)r * Hq + (size_t)g * G) * dk;
        const double *kcg = kc + ((size_t)b * Hkv + g) * (size_t)npad * dk;
        const double *vcg = vc + ((size_t)b * Hkv + g) * (size_t)npad * dv;
        const double *kg = k + ((size_t)b * Hkv + g) * (size_t)T * dk;
        const double *vg = v + ((size_t)b * Hkv + g) * (size_t)T * dv;
        double *br = NULL;
        double *tmp = NULL;
        double *lse3 = lse ? (double *)malloc(sizeof(double) * 3 * (size_t)G) : NULL;
        if (branches) tmp = (double *)malloc(sizeof(double) * 3 * (size_t)G * dv);
        orc_row(c, t, qr, kcg, vcg, kg, vg, wg + (size_t)g * G * 3 * dk, bg + (size_t)g * G * 3,
                idx_in ? idx_in + ((size_t)r * Hkv + g) * n : NULL,
                o + ((size_t)r * Hq + (size_t)g * G) * dv,
                idx_out + ((size_t)r * Hkv + g) * n,
                scores ? scores + ((size_t)r * Hkv + g) * nb : NULL, nb, tmp, NULL, lse ? lse3 : NULL);
        if (lse) {
            for (int br_i = 0; br_i < 3; br_i++)
                memcpy(lse + ((size_t)r * 3 + br_i) * Hq + (size_t)g * G, lse3 + (size_t)br_i * G,
                       sizeof(double) * (size_t)G);
            free(lse3);
        }
        if (branches) {
            for (int br_i = 0; br_i < 3; br_i++) {
                br = branches + (((size_t)r * 3 + br_i) * Hq + (size_t)g * G) * dv;
                memcpy(br, tmp + (size_t)br_i * G * dv, sizeof(double) * (size_t)G * dv);
            }
            free(tmp);
        }
    }
}

/* Decode step ([valuable12] III.3: the decode step reads a bounded token set).
 * The query of sequence b is its last cached token, t = seq_lens[b] - 1; the
 * caches hold T (capacity) raw tokens and npad compressed slots per group.
 *   q [B][Hq][dk], o [B][Hq][dv], idx_in / idx_out [B][Hkv][n] */
void orc_decode(const orc_cfg *c, const int *seq_lens, const double *q, const double *kc,
                const double *vc, int npad, const double *k, const double *v,
                const double *wg, const double *bg, const int *idx_in, double *o, int *idx_out)
{
    const int B = c->B;
    int *b_list = (int *)malloc(sizeof(int) * (size_t)B);
    int *t_list = (int *)malloc(sizeof(int) * (size_t)B);
    for (int b = 0; b < B; b++) {
        b_list[b] = b;
        t_list[b] = seq_lens[b] - 1;
    }
    orc_forward_rows(c, B, b_list, t_list, q, kc, vc, npad, k, v, wg, bg, idx_in, o, idx_out,
                     NULL, 0, NULL, NULL);
    free(t_list);
    free(b_list);
}

/* Selection only, for tests that supply their own scores S[0..t/l']. */
int orc_select(const orc_cfg *c, int t, const double *S, int *idx)
{
    return select_blocks(c, t, S, idx);
}

/* ------------------------------------------------------------------------
 * Backward pass.  Reverse mode through the gates, the three attention
 * branches and the compression, with the block selection held fixed (it is
 * piecewise constant in the inputs, so no gradient flows through the
 * importance scores).  The loss is L = sum(dO * o).
 *
 * Softmax attention over a key list with p = softmax(s), s_i = scale q.K_i,
 * o = sum_i p_i V_i and output gradient do:
 *   dV_i += p_i do;  dP_i = do.V_i;  D = sum_i p_i dP_i;  ds_i = p_i (dP_i - D)
 *   dq += scale sum_i ds_i K_i;  dK_i += scale ds_i q
 * Gate c of head h: g = sigmoid(z), z = W_g[h][c].q_h + b_g[h][c];
 *   dz = (dO.o_c) g (1 - g);  dW_g[h][c] += dz q_h;  db_g[h][c] += dz;  dq_h += dz W_g[h][c]
 * Compression: K_cmp[i] = W X_i with X_i = vec(x[16i .. 16i+31] + PE):
 *   dW += dK_cmp[i] X_i^T;  dX_i = W^T dK_cmp[i];  dx[16i + tau] += dX_i[tau];  dPE[tau] += dX_i[tau]
 * ------------------------------------------------------------------------ */

/* p over an explicit key list (returns 0 and leaves p untouched if empty) */
static int softmax_list(const double *qh, const double *K, int dk, double scale, const int *rows, int nrows,
                        double *p)
{
    if (nrows == 0) return 0;
    double mx = -INFINITY;
    for (int r = 0; r < nrows; r++) {
        const double *kr = K + (size_t)rows[r] * dk;
        double dot = 0.0;
        for (int e = 0; e < dk; e++) dot += qh[e] * kr[e];
        p[r] = scale * dot;
        if (p[r] > mx) mx = p[r];
    }
    double sum = 0.0;
    for (int r = 0; r < nrows; r++) {
        p[r] = exp(p[r] - mx);
        sum += p[r];
    }
    for (int r = 0; r < nrows; r++) p[r] /= sum;
    return nrows;
}

/* One attention branch for one head: forward output o and the backward
 * contributions for output gradient do. */
static void attend_backward(const double *qh, const double *K, const double *V, int dk, int dv, double scale,
                            const int *rows, int nrows, const double *dout, double *p, double *o, double *dq,
                            double *dK, double *dV)
{
    for (int cc = 0; cc < dv; cc++) o[cc] = 0.0;
    if (!softmax_list(qh, K, dk, scale, rows, nrows, p)) return;
    for (int r = 0; r < nrows; r++)
        for (int cc = 0; cc < dv; cc++) o[cc] += p[r] * V[(size_t)rows[r] * dv + cc];
    if (!dout || nrows <= 0) return;
    double D = 0.0;
    double *dP = (double *)malloc(sizeof(double) * (size_t)nrows);
    for (int r = 0; r < nrows; r++) {
        const double *vr = V + (size_t)rows[r] * dv;
        double x = 0.0;
        for (int cc = 0; cc < dv; cc++) x += dout[cc] * vr[cc];
        dP[r] = x;
        D += p[r] * x;
    }
    for (int r = 0; r < nrows; r++) {
        const double ds = p[r] * (dP[r] - D);
        const double *kr = K + (size_t)rows[r] * dk;
        double *dkr = dK + (size_t)rows[r] * dk;
        double *dvr = dV + (size_t)rows[r] * dv;
        for (int e = 0; e < dk; e++) {
            dq[e] += scale * ds * kr[e];
            dkr[e] += scale * ds * qh[e];
        }
        for (int cc = 0; cc < dv; cc++) dvr[cc] += p[r] * dout[cc];
    }
    free(dP);
}

/* Compression backward for one tensor: dC [BH][N][dim] -> dW [dim][l*dim],
 * dPE [l][dim], dx [BH][T][dim] (all accumulated).  With X_i the flattened
 * block i plus PE:  dX_i = W^T dC[i];  dW = sum_i dC[i] X_i^T;  token 16i+tau
 * and PE[tau] collect dX_i[tau].  dX for every block is formed first (blocks
 * are independent), then added into dx and dPE in block order. */
static void compress_backward(int BH, int T, int dim, int l, int d, int N, const double *x, const double *W,
                              const double *PE, const double *dC, double *dW, double *dPE, double *dx)
{
    const int L = l * dim;
    double *dX = (double *)malloc(sizeof(double) * (size_t)BH * N * L);
#pragma omp parallel for collapse(2) schedule(static)
    for (int bh = 0; bh < BH; bh++)
        for (int i = 0; i < N; i++) {
            const double *g = dC + ((size_t)bh * N + i) * dim;
            double *dXi = dX + ((size_t)bh * N + i) * L;
            for (int m = 0; m < L; m++) {
                double acc = 0.0;
                for (int c = 0; c < dim; c++) acc += W[(size_t)c * L + m] * g[c];
                dXi[m] = acc;
            }
        }
    for (int bh = 0; bh < BH; bh++)
        for (int i = 0; i < N; i++) {
            const double *dXi = dX + ((size_t)bh * N + i) * L;
            double *dxs = dx + (size_t)bh * T * dim;
            for (int m = 0; m < L; m++) {
                dxs[(size_t)i * d * dim + m] += dXi[m];
                dPE[m] += dXi[m];
            }
        }
    /* each thread owns whole rows c of dW */
#pragma omp parallel for schedule(static)
    for (int c = 0; c < dim; c++)
        for (int bh = 0; bh < BH; bh++)
            for (int i = 0; i < N; i++) {
                const double gc = dC[((size_t)bh * N + i) * dim + c];
                if (gc == 0.0) continue;
                const double *xs = x + ((size_t)bh * T + (size_t)i * d) * dim;
                double *row = dW + (size_t)c * L;
                for (int m = 0; m < L; m++) row[m] += gc * (xs[m] + PE[m]);
            }
    free(dX);
}

/* The three branches and the gates, backward, for given compressed K/V
 * (kc, vc: [B][Hkv][max(N,1)][dk|dv]).  Writes dq, dwg, dbg and adds into dk,
 * dv (raw keys) and dkc, dvc (compressed keys); all must start at zero. */
static void branches_backward(const orc_cfg *c, const double *q, const double *k, const double *v,
                              const double *kc, const double *vc, const double *wg, const double *bg,
                              const int *idx, const double *dO, double *dq, double *dk, double *dv,
                              double *dkc, double *dvc, double *dwg, double *dbg)
{
    const int B = c->B, T = c->T, Hkv = c->Hkv, G = c->G, Hq = Hkv * G, dk_ = c->dk, dv_ = c->dv, n = c->n;
    const int N = orc_n_cmp(T, c->l, c->d);
    const int Nn = N > 0 ? N : 1;
    const size_t nk = (size_t)B * Hkv * T * dk_, nv = (size_t)B * Hkv * T * dv_;
    const size_t nkc = (size_t)B * Hkv * Nn * dk_, nvc = (size_t)B * Hkv * Nn * dv_;

#pragma omp parallel
    {
        /* thread-private accumulators, reduced in thread order below */
        double *a_dk = (double *)calloc(nk, sizeof(double));
        double *a_dv = (double *)calloc(nv, sizeof(double));
        double *a_dkc = (double *)calloc(nkc, sizeof(double));
        double *a_dvc = (double *)calloc(nvc, sizeof(double));
        double *a_dwg = (double *)calloc((size_t)Hq * 3 * dk_, sizeof(double));
        double *a_dbg = (double *)calloc((size_t)Hq * 3, sizeof(double));
        int *rows = (int *)malloc(sizeof(int) * (size_t)(T + Nn + 1));
        double *p = (double *)malloc(sizeof(double) * (size_t)(T + Nn + 1));
        double *o3 = (double *)malloc(sizeof(double) * 3 * (size_t)dv_);
        double *dout = (double *)malloc(sizeof(double) * (size_t)dv_);
#pragma omp for schedule(dynamic, 1)
        for (long job = 0; job < (long)B * Hkv * T; job++) {
            const int t = (int)(job % T), g = (int)((job / T) % Hkv), b = (int)(job / ((long)T * Hkv));
            const size_t bg_ = (size_t)b * Hkv + g;
            const double *kcg = kc + bg_ * Nn * dk_, *vcg = vc + bg_ * Nn * dv_;
            const double *kg = k + bg_ * T * dk_, *vg = v + bg_ * T * dv_;
            double *dkcg = a_dkc + bg_ * Nn * dk_, *dvcg = a_dvc + bg_ * Nn * dv_;
            double *dkg = a_dk + bg_ * T * dk_, *dvg = a_dv + bg_ * T * dv_;
            const int nvis = (t - (c->l - 1) >= 0) ? (t - (c->l - 1)) / c->d + 1 : 0;
            const int lo = t - c->w + 1 > 0 ? t - c->w + 1 : 0;
            /* selected token list (a set of blocks, causal) */
            const int *ir = idx + (bg_ * T + t) * n;
            int jcur = t / c->lsel;
            /* a row with dO = 0 on every head of the group contributes nothing */
            int live = 0;
            for (size_t e = 0; e < (size_t)G * dv_ && !live; e++)
                live = dO[((size_t)b * T + t) * Hq * dv_ + (size_t)g * G * dv_ + e] != 0.0;
            if (!live) continue;
            for (int hh = 0; hh < G; hh++) {
                const int h = g * G + hh;
                const double *qh = q + (((size_t)b * T + t) * Hq + h) * dk_;
                const double *dOh = dO + (((size_t)b * T + t) * Hq + h) * dv_;
                double *dqh = dq + (((size_t)b * T + t) * Hq + h) * dk_;
                /* forward of the three branches */
                int nr;
                for (int i = 0; i < nvis; i++) rows[i] = i;
                attend_backward(qh, kcg, vcg, dk_, dv_, c->scale, rows, nvis, NULL, p, o3, NULL, NULL, NULL);
                nr = 0;
                for (int jj = 0; jj <= jcur; jj++) {
                    int in = 0;
                    for (int u = 0; u < n; u++) in |= ir[u] == jj;
                    if (!in) continue;
                    for (int tau = jj * c->lsel; tau < (jj + 1) * c->lsel && tau <= t; tau++) rows[nr++] = tau;
                }
                attend_backward(qh, kg, vg, dk_, dv_, c->scale, rows, nr, NULL, p, o3 + dv_, NULL, NULL, NULL);
                nr = 0;
                for (int tau = lo; tau <= t; tau++) rows[nr++] = tau;
                attend_backward(qh, kg, vg, dk_, dv_, c->scale, rows, nr, NULL, p, o3 + 2 * dv_, NULL, NULL, NULL);
                /* gates */
                double gate[3];
                for (int cc = 0; cc < 3; cc++) {
                    const double *wr = wg + ((size_t)h * 3 + cc) * dk_;
                    double z = bg[h * 3 + cc];
                    for (int e = 0; e < dk_; e++) z += wr[e] * qh[e];
                    gate[cc] = 1.0 / (1.0 + exp(-z));
                    double dg = 0.0;
                    for (int e = 0; e < dv_; e++) dg += dOh[e] * o3[cc * dv_ + e];
                    const double dz = dg * gate[cc] * (1.0 - gate[cc]);
                    for (int e = 0; e < dk_; e++) {
                        a_dwg[((size_t)h * 3 + cc) * dk_ + e] += dz * qh[e];
                        dqh[e] += dz * wr[e];
                    }
                    a_dbg[h * 3 + cc] += dz;
                }
                /* backward of the three branches with do = g_c dO */
                for (int e = 0; e < dv_; e++) dout[e] = gate[0] * dOh[e];
                for (int i = 0; i < nvis; i++) rows[i] = i;
                attend_backward(qh, kcg, vcg, dk_, dv_, c->scale, rows, nvis, dout, p, o3, dqh, dkcg, dvcg);
                for (int e = 0; e < dv_; e++) dout[e] = gate[1] * dOh[e];
                nr = 0;
                for (int jj = 0; jj <= jcur; jj++) {
                    int in = 0;
                    for (int u = 0; u < n; u++) in |= ir[u] == jj;
                    if (!in) continue;
                    for (int tau = jj * c->lsel; tau < (jj + 1) * c->lsel && tau <= t; tau++) rows[nr++] = tau;
                }
                attend_backward(qh, kg, vg, dk_, dv_, c->scale, rows, nr, dout, p, o3 + dv_, dqh, dkg, dvg);
                for (int e = 0; e < dv_; e++) dout[e] = gate[2] * dOh[e];
                nr = 0;
                for (int tau = lo; tau <= t; tau++) rows[nr++] = tau;
                attend_backward(qh, kg, vg, dk_, dv_, c->scale, rows, nr, dout, p, o3 + 2 * dv_, dqh, dkg, dvg);
            }
        }
        int nth = omp_get_num_threads(), me = omp_get_thread_num();
        for (int turn = 0; turn < nth; turn++) {
#pragma omp barrier
            if (turn == me) {
                for (size_t i = 0; i < nk; i++) dk[i] += a_dk[i];
                for (size_t i = 0; i < nv; i++) dv[i] += a_dv[i];
                for (size_t i = 0; i < nkc; i++) dkc[i] += a_dkc[i];
                for (size_t i = 0; i < nvc; i++) dvc[i] += a_dvc[i];
                for (size_t i = 0; i < (size_t)Hq * 3 * dk_; i++) dwg[i] += a_dwg[i];
                for (size_t i = 0; i < (size_t)Hq * 3; i++) dbg[i] += a_dbg[i];
            }
        }
        free(dout); free(o3); free(p); free(rows);
        free(a_dbg); free(a_dwg); free(a_dvc); free(a_dkc); free(a_dv); free(a_dk);
    }
}

/* Zeroes the gradients the backward writes. */
static void zero_grads(const orc_cfg *c, double *dq, double *dk, double *dv, double *dwck, double *dpek,
                       double *dwcv, double *dpev, double *dwg, double *dbg)
{
    const int B = c->B, T = c->T, Hkv = c->Hkv, Hq = Hkv * c->G, dk_ = c->dk, dv_ = c->dv;
    memset(dq, 0, sizeof(double) * (size_t)B * T * Hq * dk_);
    memset(dk, 0, sizeof(double) * (size_t)B * Hkv * T * dk_);
    memset(dv, 0, sizeof(double) * (size_t)B * Hkv * T * dv_);
    memset(dwck, 0, sizeof(double) * (size_t)dk_ * c->l * dk_);
    memset(dpek, 0, sizeof(double) * (size_t)c->l * dk_);
    memset(dwcv, 0, sizeof(double) * (size_t)dv_ * c->l * dv_);
    memset(dpev, 0, sizeof(double) * (size_t)c->l * dv_);
    memset(dwg, 0, sizeof(double) * (size_t)Hq * 3 * dk_);
    memset(dbg, 0, sizeof(double) * (size_t)Hq * 3);
}

/* Full backward.  Layouts as in the forward; idx [B][Hkv][T][n] is the
 * selection used by the forward.  Gradients are written (not accumulated):
 * dq [B][T][Hq][dk], dk/dv [B][Hkv][T][dk|dv], dwck [dk][l*dk], dpek [l][dk],
 * dwcv [dv][l*dv], dpev [l][dv], dwg [Hq][3][dk], dbg [Hq][3].  The
 * compressed K/V are recomputed from k/v (rounded to bf16 if round_bf16, the
 * rounding being passed straight through in reverse). */
void orc_backward(const orc_cfg *c, const double *q, const double *k, const double *v, const double *wck,
                  const double *pek, const double *wcv, const double *pev, const double *wg, const double *bg,
                  const int *idx, const double *dO, int round_bf16, double *dq, double *dk, double *dv,
                  double *dwck, double *dpek, double *dwcv, double *dpev, double *dwg, double *dbg)
{
    const int B = c->B, T = c->T, Hkv = c->Hkv, dk_ = c->dk, dv_ = c->dv;
    const int N = orc_n_cmp(T, c->l, c->d);
    const int Nn = N > 0 ? N : 1;
    double *kc = (double *)calloc((size_t)B * Hkv * Nn * dk_, sizeof(double));
    double *vc = (double *)calloc((size_t)B * Hkv * Nn * dv_, sizeof(double));
    orc_compress(B, Hkv, T, dk_, c->l, c->d, N, round_bf16, k, wck, pek, kc);
    orc_compress(B, Hkv, T, dv_, c->l, c->d, N, round_bf16, v, wcv, pev, vc);
    zero_grads(c, dq, dk, dv, dwck, dpek, dwcv, dpev, dwg, dbg);
    double *dkc = (double *)calloc((size_t)B * Hkv * Nn * dk_, sizeof(double));
    double *dvc = (double *)calloc((size_t)B * Hkv * Nn * dv_, sizeof(double));
    branches_backward(c, q, k, v, kc, vc, wg, bg, idx, dO, dq, dk, dv, dkc, dvc, dwg, dbg);
    if (N > 0) {
        compress_backward(B * Hkv, T, dk_, c->l, c->d, N, k, wck, pek, dkc, dwck, dpek, dk);
        compress_backward(B * Hkv, T, dv_, c->l, c->d, N, v, wcv, pev, dvc, dwcv, dpev, dv);
    }
    free(dvc); free(dkc); free(vc); free(kc);
}

/* Backward of the two-layer map's second layer for one tensor ([deepdaiv],
 * token compression: a small network summarises each block; its layers are
 * those of orc_compress_mlp).  With a [BH][N][dim] the first layer's output
 * (as the forward rounds it) and dC the gradient of the compressed rows:
 *   dW2[c][j] += sum_{bh,i} dC[bh][i][c] * max(a[bh][i][j], 0)
 *   dA[bh][i][j] = (sum_c W2[c][j] * dC[bh][i][c]) * (a[bh][i][j] > 0)
 * (the ReLU's derivative taken as 0 at 0). */
static void mlp2_backward(int BH, int N, int dim, const double *a, const double *W2, const double *dC,
                          double *dW2, double *dA)
{
#pragma omp parallel for schedule(static)
    for (int cc = 0; cc < dim; cc++)
        for (int j = 0; j < dim; j++) {
            double acc = 0.0;
            for (int bh = 0; bh < BH; bh++)
                for (int i = 0; i < N; i++) {
                    const double h = a[((size_t)bh * N + i) * dim + j];
                    acc += dC[((size_t)bh * N + i) * dim + cc] * (h > 0.0 ? h : 0.0);
                }
            dW2[(size_t)cc * dim + j] += acc;
        }
#pragma omp parallel for collapse(2) schedule(static)
    for (int bh = 0; bh < BH; bh++)
        for (int i = 0; i < N; i++) {
            const double *g = dC + ((size_t)bh * N + i) * dim;
            const double *ar = a + ((size_t)bh * N + i) * dim;
            double *out = dA + ((size_t)bh * N + i) * dim;
            for (int j = 0; j < dim; j++) {
                double acc = 0.0;
                for (int cc = 0; cc < dim; cc++) acc += W2[(size_t)cc * dim + j] * g[cc];
                out[j] = ar[j] > 0.0 ? acc : 0.0;
            }
        }
}

/* Full backward with the two-layer compression map (orc_compress_mlp) for K
 * and V: as orc_backward, the first layer's weights and position encodings
 * taking the place of the linear map's (dw1k, dpek, dw1v, dpev), plus the
 * second layers' gradients dw2k [dk][dk], dw2v [dv][dv].  The hidden layer
 * and the compressed K/V are recomputed from k/v, each rounded to bf16 if
 * round_bf16, the roundings passed straight through in reverse. */
void orc_backward_mlp(const orc_cfg *c, const double *q, const double *k, const double *v, const double *w1k,
                      const double *pek, const double *w2k, const double *w1v, const double *pev,
                      const double *w2v, const double *wg, const double *bg, const int *idx, const double *dO,
                      int round_bf16, double *dq, double *dk, double *dv, double *dw1k, double *dpek,
                      double *dw2k, double *dw1v, double *dpev, double *dw2v, double *dwg, double *dbg)
{
    const int B = c->B, T = c->T, Hkv = c->Hkv, dk_ = c->dk, dv_ = c->dv;
    const int N = orc_n_cmp(T, c->l, c->d);
    const int Nn = N > 0 ? N : 1;
    const size_t nkc = (size_t)B * Hkv * Nn * dk_, nvc = (size_t)B * Hkv * Nn * dv_;
    double *ak = (double *)calloc(nkc, sizeof(double)), *av = (double *)calloc(nvc, sizeof(double));
    double *kc = (double *)calloc(nkc, sizeof(double)), *vc = (double *)calloc(nvc, sizeof(double));
    orc_compress(B, Hkv, T, dk_, c->l, c->d, N, round_bf16, k, w1k, pek, ak);
    orc_compress(B, Hkv, T, dv_, c->l, c->d, N, round_bf16, v, w1v, pev, av);
    orc_compress_mlp(B, Hkv, T, dk_, c->l, c->d, N, round_bf16, k, w1k, pek, w2k, kc);
    orc_compress_mlp(B, Hkv, T, dv_, c->l, c->d, N, round_bf16, v, w1v, pev, w2v, vc);
    zero_grads(c, dq, dk, dv, dw1k, dpek, dw1v, dpev, dwg, dbg);
    memset(dw2k, 0, sizeof(double) * (size_t)dk_ * dk_);
    memset(dw2v, 0, sizeof(double) * (size_t)dv_ * dv_);
    double *dkc = (double *)calloc(nkc, sizeof(double)), *dvc = (double *)calloc(nvc, sizeof(double));
    double *dak = (double *)calloc(nkc, sizeof(double)), *dav = (double *)calloc(nvc, sizeof(double));
    branches_backward(c, q, k, v, kc, vc, wg, bg, idx, dO, dq, dk, dv, dkc, dvc, dwg, dbg);
    if (N > 0) {
        mlp2_backward(B * Hkv, N, dk_, ak, w2k, dkc, dw2k, dak);
        mlp2_backward(B * Hkv, N, dv_, av, w2v, dvc, dw2v, dav);
        compress_backward(B * Hkv, T, dk_, c->l, c->d, N, k, w1k, pek, dak, dw1k, dpek, dk);
        compress_backward(B * Hkv, T, dv_, c->l, c->d, N, v, w1v, pev, dav, dw1v, dpev, dv);
    }
    free(dav); free(dak); free(dvc); free(dkc); free(vc); free(kc); free(av); free(ak);
}
