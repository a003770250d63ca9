/*
 * oracle.c -- fp64 reference of the DFlash2 draft-block path.
 *
 * TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library.  It shares no code with the HIP side.
 * Each function follows one step of the method as the pages state it (see
 * oracle.h for the sources and the readings adopted where they are silent).
 * Loops run in the order the definitions are written; OpenMP only splits
 * independent outputs across threads and never reorders a sum.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- exact widening of the stored dtypes --------------------------------- */

static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double elem(const orc_shape* s, const void* base, int64_t i)
{
    if (s->bf16) return bf16_value(((const uint16_t*)base)[i]);
    return (double)((const float*)base)[i];
}

int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- rounding of the conv output to the dtype fed to the head ------------ */

/* bf16 keeps 8 significant bits and the fp32 exponent range.  The spacing of
 * bf16 values around x is 2^(e-8) for x = m * 2^e, 0.5 <= |m| < 1, and never
 * finer than the subnormal spacing 2^-133.  nearbyint() rounds half to even
 * under the default rounding mode. */
static uint16_t bf16_round(double x)
{
    if (x == 0.0 || !isfinite(x)) {
        float f = (float)x;
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        return (uint16_t)(u >> 16);
    }
    int e;
    (void)frexp(x, &e);
    if (e < -125) e = -125;
    double q = nearbyint(ldexp(x, 8 - e));
    float f = (float)ldexp(q, e - 8); /* exact: q has at most 9 bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void orc_round(const orc_shape* s, const double* x, void* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        if (s->bf16) ((uint16_t*)out)[i] = bf16_round(x[i]);
        else ((float*)out)[i] = (float)x[i];
    }
}

/* ---- steps 1-3: grouped dynamic depthwise causal conv --------------------- */
/* Release-note article, "two additions": a per-position (dynamic) kernel,
 * shared by each group of channels (grouped), applied channel by channel
 * (depthwise) to the current and earlier positions of the same block
 * (causal, inside the block).  The per-position kernel is generated from the
 * hidden state at that position and normalised with a softmax over the taps. */
int orc_conv(const orc_shape* s, const void* h, const void* wg,
             double* z, double* w, double* yhat)
{
    const int D = s->hidden, gs = s->group, ks = s->ksize, B = s->block;
    if (gs <= 0 || ks <= 0 || D % gs != 0 || B <= 0) return -1;
    const int G = D / gs, C = G * ks;
    const int rows = s->batch * B;

    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int row = 0; row < rows; ++row) {
        double* zr = (double*)malloc(sizeof(double) * (size_t)C);
        double* wr = (double*)malloc(sizeof(double) * (size_t)C);
        if (!zr || !wr) { free(zr); free(wr); bad = 1; continue; }
        const int t = row % B;
        /* step 1: tap logits z[t, g*ks+j] = sum_c h[t,c] * Wg[c, g*ks+j] */
        for (int col = 0; col < C; ++col) {
            double acc = 0.0;
            for (int c = 0; c < D; ++c)
                acc += elem(s, h, (int64_t)row * D + c) * elem(s, wg, (int64_t)c * C + col);
            zr[col] = acc;
        }
        /* step 2: softmax over the ks taps of each group */
        for (int g = 0; g < G; ++g) {
            double m = zr[g * ks];
            for (int j = 1; j < ks; ++j) if (zr[g * ks + j] > m) m = zr[g * ks + j];
            double den = 0.0;
            for (int j = 0; j < ks; ++j) den += exp(zr[g * ks + j] - m);
            for (int j = 0; j < ks; ++j) wr[g * ks + j] = exp(zr[g * ks + j] - m) / den;
        }
        /* step 3: y[t,c] = sum_j w[t, c/gs, j] * h[t-j, c]; positions before
         * the start of the block contribute zero */
        for (int c = 0; c < D; ++c) {
            const int g = c / gs;
            double acc = 0.0;
            for (int j = 0; j < ks; ++j)
                if (t - j >= 0) acc += wr[g * ks + j] * elem(s, h, (int64_t)(row - j) * D + c);
            yhat[(int64_t)row * D + c] = acc;
        }
        if (z) memcpy(z + (int64_t)row * C, zr, sizeof(double) * (size_t)C);
        if (w) memcpy(w + (int64_t)row * C, wr, sizeof(double) * (size_t)C);
        free(zr);
        free(wr);
    }
    return bad ? -1 : 0;
}

/* ---- steps 5-6: log-softmax and top-K ------------------------------------- */
/* The selector works on the K highest-ranked tokens of the target head at
 * each slot (release-note article, "two additions"); its node score is the
 * candidate's log-probability.
 * Order: larger logit first, equal logits by smaller vocabulary id. */
static int better(const double* L, int a, int b)
{
    return L[a] > L[b] || (L[a] == L[b] && a < b);
}

int orc_topk(int nr, int V, int K, const double* logits,
             int32_t* ids, double* logp, double* lse)
{
    if (K <= 0 || K > V) return -1;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < nr; ++i) {
        const double* L = logits + (int64_t)i * V;
        double m = -INFINITY;
        for (int v = 0; v < V; ++v) if (L[v] > m) m = L[v];
        double z;
        if (m == -INFINITY) {
            z = -INFINITY;
        } else {
            double sum = 0.0;
            for (int v = 0; v < V; ++v) sum += exp(L[v] - m);
            z = m + log(sum);
        }
        lse[i] = z;
        int32_t* out = ids + (int64_t)i * K;
        int n = 0;
        for (int v = 0; v < V; ++v) {
            if (n == K && !better(L, v, out[K - 1])) continue;
            int p = (n < K) ? n++ : K - 1;
            while (p > 0 && better(L, v, out[p - 1])) { out[p] = out[p - 1]; --p; }
            out[p] = v;
        }
        for (int k = 0; k < K; ++k) logp[(int64_t)i * K + k] = L[out[k]] - z;
    }
    return 0;
}

/* ---- step 4: vocabulary head --------------------------------------------- */
/* Logits of every row of the block against the shared target head
 * (release-note article, "two additions": the candidates come from the
 * target's head; RTX 4090 report: the drafter shares embedding and lm_head
 * with the target). */
int orc_head(const orc_shape* s, const void* y, const void* W, int r0, int nr,
             double* logits, double* lse, int32_t* ids, double* logp)
{
    const int D = s->hidden, V = s->vocab, K = s->top_k;
    if (nr <= 0 || K <= 0 || K > V) return -1;
    double* L = logits;
    if (!L) L = (double*)malloc(sizeof(double) * (size_t)nr * (size_t)V);
    double* yd = (double*)malloc(sizeof(double) * (size_t)nr * (size_t)D);
    if (!L || !yd) { if (!logits) free(L); free(yd); return -1; }
    for (int i = 0; i < nr; ++i)
        for (int c = 0; c < D; ++c) yd[(int64_t)i * D + c] = elem(s, y, (int64_t)(r0 + i) * D + c);

    int bad = 0;
#pragma omp parallel reduction(| : bad)
    {
        double* wrow = (double*)malloc(sizeof(double) * (size_t)D);
        if (!wrow) bad = 1;
#pragma omp for schedule(static)
        for (int v = 0; v < V; ++v) {
            if (!wrow) continue;
            for (int c = 0; c < D; ++c) wrow[c] = elem(s, W, (int64_t)v * D + c);
            for (int i = 0; i < nr; ++i) {
                const double* yr = yd + (int64_t)i * D;
                double acc = 0.0;
                for (int c = 0; c < D; ++c) acc += yr[c] * wrow[c];
                L[(int64_t)i * V + v] = acc;
            }
        }
        free(wrow);
    }
    int rc = bad ? -1 : orc_topk(nr, V, K, L, ids, logp, lse);
    if (!logits) free(L);
    free(yd);
    return rc;
}

/* ---- step 7: low-rank adjacent-transition scores -------------------------- */
/* Inco AI post, "lightweight path selector": the pair score of successor b
 * after predecessor a at slot t is <A(a) (*) H(h_t), B(b)>, A and B being
 * per-token rank-r embeddings and H(h_t) a context gate of slot t's hidden
 * state (elementwise product).  Here P holds A(.), Q holds B(.) and gate row t
 * holds H(h_t); with no gate, H = 1.  The first draft slot follows the
 * verified anchor. */
int orc_transitions(const orc_shape* s, int32_t anchor, const int32_t* ids,
                    const void* P, const void* Q, const double* gate, double* T)
{
    const int B = s->block, K = s->top_k, r = s->rank;
    if (B < 2 || K <= 0) return -1;
    for (int t = 1; t < B; ++t) {
        double* Tt = T + (int64_t)(t - 1) * K * K;
        const int nprev = (t == 1) ? 1 : K;
        for (int j = 0; j < K; ++j) {
            for (int k = 0; k < K; ++k) {
                if (j >= nprev) { Tt[j * K + k] = 0.0; continue; }
                const int64_t a = (t == 1) ? anchor : ids[(t - 1) * K + j];
                const int64_t b = ids[t * K + k];
                double acc = 0.0;
                for (int i = 0; i < r; ++i) {
                    const double g = gate ? gate[(int64_t)t * r + i] : 1.0;
                    acc += elem(s, P, a * r + i) * g * elem(s, Q, b * r + i);
                }
                Tt[j * K + k] = acc;
            }
        }
    }
    return 0;
}

/* ---- step 8: best path from the anchor (max-sum Viterbi) ------------------ */
/* Release-note article, "two additions": the selector picks the
 * highest-scoring path through the per-slot candidates, starting at the
 * accepted anchor.  Path score = sum over draft slots of the node score
 * plus the transition score from the previous slot's choice (the anchor for
 * slot 1).  Ties: the lowest predecessor index, and the lowest final index. */
int orc_viterbi(int B, int K, const double* logp, const double* T,
                int32_t* idx, double* score, double* margin)
{
    if (B < 2 || K <= 0) return -1;
    double* delta = (double*)malloc(sizeof(double) * (size_t)K);
    double* nd = (double*)malloc(sizeof(double) * (size_t)K);
    int32_t* bp = (int32_t*)calloc((size_t)B * (size_t)K, sizeof(int32_t));
    /* 2-best bookkeeping for the margin: best and second-best score over
     * distinct index sequences ending in each state. */
    double* s1 = (double*)malloc(sizeof(double) * (size_t)K);
    double* s2 = (double*)malloc(sizeof(double) * (size_t)K);
    double* n1 = (double*)malloc(sizeof(double) * (size_t)K);
    double* n2 = (double*)malloc(sizeof(double) * (size_t)K);
    if (!delta || !nd || !bp || !s1 || !s2 || !n1 || !n2) {
        free(delta); free(nd); free(bp); free(s1); free(s2); free(n1); free(n2);
        return -1;
    }

    for (int k = 0; k < K; ++k) {
        delta[k] = logp[1 * K + k] + T[0 * K * K + 0 * K + k];
        s1[k] = delta[k];
        s2[k] = -INFINITY;
    }
    for (int t = 2; t < B; ++t) {
        const double* Tt = T + (int64_t)(t - 1) * K * K;
        for (int k = 0; k < K; ++k) {
            double best = delta[0] + Tt[0 * K + k];
            int bj = 0;
            for (int j = 1; j < K; ++j) {
                double c = delta[j] + Tt[j * K + k];
                if (c > best) { best = c; bj = j; }
            }
            nd[k] = best + logp[t * K + k];
            bp[t * K + k] = bj;

            double a1 = -INFINITY, a2 = -INFINITY;
            for (int j = 0; j < K; ++j) {
                double c[2] = { s1[j] + Tt[j * K + k], s2[j] + Tt[j * K + k] };
                for (int u = 0; u < 2; ++u) {
                    if (c[u] > a1) { a2 = a1; a1 = c[u]; }
                    else if (c[u] > a2) { a2 = c[u]; }
                }
            }
            n1[k] = a1 + logp[t * K + k];
            n2[k] = a2 + logp[t * K + k];
        }
        memcpy(delta, nd, sizeof(double) * (size_t)K);
        memcpy(s1, n1, sizeof(double) * (size_t)K);
        memcpy(s2, n2, sizeof(double) * (size_t)K);
    }
    int kb = 0;
    for (int k = 1; k < K; ++k) if (delta[k] > delta[kb]) kb = k;
    idx[B - 1] = kb;
    for (int t = B - 1; t >= 2; --t) idx[t - 1] = bp[t * K + idx[t]];
    idx[0] = -1;
    *score = delta[kb];

    if (margin) {
        double f1 = -INFINITY, f2 = -INFINITY;
        for (int k = 0; k < K; ++k) {
            double c[2] = { s1[k], s2[k] };
            for (int u = 0; u < 2; ++u) {
                if (c[u] > f1) { f2 = f1; f1 = c[u]; }
                else if (c[u] > f2) { f2 = c[u]; }
            }
        }
        *margin = (f2 == -INFINITY) ? INFINITY : f1 - f2;
    }
    free(delta); free(nd); free(bp); free(s1); free(s2); free(n1); free(n2);
    return 0;
}

/* ---- step 8, other walk rules ----------------------------------------------- */
/* Inco AI post, "lightweight path selector": besides the best path, the
 * selector can walk greedily, taking at each slot the best successor of the
 * token chosen before it, or sample the successor from the same scores at a
 * temperature.  Score of candidate k at slot t after index p of slot t-1:
 * s_t(k) = logp[t][k] + T[t-1][p][k] (p = 0, the anchor, at t = 1).
 *  greedy: the largest s_t(k), lowest k on ties;
 *  sample: weights e_k = exp((s_t(k) - max_k s_t(k)) / temperature); with
 *          prefix sums E_k = e_0 + ... + e_k in index order, the smallest k
 *          with E_k > u_t * E_{K-1}, where u_t in [0, 1) is the caller's
 *          uniform for slot t (uniforms[t], t >= 1).
 * idx [B] receives -1 then the chosen indices; *score the sum of the chosen
 * s_t. */
int orc_walk(int B, int K, const double* logp, const double* T, int mode,
             double temperature, const double* uniforms, int32_t* idx, double* score)
{
    if (B < 2 || K <= 0 || (mode != 1 && mode != 2)) return -1;
    if (mode == 2 && (!uniforms || !(temperature > 0.0))) return -1;
    double* sc = (double*)malloc(sizeof(double) * (size_t)K);
    double* pre = (double*)malloc(sizeof(double) * (size_t)K);
    if (!sc || !pre) { free(sc); free(pre); return -1; }
    int prev = 0;
    double total = 0.0;
    idx[0] = -1;
    for (int t = 1; t < B; ++t) {
        const double* Tt = T + (int64_t)(t - 1) * K * K + (int64_t)prev * K;
        double m = -INFINITY;
        int best = 0;
        for (int k = 0; k < K; ++k) {
            sc[k] = logp[(int64_t)t * K + k] + Tt[k];
            if (sc[k] > m) { m = sc[k]; best = k; }
        }
        int pick = best;
        if (mode == 2) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) { acc += exp((sc[k] - m) / temperature); pre[k] = acc; }
            const double target = uniforms[t] * acc;
            pick = K - 1;
            for (int k = 0; k < K; ++k) if (pre[k] > target) { pick = k; break; }
        }
        idx[t] = pick;
        total += sc[pick];
        prev = pick;
    }
    *score = total;
    free(sc); free(pre);
    return 0;
}

/* ---- the whole draft block ------------------------------------------------ */

int orc_draft_block(const orc_shape* s, const void* h, const int32_t* anchor,
                    const void* wg, const void* W, const void* P, const void* Q,
                    const double* gate, int32_t* path, double* score, int32_t* ids,
                    double* logp, double* lse, int32_t* idx, double* margin)
{
    const int B = s->block, K = s->top_k, D = s->hidden, V = s->vocab;
    const int rows = s->batch * B;
    const size_t esz = s->bf16 ? 2 : 4;
    int rc = -1;
    double* yhat = (double*)malloc(sizeof(double) * (size_t)rows * D);
    void* y = malloc(esz * (size_t)rows * D);
    int32_t* cid = (int32_t*)malloc(sizeof(int32_t) * (size_t)rows * K);
    double* clp = (double*)malloc(sizeof(double) * (size_t)rows * K);
    double* cl = (double*)malloc(sizeof(double) * (size_t)rows);
    double* T = (double*)malloc(sizeof(double) * (size_t)(B - 1) * K * K);
    int32_t* bi = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
    if (!yhat || !y || !cid || !clp || !cl || !T || !bi || B < 2) goto done;

    if (orc_conv(s, h, wg, NULL, NULL, yhat)) goto done;
    orc_round(s, yhat, y, (int64_t)rows * D);
    if (orc_head(s, y, W, 0, rows, NULL, cl, cid, clp)) goto done;

    for (int b = 0; b < s->batch; ++b) {
        double sc = NAN, mg = NAN;
        if (anchor[b] < 0 || anchor[b] >= V) {
            for (int t = 0; t < B; ++t) { path[b * B + t] = -1; bi[t] = -1; }
        } else {
            const double* gb = gate ? gate + (int64_t)b * B * s->rank : NULL;
            if (orc_transitions(s, anchor[b], cid + (int64_t)b * B * K, P, Q, gb, T)) goto done;
            if (orc_viterbi(B, K, clp + (int64_t)b * B * K, T, bi, &sc, &mg)) goto done;
            path[b * B] = anchor[b];
            for (int t = 1; t < B; ++t) path[b * B + t] = cid[((int64_t)b * B + t) * K + bi[t]];
        }
        score[b] = sc;
        if (margin) margin[b] = mg;
        if (idx) memcpy(idx + (int64_t)b * B, bi, sizeof(int32_t) * (size_t)B);
    }
    if (ids) memcpy(ids, cid, sizeof(int32_t) * (size_t)rows * K);
    if (logp) memcpy(logp, clp, sizeof(double) * (size_t)rows * K);
    if (lse) memcpy(lse, cl, sizeof(double) * (size_t)rows);
    rc = 0;
done:
    free(yhat); free(y); free(cid); free(clp); free(cl); free(T); free(bi);
    return rc;
}
