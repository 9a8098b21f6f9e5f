/*
 * rom_oracle.c -- CPU oracle for the Routing Mamba (RoM) routed projections.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain, obviously correct
 * statement of what the routed projections compute. Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it. The product
 * path (the HIP library) shares no code, header, table or helper with it.
 *
 * Source of the method: "Routing Mamba: Scaling State Space Models with
 * Mixture-of-Experts Projection", landing page on chapterpal.com, Knowl 1
 * ("RoM uses one sparse routing decision for Mamba projection experts"):
 *   p_t   = Softmax(x_t W_r)                       over all N experts
 *   S_t   = indices of the K largest p_t
 *   r_t,i = p_t,i * 1[i in S_t]                    (no renormalisation over S_t)
 *   H_t   = sum_i 1[i in S_t] x_t W_in,i           (indicator only, no p scale)
 *   G_t   = SiLU(sum_i 1[i in S_t] x_t W_g,i)      (indicator only, no p scale)
 *   O_t   = sum_i r_t,i (Y_t (.) G_t) W_out,i      (scaled by the router probability)
 * SiLU is the sigmoid-weighted linear unit v * sigmoid(v) (the page's
 * reference list: Elfwing, Uchibe and Doya, 2018).
 *
 * Readings where the page is silent (each is listed in the design notes):
 *  - Storage: expert matrices are stored transposed, [out][in] (K-contiguous),
 *    so x_t W_in,i is computed as sum_k X[t][k] * W_conv[i][n][k].
 *  - Ties in "the K largest": the lowest expert index wins.
 *  - The router runs in fp32: logits are fp32 sums taken in ascending k, then
 *    the bias (a synthetic workload device; absent from the page's formula) is
 *    added. The selection is made on these fp32 logits. The probability is the
 *    softmax of those fp32 logits evaluated in double, rounded to fp32.
 *  - The projections accumulate in double (no rounding beyond fp64's).
 *  - The in-projection returns the pre-activation z; SiLU is applied where
 *    the gate meets Y, i.e. in the out-projection. h stands in for Y_t.
 *  - Grouping tokens by expert: a histogram, an exclusive prefix sum and a
 *    stable counting sort (tokens keep ascending order within an expert).
 *    The page states no grouping; a dropless grouped computation (Knowl 12:
 *    no capacity factor, no token dropping) needs one.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math, no
 * FMA contraction, so each sum is the plain left-to-right sum). OpenMP splits
 * the independent per-token loops across threads; it reorders no sum.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int orom_version(void) { return 1; }

/* Threads the OpenMP loops below use (reporting only). */
int orom_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

/* ---------------------------------------------------------------------------
 * Router (Knowl 1, first paragraph).
 *
 * X [T][dm] fp32, Wr [dm][E] fp32, bias [E] or NULL.
 * Outputs per token t: ids[t][0..K) the K selected experts in order of
 * decreasing logit (lowest index first on ties), prob[t][0..K) their softmax
 * probabilities p_t,i (not renormalised), gap[t] = l_(K) - l_(K+1), the
 * margin of the selection (+inf when K == E), and, if logits != NULL, the
 * fp32 logits [T][E].
 */
void orom_route(const float *X, int64_t T, int64_t dm, const float *Wr, const float *bias,
                int32_t E, int32_t K, int32_t *ids, float *prob, float *gap, float *logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        float *l = (float *)malloc(sizeof(float) * (size_t)E);
        char *taken = (char *)calloc((size_t)E, 1);
        const float *x = X + t * dm;
        for (int32_t j = 0; j < E; ++j) {
            float acc = 0.0f;
            for (int64_t k = 0; k < dm; ++k)
                acc = acc + x[k] * Wr[k * E + j];
            if (bias)
                acc = acc + bias[j];
            l[j] = acc;
        }
        if (logits)
            memcpy(logits + t * E, l, sizeof(float) * (size_t)E);

        /* softmax in double over all E experts */
        float lmax = l[0];
        for (int32_t j = 1; j < E; ++j)
            if (l[j] > lmax) lmax = l[j];
        double denom = 0.0;
        for (int32_t j = 0; j < E; ++j)
            denom += exp((double)l[j] - (double)lmax);

        /* the K largest, lowest index on ties (strict > scanning j upward) */
        float last = 0.0f;
        for (int32_t s = 0; s < K; ++s) {
            int32_t best = -1;
            for (int32_t j = 0; j < E; ++j) {
                if (taken[j]) continue;
                if (best < 0 || l[j] > l[best]) best = j;
            }
            taken[best] = 1;
            ids[t * K + s] = best;
            prob[t * K + s] = (float)(exp((double)l[best] - (double)lmax) / denom);
            last = l[best];
        }
        /* margin to the best unselected expert */
        int32_t next = -1;
        for (int32_t j = 0; j < E; ++j) {
            if (taken[j]) continue;
            if (next < 0 || l[j] > l[next]) next = j;
        }
        gap[t] = next < 0 ? INFINITY : last - l[next];
        free(l);
        free(taken);
    }
}

/* ---------------------------------------------------------------------------
 * Histogram and stable counting sort of n assignments (n = T*K; assignment a
 * belongs to token a / K) by expert id.
 *   counts[e]   = #{a : ids[a] = e}
 *   offsets[0]  = 0, offsets[e+1] = offsets[e] + counts[e]
 *   perm[pos]   = a, inv_perm[a] = pos, with pos = offsets[ids[a]] + #{a' < a : ids[a'] = ids[a]}
 * Returns 0, or -1 if an id lies outside [0, E).
 */
int orom_sort(const int32_t *ids, int64_t n, int32_t E, int32_t *counts, int32_t *offsets,
              int32_t *perm, int32_t *inv_perm)
{
    for (int32_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t a = 0; a < n; ++a) {
        if (ids[a] < 0 || ids[a] >= E) return -1;
        counts[ids[a]] += 1;
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    for (int32_t e = 0; e < E; ++e)
        next[e] = offsets[e];
    for (int64_t a = 0; a < n; ++a) {
        int32_t pos = next[ids[a]]++;
        perm[pos] = (int32_t)a;
        inv_perm[a] = pos;
    }
    free(next);
    return 0;
}

/* Permute: Xp[pos] = X[perm[pos] / K], rows of dm floats (slot order). */
void orom_permute(const float *X, int64_t n, int32_t K, int64_t dm, const int32_t *perm, float *Xp)
{
    for (int64_t pos = 0; pos < n; ++pos)
        memcpy(Xp + pos * dm, X + (int64_t)(perm[pos] / K) * dm, sizeof(float) * (size_t)dm);
}

/* ---------------------------------------------------------------------------
 * In-projection (Knowl 1, H_t and the argument of SiLU in G_t) for n tokens.
 *
 * X [n][dm]; ids [n][K]; Wc, Wg [E][di][dm] (row n of expert i is column n
 * of the page's W_in,i / W_g,i). Outputs x_out, z_out [n][di] in double:
 *   x[t][c] = sum_{s<K} sum_k X[t][k] * Wc[ids[t][s]][c][k]
 *   z[t][c] = sum_{s<K} sum_k X[t][k] * Wg[ids[t][s]][c][k]
 * The indicator 1[i in S_t] admits exactly the K selected experts, unscaled.
 */
void orom_in_proj(const float *X, int64_t n, int64_t dm, int64_t di, const int32_t *ids, int32_t K,
                  const float *Wc, const float *Wg, int32_t E, double *x_out, double *z_out)
{
    (void)E;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const float *x = X + t * dm;
        for (int64_t c = 0; c < di; ++c) {
            double hx = 0.0, hz = 0.0;
            for (int32_t s = 0; s < K; ++s) {
                const int64_t i = ids[t * K + s];
                const float *wc = Wc + (i * di + c) * dm;
                const float *wg = Wg + (i * di + c) * dm;
                for (int64_t k = 0; k < dm; ++k) {
                    hx += (double)x[k] * (double)wc[k];
                    hz += (double)x[k] * (double)wg[k];
                }
            }
            x_out[t * di + c] = hx;
            z_out[t * di + c] = hz;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Out-projection (Knowl 1, O_t) for n tokens, with h standing in for Y_t.
 *
 * z [n][di] (pre-activation gate), h [n][di], ids and prob [n][K],
 * Wo [E][dm][di] (row m of expert i is column m of the page's W_out,i).
 *   a[t][c]   = SiLU(z[t][c]) * h[t][c],  SiLU(v) = v / (1 + exp(-v))
 *   out[t][m] = sum_{s<K} prob[t][s] * sum_c a[t][c] * Wo[ids[t][s]][m][c]
 */
void orom_out_proj(const double *z, const float *h, int64_t n, int64_t di, int64_t dm,
                   const int32_t *ids, const float *prob, int32_t K, const float *Wo, int32_t E,
                   double *out)
{
    (void)E;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        double *a = (double *)malloc(sizeof(double) * (size_t)di);
        for (int64_t c = 0; c < di; ++c) {
            const double v = z[t * di + c];
            a[c] = v / (1.0 + exp(-v)) * (double)h[t * di + c];
        }
        for (int64_t m = 0; m < dm; ++m) {
            double o = 0.0;
            for (int32_t s = 0; s < K; ++s) {
                const int64_t i = ids[t * K + s];
                const float *wo = Wo + (i * dm + m) * di;
                double acc = 0.0;
                for (int64_t c = 0; c < di; ++c)
                    acc += a[c] * (double)wo[c];
                o += (double)prob[t * K + s] * acc;
            }
            out[t * dm + m] = o;
        }
        free(a);
    }
}

/* ---------------------------------------------------------------------------
 * Routing-weighted in-projection of Switch Mamba (Swimba project page,
 * extended abstract): the in-projection is a set of expert projections behind a
 * token-level softmax router, and the experts' streams, each weighted by its
 * routing weight, are summed into the one input of the SSM kernel. The routing
 * weight is read as Knowl 1's r_t,i of the RoM page, i.e. the softmax
 * probability of a selected expert, not renormalised over the selection.
 *
 * X [n][dm]; ids, prob [n][K]; W [E][dout][dm] (row c of expert i is column c
 * of that expert's in-projection). Output y [n][dout] in double:
 *   y[t][c] = sum_{s<K} prob[t][s] * sum_k X[t][k] * W[ids[t][s]][c][k]
 */
void orom_in_proj_weighted(const float *X, int64_t n, int64_t dm, int64_t dout, const int32_t *ids,
                           const float *prob, int32_t K, const float *W, int32_t E, double *y)
{
    (void)E;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const float *x = X + t * dm;
        for (int64_t c = 0; c < dout; ++c) {
            double yc = 0.0;
            for (int32_t s = 0; s < K; ++s) {
                const int64_t i = ids[t * K + s];
                const float *w = W + (i * dout + c) * dm;
                double stream = 0.0;
                for (int64_t k = 0; k < dm; ++k)
                    stream += (double)x[k] * (double)w[k];
                yc += (double)prob[t * K + s] * stream;
            }
            y[t * dout + c] = yc;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Shared short causal convolution (Routing Mamba landing page, Knowl 1: the
 * short convolution applied to H_t before the selective SSM; Knowl 9: the 1D
 * convolution is shared across experts, not expertized). The page gives no
 * width, no bias convention and no activation; the reading taken here is a
 * depthwise (per-channel) causal convolution of width w over each sequence
 * separately, with zeros before a sequence's first token, an optional
 * per-channel bias, and an optional SiLU on the result:
 *   u[b][t][c] = bias[c] + sum_{j<w} W[c][j] * H[b][t - (w-1) + j][c]
 *   y[b][t][c] = act ? SiLU(u) : u,   H[b][s][c] = 0 for s < 0
 * so W[c][w-1] multiplies the current token and W[c][0] the oldest.
 * H [nseq][L][C] fp32 (token order, sequences contiguous), W [C][w],
 * bias [C] or NULL. Output y in double.
 */
void orom_conv1d(const float *H, int64_t nseq, int64_t L, int64_t C, const float *W, const float *bias,
                 int32_t w, int32_t act, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t bt = 0; bt < nseq * L; ++bt) {
        const int64_t b = bt / L, t = bt % L;
        for (int64_t c = 0; c < C; ++c) {
            double u = bias ? (double)bias[c] : 0.0;
            for (int32_t j = 0; j < w; ++j) {
                const int64_t s = t - (w - 1) + j;
                if (s < 0) continue;
                u += (double)W[c * w + j] * (double)H[(b * L + s) * C + c];
            }
            y[bt * C + c] = act ? u / (1.0 + exp(-u)) : u;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Backward of the routed projections: the exact derivatives of Knowl 1's
 * H_t, G_t (pre-activation z) and O_t with respect to their inputs and expert
 * weights, for n tokens. The router's probabilities are treated as given (the
 * gradient that reaches the router through p, and through the selection S_t,
 * is not computed here).
 *
 * Out-projection, with g = dL/dout [n][dm] and a = SiLU(z) * h:
 *   da[t][c]      = sum_{s<K} prob[t][s] * sum_m Wo[ids[t][s]][m][c] * g[t][m]
 *   dz[t][c]      = da[t][c] * h[t][c] * SiLU'(z[t][c]),
 *                   SiLU'(v) = sig(v) * (1 + v * (1 - sig(v))), sig(v) = 1 / (1 + exp(-v))
 *   dh[t][c]      = da[t][c] * SiLU(z[t][c])
 *   dWo[i][m][c]  = sum over (t, s) with ids[t][s] = i of prob[t][s] * g[t][m] * a[t][c]
 */
void orom_out_proj_dgrad(const float *g, const double *z, const float *h, int64_t n, int64_t di, int64_t dm,
                         const int32_t *ids, const float *prob, int32_t K, const float *Wo, int32_t E,
                         double *dz, double *dh)
{
    (void)E;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        for (int64_t c = 0; c < di; ++c) {
            double da = 0.0;
            for (int32_t s = 0; s < K; ++s) {
                const int64_t i = ids[t * K + s];
                double col = 0.0;
                for (int64_t m = 0; m < dm; ++m)
                    col += (double)Wo[(i * dm + m) * di + c] * (double)g[t * dm + m];
                da += (double)prob[t * K + s] * col;
            }
            const double v = z[t * di + c];
            const double sg = 1.0 / (1.0 + exp(-v));
            dz[t * di + c] = da * (double)h[t * di + c] * (sg * (1.0 + v * (1.0 - sg)));
            dh[t * di + c] = da * (v * sg);
        }
    }
}

/* One weight-gradient entry dWo[i][m][c], summed over the tokens in ascending order. */
static double out_wgrad_entry(const float *g, const double *z, const float *h, int64_t n, int64_t di, int64_t dm,
                              const int32_t *ids, const float *prob, int32_t K, int64_t i, int64_t m, int64_t c)
{
    double acc = 0.0;
    for (int64_t t = 0; t < n; ++t)
        for (int32_t s = 0; s < K; ++s) {
            if (ids[t * K + s] != i) continue;
            const double v = z[t * di + c];
            const double a = v / (1.0 + exp(-v)) * (double)h[t * di + c];
            acc += (double)prob[t * K + s] * (double)g[t * dm + m] * a;
        }
    return acc;
}

/* The full dWo [E][dm][di]. */
void orom_out_proj_wgrad(const float *g, const double *z, const float *h, int64_t n, int64_t di, int64_t dm,
                         const int32_t *ids, const float *prob, int32_t K, int32_t E, double *dWo)
{
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < (int64_t)E * dm * di; ++q) {
        const int64_t i = q / (dm * di), m = (q / di) % dm, c = q % di;
        dWo[q] = out_wgrad_entry(g, z, h, n, di, dm, ids, prob, K, i, m, c);
    }
}

/* Selected entries: entry j is dWo[ent[3j]][ent[3j+1]][ent[3j+2]]. */
void orom_out_proj_wgrad_entries(const float *g, const double *z, const float *h, int64_t n, int64_t di,
                                 int64_t dm, const int32_t *ids, const float *prob, int32_t K, const int64_t *ent,
                                 int64_t nent, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nent; ++j)
        out[j] = out_wgrad_entry(g, z, h, n, di, dm, ids, prob, K, ent[3 * j], ent[3 * j + 1], ent[3 * j + 2]);
}

/* In-projection, with dx = dL/dH and dzg = dL/dz (the pre-activation gate):
 *   dX[t][k]       = sum_{s<K} sum_c (Wc[ids[t][s]][c][k] * dx[t][c] + Wg[ids[t][s]][c][k] * dzg[t][c])
 *   dWc[i][c][k]   = sum over (t, s) with ids[t][s] = i of dx[t][c] * X[t][k]   (dWg likewise with dzg)
 * (the indicator 1[i in S_t] carries no probability, so neither does its derivative).
 */
void orom_in_proj_dgrad(const float *dx, const float *dzg, int64_t n, int64_t dm, int64_t di, const int32_t *ids,
                        int32_t K, const float *Wc, const float *Wg, int32_t E, double *dX)
{
    (void)E;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        for (int64_t k = 0; k < dm; ++k) {
            double acc = 0.0;
            for (int32_t s = 0; s < K; ++s) {
                const int64_t i = ids[t * K + s];
                for (int64_t c = 0; c < di; ++c)
                    acc += (double)Wc[(i * di + c) * dm + k] * (double)dx[t * di + c]
                         + (double)Wg[(i * di + c) * dm + k] * (double)dzg[t * di + c];
            }
            dX[t * dm + k] = acc;
        }
    }
}

/* One entry of dWc (gate = 0) or dWg (gate = 1) [i][c][k], summed over the tokens in ascending order. */
static double in_wgrad_entry(const float *X, const float *dy, int64_t n, int64_t dm, int64_t di,
                             const int32_t *ids, int32_t K, int64_t i, int64_t c, int64_t k)
{
    double acc = 0.0;
    for (int64_t t = 0; t < n; ++t)
        for (int32_t s = 0; s < K; ++s) {
            if (ids[t * K + s] != i) continue;
            acc += (double)dy[t * di + c] * (double)X[t * dm + k];
        }
    return acc;
}

void orom_in_proj_wgrad(const float *X, const float *dx, const float *dzg, int64_t n, int64_t dm, int64_t di,
                        const int32_t *ids, int32_t K, int32_t E, double *dWc, double *dWg)
{
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < (int64_t)E * di * dm; ++q) {
        const int64_t i = q / (di * dm), c = (q / dm) % di, k = q % dm;
        dWc[q] = in_wgrad_entry(X, dx, n, dm, di, ids, K, i, c, k);
        dWg[q] = in_wgrad_entry(X, dzg, n, dm, di, ids, K, i, c, k);
    }
}

/* Selected entries (i, c, k) of dWc and dWg. */
void orom_in_proj_wgrad_entries(const float *X, const float *dx, const float *dzg, int64_t n, int64_t dm,
                                int64_t di, const int32_t *ids, int32_t K, const int64_t *ent, int64_t nent,
                                double *outc, double *outg)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nent; ++j) {
        outc[j] = in_wgrad_entry(X, dx, n, dm, di, ids, K, ent[3 * j], ent[3 * j + 1], ent[3 * j + 2]);
        outg[j] = in_wgrad_entry(X, dzg, n, dm, di, ids, K, ent[3 * j], ent[3 * j + 1], ent[3 * j + 2]);
    }
}
