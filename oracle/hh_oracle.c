/*
 * hh_oracle.c -- plain, slow, fp64 CPU oracle for Hedgehog-style linear
 * attention.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark call it to check and to time the HIP
 * library.  The library never calls, links or includes this file, and this
 * file shares no code with it.
 *
 * Sources (all on "The Hedgehog & the Porcupine: Expressive Linear Attentions
 * with Softmax Mimicry", the paper-graph-ui walkthrough of arXiv 2402.04347,
 * and the paperlayer.ai summary of the same paper):
 *   - Eq. 2 (section 2, Context and Motivation; restated in section 3.4,
 *     "Complexity Analysis"): y_i = phi(q_i)^T sum_{j<=i} phi(k_j) v_j^T
 *     divided by phi(q_i)^T sum_{j<=i} phi(k_j).
 *   - Running sums S_i, z_i and their per-token update (section 3.4,
 *     "Complexity Analysis", the bullet list of costs).
 *   - Hedgehog map phi(x) = exp(W x + b) with one output per row w_l of W
 *     (section 3.4, "The Hedgehog MLP Feature Map", Choice 1) extended with the
 *     negated half exp(-(W x + b)) to R^{2d} (Choice 3; paperlayer A.1).
 *   - Degree-2 Taylor map [1, x, x_i x_j] with kernel 1 + q.k + (q.k)^2/2
 *     (section 3.4, "The Taylor Exponential as a Bridge Result").
 *   - Generalised quadratic kernel p(s) = a + b s + c s^2 of the learned global
 *     quadratic (paperlayer.ai summary of arXiv 2610.13674, section 2 and App. D,
 *     "Global Reference and HD Realization"), realised by the feature map
 *     [sqrt(a), sqrt(b) x, sqrt(c) x_i x_j] so that phi(q).phi(k) = p(q.k); the
 *     Taylor map is the case (a, b, c) = (1, 1, 1/2).  The coefficients are
 *     per head and must be >= 0.
 *   - Bidirectional (encoder) attention: the same sums taken over every key
 *     (paperlayer section 1: bidirectional BERT conversions).
 *   - Attention-weight distillation loss, Eq. 4 (section 3.4, "The Attention
 *     Weight Distillation Loss"): for query i, the cross-entropy between the
 *     causal softmax weights of q_i.k_j / sqrt(d) over j <= i (the raw q, k, not
 *     their features) and the linear weights phi(q_i).phi(k_j) normalised over
 *     the same keys.
 *
 * Readings taken where the pages are silent or garbled:
 *   - W is stored [d_out][d_in] row-major and u = W x + b (the pages call w_l
 *     "the l-th row of W").
 *   - Feature order: positive half first, then the negated half; the negation
 *     covers the bias too.
 *   - Taylor quadratic block carries 1/sqrt(2) so that phi(q).phi(k) equals
 *     1 + s + s^2/2 exactly; pairs in row-major order a*d + c, all d*d kept.
 *   - Causal sums are inclusive (j <= i); a decode step updates, then reads.
 *   - No scaling of q or k inside the method, no epsilon in the denominator.
 *
 * Everything is computed in double.  Inputs arrive as double arrays that
 * hold the exact values the library receives.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define HHO_HEDGEHOG 0
#define HHO_TAYLOR2 1
#define HHO_HEDGEHOG_SOFTMAX 2
#define HHO_EXP 3
#define HHO_SOFTMAX 4
#define HHO_QUADRATIC 5

int hho_feature_dim(int map, int d) {
    if (map == HHO_HEDGEHOG || map == HHO_HEDGEHOG_SOFTMAX) return 2 * d;
    if (map == HHO_TAYLOR2 || map == HHO_QUADRATIC) return 1 + d + d * d;
    if (map == HHO_EXP || map == HHO_SOFTMAX) return d;
    return -1;
}

/* Hedgehog feature map (Choices 1 and 3): u_l = b_l + sum_m W[l][m] x_m,
 * phi = (exp(u_0), ..., exp(u_{d-1}), exp(-u_0), ..., exp(-u_{d-1})). */
static void phi_hedgehog(int d, const double *x, const double *W, const double *b, double *out) {
    for (int l = 0; l < d; l++) {
        double u = b ? b[l] : 0.0;
        for (int m = 0; m < d; m++) u += W[(size_t)l * d + m] * x[m];
        out[l] = exp(u);
        out[d + l] = exp(-u);
    }
}

/* Degree-2 Taylor feature map: (1, x_0..x_{d-1}, x_a x_c / sqrt(2) for a, c in [d]). */
static void phi_taylor(int d, const double *x, double *out) {
    const double r = 1.0 / sqrt(2.0);
    out[0] = 1.0;
    for (int m = 0; m < d; m++) out[1 + m] = x[m];
    for (int a = 0; a < d; a++)
        for (int c = 0; c < d; c++) out[1 + d + (size_t)a * d + c] = x[a] * x[c] * r;
}

/* Generalised quadratic map, coefficients abc = (a, b, c):
 * (sqrt(a), sqrt(b) x_0..x_{d-1}, sqrt(c) x_a x_c for a, c in [d]), so that
 * phi(q).phi(k) = a + b s + c s^2 with s = q.k. */
static void phi_quadratic(int d, const double *x, const double *abc, double *out) {
    const double sa = sqrt(abc[0]), sb = sqrt(abc[1]), sc = sqrt(abc[2]);
    out[0] = sa;
    for (int m = 0; m < d; m++) out[1 + m] = sb * x[m];
    for (int a = 0; a < d; a++)
        for (int c = 0; c < d; c++) out[1 + d + (size_t)a * d + c] = sc * x[a] * x[c];
}

/* Single-sided exponential map (Choice 1, the default d' = d): phi_l = exp(w_l.x + b_l). */
static void phi_exp(int d, const double *x, const double *W, const double *b, double *out) {
    for (int l = 0; l < d; l++) {
        double u = b ? b[l] : 0.0;
        for (int m = 0; m < d; m++) u += W[(size_t)l * d + m] * x[m];
        out[l] = exp(u);
    }
}

/* Softmax over the d feature directions (Choice 4, no bias): out_l = exp(s u_l) / sum_i exp(s u_i)
 * with u = W x and sign s = +1 or -1.  Evaluated with the largest s u_i subtracted first (the
 * same value). */
static void softmax_dirs(int d, const double *x, const double *W, double sgn, double *out) {
    double mx = -INFINITY;
    for (int l = 0; l < d; l++) {
        double u = 0.0;
        for (int m = 0; m < d; m++) u += W[(size_t)l * d + m] * x[m];
        out[l] = sgn * u;
        if (out[l] > mx) mx = out[l];
    }
    double sum = 0.0;
    for (int l = 0; l < d; l++) {
        out[l] = exp(out[l] - mx);
        sum += out[l];
    }
    for (int l = 0; l < d; l++) out[l] /= sum;
}

static void phi_one(int map, int d, const double *x, const double *W, const double *b, double *out) {
    switch (map) {
    case HHO_HEDGEHOG: phi_hedgehog(d, x, W, b, out); break;
    case HHO_TAYLOR2: phi_taylor(d, x, out); break;
    case HHO_QUADRATIC: phi_quadratic(d, x, W, out); break;
    case HHO_EXP: phi_exp(d, x, W, b, out); break;
    case HHO_SOFTMAX: softmax_dirs(d, x, W, 1.0, out); break;
    case HHO_HEDGEHOG_SOFTMAX:
        /* Choice 4 with the negation mapping of Choice 3: one softmax over the d projections,
         * one over their negations (each half sums to 1) */
        softmax_dirs(d, x, W, 1.0, out);
        softmax_dirs(d, x, W, -1.0, out + d);
        break;
    }
}

/* Feature map of ntok tokens of one head: x [ntok][d] -> phi [ntok][d']. */
void hho_featuremap_head(int map, int d, long ntok, const double *x, const double *W, const double *b,
                         double *phi) {
    int dp = hho_feature_dim(map, d);
    for (long t = 0; t < ntok; t++) phi_one(map, d, x + t * d, W, b, phi + t * dp);
}

/* Chain rule through one feature map: given x, the map's parameters and dL/dphi, add dL/dx to
 * dx and (maps with parameters) dL/dW, dL/db to dW [d][d], db [d].
 *   Hedgehog: u = W x + b, phi = [e^u, e^-u]: dL/du_l = dphi_l e^u_l - dphi_{d+l} e^-u_l.
 *   exp (single-sided): dL/du_l = dphi_l e^u_l.
 *   softmax over directions p = softmax(s u), u = W x: dL/du = s p (dphi - <dphi, p>); the
 *   two-sided softmax map adds its s = +1 and s = -1 halves.
 *   Taylor: phi = [1, x_m, x_a x_c / sqrt 2]: dL/dx_m = dphi_{1+m} + sum_c (dphi_{mc} + dphi_{cm}) x_c / sqrt 2.
 * Then dx = W^T du, dW += du x^T, db += du. */
static void phi_backward(int map, int d, const double *x, const double *W, const double *b, const double *dphi,
                         double *dx, double *dW, double *db) {
    if (map == HHO_QUADRATIC) {  /* phi = [sqrt a, sqrt b x_m, sqrt c x_a x_c]; only dx (no W) */
        const double sb = sqrt(W[1]), sc = sqrt(W[2]);
        for (int m = 0; m < d; m++) {
            double g = sb * dphi[1 + m];
            for (int c = 0; c < d; c++)
                g += (dphi[1 + d + (size_t)m * d + c] + dphi[1 + d + (size_t)c * d + m]) * x[c] * sc;
            dx[m] += g;
        }
        return;
    }
    if (map == HHO_TAYLOR2) {
        const double r = 1.0 / sqrt(2.0);
        for (int m = 0; m < d; m++) {
            double g = dphi[1 + m];
            for (int c = 0; c < d; c++)
                g += (dphi[1 + d + (size_t)m * d + c] + dphi[1 + d + (size_t)c * d + m]) * x[c] * r;
            dx[m] += g;
        }
        return;
    }
    double *u = malloc(sizeof(double) * d), *du = malloc(sizeof(double) * d), *p = malloc(sizeof(double) * d);
    const int with_b = map == HHO_HEDGEHOG || map == HHO_EXP;
    for (int l = 0; l < d; l++) {
        double a = (with_b && b) ? b[l] : 0.0;
        for (int m = 0; m < d; m++) a += W[(size_t)l * d + m] * x[m];
        u[l] = a;
        du[l] = 0.0;
    }
    if (map == HHO_HEDGEHOG) {
        for (int l = 0; l < d; l++) du[l] = dphi[l] * exp(u[l]) - dphi[d + l] * exp(-u[l]);
    } else if (map == HHO_EXP) {
        for (int l = 0; l < d; l++) du[l] = dphi[l] * exp(u[l]);
    } else {
        const int halves = map == HHO_HEDGEHOG_SOFTMAX ? 2 : 1;
        for (int hf = 0; hf < halves; hf++) {
            const double sgn = hf == 0 ? 1.0 : -1.0;
            softmax_dirs(d, x, W, sgn, p);
            const double *dp_ = dphi + (size_t)hf * d;
            double dot = 0.0;
            for (int l = 0; l < d; l++) dot += dp_[l] * p[l];
            for (int l = 0; l < d; l++) du[l] += sgn * p[l] * (dp_[l] - dot);
        }
    }
    for (int m = 0; m < d; m++) {
        double g = 0.0;
        for (int l = 0; l < d; l++) g += W[(size_t)l * d + m] * du[l];
        dx[m] += g;
    }
    for (int l = 0; l < d; l++) {
        for (int m = 0; m < d; m++) dW[(size_t)l * d + m] += du[l] * x[m];
        if (with_b) db[l] += du[l];
    }
    free(u); free(du); free(p);
}

/* ---- one (batch, head) sequence ------------------------------------------ */

/* Causal attention by running sums (Eq. 2 in its recurrent form).
 * S [d'][d], z [d'] start at S0/z0 (or zero) and end as the inclusive sums.
 * For each token i: f = phi(k_i); S += f v_i^T; z += f; g = phi(q_i);
 * y_i = (g^T S) / (g^T z). */
static void causal_one(int map, int d, long N, const double *q, const double *k, const double *v,
                       const double *W, const double *b, const double *S0, const double *z0,
                       double *y, double *S_out, double *z_out) {
    int dp = hho_feature_dim(map, d);
    double *S = calloc((size_t)dp * d, sizeof(double));
    double *z = calloc((size_t)dp, sizeof(double));
    double *f = malloc(sizeof(double) * dp);
    double *g = malloc(sizeof(double) * dp);
    double *num = malloc(sizeof(double) * d);
    if (S0) memcpy(S, S0, sizeof(double) * dp * d);
    if (z0) memcpy(z, z0, sizeof(double) * dp);
    for (long i = 0; i < N; i++) {
        phi_one(map, d, k + i * d, W, b, f);
        const double *vi = v + i * d;
        for (int a = 0; a < dp; a++) {
            double *Sa = S + (size_t)a * d;
            for (int c = 0; c < d; c++) Sa[c] += f[a] * vi[c];
            z[a] += f[a];
        }
        phi_one(map, d, q + i * d, W, b, g);
        double den = 0.0;
        for (int c = 0; c < d; c++) num[c] = 0.0;
        for (int a = 0; a < dp; a++) {
            const double *Sa = S + (size_t)a * d;
            for (int c = 0; c < d; c++) num[c] += g[a] * Sa[c];
            den += g[a] * z[a];
        }
        for (int c = 0; c < d; c++) y[i * d + c] = num[c] / den;
    }
    if (S_out) memcpy(S_out, S, sizeof(double) * dp * d);
    if (z_out) memcpy(z_out, z, sizeof(double) * dp);
    free(S); free(z); free(f); free(g); free(num);
}

/* Causal attention by running sums from given features: the same recurrence as causal_one
 * with f = phik[i] and g = phiq[i] ([N][d'] each) instead of the feature map. */
static void causal_feat_one(int d, int dp, long N, const double *phiq, const double *phik, const double *v,
                            const double *S0, const double *z0, double *y, double *S_out, double *z_out) {
    double *S = calloc((size_t)dp * d, sizeof(double));
    double *z = calloc((size_t)dp, sizeof(double));
    double *num = malloc(sizeof(double) * d);
    if (S0) memcpy(S, S0, sizeof(double) * dp * d);
    if (z0) memcpy(z, z0, sizeof(double) * dp);
    for (long i = 0; i < N; i++) {
        const double *f = phik + (size_t)i * dp, *g = phiq + (size_t)i * dp, *vi = v + i * d;
        for (int a = 0; a < dp; a++) {
            double *Sa = S + (size_t)a * d;
            for (int c = 0; c < d; c++) Sa[c] += f[a] * vi[c];
            z[a] += f[a];
        }
        double den = 0.0;
        for (int c = 0; c < d; c++) num[c] = 0.0;
        for (int a = 0; a < dp; a++) {
            const double *Sa = S + (size_t)a * d;
            for (int c = 0; c < d; c++) num[c] += g[a] * Sa[c];
            den += g[a] * z[a];
        }
        for (int c = 0; c < d; c++) y[i * d + c] = num[c] / den;
    }
    if (S_out) memcpy(S_out, S, sizeof(double) * dp * d);
    if (z_out) memcpy(z_out, z, sizeof(double) * dp);
    free(S); free(z); free(num);
}

/* Bidirectional attention: S and z summed over every key, then each query reads them. */
static void bidir_one(int map, int d, long N, const double *q, const double *k, const double *v,
                      const double *W, const double *b, double *y) {
    int dp = hho_feature_dim(map, d);
    double *S = calloc((size_t)dp * d, sizeof(double));
    double *z = calloc((size_t)dp, sizeof(double));
    double *f = malloc(sizeof(double) * dp);
    double *num = malloc(sizeof(double) * d);
    for (long j = 0; j < N; j++) {
        phi_one(map, d, k + j * d, W, b, f);
        for (int a = 0; a < dp; a++) {
            for (int c = 0; c < d; c++) S[(size_t)a * d + c] += f[a] * v[j * d + c];
            z[a] += f[a];
        }
    }
    for (long i = 0; i < N; i++) {
        phi_one(map, d, q + i * d, W, b, f);
        double den = 0.0;
        for (int c = 0; c < d; c++) num[c] = 0.0;
        for (int a = 0; a < dp; a++) {
            for (int c = 0; c < d; c++) num[c] += f[a] * S[(size_t)a * d + c];
            den += f[a] * z[a];
        }
        for (int c = 0; c < d; c++) y[i * d + c] = num[c] / den;
    }
    free(S); free(z); free(f); free(num);
}

/* Explicit quadratic form, no running sums: a_ij = phi(q_i)^T phi(k_j) for the
 * keys a query sees (j <= i when causal, all j otherwise); y_i = sum_j a_ij v_j /
 * sum_j a_ij.  Rows listed in `rows` only (all rows when rows == NULL). */
static void quadratic_rows_one(int map, int d, long N, int causal, const double *q, const double *k,
                               const double *v, const double *W, const double *b, long nrows,
                               const long *rows, double *y) {
    int dp = hho_feature_dim(map, d);
    double *g = malloc(sizeof(double) * dp);
    double *f = malloc(sizeof(double) * dp);
    double *num = malloc(sizeof(double) * d);
    long count = rows ? nrows : N;
    for (long r = 0; r < count; r++) {
        long i = rows ? rows[r] : r;
        phi_one(map, d, q + i * d, W, b, g);
        long jend = causal ? i + 1 : N;
        double den = 0.0;
        for (int c = 0; c < d; c++) num[c] = 0.0;
        for (long j = 0; j < jend; j++) {
            phi_one(map, d, k + j * d, W, b, f);
            double a = 0.0;
            for (int t = 0; t < dp; t++) a += g[t] * f[t];
            for (int c = 0; c < d; c++) num[c] += a * v[j * d + c];
            den += a;
        }
        for (int c = 0; c < d; c++) y[r * d + c] = num[c] / den;
    }
    free(g); free(f); free(num);
}

/* Gradients of L = sum_i dy_i . y_i through Eq. 2, from its explicit form: with
 * a_ij = phi(q_i).phi(k_j) over the keys query i sees (j <= i, or all j), den_i = sum_j a_ij and
 * y_i = sum_j a_ij v_j / den_i, the chain rule gives
 *   dL/da_ij = dy_i . (v_j - y_i) / den_i,
 *   dL/dphi(q_i) = sum_j dL/da_ij phi(k_j),   dL/dphi(k_j) = sum_i dL/da_ij phi(q_i),
 *   dL/dv_j = sum_i (a_ij / den_i) dy_i,
 * then phi_backward takes dL/dphi to dL/dq, dL/dk and the parameters.  dq, dk, dv [N][d] are
 * written; dW [d][d] and db [d] are accumulated (they sum over every token and both q and k). */
static void backward_one(int map, int d, long N, int causal, const double *q, const double *k, const double *v,
                         const double *W, const double *b, const double *dy, double *dq, double *dk, double *dv,
                         double *dW, double *db) {
    const int dp = hho_feature_dim(map, d);
    double *fq = malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * dp);
    double *fk = malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * dp);
    double *dfq = calloc((size_t)(N > 0 ? N : 1) * dp, sizeof(double));
    double *dfk = calloc((size_t)(N > 0 ? N : 1) * dp, sizeof(double));
    double *a = malloc(sizeof(double) * (N > 0 ? N : 1));
    double *y = malloc(sizeof(double) * d);
    for (long t = 0; t < N; t++) {
        phi_one(map, d, q + t * d, W, b, fq + (size_t)t * dp);
        phi_one(map, d, k + t * d, W, b, fk + (size_t)t * dp);
    }
    memset(dv, 0, sizeof(double) * N * d);
    for (long i = 0; i < N; i++) {
        const long jend = causal ? i + 1 : N;
        double den = 0.0;
        for (int c = 0; c < d; c++) y[c] = 0.0;
        for (long j = 0; j < jend; j++) {
            double s = 0.0;
            for (int t = 0; t < dp; t++) s += fq[(size_t)i * dp + t] * fk[(size_t)j * dp + t];
            a[j] = s;
            den += s;
            for (int c = 0; c < d; c++) y[c] += s * v[j * d + c];
        }
        for (int c = 0; c < d; c++) y[c] /= den;
        for (long j = 0; j < jend; j++) {
            double tij = 0.0;
            for (int c = 0; c < d; c++) tij += dy[i * d + c] * (v[j * d + c] - y[c]);
            tij /= den;
            for (int t = 0; t < dp; t++) {
                dfq[(size_t)i * dp + t] += tij * fk[(size_t)j * dp + t];
                dfk[(size_t)j * dp + t] += tij * fq[(size_t)i * dp + t];
            }
            for (int c = 0; c < d; c++) dv[j * d + c] += a[j] / den * dy[i * d + c];
        }
    }
    memset(dq, 0, sizeof(double) * N * d);
    memset(dk, 0, sizeof(double) * N * d);
    for (long t = 0; t < N; t++) {
        phi_backward(map, d, q + t * d, W, b, dfq + (size_t)t * dp, dq + t * d, dW, db);
        phi_backward(map, d, k + t * d, W, b, dfk + (size_t)t * dp, dk + t * d, dW, db);
    }
    free(fq); free(fk); free(dfq); free(dfk); free(a); free(y);
}

/* Distillation loss of the listed query rows (all rows when rows == NULL), directly from Eq. 4:
 * p_ij = exp(q_i.k_j / sqrt(d)) / sum_{m<=i} exp(q_i.k_m / sqrt(d)),
 * a_ij = phi(q_i).phi(k_j),
 * L_i = -sum_{j<=i} p_ij log(a_ij / sum_{m<=i} a_im).
 * The softmax is evaluated with its maximum logit subtracted (the same weights). */
static void distill_rows_one(int map, int d, long N, const double *q, const double *k, const double *W,
                             const double *b, long nrows, const long *rows, double *loss) {
    int dp = hho_feature_dim(map, d);
    double *g = malloc(sizeof(double) * dp);
    double *f = malloc(sizeof(double) * dp);
    double *logit = malloc(sizeof(double) * (N > 0 ? N : 1));
    double *a = malloc(sizeof(double) * (N > 0 ? N : 1));
    const double scale = 1.0 / sqrt((double)d);
    long count = rows ? nrows : N;
    for (long r = 0; r < count; r++) {
        long i = rows ? rows[r] : r;
        phi_one(map, d, q + i * d, W, b, g);
        double mx = -INFINITY, asum = 0.0;
        for (long j = 0; j <= i; j++) {
            double s = 0.0;
            for (int c = 0; c < d; c++) s += q[i * d + c] * k[j * d + c];
            logit[j] = s * scale;
            if (logit[j] > mx) mx = logit[j];
            phi_one(map, d, k + j * d, W, b, f);
            double aij = 0.0;
            for (int t = 0; t < dp; t++) aij += g[t] * f[t];
            a[j] = aij;
            asum += aij;
        }
        double psum = 0.0;
        for (long j = 0; j <= i; j++) psum += exp(logit[j] - mx);
        double L = 0.0;
        for (long j = 0; j <= i; j++) L -= (exp(logit[j] - mx) / psum) * log(a[j] / asum);
        loss[r] = L;
    }
    free(g); free(f); free(logit); free(a);
}

/* One decode step from (S, z), in place: S += phi(k) v^T; z += phi(k); y = phi(q)^T S / phi(q)^T z. */
static void decode_one(int map, int d, const double *q, const double *k, const double *v,
                       const double *W, const double *b, double *S, double *z, double *y) {
    int dp = hho_feature_dim(map, d);
    double *f = malloc(sizeof(double) * dp);
    phi_one(map, d, k, W, b, f);
    for (int a = 0; a < dp; a++) {
        for (int c = 0; c < d; c++) S[(size_t)a * d + c] += f[a] * v[c];
        z[a] += f[a];
    }
    phi_one(map, d, q, W, b, f);
    double den = 0.0;
    for (int c = 0; c < d; c++) y[c] = 0.0;
    for (int a = 0; a < dp; a++) {
        for (int c = 0; c < d; c++) y[c] += f[a] * S[(size_t)a * d + c];
        den += f[a] * z[a];
    }
    for (int c = 0; c < d; c++) y[c] /= den;
    free(f);
}

/* ---- batched entry points: B*H independent sequences, threads over them ---- */

typedef struct {
    int op;        /* 0 causal, 1 bidirectional, 2 decode, 3 quadratic rows, 4 featuremap, 5 distillation loss,
                      6 causal from given features, 7 backward */
    int map, d, dp, H, causal;
    long BH, N;
    const double *q, *k, *v, *W, *b, *S0, *z0, *dy;
    double *y, *S_out, *z_out, *dq, *dk, *dv, *dW, *db;
    long nrows;
    const long *rows;
    long next;     /* shared work counter */
    pthread_mutex_t mu;
} job_t;

static void run_pair(job_t *j, long p) {
    int d = j->d;
    int dp = hho_feature_dim(j->map, d);
    long h = p % j->H;
    const int has_W = j->map != HHO_TAYLOR2;
    const int has_b = j->map == HHO_HEDGEHOG || j->map == HHO_EXP;
    /* the quadratic map's parameters are its three coefficients per head */
    const double *W = !has_W ? NULL : j->map == HHO_QUADRATIC ? j->W + (size_t)h * 3 : j->W + (size_t)h * d * d;
    const double *b = (has_b && j->b) ? j->b + (size_t)h * d : NULL;
    size_t seq = (size_t)j->N * d;
    switch (j->op) {
    case 0:
        causal_one(j->map, d, j->N, j->q + p * seq, j->k + p * seq, j->v + p * seq, W, b,
                   j->S0 ? j->S0 + (size_t)p * dp * d : NULL, j->z0 ? j->z0 + (size_t)p * dp : NULL,
                   j->y + p * seq, j->S_out ? j->S_out + (size_t)p * dp * d : NULL,
                   j->z_out ? j->z_out + (size_t)p * dp : NULL);
        break;
    case 1:
        bidir_one(j->map, d, j->N, j->q + p * seq, j->k + p * seq, j->v + p * seq, W, b, j->y + p * seq);
        break;
    case 2:
        decode_one(j->map, d, j->q + (size_t)p * d, j->k + (size_t)p * d, j->v + (size_t)p * d, W, b,
                   j->S_out + (size_t)p * dp * d, j->z_out + (size_t)p * dp, j->y + (size_t)p * d);
        break;
    case 3:
        quadratic_rows_one(j->map, d, j->N, j->causal, j->q + p * seq, j->k + p * seq, j->v + p * seq,
                           W, b, j->nrows, j->rows, j->y + (size_t)p * (j->rows ? j->nrows : j->N) * d);
        break;
    case 4:
        hho_featuremap_head(j->map, d, j->N, j->q + p * seq, W, b, j->y + (size_t)p * j->N * dp);
        break;
    case 6:
        causal_feat_one(d, j->dp, j->N, j->q + p * j->N * j->dp, j->k + p * j->N * j->dp, j->v + p * seq,
                        j->S0 ? j->S0 + (size_t)p * j->dp * d : NULL, j->z0 ? j->z0 + (size_t)p * j->dp : NULL,
                        j->y + p * seq, j->S_out ? j->S_out + (size_t)p * j->dp * d : NULL,
                        j->z_out ? j->z_out + (size_t)p * j->dp : NULL);
        break;
    case 7:  /* per-pair parameter gradients: dW [BH][d][d], db [BH][d] (summed by the caller) */
        backward_one(j->map, d, j->N, j->causal, j->q + p * seq, j->k + p * seq, j->v + p * seq, W, b,
                     j->dy + p * seq, j->dq + p * seq, j->dk + p * seq, j->dv + p * seq,
                     j->dW + (size_t)p * d * d, j->db + (size_t)p * d);
        break;
    case 5:
        distill_rows_one(j->map, d, j->N, j->q + p * seq, j->k + p * seq, W, b, j->nrows, j->rows,
                         j->y + (size_t)p * (j->rows ? j->nrows : j->N));
        break;
    }
}

static void *worker(void *arg) {
    job_t *j = (job_t *)arg;
    for (;;) {
        pthread_mutex_lock(&j->mu);
        long p = j->next++;
        pthread_mutex_unlock(&j->mu);
        if (p >= j->BH) break;
        run_pair(j, p);
    }
    return NULL;
}

static void run_job(job_t *j, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > j->BH) nthreads = (int)j->BH;
    j->next = 0;
    pthread_mutex_init(&j->mu, NULL);
    if (nthreads <= 1) {
        worker(j);
    } else {
        pthread_t th[256];
        for (int t = 0; t < nthreads; t++) pthread_create(&th[t], NULL, worker, j);
        for (int t = 0; t < nthreads; t++) pthread_join(th[t], NULL);
    }
    pthread_mutex_destroy(&j->mu);
}

/* q,k,v,y: [B*H][N][d]; W: [H][d][d]; b: [H][d] or NULL; S0/S_out: [B*H][d'][d] or NULL;
 * z0/z_out: [B*H][d'] or NULL. */
void hho_causal(int map, int d, long B, long H, long N, const double *q, const double *k,
                const double *v, const double *W, const double *b, const double *S0, const double *z0,
                double *y, double *S_out, double *z_out, int nthreads) {
    job_t j;
    memset(&j, 0, sizeof j);
    j.op = 0; j.map = map; j.d = d; j.H = (int)H; j.BH = B * H; j.N = N;
    j.q = q; j.k = k; j.v = v; j.W = W; j.b = b; j.S0 = S0; j.z0 = z0;
    j.y = y; j.S_out = S_out; j.z_out = z_out;
    run_job(&j, nthreads);
}

void hho_bidir(int map, int d, long B, long H, long N, const double *q, const double *k,
               const double *v, const double *W, const double *b, double *y, int nthreads) {
    job_t j;
    memset(&j, 0, sizeof j);
    j.op = 1; j.map = map; j.d = d; j.H = (int)H; j.BH = B * H; j.N = N;
    j.q = q; j.k = k; j.v = v; j.W = W; j.b = b; j.y = y;
    run_job(&j, nthreads);
}

/* q,k,v,y: [B*H][d]; S: [B*H][d'][d] and z: [B*H][d'] updated in place. */
void hho_decode_step(int map, int d, long B, long H, const double *q, const double *k,
                     const double *v, const double *W, const double *b, double *S, double *z,
                     double *y, int nthreads) {
    job_t j;
    memset(&j, 0, sizeof j);
    j.op = 2; j.map = map; j.d = d; j.H = (int)H; j.BH = B * H; j.N = 1;
    j.q = q; j.k = k; j.v = v; j.W = W; j.b = b; j.S_out = S; j.z_out = z; j.y = y;
    run_job(&j, nthreads);
}

/* Quadratic form for selected rows (rows == NULL: all rows); y: [B*H][nrows or N][d]. */
void hho_quadratic(int map, int d, long B, long H, long N, int causal, const double *q,
                   const double *k, const double *v, const double *W, const double *b, long nrows,
                   const long *rows, double *y, int nthreads) {
    job_t j;
    memset(&j, 0, sizeof j);
    j.op = 3; j.map = map; j.d = d; j.H = (int)H; j.BH = B * H; j.N = N; j.causal = causal;
    j.q = q; j.k = k; j.v = v; j.W = W; j.b = b; j.y = y; j.nrows = nrows; j.rows = rows;
    run_job(&j, nthreads);
}

/* Feature map of x [B*H][N][d] -> phi [B*H][N][d']. */
void hho_featuremap(int map, int d, long B, long H, long N, const double *x, const double *W,
                    const double *b, double *phi, int nthreads) {
    job_t j;
    memset(&j, 0, sizeof j);
    j.op = 4; j.map = map; j.d = d; j.H = (int)H; j.BH = B * H; j.N = N;
    j.q = x; j.W = W; j.b = b; j.y = phi;
    run_job(&j, nthreads);
}

/* Distillation loss (Eq. 4) of q, k [B*H][N][d] -> loss [B*H][nrows or N] for the listed query rows
 * (rows == NULL: all rows). */
void hho_distill(int map, int d, long B, long H, long N, const double *q, const double *k, const double *W,
                 const double *b, long nrows, const long *rows, double *loss, int nthreads) {
    job_t j;
    memset(&j, 0, sizeof j);
    j.op = 5; j.map = map; j.d = d; j.H = (int)H; j.BH = B * H; j.N = N;
    j.q = q; j.k = k; j.W = W; j.b = b; j.y = loss; j.nrows = nrows; j.rows = rows;
    run_job(&j, nthreads);
}

/* Causal Eq. 2 from given features: phiq, phik [B*H][N][dp], v, y [B*H][N][d]; optional
 * S0/S_out [B*H][dp][d], z0/z_out [B*H][dp]. */
void hho_causal_features(int d, int dp, long BH, long N, const double *phiq, const double *phik, const double *v,
                         const double *S0, const double *z0, double *y, double *S_out, double *z_out,
                         int nthreads) {
    job_t j;
    memset(&j, 0, sizeof j);
    j.op = 6; j.d = d; j.dp = dp; j.H = 1; j.BH = BH; j.N = N;
    j.q = phiq; j.k = phik; j.v = v; j.S0 = S0; j.z0 = z0;
    j.y = y; j.S_out = S_out; j.z_out = z_out;
    run_job(&j, nthreads);
}

/* Backward of the forward (causal or bidirectional): q, k, v, dy, dq, dk, dv [B*H][N][d];
 * dW [B*H][d][d] and db [B*H][d] receive each sequence's parameter gradient (zeroed here). */
void hho_backward(int map, int d, long B, long H, long N, int causal, const double *q, const double *k,
                  const double *v, const double *W, const double *b, const double *dy, double *dq, double *dk,
                  double *dv, double *dW, double *db, int nthreads) {
    job_t j;
    memset(&j, 0, sizeof j);
    memset(dW, 0, sizeof(double) * B * H * d * d);
    memset(db, 0, sizeof(double) * B * H * d);
    j.op = 7; j.map = map; j.d = d; j.H = (int)H; j.BH = B * H; j.N = N; j.causal = causal;
    j.q = q; j.k = k; j.v = v; j.W = W; j.b = b; j.dy = dy;
    j.dq = dq; j.dk = dk; j.dv = dv; j.dW = dW; j.db = db;
    run_job(&j, nthreads);
}
