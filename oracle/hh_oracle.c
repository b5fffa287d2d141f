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

int hho_feature_dim(int map, int d) {
    if (map == HHO_HEDGEHOG) return 2 * d;
    if (map == HHO_TAYLOR2) return 1 + d + d * d;
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

static void phi_one(int map, int d, const double *x, const double *W, const double *b, double *out) {
    if (map == HHO_HEDGEHOG) phi_hedgehog(d, x, W, b, out);
    else phi_taylor(d, x, out);
}

/* Feature map of ntok tokens of one head: x [ntok][d] -> phi [ntok][d']. */
void hho_featuremap_head(int map, int d, long ntok, const double *x, const double *W, const double *b,
                         double *phi) {
    int dp = hho_feature_dim(map, d);
    for (long t = 0; t < ntok; t++) phi_one(map, d, x + t * d, W, b, phi + t * dp);
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
    int op;        /* 0 causal, 1 bidirectional, 2 decode, 3 quadratic rows, 4 featuremap, 5 distillation loss */
    int map, d, H, causal;
    long BH, N;
    const double *q, *k, *v, *W, *b, *S0, *z0;
    double *y, *S_out, *z_out;
    long nrows;
    const long *rows;
    long next;     /* shared work counter */
    pthread_mutex_t mu;
} job_t;

static void run_pair(job_t *j, long p) {
    int d = j->d;
    int dp = hho_feature_dim(j->map, d);
    long h = p % j->H;
    const double *W = j->map == HHO_HEDGEHOG ? j->W + (size_t)h * d * d : NULL;
    const double *b = (j->map == HHO_HEDGEHOG && j->b) ? j->b + (size_t)h * d : NULL;
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
