/*
 * fp64 CPU oracle for the fast-weight delta-rule layer with DPFP projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls this
 * file; only the tests, the package's smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or helper with the HIP kernels.
 *
 * Sources (web pages; cited by page title and section):
 *   [FWT]  "Fast Weights Transformer" technical guide for the labml annotated implementation,
 *          xdnf.cn/news/308600.
 *            - section "DPFP / projection formula and hyper-parameters": the map itself,
 *              d_dot = 2 * d_key * nu, the cyclic wrap, and the code that realises the wrap
 *              as a roll of relu([k, -k]) by +i;
 *            - section "DPFP / normalisation": phi <- phi / (sum_j phi_j + eps), eps = 1e-6;
 *            - section "FastWeightsAttention / update formula": v_bar = W phi(k),
 *              beta = sigmoid(.), W += beta (v - v_bar) (x) phi(k), y = W phi(q);
 *            - section "FastWeightsAttention / module structure and source walkthrough":
 *              W starts at zero with shape [batch, heads, d_value, d_key(=d_dot)], and each
 *              time step does retrieve, then write, then read (the read uses the new W).
 *
 * Readings taken where the pages are garbled or silent (each is listed in the design notes):
 *   - the wrap direction is the one the code uses: block i (i = 1..nu) at offset
 *     (i-1)*2*d_k holds x[j] * x[(j - i) mod 2*d_k], x = relu([k, -k]);
 *   - eps is added to the sum (not a max), and is not a parameter;
 *   - beta_logit is the pre-sigmoid value; beta = 1/(1+exp(-l)) evaluated stably;
 *   - layout is [B, H, T, d] row-major; W is [B, H, d_v, D] with D = 2*d_k*nu.
 *
 * Everything is plain fp64 with no blocking, fusion or reordering beyond the definition.
 * The only parallelism is OpenMP over independent vectors / (batch, head) slices.
 * Pins that tie this file to the pages live in tests/test_oracle_pins.py; none of the
 * functions below is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DPFP_EPS 1e-6

/* Number of OpenMP threads a parallel region of this library uses (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* sigmoid(l) = 1 / (1 + exp(-l)), written so that neither branch overflows:
 * for l < 0 use exp(l) / (1 + exp(l)).  sigmoid(-inf) = 0, sigmoid(+inf) = 1.
 * [FWT] section "FastWeightsAttention / update formula" (beta = sigma(W_beta x)). */
double oracle_sigmoid(double l)
{
    if (l >= 0.0) return 1.0 / (1.0 + exp(-l));
    double e = exp(l);
    return e / (1.0 + e);
}

/* DPFP of one vector k[0..d_k) into phi[0..2*d_k*nu).
 * [FWT] section "DPFP / projection formula and hyper-parameters" and "DPFP / normalisation".
 * x = relu([k, -k]) (length 2*d_k); for shift i = 1..nu the block at offset (i-1)*2*d_k is
 * x multiplied elementwise by x rolled by +i, i.e. x[j] * x[(j - i) mod 2*d_k];
 * then every entry is divided by (sum of all entries + eps). */
static void dpfp_one(const double* k, double* phi, int d_k, int nu, double* x)
{
    const int two_dk = 2 * d_k;
    for (int j = 0; j < d_k; ++j) {
        x[j] = k[j] > 0.0 ? k[j] : 0.0;
        x[d_k + j] = -k[j] > 0.0 ? -k[j] : 0.0;
    }
    double sum = 0.0;
    for (int i = 1; i <= nu; ++i) {
        for (int j = 0; j < two_dk; ++j) {
            int src = ((j - i) % two_dk + two_dk) % two_dk;
            double p = x[j] * x[src];
            phi[(i - 1) * two_dk + j] = p;
            sum += p;
        }
    }
    const int D = two_dk * nu;
    for (int d = 0; d < D; ++d) phi[d] = phi[d] / (sum + ORACLE_DPFP_EPS);
}

/* phi[n, :] = DPFP(x[n, :]) for n in [0, n_vec). x is [n_vec, d_k], phi is [n_vec, 2*d_k*nu]. */
void oracle_dpfp(const double* x, double* phi, int64_t n_vec, int d_k, int nu)
{
    const int64_t D = 2 * (int64_t)d_k * nu;
#pragma omp parallel
    {
        double* work = (double*)malloc(sizeof(double) * 2 * (size_t)d_k);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < n_vec; ++n) dpfp_one(x + n * d_k, phi + n * D, d_k, nu, work);
        free(work);
    }
}

/* The zero/nonzero pattern of DPFP by sign alone: entry (i, j) is nonzero exactly when both
 * factors x[j] and x[(j - i) mod 2*d_k] are strictly positive.  mask is [n_vec, D] bytes. */
void oracle_dpfp_mask(const double* x, uint8_t* mask, int64_t n_vec, int d_k, int nu)
{
    const int two_dk = 2 * d_k;
    const int64_t D = (int64_t)two_dk * nu;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_vec; ++n) {
        const double* k = x + n * d_k;
        for (int i = 1; i <= nu; ++i) {
            for (int j = 0; j < two_dk; ++j) {
                int src = ((j - i) % two_dk + two_dk) % two_dk;
                int pos_j = j < d_k ? (k[j] > 0.0) : (k[j - d_k] < 0.0);
                int pos_s = src < d_k ? (k[src] > 0.0) : (k[src - d_k] < 0.0);
                mask[n * D + (int64_t)(i - 1) * two_dk + j] = (uint8_t)(pos_j && pos_s);
            }
        }
    }
}

/* One time step of the delta rule on one (batch, head) slice, in the order of
 * [FWT] section "FastWeightsAttention / module structure and source walkthrough":
 *   retrieve  v_bar = W phi_k
 *   write     W <- W + beta * (v - v_bar) (outer) phi_k
 *   read      y = W phi_q          (with the W just written)
 * W is [d_v, D] row-major.  vbar is scratch of length d_v. */
static void delta_step_one(double* W, const double* phi_k, const double* phi_q, const double* v,
                           double beta, double* y, double* vbar, int d_v, int D)
{
    for (int r = 0; r < d_v; ++r) {
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += W[(size_t)r * D + d] * phi_k[d];
        vbar[r] = s;
    }
    for (int r = 0; r < d_v; ++r) {
        double c = beta * (v[r] - vbar[r]);
        for (int d = 0; d < D; ++d) W[(size_t)r * D + d] += c * phi_k[d];
    }
    for (int r = 0; r < d_v; ++r) {
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += W[(size_t)r * D + d] * phi_q[d];
        y[r] = s;
    }
}

/* Full causal forward over T steps for every (b, h) slice.
 *   q, k        [B, H, T, d_k]
 *   v, y        [B, H, T, d_v]
 *   beta_logit  [B, H, T]
 *   W0, W_final [B, H, d_v, D]; W0 == NULL means W starts at zero (the page's default);
 *               W_final may be NULL (not written) and may equal W0.
 * Each slice runs the literal per-time-step recurrence of delta_step_one. */
void oracle_delta_forward(const double* q, const double* k, const double* v,
                          const double* beta_logit, const double* W0, double* y,
                          double* W_final, int B, int H, int T, int d_k, int d_v, int nu)
{
    const int D = 2 * d_k * nu;
    const int64_t BH = (int64_t)B * H;
#pragma omp parallel
    {
        double* W = (double*)malloc(sizeof(double) * (size_t)d_v * D);
        double* pk = (double*)malloc(sizeof(double) * (size_t)D);
        double* pq = (double*)malloc(sizeof(double) * (size_t)D);
        double* vbar = (double*)malloc(sizeof(double) * (size_t)d_v);
        double* work = (double*)malloc(sizeof(double) * 2 * (size_t)d_k);
#pragma omp for schedule(dynamic, 1)
        for (int64_t s = 0; s < BH; ++s) {
            if (W0) memcpy(W, W0 + s * d_v * D, sizeof(double) * (size_t)d_v * D);
            else memset(W, 0, sizeof(double) * (size_t)d_v * D);
            for (int t = 0; t < T; ++t) {
                const int64_t row = s * T + t;
                dpfp_one(k + row * d_k, pk, d_k, nu, work);
                dpfp_one(q + row * d_k, pq, d_k, nu, work);
                double beta = oracle_sigmoid(beta_logit[row]);
                delta_step_one(W, pk, pq, v + row * d_v, beta, y + row * d_v, vbar, d_v, D);
            }
            if (W_final) memcpy(W_final + s * d_v * D, W, sizeof(double) * (size_t)d_v * D);
        }
        free(W); free(pk); free(pq); free(vbar); free(work);
    }
}

/* One decode step for every (b, h): the single-token case of the forward, with the state
 * carried in and out through W (updated in place).  This is the token-by-token mode of
 * [FWT] sections "token_wise variant" and "Inference and sampling".
 *   q, k [B, H, d_k]; v, y [B, H, d_v]; beta_logit [B, H]; W [B, H, d_v, D]. */
void oracle_delta_step(const double* q, const double* k, const double* v,
                       const double* beta_logit, double* W, double* y,
                       int B, int H, int d_k, int d_v, int nu)
{
    const int D = 2 * d_k * nu;
    const int64_t BH = (int64_t)B * H;
#pragma omp parallel
    {
        double* pk = (double*)malloc(sizeof(double) * (size_t)D);
        double* pq = (double*)malloc(sizeof(double) * (size_t)D);
        double* vbar = (double*)malloc(sizeof(double) * (size_t)d_v);
        double* work = (double*)malloc(sizeof(double) * 2 * (size_t)d_k);
#pragma omp for schedule(static)
        for (int64_t s = 0; s < BH; ++s) {
            dpfp_one(k + s * d_k, pk, d_k, nu, work);
            dpfp_one(q + s * d_k, pq, d_k, nu, work);
            double beta = oracle_sigmoid(beta_logit[s]);
            delta_step_one(W + s * d_v * D, pk, pq, v + s * d_v, beta, y + s * d_v, vbar, d_v, D);
        }
        free(pk); free(pq); free(vbar); free(work);
    }
}
