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

/* ------------------------------------------------------------------------------------------
 * Gradient of the forward.  The pages train this layer ([FWT] section "Training experiment":
 * a cross-entropy loss, gradient-norm clipping), which needs the derivatives of the forward
 * above with respect to every input.  This is that derivative written out: reverse-mode
 * differentiation of the literal per-step recurrence, one step at a time from t = T-1 down
 * to 0.  With f = phi(k_t), g = phi(q_t), beta = sigmoid(l_t), P the memory before step t
 * and N = P + u f^T (u = beta (v - P f)) the memory after it, and G the gradient of the loss
 * with respect to N (the running gradient, which starts as dW_final):
 *   y_t = N g          G += dy_t g^T;   dg = N^T dy_t
 *   N = P + u f^T      du = G f;        df = G^T u
 *   u = beta (v - vb)  dv_t = beta du;  dbeta = du . (v - vb);  dvb = -beta du
 *   vb = P f           G <- G + dvb f^T (now the gradient for P);  df += P^T dvb
 *   beta = sigmoid(l)  dl_t = dbeta * beta * (1 - beta)
 * and the DPFP derivative takes df, dg back to dk_t, dq_t (dpfp_vjp_one).  dW0 is the final G.
 * The memories P, N are recomputed from copies kept every ORACLE_CHECKPOINT steps: the
 * recomputation repeats the forward's operations in the same order, so every value equals the
 * forward's own.
 * ------------------------------------------------------------------------------------------ */
#define ORACLE_CHECKPOINT 64

/* Derivative of DPFP: given k (length d_k) and dphi (length D), adds nothing and writes
 * dk = (d phi / d k)^T dphi.  phi = raw / (S + eps) with S = sum(raw), so
 * draw_m = (dphi_m - sum_j dphi_j phi_j) / (S + eps); raw[(i-1)*2d_k + j] = x[j] x[(j-i) mod 2d_k]
 * sends draw * x[src] to x[j] and draw * x[j] to x[src]; x = relu([k, -k]) passes dx[j] to
 * k_j where k_j > 0 and -dx[d_k + j] where k_j < 0 (zero where k_j = 0). */
static void dpfp_vjp_one(const double* k, const double* dphi, double* dk, int d_k, int nu,
                         double* x, double* raw, double* dx)
{
    const int two_dk = 2 * d_k;
    const int D = two_dk * nu;
    for (int j = 0; j < d_k; ++j) {
        x[j] = k[j] > 0.0 ? k[j] : 0.0;
        x[d_k + j] = k[j] < 0.0 ? -k[j] : 0.0;
    }
    double S = 0.0;
    for (int i = 1; i <= nu; ++i)
        for (int j = 0; j < two_dk; ++j) {
            int src = ((j - i) % two_dk + two_dk) % two_dk;
            raw[(i - 1) * two_dk + j] = x[j] * x[src];
            S += raw[(i - 1) * two_dk + j];
        }
    const double den = S + ORACLE_DPFP_EPS;
    double dot = 0.0;  /* sum_j dphi_j phi_j */
    for (int d = 0; d < D; ++d) dot += dphi[d] * (raw[d] / den);
    for (int m = 0; m < two_dk; ++m) dx[m] = 0.0;
    for (int i = 1; i <= nu; ++i)
        for (int j = 0; j < two_dk; ++j) {
            int src = ((j - i) % two_dk + two_dk) % two_dk;
            double draw = (dphi[(i - 1) * two_dk + j] - dot) / den;
            dx[j] += draw * x[src];
            dx[src] += draw * x[j];
        }
    for (int j = 0; j < d_k; ++j) {
        double g = 0.0;
        if (k[j] > 0.0) g += dx[j];
        if (k[j] < 0.0) g -= dx[d_k + j];
        dk[j] = g;
    }
}

/* Gradients of L = <dy, y> + <dW_final, W_final> through oracle_delta_forward.
 *   q, k, v, beta_logit, W0   the forward's inputs (W0 may be NULL: zeros)
 *   dy        [B, H, T, d_v]  gradient with respect to y
 *   dW_final  [B, H, d_v, D]  gradient with respect to W_final, or NULL (zeros)
 *   dq, dk    [B, H, T, d_k]; dv [B, H, T, d_v]; dbeta_logit [B, H, T]  outputs
 *   dW0       [B, H, d_v, D]  output (gradient with respect to W0), or NULL to skip it */
void oracle_delta_backward(const double* q, const double* k, const double* v,
                           const double* beta_logit, const double* W0, const double* dy,
                           const double* dW_final, double* dq, double* dk, double* dv,
                           double* dbeta_logit, double* dW0, int B, int H, int T, int d_k,
                           int d_v, int nu)
{
    const int D = 2 * d_k * nu;
    const int64_t BH = (int64_t)B * H;
    const size_t WS = (size_t)d_v * D;
    const int nck = (T + ORACLE_CHECKPOINT - 1) / ORACLE_CHECKPOINT;
#pragma omp parallel
    {
        double* ck = (double*)malloc(sizeof(double) * WS * (size_t)(nck > 0 ? nck : 1));
        double* seg = (double*)malloc(sizeof(double) * WS * (ORACLE_CHECKPOINT + 1));
        double* G = (double*)malloc(sizeof(double) * WS);
        double* pk = (double*)malloc(sizeof(double) * (size_t)D);
        double* pq = (double*)malloc(sizeof(double) * (size_t)D);
        double* df = (double*)malloc(sizeof(double) * (size_t)D);
        double* dg = (double*)malloc(sizeof(double) * (size_t)D);
        double* raw = (double*)malloc(sizeof(double) * (size_t)D);
        double* vbar = (double*)malloc(sizeof(double) * (size_t)d_v);
        double* u = (double*)malloc(sizeof(double) * (size_t)d_v);
        double* du = (double*)malloc(sizeof(double) * (size_t)d_v);
        double* ytmp = (double*)malloc(sizeof(double) * (size_t)d_v);
        double* work = (double*)malloc(sizeof(double) * 2 * (size_t)d_k);
        double* dxw = (double*)malloc(sizeof(double) * 2 * (size_t)d_k);
#pragma omp for schedule(dynamic, 1)
        for (int64_t s = 0; s < BH; ++s) {
            /* forward once, keeping the memory at the start of every segment */
            double* W = seg;
            if (W0) memcpy(W, W0 + s * WS, sizeof(double) * WS);
            else memset(W, 0, sizeof(double) * WS);
            for (int t = 0; t < T; ++t) {
                if (t % ORACLE_CHECKPOINT == 0)
                    memcpy(ck + (size_t)(t / ORACLE_CHECKPOINT) * WS, W, sizeof(double) * WS);
                const int64_t row = s * T + t;
                dpfp_one(&k[row * d_k], pk, d_k, nu, work);
                dpfp_one(&q[row * d_k], pq, d_k, nu, work);
                delta_step_one(W, pk, pq, v + row * d_v, oracle_sigmoid(beta_logit[row]), ytmp,
                               vbar, d_v, D);
            }
            if (dW_final) memcpy(G, dW_final + s * WS, sizeof(double) * WS);
            else memset(G, 0, sizeof(double) * WS);
            for (int c = nck - 1; c >= 0; --c) {
                const int t0 = c * ORACLE_CHECKPOINT;
                const int t1 = t0 + ORACLE_CHECKPOINT < T ? t0 + ORACLE_CHECKPOINT : T;
                /* seg[i] = memory after step t0 + i - 1 (seg[0] = memory before step t0) */
                memcpy(seg, ck + (size_t)c * WS, sizeof(double) * WS);
                for (int t = t0; t < t1; ++t) {
                    const int64_t row = s * T + t;
                    double* Wn = seg + (size_t)(t - t0 + 1) * WS;
                    memcpy(Wn, seg + (size_t)(t - t0) * WS, sizeof(double) * WS);
                    dpfp_one(&k[row * d_k], pk, d_k, nu, work);
                    dpfp_one(&q[row * d_k], pq, d_k, nu, work);
                    delta_step_one(Wn, pk, pq, v + row * d_v, oracle_sigmoid(beta_logit[row]),
                                   ytmp, vbar, d_v, D);
                }
                for (int t = t1 - 1; t >= t0; --t) {
                    const int64_t row = s * T + t;
                    const double* P = seg + (size_t)(t - t0) * WS;
                    const double* N = seg + (size_t)(t - t0 + 1) * WS;
                    const double* vt = v + row * d_v;
                    const double* dyt = dy + row * d_v;
                    dpfp_one(&k[row * d_k], pk, d_k, nu, work);
                    dpfp_one(&q[row * d_k], pq, d_k, nu, work);
                    const double beta = oracle_sigmoid(beta_logit[s * T + t]);
                    for (int r = 0; r < d_v; ++r) {
                        double sacc = 0.0;
                        for (int d = 0; d < D; ++d) sacc += P[(size_t)r * D + d] * pk[d];
                        vbar[r] = sacc;
                        u[r] = beta * (vt[r] - vbar[r]);
                    }
                    /* y_t = N g */
                    for (int d = 0; d < D; ++d) {
                        double sacc = 0.0;
                        for (int r = 0; r < d_v; ++r) sacc += N[(size_t)r * D + d] * dyt[r];
                        dg[d] = sacc;
                    }
                    for (int r = 0; r < d_v; ++r)
                        for (int d = 0; d < D; ++d) G[(size_t)r * D + d] += dyt[r] * pq[d];
                    /* N = P + u f^T */
                    for (int r = 0; r < d_v; ++r) {
                        double sacc = 0.0;
                        for (int d = 0; d < D; ++d) sacc += G[(size_t)r * D + d] * pk[d];
                        du[r] = sacc;
                    }
                    for (int d = 0; d < D; ++d) {
                        double sacc = 0.0;
                        for (int r = 0; r < d_v; ++r) sacc += G[(size_t)r * D + d] * u[r];
                        df[d] = sacc;
                    }
                    /* u = beta (v - vb) */
                    double dbeta = 0.0;
                    for (int r = 0; r < d_v; ++r) {
                        dv[row * d_v + r] = beta * du[r];
                        dbeta += du[r] * (vt[r] - vbar[r]);
                    }
                    /* vb = P f: G becomes the gradient for P */
                    for (int r = 0; r < d_v; ++r) {
                        const double dvb = -beta * du[r];
                        for (int d = 0; d < D; ++d) G[(size_t)r * D + d] += dvb * pk[d];
                    }
                    for (int d = 0; d < D; ++d) {
                        double sacc = 0.0;
                        for (int r = 0; r < d_v; ++r) sacc += P[(size_t)r * D + d] * (-beta * du[r]);
                        df[d] += sacc;
                    }
                    dbeta_logit[row] = dbeta * beta * (1.0 - beta);
                    dpfp_vjp_one(k + row * d_k, df, dk + row * d_k, d_k, nu, work, raw, dxw);
                    dpfp_vjp_one(q + row * d_k, dg, dq + row * d_k, d_k, nu, work, raw, dxw);
                }
            }
            if (dW0) memcpy(dW0 + s * WS, G, sizeof(double) * WS);
        }
        free(ck); free(seg); free(G); free(pk); free(pq); free(df); free(dg); free(raw);
        free(vbar); free(u); free(du); free(ytmp); free(work); free(dxw);
    }
}

/* ------------------------------------------------------------------------------------------
 * Sum-update linear attention with the z normaliser: [FWT] section "Background / fast
 * computation form of linear self-attention".  Replacing the softmax kernel by
 * phi(k)^T phi(q) turns causal attention into the recurrence
 *   W_t = W_{t-1} + v_t phi(k_t)^T,   z_t = z_{t-1} + phi(k_t),   y_t = W_t phi(q_t) / (z_t . phi(q_t))
 * with phi = DPFP.  Readings: W_0, z_0 are given or zero; where the denominator z_t . phi(q_t)
 * is exactly 0 (phi(q_t) = 0, or no earlier key shares a feature with q_t) y_t is 0.
 *   q, k [B, H, T, d_k]; v, y [B, H, T, d_v]; W0, W_final [B, H, d_v, D]; z0, z_final [B, H, D]
 *   (W0, z0 may be NULL; W_final, z_final may be NULL: not written).
 * ------------------------------------------------------------------------------------------ */
void oracle_sum_forward(const double* q, const double* k, const double* v, const double* W0,
                        const double* z0, double* y, double* W_final, double* z_final, int B,
                        int H, int T, int d_k, int d_v, int nu)
{
    const int D = 2 * d_k * nu;
    const int64_t BH = (int64_t)B * H;
#pragma omp parallel
    {
        double* W = (double*)malloc(sizeof(double) * (size_t)d_v * D);
        double* z = (double*)malloc(sizeof(double) * (size_t)D);
        double* pk = (double*)malloc(sizeof(double) * (size_t)D);
        double* pq = (double*)malloc(sizeof(double) * (size_t)D);
        double* work = (double*)malloc(sizeof(double) * 2 * (size_t)d_k);
#pragma omp for schedule(dynamic, 1)
        for (int64_t s = 0; s < BH; ++s) {
            if (W0) memcpy(W, W0 + (size_t)s * d_v * D, sizeof(double) * (size_t)d_v * D);
            else memset(W, 0, sizeof(double) * (size_t)d_v * D);
            if (z0) memcpy(z, z0 + s * D, sizeof(double) * (size_t)D);
            else memset(z, 0, sizeof(double) * (size_t)D);
            for (int t = 0; t < T; ++t) {
                const int64_t row = s * T + t;
                dpfp_one(k + (size_t)row * d_k, pk, d_k, nu, work);
                dpfp_one(q + (size_t)row * d_k, pq, d_k, nu, work);
                const double* vt = v + row * d_v;
                /* write */
                for (int r = 0; r < d_v; ++r)
                    for (int d = 0; d < D; ++d) W[(size_t)r * D + d] += vt[r] * pk[d];
                for (int d = 0; d < D; ++d) z[d] += pk[d];
                /* read, normalised */
                double den = 0.0;
                for (int d = 0; d < D; ++d) den += z[d] * pq[d];
                for (int r = 0; r < d_v; ++r) {
                    double num = 0.0;
                    for (int d = 0; d < D; ++d) num += W[(size_t)r * D + d] * pq[d];
                    y[row * d_v + r] = den != 0.0 ? num / den : 0.0;
                }
            }
            if (W_final) memcpy(W_final + s * d_v * D, W, sizeof(double) * (size_t)d_v * D);
            if (z_final) memcpy(z_final + s * D, z, sizeof(double) * (size_t)D);
        }
        free(W); free(z); free(pk); free(pq); free(work);
    }
}

/* ------------------------------------------------------------------------------------------
 * The projections around the layer: [FWT] section "FastWeightsAttention / module structure
 * and source walkthrough".  The query, key and value maps are bias-free linear maps from
 * d_model to heads * d (then split by head), the interpolation weight is a bias-free linear map
 * to one scalar per head (squashed by the sigmoid inside the layer), and the output is a linear
 * map (with bias) of the heads' concatenated outputs back to d_model; the Transformer layer
 * adds it to its input (the attention residual).
 *   x     [B, T, d_model]
 *   Wqkvb [3 rows blocks + 1]: rows 0 .. H*d_k - 1 query, H*d_k .. 2*H*d_k - 1 key,
 *         then H*d_v value rows, then H beta rows; each row has d_model entries (out = x W^T)
 *   q, k  [B, H, T, d_k]; v [B, H, T, d_v]; beta_logit [B, H, T]
 * ------------------------------------------------------------------------------------------ */
void oracle_layer_project(const double* x, const double* Wqkvb, double* q, double* k, double* v,
                          double* beta_logit, int B, int T, int d_model, int H, int d_k, int d_v)
{
    const int nq = H * d_k, nv = H * d_v;
    const int N = 2 * nq + nv + H;
#pragma omp parallel for schedule(static)
    for (int64_t bt = 0; bt < (int64_t)B * T; ++bt) {
        const int64_t b = bt / T, t = bt % T;
        const double* xr = x + bt * d_model;
        for (int n = 0; n < N; ++n) {
            double s = 0.0;
            for (int c = 0; c < d_model; ++c) s += xr[c] * Wqkvb[(int64_t)n * d_model + c];
            if (n < nq) {
                q[((b * H + n / d_k) * T + t) * d_k + n % d_k] = s;
            } else if (n < 2 * nq) {
                const int m = n - nq;
                k[((b * H + m / d_k) * T + t) * d_k + m % d_k] = s;
            } else if (n < 2 * nq + nv) {
                const int m = n - 2 * nq;
                v[((b * H + m / d_v) * T + t) * d_v + m % d_v] = s;
            } else {
                const int h = n - 2 * nq - nv;
                beta_logit[(b * H + h) * T + t] = s;
            }
        }
    }
}

/* out[b, t, :] = residual[b, t, :] + bo + Wo concat_h(y[b, h, t, :]) with Wo [d_model, H*d_v]
 * (bo, residual may be NULL: zero). */
void oracle_layer_output(const double* y, const double* Wo, const double* bo,
                         const double* residual, double* out, int B, int T, int H, int d_v,
                         int d_model)
{
    const int Kc = H * d_v;
#pragma omp parallel for schedule(static)
    for (int64_t bt = 0; bt < (int64_t)B * T; ++bt) {
        const int64_t b = bt / T, t = bt % T;
        for (int n = 0; n < d_model; ++n) {
            double s = 0.0;
            for (int kk = 0; kk < Kc; ++kk)
                s += y[((b * H + kk / d_v) * T + t) * d_v + kk % d_v] * Wo[(int64_t)n * Kc + kk];
            if (bo) s += bo[n];
            if (residual) s += residual[bt * d_model + n];
            out[bt * d_model + n] = s;
        }
    }
}
