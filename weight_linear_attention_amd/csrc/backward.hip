// Gradient of the chunked forward: dq, dk, dv, dbeta_logit and dW0 from dy and dW_final.
//
// The layer is trained ("Fast Weights Transformer" guide, xdnf.cn/news/308600, section
// "Training experiment"), so its forward -- the delta rule of section "FastWeightsAttention /
// update formula" over the DPFP features of section "DPFP" -- needs its derivatives.  They are
// taken through the chunk form of the recurrence.  For a chunk of C rows starting from memory
// W0 (d_v x D) with normalised features K, Q (C x D), beta (C):
//   G = K K^T,  P = lower_incl(Q K^T),  A = I + diag(beta) strict_lower(G),  T = A^-1 diag(beta)
//   U = T (V - K W0^T),  Y = Q W0^T + P U,  W1 = W0 + U^T K.
// With Wy = T K and Uy = T V this is U = Uy - Wy W0^T.  Given dY and dW1 (the gradient of the
// chunk-end memory), with Ainv = A^-1:
//   dU = P^T dY + K dW1^T;  lam = Ainv^T dU;  dV = diag(beta) lam
//   dW0 = dW1 + dY^T Q' - dW1 K^T Wy,  Q' = Q - P Wy           (the reverse chain)
//   dP = lower_incl(dY U^T);  Z = lam U^T;  dG_ij = -beta_i Z_ij (j < i)
//   dQ = dY W0 + dP K
//   dK = U dW1 - diag(beta) lam W0 + dP^T Q + (dG + dG^T) K
//   dbeta_i = lam_i.V_i - (lam W0)_i.K_i - sum_{j<i} G_ij Z_ij,   dlogit = dbeta beta (1 - beta)
// and the derivative of DPFP takes dK, dQ to dk, dq.
//
// Both chains are row-separable: row r of the memory (and of its gradient) moves with its own
// column of V (of dY) alone, so the serial passes run one wave per row.  Five launches:
//   1. bwd_prep         per chunk: K, Q, G, P, Ainv, Wy, Q', Uy, beta           (parallel)
//   2. bwd_fwd_states   per (b, h, 8 rows): chunk-start memories and U          (serial)
//   3. bwd_grad_states  per (b, h, 8 rows): chunk-end gradients, K dW1^T, dW0   (serial)
//   4. bwd_chunk_grads  per chunk: dK, dQ (over 2, 3), dv, dbeta_logit           (parallel)
//   5. bwd_dpfp         per vector: dk, dq                                      (parallel)
// Arithmetic is fp32 on the vector ALU; chunk C = 32.
#include "chunk_f32.h"
#include "fwa_internal.h"

namespace fwa {

constexpr int kPrepThreads2 = 256;
constexpr int kCS = kBC + 4; // row stride of the C x C tiles (16-byte rows, few bank clashes)

// Workspace regions (fp32), each indexed by the chunk u = bh * NC + n.
struct BwdLayout {
    int64_t kt, qt, wy, qp, ai, pm, gm, be, uy, uu, aa, ws, gs, end;
};

__host__ __device__ inline BwdLayout bwd_layout(int64_t NU, int D, int d_v) {
    BwdLayout L;
    int64_t o = 0;
    const int64_t CD = int64_t(kBC) * D, CC = int64_t(kBC) * kBC, CV = int64_t(kBC) * d_v;
    const int64_t VD = int64_t(d_v) * D;
    L.kt = o; o += NU * CD;
    L.qt = o; o += NU * CD;
    L.wy = o; o += NU * CD;      // Wy, then dK (bwd_chunk_grads)
    L.qp = o; o += NU * CD;      // Q', then dQ
    L.ai = o; o += NU * CC;
    L.pm = o; o += NU * CC;
    L.gm = o; o += NU * CC;
    L.be = o; o += NU * kBC;
    L.uy = o; o += NU * CV;      // [c][r]
    L.uu = o; o += NU * CV;      // [r][c]
    L.aa = o; o += NU * CV;      // [r][c]
    L.ws = o; o += NU * VD;      // chunk-start memory [r][d]
    L.gs = o; o += NU * VD;      // chunk-end memory gradient [r][d]
    L.end = o;
    return L;
}

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* bl;
    const float* W0;
    const void* dy;
    const float* dWf;
    void* dq;
    void* dk;
    void* dv;
    void* dbl;
    float* dW0;
    float* ws;
    int BH, T, NC, d_k, d_v, nu, D;
    BwdLayout L;
};

// ------------------------------------------------------------------------------ 1. prep

// LDS: x rows of k and q (relu([., -.]), C x 2 d_k each; T = Ainv diag(beta) over them once
// they are dead), K and Q (C x SD, SD = D + 8; W_y over K once it is dead), G, P, Ainv
// (C x kCS), beta, V (C x d_v).  The products G = K K^T, P = Q K^T, W_y = T K, P W_y and
// U_y = T V run on the fp32 MFMA (16x16x4; lane group g supplies k = 4 g + s to sub-step s
// for both operands: A as one 16-byte read of a row, B as four reads down a column).
template <bool BF16>
__global__ __launch_bounds__(kPrepThreads2) void bwd_prep_kernel(BwdArgs a) {
    extern __shared__ float lds[];
    const int D = a.D, d_k = a.d_k, d_v = a.d_v, two = 2 * d_k;
    const int u = blockIdx.x;
    const int bh = u / a.NC, n = u % a.NC;
    const int t0 = n * kBC;
    const int tid = threadIdx.x;
    const int wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    constexpr int CS = kCS;
    const int SD = tile_stride(D);
    float* xk = lds;                         // [C][2 d_k]
    float* xq = xk + kBC * two;
    float* Ts = xk;                          // [C][CS] T = Ainv diag(beta), after DPFP
    float* Kt = xq + kBC * two;              // [C][SD]; W_y once K is dead
    float* Qt = Kt + kBC * SD;
    float* Gm = Qt + kBC * SD;               // [C][CS]
    float* Pm = Gm + kBC * CS;
    float* Ai = Pm + kBC * CS;
    float* be = Ai + kBC * CS;               // [C]
    float* Vs = be + kBC;                    // [C][d_v]

    // relu'd raw rows (zero past the sequence end), beta (zero past the end), v
    load_relu_rows<BF16>(a.k, xk, int64_t(bh) * a.T, a.T - t0 < kBC ? a.T - t0 : kBC, t0, d_k,
                         tid, kPrepThreads2);
    load_relu_rows<BF16>(a.q, xq, int64_t(bh) * a.T, a.T - t0 < kBC ? a.T - t0 : kBC, t0, d_k,
                         tid, kPrepThreads2);
    for (int c = tid; c < kBC; c += kPrepThreads2)
        be[c] = t0 + c < a.T ? sigmoid_stable(load_elem<BF16>(a.bl, int64_t(bh) * a.T + t0 + c)) : 0.0f;
    for (int c = wv; c < kBC; c += kPrepThreads2 / 64)
        for (int r = lane; r < d_v; r += 64)
            Vs[c * d_v + r] = t0 + c < a.T ? load_elem<BF16>(a.v, (int64_t(bh) * a.T + t0 + c) * d_v + r) : 0.0f;
    dpfp_tiles(xk, xq, Kt, Qt, D, d_k, tid);
    const int64_t CD = int64_t(kBC) * D;
    float* gK = a.ws + a.L.kt + int64_t(u) * CD;
    float* gQ = a.ws + a.L.qt + int64_t(u) * CD;
    for (int c = wv; c < kBC; c += kPrepThreads2 / 64)
        for (int p = lane; p < D; p += 64) {
            gK[c * D + p] = Kt[c * SD + p];
            gQ[c * D + p] = Qt[c * SD + p];
        }
    // G = K K^T (all four tiles) and P = lower_incl(Q K^T) (tiles (0,0), (1,0), (1,1));
    // wave w takes tiles w and w + 4 of that list
    for (int tau = wv; tau < 7; tau += 4) {
        const bool isP = tau >= 4;
        const int it = isP ? (tau == 4 ? 0 : 1) : tau >> 1;
        const int jt = isP ? (tau == 6 ? 1 : 0) : tau & 1;
        const float* X = isP ? Qt : Kt;
        f32x4 acc = zero4();
        for (int kb = 0; kb < D; kb += 16) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(X + (16 * it + l16) * SD + kb + 4 * g4);
            const f32x4 bv = *reinterpret_cast<const f32x4*>(Kt + (16 * jt + l16) * SD + kb + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma_f32_k4(av[s], bv[s], acc);
        }
        const int col = 16 * jt + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * it + 4 * g4 + e;
            if (isP) Pm[row * CS + col] = col <= row ? acc[e] : 0.0f;
            else Gm[row * CS + col] = acc[e];
        }
    }
    for (int e = tid; e < 16 * 16; e += kPrepThreads2)         // P tile (0, 1): above the diagonal
        Pm[(e >> 4) * CS + 16 + (e & 15)] = 0.0f;
    __syncthreads();
    // Ainv = (I + diag(beta) strict_lower(G))^-1 by forward substitution, one column per thread
    if (tid < kBC) {
        const int j = tid;
        float x[kBC];
#pragma unroll
        for (int i = 0; i < kBC; ++i) x[i] = 0.0f;
#pragma unroll
        for (int i = 0; i < kBC; ++i) {
            if (i == j) x[i] = 1.0f;
            if (i > j) {
                float s = 0.0f;
#pragma unroll
                for (int m = 0; m < i; ++m) s += Gm[i * CS + m] * x[m];
                x[i] = -be[i] * s;
            }
        }
#pragma unroll
        for (int i = 0; i < kBC; ++i) Ai[i * CS + j] = x[i];
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kPrepThreads2) {       // T = Ainv diag(beta)
        const int i = e >> 5, j = e & (kBC - 1);
        Ts[i * CS + j] = Ai[i * CS + j] * be[j];
    }
    __syncthreads();
    // W_y = T K: tiles (it, pt) w + 4 q, accumulators kept until every wave has read K
    const int NPT = D / 16;
    constexpr int kMaxWy = 384 / 16 * 2 / 4;                     // tiles per wave at D <= 384
    f32x4 wy[kMaxWy];
    float* gWy = a.ws + a.L.wy + int64_t(u) * CD;
#pragma unroll
    for (int q = 0; q < kMaxWy; ++q) {
        const int tau = wv + 4 * q;
        wy[q] = zero4();
        if (tau >= 2 * NPT) continue;
        const int it = tau & 1, pt = tau >> 1;
#pragma unroll
        for (int kb = 0; kb < kBC; kb += 16) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(Ts + (16 * it + l16) * CS + kb + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                wy[q] = mfma_f32_k4(av[s], Kt[(kb + 4 * g4 + s) * SD + 16 * pt + l16], wy[q]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) gWy[int64_t(16 * it + 4 * g4 + e) * D + 16 * pt + l16] = wy[q][e];
    }
    __syncthreads();                                             // K is dead: W_y over it
#pragma unroll
    for (int q = 0; q < kMaxWy; ++q) {
        const int tau = wv + 4 * q;
        if (tau >= 2 * NPT) continue;
        const int it = tau & 1, pt = tau >> 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) Kt[(16 * it + 4 * g4 + e) * SD + 16 * pt + l16] = wy[q][e];
    }
    __syncthreads();
    // Q' = Q - P W_y
    float* gQp = a.ws + a.L.qp + int64_t(u) * CD;
    for (int tau = wv; tau < 2 * NPT; tau += 4) {
        const int it = tau & 1, pt = tau >> 1;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < kBC; kb += 16) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(Pm + (16 * it + l16) * CS + kb + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = mfma_f32_k4(av[s], Kt[(kb + 4 * g4 + s) * SD + 16 * pt + l16], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * it + 4 * g4 + e, col = 16 * pt + l16;
            gQp[int64_t(row) * D + col] = Qt[row * SD + col] - acc[e];
        }
    }
    // Uy = T V ([c][r])
    float* gUy = a.ws + a.L.uy + int64_t(u) * kBC * d_v;
    for (int tau = wv; tau < 2 * ((d_v + 15) / 16); tau += 4) {
        const int it = tau & 1, rt = tau >> 1;
        const int r = 16 * rt + l16;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < kBC; kb += 16) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(Ts + (16 * it + l16) * CS + kb + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = mfma_f32_k4(av[s], r < d_v ? Vs[(kb + 4 * g4 + s) * d_v + r] : 0.0f, acc);
        }
        if (r < d_v) {
#pragma unroll
            for (int e = 0; e < 4; ++e) gUy[(16 * it + 4 * g4 + e) * d_v + r] = acc[e];
        }
    }
    // Ainv, P, G, beta
    float* gAi = a.ws + a.L.ai + int64_t(u) * kBC * kBC;
    float* gPm = a.ws + a.L.pm + int64_t(u) * kBC * kBC;
    float* gGm = a.ws + a.L.gm + int64_t(u) * kBC * kBC;
    for (int e = tid; e < kBC * kBC; e += kPrepThreads2) {
        const int i = e >> 5, j = e & (kBC - 1);
        gAi[e] = Ai[i * CS + j];
        gPm[e] = Pm[i * CS + j];
        gGm[e] = Gm[i * CS + j];
    }
    if (tid < kBC) a.ws[a.L.be + int64_t(u) * kBC + tid] = be[tid];
}

// ------------------------------------------------------------------------------ row chains

// Chunk-start memories and U: row r of the memory moves as w <- w + K^T u with
// u = Uy[:, r] - Wy w.  Lane l holds w[l + 64 m], m < NPL.  The next chunk's Wy and K tiles load
// into registers while the current chunk computes.
template <int NPL>
__global__ __launch_bounds__(64 * kRowWaves) void bwd_fwd_states_kernel(BwdArgs a) {
    extern __shared__ float lds[];
    const int D = a.D, d_v = a.d_v;
    const int rgroups = (d_v + kRowWaves - 1) / kRowWaves;
    const int bh = blockIdx.x / rgroups;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = (blockIdx.x % rgroups) * kRowWaves + wave;
    const bool live = r < d_v;
    constexpr int SDP = 64 * NPL;     // padded LDS row stride of the staged tiles
    float* Wy = lds;                  // [C][SDP]
    float* Kt = Wy + kBC * SDP;       // [C][SDP]
    int slot[NPL];
    tile_slots<NPL>(slot, D, tid);
    zero_tile_pads<NPL>(Wy, D, tid);
    zero_tile_pads<NPL>(Kt, D, tid);
    float w[NPL];
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
        const int p = lane + 64 * m;
        w[m] = (live && a.W0 && p < D) ? a.W0[(int64_t(bh) * d_v + r) * D + p] : 0.0f;
    }
    const int64_t CD = int64_t(kBC) * D;
    const int n_tile = kBC * D;
    f32x4 rwy[NPL], rk[NPL];
    float uy_next = 0.0f;
#define FWA_BWD_FWD_FETCH(nn)                                                                   \
    do {                                                                                       \
        const int64_t uf = int64_t(bh) * a.NC + (nn);                                          \
        prefetch_tile<NPL>(rwy, a.ws + a.L.wy + uf * CD, n_tile, tid);                         \
        prefetch_tile<NPL>(rk, a.ws + a.L.kt + uf * CD, n_tile, tid);                          \
        uy_next = live ? a.ws[a.L.uy + uf * kBC * d_v + (lane >> 1) * d_v + r] : 0.0f;        \
    } while (0)
    if (a.NC > 0) FWA_BWD_FWD_FETCH(0);
    for (int n = 0; n < a.NC; ++n) {
        const int64_t u = int64_t(bh) * a.NC + n;
        if (live) {
            float* gw = a.ws + a.L.ws + (u * d_v + r) * D;
#pragma unroll
            for (int m = 0; m < NPL; ++m)
                if (lane + 64 * m < D) gw[lane + 64 * m] = w[m];
        }
        lds_barrier();
        commit_tile<NPL>(Wy, rwy, slot);
        commit_tile<NPL>(Kt, rk, slot);
        const float uy = uy_next;
        lds_barrier();
        if (n + 1 < a.NC) FWA_BWD_FWD_FETCH(n + 1);
        float part[kBC];
#pragma unroll
        for (int c = 0; c < kBC; ++c) {
            float sacc = 0.0f;
#pragma unroll
            for (int m = 0; m < NPL; ++m) sacc += Wy[c * SDP + lane + 64 * m] * w[m];
            part[c] = sacc;
        }
        const float x = wave_reduce_scatter32(part);          // (Wy w)[lane >> 1]
        const float uc = uy - x;
        if (live && (lane & 1) == 0) a.ws[a.L.uu + (u * d_v + r) * kBC + (lane >> 1)] = uc;
#pragma unroll
        for (int c = 0; c < kBC; ++c) {
            const float uv = lane_value(uc, 2 * c);
#pragma unroll
            for (int m = 0; m < NPL; ++m) w[m] += uv * Kt[c * SDP + lane + 64 * m];
        }
    }
#undef FWA_BWD_FWD_FETCH
}

// Chunk-end gradients of the memory, K dW1^T and dW0, chunks in reverse: row r of the
// gradient moves as g <- g + Q'^T dY[:, r] - Wy^T (K g).  The previous chunk's tiles load into
// registers while the current chunk computes.
template <bool BF16, int NPL>
__global__ __launch_bounds__(64 * kRowWaves) void bwd_grad_states_kernel(BwdArgs a) {
    extern __shared__ float lds[];
    const int D = a.D, d_v = a.d_v;
    const int rgroups = (d_v + kRowWaves - 1) / kRowWaves;
    const int bh = blockIdx.x / rgroups;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = (blockIdx.x % rgroups) * kRowWaves + wave;
    const bool live = r < d_v;
    constexpr int SDP = 64 * NPL;     // padded LDS row stride of the staged tiles
    float* Kt = lds;                  // [C][SDP]
    float* Qp = Kt + kBC * SDP;
    float* Wy = Qp + kBC * SDP;
    int slot[NPL];
    tile_slots<NPL>(slot, D, tid);
    zero_tile_pads<NPL>(Kt, D, tid);
    zero_tile_pads<NPL>(Qp, D, tid);
    zero_tile_pads<NPL>(Wy, D, tid);
    float g[NPL];
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
        const int p = lane + 64 * m;
        g[m] = (live && a.dWf && p < D) ? a.dWf[(int64_t(bh) * d_v + r) * D + p] : 0.0f;
    }
    const int64_t CD = int64_t(kBC) * D;
    const int n_tile = kBC * D;
    f32x4 rk[NPL], rq[NPL], rwy[NPL];
    float dy_next = 0.0f;
    // dY[c, r] of the fetched chunk in lane c (zero past the end)
#define FWA_BWD_GRAD_FETCH(nn)                                                                  \
    do {                                                                                       \
        const int64_t uf = int64_t(bh) * a.NC + (nn);                                          \
        prefetch_tile<NPL>(rk, a.ws + a.L.kt + uf * CD, n_tile, tid);                          \
        prefetch_tile<NPL>(rq, a.ws + a.L.qp + uf * CD, n_tile, tid);                          \
        prefetch_tile<NPL>(rwy, a.ws + a.L.wy + uf * CD, n_tile, tid);                         \
        const int tf = (nn) * kBC + lane;                                                      \
        dy_next = (live && lane < kBC && tf < a.T)                                            \
                      ? load_elem<BF16>(a.dy, (int64_t(bh) * a.T + tf) * d_v + r) : 0.0f;     \
    } while (0)
    if (a.NC > 0) FWA_BWD_GRAD_FETCH(a.NC - 1);
    for (int n = a.NC - 1; n >= 0; --n) {
        const int64_t u = int64_t(bh) * a.NC + n;
        if (live) {
            float* gg = a.ws + a.L.gs + (u * d_v + r) * D;
#pragma unroll
            for (int m = 0; m < NPL; ++m)
                if (lane + 64 * m < D) gg[lane + 64 * m] = g[m];
        }
        lds_barrier();
        commit_tile<NPL>(Kt, rk, slot);
        commit_tile<NPL>(Qp, rq, slot);
        commit_tile<NPL>(Wy, rwy, slot);
        const float dyc = dy_next;
        lds_barrier();
        if (n > 0) FWA_BWD_GRAD_FETCH(n - 1);
        float part[kBC];
#pragma unroll
        for (int c = 0; c < kBC; ++c) {
            float sacc = 0.0f;
#pragma unroll
            for (int m = 0; m < NPL; ++m) sacc += Kt[c * SDP + lane + 64 * m] * g[m];
            part[c] = sacc;
        }
        const float ac = wave_reduce_scatter32(part);         // (K g)[lane >> 1]
        if (live && (lane & 1) == 0) a.ws[a.L.aa + (u * d_v + r) * kBC + (lane >> 1)] = ac;
        // partly unrolled: a full unroll hoists all 2 * 32 * NPL tile reads and spills at NPL >= 4
#pragma unroll 4
        for (int c = 0; c < kBC; ++c) {
            const float dy = lane_value(dyc, c), av = lane_value(ac, 2 * c);
#pragma unroll
            for (int m = 0; m < NPL; ++m)
                g[m] += dy * Qp[c * SDP + lane + 64 * m] - av * Wy[c * SDP + lane + 64 * m];
        }
    }
    if (live && a.dW0) {
#pragma unroll
        for (int m = 0; m < NPL; ++m)
            if (lane + 64 * m < D) a.dW0[(int64_t(bh) * d_v + r) * D + lane + 64 * m] = g[m];
    }
#undef FWA_BWD_GRAD_FETCH
}

// ------------------------------------------------------------------------------ 4. chunk grads

constexpr int kSlice = 64;   // columns of D per pass in bwd_chunk_grads

// Padded d_v: the d_v contraction runs in 16-deep blocks; the row stride adds 4 floats.
__host__ __device__ inline int grads_dv16(int d_v) { return (d_v + 15) & ~15; }
__host__ __device__ inline int grads_dvp(int d_v) { return grads_dv16(d_v) + 4; }

// One chunk per workgroup of 4 waves, every contraction on the fp32 MFMA (16x16x4; a 16-deep k
// block feeds four products, lane group g supplying k = 4 g + s to sub-step s for both operands,
// so each lane reads its A and B values as one 16-byte LDS read each: A operands row-major
// [row][k], B operands transposed [column][k]):
//   dU = P^T dY + (K dW1^T, from the row pass)      lam = Ainv^T dU      dv = diag(beta) lam
//   dP = lower_incl(dY U^T)      Z = lam U^T      dG_ij = -beta_i Z_ij (j < i), symmetrised
// then, per 64-column slice of D (wave w: column tile w, both row tiles),
//   dQ = dY W0 + dP K,   M = lam W0,   dK = U dW1 + dP^T Q + (dG + dG^T) K - diag(beta) M.
// The chunk's operands are loaded into registers in one batch before any LDS store; the next
// slice's W0, dW1, K and Q load into registers while the current slice computes.
template <bool BF16>
__global__ __launch_bounds__(kPrepThreads2) void bwd_chunk_grads_kernel(BwdArgs a) {
    extern __shared__ float lds[];
    const int D = a.D, d_v = a.d_v;
    const int u = blockIdx.x;
    const int bh = u / a.NC, n = u % a.NC;
    const int t0 = n * kBC;
    const int tid = threadIdx.x;
    const int wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    constexpr int CS = kCS;
    const int DV16 = grads_dv16(d_v), SV = grads_dvp(d_v);   // padded [C][d_v] rows
    const int NR = DV16 / 16;                                  // 16-column tiles of d_v
    const int CV = kBC * SV;
    float* dYs = lds;                 // [C][SV] row-major, zero past d_v
    float* Us = dYs + CV;             // U
    float* Ls = Us + CV;              // lam
    float* Vs = Ls + CV;
    float* dYT = Vs + CV;             // [DV16][CS]: dY^T
    float* dUT = dYT + DV16 * CS;     // dU^T
    float* PmT = dUT + DV16 * CS;     // [C][CS]: P^T
    float* AiT = PmT + kBC * CS;      // Ainv^T
    float* Gm = AiT + kBC * CS;       // G
    float* Zs = Gm + kBC * CS;        // Z
    float* dP = Zs + kBC * CS;
    float* dPT = dP + kBC * CS;       // dP^T
    float* dG = dPT + kBC * CS;       // dG + dG^T
    float* be = dG + kBC * CS;        // [C]
    float* bpart = be + kBC;          // [C]: lam_i.V_i - sum_{j<i} G_ij Z_ij
    float* mkb = bpart + kBC;         // [4][C]: per-wave partial sums of M_i . K_i
    float* W0T = mkb + 4 * kBC;       // [kSlice][SV]: W0 slice transposed
    float* G1T = W0T + kSlice * SV;   // dW1 slice transposed
    float* KT = G1T + kSlice * SV;    // [kSlice][CS]: K slice transposed
    float* QT = KT + kSlice * CS;

    const int64_t u64 = u;
    // ---- the chunk's operands, all loads first.  dy, v: (row c = tid / 64 + 4 m, entry r =
    //      tid % 64); U, K dW1^T: workspace [r][c] units tid + 256 m; Ainv, P, G: [i][j] units
    //      tid + 256 m
    {
        constexpr int MR = kBC / (kPrepThreads2 / 64);           // 8 rows per thread
        constexpr int MU = kBC * 64 / kPrepThreads2;              // 8 units (d_v <= 64)
        constexpr int MC = kBC * kBC / kPrepThreads2;             // 4 units
        const int r = tid & 63;
        float fy[MR], fv[MR], fu[MU], fa[MU], fi[MC], fp[MC], fg[MC];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int c = (tid >> 6) + 4 * m;
            const bool in = t0 + c < a.T && r < d_v;
            const int64_t g = (int64_t(bh) * a.T + t0 + (in ? c : 0)) * d_v + (in ? r : 0);
            fy[m] = in ? load_elem<BF16>(a.dy, g) : 0.0f;
            fv[m] = in ? load_elem<BF16>(a.v, g) : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < MU; ++m) {
            const int e = tid + kPrepThreads2 * m;
            const bool in = e < kBC * d_v;
            fu[m] = in ? a.ws[a.L.uu + u64 * kBC * d_v + e] : 0.0f;
            fa[m] = in ? a.ws[a.L.aa + u64 * kBC * d_v + e] : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            const int e = tid + kPrepThreads2 * m;
            fi[m] = a.ws[a.L.ai + u64 * kBC * kBC + e];
            fp[m] = a.ws[a.L.pm + u64 * kBC * kBC + e];
            fg[m] = a.ws[a.L.gm + u64 * kBC * kBC + e];
        }
        const float fb = tid < kBC ? a.ws[a.L.be + u64 * kBC + tid] : 0.0f;
        // zero padding: rows past d_v of the transposed tiles, entries past d_v of the row tiles
        for (int e = tid; e < (DV16 - d_v) * CS; e += kPrepThreads2) {
            dYT[d_v * CS + e] = 0.0f;
            dUT[d_v * CS + e] = 0.0f;
        }
        for (int e = tid; e < kBC * (SV - d_v); e += kPrepThreads2) {
            const int c = e / (SV - d_v), rr = d_v + e % (SV - d_v);
            dYs[c * SV + rr] = 0.0f;
            Us[c * SV + rr] = 0.0f;
            Ls[c * SV + rr] = 0.0f;
            Vs[c * SV + rr] = 0.0f;
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int c = (tid >> 6) + 4 * m;
            if (r < d_v) {
                dYs[c * SV + r] = fy[m];
                dYT[r * CS + c] = fy[m];
                Vs[c * SV + r] = fv[m];
            }
        }
#pragma unroll
        for (int m = 0; m < MU; ++m) {
            const int e = tid + kPrepThreads2 * m, rr = e >> 5, c = e & (kBC - 1);
            if (e < kBC * d_v) {
                Us[c * SV + rr] = fu[m];
                dUT[rr * CS + c] = fa[m];                  // K dW1^T, P^T dY added below
            }
        }
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            const int e = tid + kPrepThreads2 * m, i = e >> 5, j = e & (kBC - 1);
            AiT[j * CS + i] = fi[m];
            PmT[j * CS + i] = fp[m];
            Gm[i * CS + j] = fg[m];
        }
        if (tid < kBC) be[tid] = fb;
    }
    __syncthreads();
    // ---- dU = P^T dY + K dW1^T (tiles (it, rt) of dU, stored transposed)
    for (int tau = wv; tau < 2 * NR; tau += 4) {
        const int it = tau & 1, rt = tau >> 1;
        float* out = dUT + (16 * rt + l16) * CS + 16 * it + 4 * g4;
        f32x4 acc = *reinterpret_cast<const f32x4*>(out);
#pragma unroll
        for (int kb = 0; kb < kBC; kb += 16) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(PmT + (16 * it + l16) * CS + kb + 4 * g4);
            const f32x4 bv = *reinterpret_cast<const f32x4*>(dYT + (16 * rt + l16) * CS + kb + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma_f32_k4(av[s], bv[s], acc);
        }
        *reinterpret_cast<f32x4*>(out) = acc;
    }
    __syncthreads();
    // ---- lam = Ainv^T dU; dv = diag(beta) lam
    for (int tau = wv; tau < 2 * NR; tau += 4) {
        const int it = tau & 1, rt = tau >> 1;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < kBC; kb += 16) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(AiT + (16 * it + l16) * CS + kb + 4 * g4);
            const f32x4 bv = *reinterpret_cast<const f32x4*>(dUT + (16 * rt + l16) * CS + kb + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma_f32_k4(av[s], bv[s], acc);
        }
        const int r = 16 * rt + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * it + 4 * g4 + e;
            Ls[i * SV + r] = acc[e];
            if (r < d_v && t0 + i < a.T)
                store_elem<BF16>(a.dv, (int64_t(bh) * a.T + t0 + i) * d_v + r, be[i] * acc[e]);
        }
    }
    __syncthreads();
    // ---- dP = lower_incl(dY U^T) (and its transpose), Z = lam U^T, dG: wave w -> tile
    //      (w % 2, w / 2) of both
    {
        const int it = wv & 1, jt = wv >> 1;
        f32x4 sp = zero4(), sz = zero4();
        for (int kb = 0; kb < DV16; kb += 16) {
            const f32x4 bu = *reinterpret_cast<const f32x4*>(Us + (16 * jt + l16) * SV + kb + 4 * g4);
            const f32x4 ay = *reinterpret_cast<const f32x4*>(dYs + (16 * it + l16) * SV + kb + 4 * g4);
            const f32x4 al = *reinterpret_cast<const f32x4*>(Ls + (16 * it + l16) * SV + kb + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                sp = mfma_f32_k4(ay[s], bu[s], sp);
                sz = mfma_f32_k4(al[s], bu[s], sz);
            }
        }
        const int j = 16 * jt + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * it + 4 * g4 + e;
            const float p = j <= i ? sp[e] : 0.0f;
            dP[i * CS + j] = p;
            dPT[j * CS + i] = p;
            dG[i * CS + j] = j < i ? -be[i] * sz[e] : 0.0f;     // strict lower part for now
            Zs[i * CS + j] = sz[e];
        }
    }
    __syncthreads();
    // ---- dG's upper part = its transpose; beta partials lam_i.V_i - sum_{j<i} G_ij Z_ij over
    //      the 8 adjacent lanes of row i
    for (int e = tid; e < kBC * kBC; e += kPrepThreads2) {
        const int i = e >> 5, j = e & (kBC - 1);
        if (j > i) dG[i * CS + j] = dG[j * CS + i];
    }
    {
        const int i = tid >> 3, p8 = tid & 7;
        float s = 0.0f;
        for (int r = p8; r < d_v; r += 8) s += Ls[i * SV + r] * Vs[i * SV + r];
        for (int j = p8; j < i; j += 8) s -= Gm[i * CS + j] * Zs[i * CS + j];
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        if (p8 == 0) bpart[i] = s;
    }

    // ---- D-wide products per 64-column slice
    const int64_t CD = int64_t(kBC) * D;
    // staging: thread -> (column nn, 4 consecutive k) units u = tid + 256 p: nn = u % 64, k0 =
    // 4 (u / 64); four global loads down the k rows (coalesced along D over the lanes) become one
    // 16-byte LDS store of the transposed row.  W0 and dW1: k = the d_v index; K and Q: k = the
    // chunk row.
    constexpr int NW = 16 * kSlice / kPrepThreads2;      // W0 / dW1 units per thread (d_v <= 64)
    constexpr int NK = (kBC / 4) * kSlice / kPrepThreads2;   // K / Q units per thread
    f32x4 pw[NW], pg[NW], pk[NK], pq[NK];
    auto fetch = [&](int s0) {
#pragma unroll
        for (int p = 0; p < NW; ++p) {
            const int e = tid + kPrepThreads2 * p, k0 = 4 * (e / kSlice), nn = e % kSlice;
            const bool cin = s0 + nn < D;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool in = cin && k0 + q < d_v;
                const int64_t o = (u64 * d_v + (in ? k0 + q : 0)) * D + (in ? s0 + nn : 0);
                pw[p][q] = in ? a.ws[a.L.ws + o] : 0.0f;
                pg[p][q] = in ? a.ws[a.L.gs + o] : 0.0f;
            }
        }
#pragma unroll
        for (int p = 0; p < NK; ++p) {
            const int e = tid + kPrepThreads2 * p, c0 = 4 * (e / kSlice), nn = e % kSlice;
            const bool in = s0 + nn < D;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t o = u64 * CD + (c0 + q) * D + (in ? s0 + nn : 0);
                pk[p][q] = in ? a.ws[a.L.kt + o] : 0.0f;
                pq[p][q] = in ? a.ws[a.L.qt + o] : 0.0f;
            }
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int p = 0; p < NW; ++p) {
            const int e = tid + kPrepThreads2 * p, k0 = 4 * (e / kSlice), nn = e % kSlice;
            if (k0 < DV16) {
                *reinterpret_cast<f32x4*>(W0T + nn * SV + k0) = pw[p];
                *reinterpret_cast<f32x4*>(G1T + nn * SV + k0) = pg[p];
            }
        }
#pragma unroll
        for (int p = 0; p < NK; ++p) {
            const int e = tid + kPrepThreads2 * p, c0 = 4 * (e / kSlice), nn = e % kSlice;
            *reinterpret_cast<f32x4*>(KT + nn * CS + c0) = pk[p];
            *reinterpret_cast<f32x4*>(QT + nn * CS + c0) = pq[p];
        }
    };
    float mkp[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mkp[rt][e] = 0.0f;
    const int ncol = 16 * wv + l16;                         // the lane's column in the slice
    fetch(0);
    for (int s0 = 0; s0 < D; s0 += kSlice) {
        __syncthreads();                                    // the previous slice's reads are done
        commit();
        if (s0 + kSlice < D) fetch(s0 + kSlice);
        __syncthreads();
        f32x4 dq[2], mm[2], dk[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) dq[rt] = mm[rt] = dk[rt] = zero4();
        // k over d_v
        for (int kb = 0; kb < DV16; kb += 16) {
            const f32x4 bw = *reinterpret_cast<const f32x4*>(W0T + ncol * SV + kb + 4 * g4);
            const f32x4 bg = *reinterpret_cast<const f32x4*>(G1T + ncol * SV + kb + 4 * g4);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int ro = (16 * rt + l16) * SV + kb + 4 * g4;
                const f32x4 ady = *reinterpret_cast<const f32x4*>(dYs + ro);
                const f32x4 al = *reinterpret_cast<const f32x4*>(Ls + ro);
                const f32x4 au = *reinterpret_cast<const f32x4*>(Us + ro);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    dq[rt] = mfma_f32_k4(ady[s], bw[s], dq[rt]);
                    mm[rt] = mfma_f32_k4(al[s], bw[s], mm[rt]);
                    dk[rt] = mfma_f32_k4(au[s], bg[s], dk[rt]);
                }
            }
        }
        // k over the chunk rows
#pragma unroll
        for (int kb = 0; kb < kBC; kb += 16) {
            const f32x4 bk = *reinterpret_cast<const f32x4*>(KT + ncol * CS + kb + 4 * g4);
            const f32x4 bq = *reinterpret_cast<const f32x4*>(QT + ncol * CS + kb + 4 * g4);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int ro = (16 * rt + l16) * CS + kb + 4 * g4;
                const f32x4 ap = *reinterpret_cast<const f32x4*>(dP + ro);
                const f32x4 apt = *reinterpret_cast<const f32x4*>(dPT + ro);
                const f32x4 ag = *reinterpret_cast<const f32x4*>(dG + ro);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    dq[rt] = mfma_f32_k4(ap[s], bk[s], dq[rt]);
                    dk[rt] = mfma_f32_k4(apt[s], bq[s], dk[rt]);
                    dk[rt] = mfma_f32_k4(ag[s], bk[s], dk[rt]);
                }
            }
        }
        // result slot e of row tile rt: row i = 16 rt + 4 g4 + e, column s0 + ncol
        const int col = s0 + ncol;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * rt + 4 * g4 + e;
                const float m = mm[rt][e];
                mkp[rt][e] += m * KT[ncol * CS + i];
                if (col < D) {
                    a.ws[a.L.wy + u64 * CD + int64_t(i) * D + col] = dk[rt][e] - be[i] * m;
                    a.ws[a.L.qp + u64 * CD + int64_t(i) * D + col] = dq[rt][e];
                }
            }
        }
    }
    // M_i . K_i: the 16 lanes of a row group hold its columns; then the four waves
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float s = mkp[rt][e];
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            s += __shfl_xor(s, 4);
            s += __shfl_xor(s, 8);
            if (l16 == 0) mkb[wv * kBC + 16 * rt + 4 * g4 + e] = s;
        }
    __syncthreads();
    if (tid < kBC && t0 + tid < a.T) {
        // beta (1 - beta) as sigmoid(l) sigmoid(-l): 1 - beta cancels where beta rounds to 1
        const int i = tid;
        const float mk = (mkb[i] + mkb[kBC + i]) + (mkb[2 * kBC + i] + mkb[3 * kBC + i]);
        const int64_t g = int64_t(bh) * a.T + t0 + i;
        const float l = load_elem<BF16>(a.bl, g);
        const float dbeta = bpart[i] - mk;
        store_elem<BF16>(a.dbl, g, dbeta * sigmoid_stable(l) * sigmoid_stable(-l));
    }
}

// ------------------------------------------------------------------------------ 5. DPFP'

// One wave per vector: dx = (d phi / d x)^T dphi for x = k (blockIdx.y == 0, dphi = dK) or
// x = q (blockIdx.y == 1, dphi = dQ).  phi = raw / (S + eps), so
// draw_p = (dphi_p - dphi . phi) / (S + eps); with raw(i, j) = x[j] x[(j - i) mod 2 d_k], the
// relu'd entry m receives sum_i draw(i, m) x[m - i] + draw(i, m + i) x[m + i] (indices mod
// 2 d_k), and k_j receives that of entry j where k_j > 0 and minus that of entry d_k + j where
// k_j < 0.
constexpr int kDpfpWaves = 4;

template <bool BF16>
__global__ __launch_bounds__(64 * kDpfpWaves) void bwd_dpfp_kernel(BwdArgs a) {
    __shared__ float xs_all[kDpfpWaves][128];
    __shared__ float dr_all[kDpfpWaves][512];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t vec = int64_t(blockIdx.x) * kDpfpWaves + wave;      // (bh, t) flat
    const int64_t nvec = int64_t(a.BH) * a.T;
    const bool live = vec < nvec;
    const bool isq = blockIdx.y == 1;
    const void* x = isq ? a.q : a.k;
    void* dx_out = isq ? a.dq : a.dk;
    const int d_k = a.d_k, two = 2 * d_k, D = a.D;
    float* xs = xs_all[wave];
    float* dr = dr_all[wave];
    const int64_t bh = live ? vec / a.T : 0, t = live ? vec % a.T : 0;
    const float* dphi = a.ws + (isq ? a.L.qp : a.L.wy) +
                        ((bh * a.NC + t / kBC) * kBC + t % kBC) * int64_t(D);
    for (int m = lane; m < two; m += 64) {
        const float kv = live ? load_elem<BF16>(x, vec * d_k + (m % d_k)) : 0.0f;
        xs[m] = m < d_k ? relu(kv) : relu(-kv);
    }
    __syncthreads();
    float S = 0.0f, dot = 0.0f;
    for (int p = lane; p < D; p += 64) {
        const int i = p / two + 1, j = p % two;
        int src = j - i;
        src += src < 0 ? two : 0;
        const float raw = xs[j] * xs[src];
        S += raw;
        dot += live ? dphi[p] * raw : 0.0f;
    }
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) {
        S += __shfl_xor(S, mask);
        dot += __shfl_xor(dot, mask);
    }
    const float den = S + kDpfpEps;
    const float dphin = dot / den;                          // dphi . phi
    for (int p = lane; p < D; p += 64) dr[p] = live ? (dphi[p] - dphin) / den : 0.0f;
    __syncthreads();
    if (live && lane < d_k) {
        float dxv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int m = lane + h * d_k;
            float s = 0.0f;
            for (int i = 1; i <= a.nu; ++i) {
                const int base = (i - 1) * two;
                int mi = m - i;
                mi += mi < 0 ? two : 0;
                int pi = m + i;
                pi -= pi >= two ? two : 0;
                s += dr[base + m] * xs[mi] + dr[base + pi] * xs[pi];
            }
            dxv[h] = s;
        }
        const float kv = load_elem<BF16>(x, vec * d_k + lane);
        const float gk = (kv > 0.0f ? dxv[0] : 0.0f) - (kv < 0.0f ? dxv[1] : 0.0f);
        store_elem<BF16>(dx_out, vec * d_k + lane, gk);
    }
}

// ------------------------------------------------------------------------------ host

static int bwd_npl(int D) { return (D + 63) / 64; }

bool plan_backward(int BH, int T, int d_k, int d_v, int nu, int64_t* ws_bytes) {
    const int D = 2 * d_k * nu;
    if (d_k != 16 && d_k != 32 && d_k != 64) return false;
    if (d_v < 1 || d_v > 64 || D > 384 || nu > 64) return false;
    const int NC = (T + kBC - 1) / kBC;
    const BwdLayout L = bwd_layout(int64_t(BH) * NC, D, d_v);
    *ws_bytes = L.end * 4;
    return true;
}

static int lds_prep_bytes(int D, int d_k, int d_v) {
    return 4 * (2 * kBC * 2 * d_k + 2 * kBC * tile_stride(D) + 3 * kBC * kCS + kBC +
                kBC * d_v);
}
static int lds_grads_bytes(int d_v) {
    const int SV = grads_dvp(d_v), DV16 = grads_dv16(d_v);
    return 4 * (4 * kBC * SV + 2 * DV16 * kCS + 7 * kBC * kCS + 2 * kBC + 4 * kBC +
                2 * kSlice * SV + 2 * kSlice * kCS);
}

template <int NPL, bool BF16>
static hipError_t launch_rows(const BwdArgs& a, hipStream_t stream) {
    const int rgroups = (a.d_v + kRowWaves - 1) / kRowWaves;
    const dim3 grid(static_cast<unsigned>(int64_t(a.BH) * rgroups));
    auto kf = bwd_fwd_states_kernel<NPL>;
    auto kg = bwd_grad_states_kernel<BF16, NPL>;
    const int lf = 4 * 2 * kBC * 64 * NPL, lg = 4 * 3 * kBC * 64 * NPL;
    hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kf), lf);
    if (e != hipSuccess) return e;
    if ((e = ensure_lds_attr(reinterpret_cast<const void*>(kg), lg)) != hipSuccess) return e;
    hipLaunchKernelGGL(kf, grid, dim3(64 * kRowWaves), lf, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(kg, grid, dim3(64 * kRowWaves), lg, stream, a);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_backward_t(BwdArgs a, hipStream_t stream) {
    const int64_t NU = int64_t(a.BH) * a.NC;
    hipError_t e;
    if (NU > 0) {
        const int lp = lds_prep_bytes(a.D, a.d_k, a.d_v);
        auto kp = bwd_prep_kernel<BF16>;
        if ((e = ensure_lds_attr(reinterpret_cast<const void*>(kp), lp)) != hipSuccess) return e;
        hipLaunchKernelGGL(kp, dim3(static_cast<unsigned>(NU)), dim3(kPrepThreads2), lp, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    switch (bwd_npl(a.D)) {
        case 1: e = launch_rows<1, BF16>(a, stream); break;
        case 2: e = launch_rows<2, BF16>(a, stream); break;
        case 3: e = launch_rows<3, BF16>(a, stream); break;
        case 4: e = launch_rows<4, BF16>(a, stream); break;
        case 5: e = launch_rows<5, BF16>(a, stream); break;
        case 6: e = launch_rows<6, BF16>(a, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || NU == 0) return e;
    const int lg = lds_grads_bytes(a.d_v);
    auto kc = bwd_chunk_grads_kernel<BF16>;
    if ((e = ensure_lds_attr(reinterpret_cast<const void*>(kc), lg)) != hipSuccess) return e;
    hipLaunchKernelGGL(kc, dim3(static_cast<unsigned>(NU)), dim3(kPrepThreads2), lg, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nvec = int64_t(a.BH) * a.T;
    const dim3 grid(static_cast<unsigned>((nvec + kDpfpWaves - 1) / kDpfpWaves), 2);
    hipLaunchKernelGGL((bwd_dpfp_kernel<BF16>), grid, dim3(64 * kDpfpWaves), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_backward(const void* q, const void* k, const void* v, const void* bl,
                           const float* W0, const void* dy, const float* dWf, void* dq, void* dk,
                           void* dv, void* dbl, float* dW0, int BH, int T, int d_k, int d_v,
                           int nu, bool bf16, void* workspace, hipStream_t stream) {
    BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.bl = bl; a.W0 = W0; a.dy = dy; a.dWf = dWf;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dbl = dbl; a.dW0 = dW0;
    a.ws = static_cast<float*>(workspace);
    a.BH = BH; a.T = T; a.NC = (T + kBC - 1) / kBC; a.d_k = d_k; a.d_v = d_v; a.nu = nu;
    a.D = 2 * d_k * nu;
    a.L = bwd_layout(int64_t(BH) * a.NC, a.D, d_v);
    return bf16 ? launch_backward_t<true>(a, stream) : launch_backward_t<false>(a, stream);
}

}  // namespace fwa
