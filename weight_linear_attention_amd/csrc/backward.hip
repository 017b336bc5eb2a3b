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
    L.kt = o; o += NU * CD;      // K^T [d][c]
    L.qt = o; o += NU * CD;      // Q^T [d][c]
    L.wy = o; o += NU * CD;      // Wy^T [d][c], then dK [c][d] (bwd_chunk_grads)
    L.qp = o; o += NU * CD;      // Q'^T [d][c], then dQ [c][d]
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

// Floats of the prep's two LDS regions (see below).
__host__ __device__ inline int bwd_prep_region_a(int d_k) {
    const int x = 2 * kBC * 2 * d_k, t = 2 * (2 * d_k) * kCS;
    return x > t ? x : t;
}
__host__ __device__ inline int bwd_prep_region_b(int d_k) {
    const int sl = 2 * kBC * (2 * d_k + 4), m = 4 * kBC * kCS;
    return sl > m ? sl : m;
}

// LDS (77 KB at d_k = 64, d_v = 64: two workgroups per CU):
//   region A: the relu'd raw rows of k and q (C x 2 d_k each) in the first pass; in the second
//             one shift slice of K^T and of Q^T read back ([2 d_k][kCS] each), W_y^T of the
//             slice over K^T once it is read;
//   region B: one shift slice of K and of Q (C x (2 d_k + 4)) in the first pass; then G, P,
//             Ainv and T = Ainv diag(beta) (C x kCS each);
//   beta (C), V (C x d_v).
// The row sums of the raw features come first (the order dpfp_tiles uses).  First pass, one
// shift i at a time: the slice's normalised features (columns (i - 1) 2 d_k .. + 2 d_k - 1) go
// to the workspace transposed and into the G = K K^T and P = lower_incl(Q K^T) accumulators.
// Then Ainv and T.  Second pass, per slice: K^T and Q^T back from the workspace (written by this
// workgroup, visible after the workgroup barrier), W_y = T K and Q' = Q - P W_y.  Every product
// runs on the fp32 MFMA (16x16x4; lane group g supplies k = 4 g + s to sub-step s).
template <bool BF16>
__global__ __launch_bounds__(kPrepThreads2, 2) void bwd_prep_kernel(BwdArgs a) {
    extern __shared__ float lds[];
    const int D = a.D, d_k = a.d_k, d_v = a.d_v, two = 2 * d_k;
    const int u = blockIdx.x;
    const int bh = u / a.NC, n = u % a.NC;
    const int t0 = n * kBC;
    const int tid = threadIdx.x;
    const int wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    constexpr int CS = kCS;
    const int SS = two + 4;
    const int regA = bwd_prep_region_a(d_k), regB = bwd_prep_region_b(d_k);
    float* xk = lds;                         // [C][2 d_k]
    float* xq = xk + kBC * two;
    float* KT = lds;                         // [2 d_k][CS] (second pass)
    float* QT = KT + two * CS;
    float* Ks = lds + regA;                  // [C][SS] (first pass)
    float* Qs = Ks + kBC * SS;
    float* Gm = lds + regA;                  // [C][CS] each
    float* Pm = Gm + kBC * CS;
    float* Ai = Pm + kBC * CS;
    float* Ts = Ai + kBC * CS;
    float* be = lds + regA + regB;           // [C]
    float* Vs = be + kBC;                    // [C][d_v]

    // relu'd raw rows (zero past the sequence end), beta (zero past the end), v
    const int rows = a.T - t0 < kBC ? a.T - t0 : kBC;
    const float blv = load_elem<BF16>(a.bl, int64_t(bh) * a.T + t0 + min(tid & (kBC - 1), rows - 1));
    load_chunk_inputs<BF16, kPrepThreads2, 64>(a.k, a.q, a.v, xk, xq, Vs, int64_t(bh) * a.T, rows,
                                               t0, d_k, d_v, tid);
    if (tid < kBC) be[tid] = tid < rows ? sigmoid_stable(blv) : 0.0f;
    __syncthreads();
    // row sums: row c = tid / 8 by its eight adjacent threads, entries p = tid % 8 + 8 m
    const int c = tid >> 3, s0 = tid & 7;
    const float* xrk = xk + c * two;
    const float* xrq = xq + c * two;
    float sk = 0.0f, sq = 0.0f;
    for (int i = 1; i <= a.nu; ++i)
        for (int jj = s0; jj < two; jj += 8) {
            int src = jj - i;
            src += (src < 0) ? two : 0;
            sk += xrk[jj] * xrk[src];
            sq += xrq[jj] * xrq[src];
        }
    sk = sum8_dpp(sk);
    sq = sum8_dpp(sq);
    const float ik = 1.0f / (sk + kDpfpEps), iq = 1.0f / (sq + kDpfpEps);
    const int64_t CD = int64_t(kBC) * D;
    float* gK = a.ws + a.L.kt + int64_t(u) * CD;
    float* gQ = a.ws + a.L.qt + int64_t(u) * CD;
    // G (all four tiles) and P (tiles (0,0), (1,0), (1,1)): wave w takes tiles w and w + 4
    f32x4 gacc[2] = {zero4(), zero4()};
    for (int i = 1; i <= a.nu; ++i) {
        const int col0 = (i - 1) * two;
        for (int jj = s0; jj < two; jj += 8) {
            int src = jj - i;
            src += (src < 0) ? two : 0;
            Ks[c * SS + jj] = xrk[jj] * xrk[src] * ik;
            Qs[c * SS + jj] = xrq[jj] * xrq[src] * iq;
        }
        __syncthreads();
        // K and Q leave transposed ([D][C]): unit e = 4 consecutive rows of column col0 + e / 8
        for (int e = tid; e < 8 * two; e += kPrepThreads2) {
            const int f = e >> 3, c0 = 4 * (e & 7);
            f32x4 kv, qv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kv[j] = Ks[(c0 + j) * SS + f];
                qv[j] = Qs[(c0 + j) * SS + f];
            }
            *reinterpret_cast<f32x4*>(gK + (col0 + f) * kBC + c0) = kv;
            *reinterpret_cast<f32x4*>(gQ + (col0 + f) * kBC + c0) = qv;
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tau = wv + 4 * q;
            if (tau >= 7) continue;
            const bool isP = tau >= 4;
            const int it = isP ? (tau == 4 ? 0 : 1) : tau >> 1;
            const int jt = isP ? (tau == 6 ? 1 : 0) : tau & 1;
            const float* X = isP ? Qs : Ks;
            for (int kb = 0; kb < two; kb += 16) {
                const f32x4 av = *reinterpret_cast<const f32x4*>(X + (16 * it + l16) * SS + kb + 4 * g4);
                const f32x4 bv = *reinterpret_cast<const f32x4*>(Ks + (16 * jt + l16) * SS + kb + 4 * g4);
#pragma unroll
                for (int s = 0; s < 4; ++s) gacc[q] = mfma_f32_k4(av[s], bv[s], gacc[q]);
            }
        }
        __syncthreads();                                         // the slice is dead
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int tau = wv + 4 * q;
        if (tau >= 7) continue;
        const bool isP = tau >= 4;
        const int it = isP ? (tau == 4 ? 0 : 1) : tau >> 1;
        const int jt = isP ? (tau == 6 ? 1 : 0) : tau & 1;
        const int col = 16 * jt + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * it + 4 * g4 + e;
            if (isP) Pm[row * CS + col] = col <= row ? gacc[q][e] : 0.0f;
            else Gm[row * CS + col] = gacc[q][e];
        }
    }
    for (int e = tid; e < 16 * 16; e += kPrepThreads2)         // P tile (0, 1): above the diagonal
        Pm[(e >> 4) * CS + 16 + (e & 15)] = 0.0f;
    __syncthreads();
    // Ainv = (I + diag(beta) strict_lower(G))^-1 by forward substitution: column j = tid / 8 by
    // the 8 adjacent threads s = tid % 8, thread s holding x[m] for m = s mod 8; each row's sum
    // adds the 8 threads' parts over the lanes
    {
        const int j = tid >> 3, s = tid & 7;
        float xs[kBC / 8];
#pragma unroll
        for (int k = 0; k < kBC / 8; ++k) xs[k] = 0.0f;
#pragma unroll
        for (int i = 0; i < kBC; ++i) {
            float p = 0.0f;
#pragma unroll
            for (int k = 0; k < kBC / 8; ++k)
                if (8 * k < i && s + 8 * k < i) p += Gm[i * CS + s + 8 * k] * xs[k];
            p = sum8_dpp(p);
            const float xi = i == j ? 1.0f : (i > j ? -be[i] * p : 0.0f);
            if (s == (i & 7)) xs[i >> 3] = xi;
        }
#pragma unroll
        for (int k = 0; k < kBC / 8; ++k) Ai[(s + 8 * k) * CS + j] = xs[k];
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kPrepThreads2) {       // T = Ainv diag(beta)
        const int i = e >> 5, j = e & (kBC - 1);
        Ts[i * CS + j] = Ai[i * CS + j] * be[j];
    }
    // second pass: W_y = T K and Q' = Q - P W_y per slice; tiles (it, pt) w + 4 q of the slice
    float* gWy = a.ws + a.L.wy + int64_t(u) * CD;
    float* gQp = a.ws + a.L.qp + int64_t(u) * CD;
    const int NPT = two / 16;
    constexpr int kMaxWy = 128 / 16 * 2 / 4;                     // tiles per wave, 2 d_k <= 128
    for (int i = 1; i <= a.nu; ++i) {
        const int col0 = (i - 1) * two;
        __syncthreads();                                         // T written; last slice dead
        for (int e = tid; e < 8 * two; e += kPrepThreads2) {
            const int f = e >> 3, c0 = 4 * (e & 7);
            *reinterpret_cast<f32x4*>(KT + f * CS + c0) = *reinterpret_cast<const f32x4*>(gK + (col0 + f) * kBC + c0);
            *reinterpret_cast<f32x4*>(QT + f * CS + c0) = *reinterpret_cast<const f32x4*>(gQ + (col0 + f) * kBC + c0);
        }
        __syncthreads();
        f32x4 wy[kMaxWy];
#pragma unroll
        for (int q = 0; q < kMaxWy; ++q) {
            const int tau = wv + 4 * q;
            wy[q] = zero4();
            if (tau >= 2 * NPT) continue;
            const int it = tau & 1, pt = tau >> 1;
#pragma unroll
            for (int kb = 0; kb < kBC; kb += 16) {
                const f32x4 av = *reinterpret_cast<const f32x4*>(Ts + (16 * it + l16) * CS + kb + 4 * g4);
                const f32x4 bv = *reinterpret_cast<const f32x4*>(KT + (16 * pt + l16) * CS + kb + 4 * g4);
#pragma unroll
                for (int s = 0; s < 4; ++s) wy[q] = mfma_f32_k4(av[s], bv[s], wy[q]);
            }
            *reinterpret_cast<f32x4*>(gWy + (col0 + 16 * pt + l16) * kBC + 16 * it + 4 * g4) = wy[q];   // [D][C]
        }
        __syncthreads();                                         // K^T is dead: W_y^T over it
#pragma unroll
        for (int q = 0; q < kMaxWy; ++q) {
            const int tau = wv + 4 * q;
            if (tau >= 2 * NPT) continue;
            const int it = tau & 1, pt = tau >> 1;
            *reinterpret_cast<f32x4*>(KT + (16 * pt + l16) * CS + 16 * it + 4 * g4) = wy[q];
        }
        __syncthreads();
        for (int tau = wv; tau < 2 * NPT; tau += 4) {
            const int it = tau & 1, pt = tau >> 1;
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < kBC; kb += 16) {
                const f32x4 av = *reinterpret_cast<const f32x4*>(Pm + (16 * it + l16) * CS + kb + 4 * g4);
                const f32x4 bv = *reinterpret_cast<const f32x4*>(KT + (16 * pt + l16) * CS + kb + 4 * g4);
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mfma_f32_k4(av[s], bv[s], acc);
            }
            const f32x4 qv = *reinterpret_cast<const f32x4*>(QT + (16 * pt + l16) * CS + 16 * it + 4 * g4);
            *reinterpret_cast<f32x4*>(gQp + (col0 + 16 * pt + l16) * kBC + 16 * it + 4 * g4) = qv - acc;   // [D][C]
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

// ------------------------------------------------------------------------------ state chains

// The two chains over the chunks, one launch: workgroups [0, G) run the forward chain of the
// chunk-start memories, workgroups [G, 2 G) the reverse chain of the chunk-end memory
// gradients (G = B H ceil(d_v / 16)); neither reads what the other writes.  A workgroup of 8
// waves owns 16 rows r of one memory, held transposed (D x 16) in fp32 MFMA accumulators: wave
// w holds d-tiles dt = w + 8 q (rows d = 16 dt + 4 (l / 16) + e, column l % 16 of lane l, slot
// e), which is the B operand of a 16x16x4 product over those d as it stands (lane group g
// supplies k = 4 g + s to sub-step s).  Per chunk each wave forms its part of a 32 x 16 product
// over its d-tiles, waves 0 and 1 sum the eight parts of one 16-row tile each into LDS (in the
// layout of the update's B operand), and each wave updates its d-tiles.  The per-chunk [D][C]
// tiles are stored transposed in the workspace and staged as they are into LDS rows of kTS
// floats; the next chunk's tiles load into registers while the current chunk computes.
constexpr int kStWaves = 8;
constexpr int kStThreads = 64 * kStWaves;
constexpr int kTS = kBC + 4;     // LDS row stride of the transposed tiles and the [16][C] operands

// LDS floats of the state chains: two [D][kTS] tiles, two [16][kTS] operands, the per-wave
// partial products (8 waves x 2 row tiles x 64 lanes x 4)
__host__ __device__ inline int states_lds_floats(int D) {
    return 2 * D * kTS + 2 * 16 * kTS + kStWaves * 2 * 64 * 4;
}

// Every lane issues the same loads (a unit past the tile loads the last one again and is not
// committed), so the in-order load counter lets each commit wait for its own tile only.
template <int NUM>
__device__ __forceinline__ void fetch_tile_t(f32x4 (&r)[NUM], const float* g, int units, int tid) {
    const f32x4* g4 = reinterpret_cast<const f32x4*>(g);
#pragma unroll
    for (int m = 0; m < NUM; ++m) r[m] = g4[min(tid + kStThreads * m, units - 1)];
}

// unit uu = 4 consecutive c of row d = uu / 8
template <int NUM>
__device__ __forceinline__ void commit_tile_t(float* s, const f32x4 (&r)[NUM], int units, int tid) {
#pragma unroll
    for (int m = 0; m < NUM; ++m) {
        const int uu = tid + kStThreads * m;
        if (uu < units) *reinterpret_cast<f32x4*>(s + (uu >> 3) * kTS + 4 * (uu & 7)) = r[m];
    }
}

// This wave's part of X^T = A S^T over its d-tiles, A ([C][D]) read from its transposed LDS copy
// AT ([D][kTS]) and S^T in the accumulators, into red: rows c = 16 rt + 4 (l / 16) + e of X^T
// in red[wave][rt][lane].
template <int NDW>
__device__ __forceinline__ void states_partial(const float* AT, const f32x4 (&S)[NDW], int NDT,
                                               int wv, int lane, f32x4* red) {
    const int l16 = lane & 15, g4 = lane >> 4;
    f32x4 P0 = zero4(), P1 = zero4();
#pragma unroll
    for (int q = 0; q < NDW; ++q) {
        const int dt = wv + kStWaves * q;
        if (dt >= NDT) continue;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float* row = AT + (16 * dt + 4 * g4 + s) * kTS;
            P0 = mfma_f32_k4(row[l16], S[q][s], P0);
            P1 = mfma_f32_k4(row[16 + l16], S[q][s], P1);
        }
    }
    red[(wv * 2 + 0) * 64 + lane] = P0;
    red[(wv * 2 + 1) * 64 + lane] = P1;
}

// The sum of the eight waves' parts of row tile rt, in this lane's accumulator slots.
__device__ __forceinline__ f32x4 states_sum(const f32x4* red, int rt, int lane) {
    f32x4 x = red[rt * 64 + lane];
#pragma unroll
    for (int w = 1; w < kStWaves; ++w) x += red[(w * 2 + rt) * 64 + lane];
    return x;
}

// Row r of the memory moves as w <- w + K^T u with u = Uy[:, r] - Wy w (the chunk's own
// correction of the values, "Linear Transformers Are Secretly Fast Weight Programmers",
// delta rule in chunked form); writes each chunk-start memory and u.
template <int NDW>
__device__ __forceinline__ void fwd_states_chain(const BwdArgs& a, float* lds, int bh, int r0) {
    const int D = a.D, d_v = a.d_v, NDT = D / 16;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int r = r0 + l16;
    const bool rok = r < d_v;
    float* WyT = lds;                             // [D][kTS]
    float* KT = WyT + D * kTS;                    // [D][kTS]
    float* UyT = KT + D * kTS;                    // [16][kTS]: Uy^T, then u^T
    f32x4* red = reinterpret_cast<f32x4*>(UyT + 2 * 16 * kTS);  // [8 waves][2][64 lanes]
    f32x4 W[NDW];
#pragma unroll
    for (int q = 0; q < NDW; ++q) {
        const int dt = wv + kStWaves * q;
        W[q] = zero4();
        if (a.W0 && rok && dt < NDT)
            W[q] = *reinterpret_cast<const f32x4*>(a.W0 + (int64_t(bh) * d_v + r) * D + 16 * dt + 4 * g4);
    }
    const int64_t CD = int64_t(kBC) * D;
    const int units = 8 * D;
    constexpr int NUM = 2 * NDW;
    f32x4 rwy[NUM], rk[NUM];
    // Uy^T element of this thread: row yr = tid % 16 of the 16, chunk row yc = tid / 16 (rows
    // past d_v load row d_v - 1 and commit 0)
    const int yc = tid >> 4, yr = tid & 15;
    const bool yok = r0 + yr < d_v;
    const int yrc = min(r0 + yr, d_v - 1);
    float uy_next;
    auto fetch = [&](int nn) {
        const int64_t uf = int64_t(bh) * a.NC + nn;
        fetch_tile_t(rwy, a.ws + a.L.wy + uf * CD, units, tid);
        fetch_tile_t(rk, a.ws + a.L.kt + uf * CD, units, tid);
        uy_next = a.ws[a.L.uy + (uf * kBC + yc) * d_v + yrc];
    };
    if (a.NC > 0) fetch(0);
    for (int n = 0; n < a.NC; ++n) {
        const int64_t u = int64_t(bh) * a.NC + n;
        if (rok) {
            float* gw = a.ws + a.L.ws + (u * d_v + r) * D;
#pragma unroll
            for (int q = 0; q < NDW; ++q) {
                const int dt = wv + kStWaves * q;
                if (dt < NDT) *reinterpret_cast<f32x4*>(gw + 16 * dt + 4 * g4) = W[q];
            }
        }
        lds_barrier();                            // the previous chunk's reads are done
        commit_tile_t(WyT, rwy, units, tid);
        commit_tile_t(KT, rk, units, tid);
        UyT[yr * kTS + yc] = yok ? uy_next : 0.0f;
        lds_barrier();
        fetch(n + 1 < a.NC ? n + 1 : n);          // unconditional: the load counts stay fixed
        states_partial(WyT, W, NDT, wv, lane, red);
        lds_barrier();
        // u^T = Uy^T - (Wy W^T)^T: waves 0 and 1 sum row tile wv, each lane rewriting its own
        // 16 bytes of UyT
        if (wv < 2) {
            f32x4* up = reinterpret_cast<f32x4*>(UyT + l16 * kTS + 16 * wv + 4 * g4);
            const f32x4 uc = *up - states_sum(red, wv, lane);
            *up = uc;
            if (rok)
                *reinterpret_cast<f32x4*>(a.ws + a.L.uu + (u * d_v + r) * kBC + 16 * wv + 4 * g4) = uc;
        }
        lds_barrier();
        // W^T += K^T u on this wave's d-tiles
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const f32x4 bv = *reinterpret_cast<const f32x4*>(UyT + l16 * kTS + 16 * rt + 4 * g4);
#pragma unroll
            for (int q = 0; q < NDW; ++q) {
                const int dt = wv + kStWaves * q;
                if (dt >= NDT) continue;
                const f32x4 av = *reinterpret_cast<const f32x4*>(KT + (16 * dt + l16) * kTS + 16 * rt + 4 * g4);
#pragma unroll
                for (int s = 0; s < 4; ++s) W[q] = mfma_f32_k4(av[s], bv[s], W[q]);
            }
        }
    }
}

// Row r of the memory gradient moves backwards as g <- g + Q'^T dY[:, r] - Wy^T (K g); writes
// each chunk-end gradient, K g, and the gradient of the initial memory.  The K tile's LDS rows
// take the Wy tile once the products with K are done.
template <bool BF16, int NDW>
__device__ __forceinline__ void grad_states_chain(const BwdArgs& a, float* lds, int bh, int r0) {
    const int D = a.D, d_v = a.d_v, NDT = D / 16;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int r = r0 + l16;
    const bool rok = r < d_v;
    float* KT = lds;                              // [D][kTS]: K^T, then Wy^T
    float* WyT = KT;
    float* QpT = KT + D * kTS;                    // [D][kTS]
    float* dYT = QpT + D * kTS;                   // [16][kTS]: dY^T of the 16 rows
    float* AT = dYT + 16 * kTS;                   // [16][kTS]: -(K g)^T
    f32x4* red = reinterpret_cast<f32x4*>(AT + 16 * kTS);
    f32x4 G[NDW];
#pragma unroll
    for (int q = 0; q < NDW; ++q) {
        const int dt = wv + kStWaves * q;
        G[q] = zero4();
        if (a.dWf && rok && dt < NDT)
            G[q] = *reinterpret_cast<const f32x4*>(a.dWf + (int64_t(bh) * d_v + r) * D + 16 * dt + 4 * g4);
    }
    const int64_t CD = int64_t(kBC) * D;
    const int units = 8 * D;
    constexpr int NUM = 2 * NDW;
    f32x4 rk[NUM], rq[NUM], rwy[NUM];
    // dY^T element of this thread: row yr = tid % 16 of the 16, chunk row yc = tid / 16, loaded
    // as stored (clamped into the sequence) and converted when committed
    using YT = std::conditional_t<BF16, u16, float>;
    const int yc = tid >> 4, yr = tid & 15;
    const bool yok = r0 + yr < d_v;
    const int yrc = min(r0 + yr, d_v - 1);
    YT dy_next{};
    auto fetch_kq = [&](int nn) {
        const int64_t uf = int64_t(bh) * a.NC + nn;
        fetch_tile_t(rk, a.ws + a.L.kt + uf * CD, units, tid);
        fetch_tile_t(rq, a.ws + a.L.qp + uf * CD, units, tid);
        const int tf = min(nn * kBC + yc, a.T - 1);
        dy_next = static_cast<const YT*>(a.dy)[(int64_t(bh) * a.T + tf) * d_v + yrc];
    };
    auto fetch_wy = [&](int nn) {
        fetch_tile_t(rwy, a.ws + a.L.wy + (int64_t(bh) * a.NC + nn) * CD, units, tid);
    };
    if (a.NC > 0) {
        fetch_kq(a.NC - 1);
        fetch_wy(a.NC - 1);
    }
    for (int n = a.NC - 1; n >= 0; --n) {
        const int64_t u = int64_t(bh) * a.NC + n;
        const int nn = n > 0 ? n - 1 : 0;         // unconditional prefetch: load counts stay fixed
        if (rok) {
            float* gg = a.ws + a.L.gs + (u * d_v + r) * D;
#pragma unroll
            for (int q = 0; q < NDW; ++q) {
                const int dt = wv + kStWaves * q;
                if (dt < NDT) *reinterpret_cast<f32x4*>(gg + 16 * dt + 4 * g4) = G[q];
            }
        }
        lds_barrier();                            // the previous chunk's reads are done
        commit_tile_t(KT, rk, units, tid);
        commit_tile_t(QpT, rq, units, tid);
        dYT[yr * kTS + yc] = (yok && n * kBC + yc < a.T) ? to_f32(dy_next) : 0.0f;
        lds_barrier();
        fetch_kq(nn);
        states_partial(KT, G, NDT, wv, lane, red);
        lds_barrier();
        // -(K g)^T: waves 0 and 1 sum row tile wv
        if (wv < 2) {
            const f32x4 ac = states_sum(red, wv, lane);
            *reinterpret_cast<f32x4*>(AT + l16 * kTS + 16 * wv + 4 * g4) = -ac;
            if (rok)
                *reinterpret_cast<f32x4*>(a.ws + a.L.aa + (u * d_v + r) * kBC + 16 * wv + 4 * g4) = ac;
        }
        commit_tile_t(WyT, rwy, units, tid);      // K^T is dead
        fetch_wy(nn);
        lds_barrier();
        // G^T += Q'^T dY - Wy^T (K g) on this wave's d-tiles
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const f32x4 by = *reinterpret_cast<const f32x4*>(dYT + l16 * kTS + 16 * rt + 4 * g4);
            const f32x4 ba = *reinterpret_cast<const f32x4*>(AT + l16 * kTS + 16 * rt + 4 * g4);
#pragma unroll
            for (int q = 0; q < NDW; ++q) {
                const int dt = wv + kStWaves * q;
                if (dt >= NDT) continue;
                const int ro = (16 * dt + l16) * kTS + 16 * rt + 4 * g4;
                const f32x4 aq = *reinterpret_cast<const f32x4*>(QpT + ro);
                const f32x4 aw = *reinterpret_cast<const f32x4*>(WyT + ro);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    G[q] = mfma_f32_k4(aq[s], by[s], G[q]);
                    G[q] = mfma_f32_k4(aw[s], ba[s], G[q]);
                }
            }
        }
    }
    if (a.dW0 && rok) {
#pragma unroll
        for (int q = 0; q < NDW; ++q) {
            const int dt = wv + kStWaves * q;
            if (dt < NDT)
                *reinterpret_cast<f32x4*>(a.dW0 + (int64_t(bh) * d_v + r) * D + 16 * dt + 4 * g4) = G[q];
        }
    }
}

// Workgroups are dispatched to the 8 XCDs round robin by index: logical index L counts the
// workgroups of XCD 0 first, then XCD 1, ..., so the row groups of one (b, h) and role, which
// stage the same tiles in step, share an L2.
template <bool BF16, int NDW>
__global__ __launch_bounds__(kStThreads) void bwd_states_kernel(BwdArgs a) {
    extern __shared__ float lds[];
    const int rgroups = (a.d_v + 15) / 16;
    const int G = a.BH * rgroups, N = 2 * G;
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int L = x * (N >> 3) + min(x, N & 7) + j;
    const int b = L < G ? L : L - G;
    const int bh = b / rgroups, r0 = (b % rgroups) * 16;
    if (L < G) fwd_states_chain<NDW>(a, lds, bh, r0);
    else grad_states_chain<BF16, NDW>(a, lds, bh, r0);
}

// ------------------------------------------------------------------------------ 4. chunk grads

constexpr int kSlice = 64;   // columns of D per pass in bwd_chunk_grads
constexpr int kGradThreads = 512;                 // bwd_chunk_grads: 8 waves
constexpr int kGradWaves = kGradThreads / 64;

// Padded d_v: the d_v contraction runs in 16-deep blocks; the row stride adds 4 floats.
__host__ __device__ inline int grads_dv16(int d_v) { return (d_v + 15) & ~15; }
__host__ __device__ inline int grads_dvp(int d_v) { return grads_dv16(d_v) + 4; }

// One chunk per workgroup of 8 waves (two per SIMD, so one wave's MFMA chain overlaps the other's
// LDS reads), every contraction on the fp32 MFMA (16x16x4; a 16-deep k
// block feeds four products, lane group g supplying k = 4 g + s to sub-step s for both operands,
// so each lane reads its A and B values as one 16-byte LDS read each: A operands row-major
// [row][k], B operands transposed [column][k]):
//   dU = P^T dY + (K dW1^T, from the row pass)      lam = Ainv^T dU      dv = diag(beta) lam
//   dP = lower_incl(dY U^T)      Z = lam U^T      dG_ij = -beta_i Z_ij (j < i), symmetrised
// then, per 64-column slice of D (wave w: column tile w % 4, row tile w / 4),
//   dQ = dY W0 + dP K,   M = lam W0,   dK = U dW1 + dP^T Q + (dG + dG^T) K - diag(beta) M.
// One chunk per workgroup, or, with PERSIST (more chunks than workgroups fit at once), the
// resident workgroups walk the chunks with the grid as stride and each chunk's operands load into
// registers during the previous chunk; the next slice's W0, dW1, K and Q load into registers
// while the current slice computes.
template <bool BF16, bool PERSIST>
__global__ __launch_bounds__(kGradThreads) void bwd_chunk_grads_kernel(BwdArgs a) {
    extern __shared__ float lds[];
    const int D = a.D, d_v = a.d_v;
    const int64_t NU = int64_t(a.BH) * a.NC;
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
    float* mkb = bpart + kBC;         // [4][C]: partial sums of M_i . K_i per column tile
    float* W0T = mkb + 4 * kBC;       // [kSlice][SV]: W0 slice transposed
    float* G1T = W0T + kSlice * SV;   // dW1 slice transposed
    float* KT = G1T + kSlice * SV;    // [kSlice][CS]: K slice transposed
    float* QT = KT + kSlice * CS;

    // ---- a chunk's operands in registers.  dy, v: (row c = tid / 64 + 8 m, entry r =
    //      tid % 64); U, K dW1^T: workspace [r][c] units tid + 512 m; Ainv, P, G: [i][j] units
    //      tid + 512 m.  Every lane issues every load (an entry outside the chunk reads the
    //      chunk's first one and is zeroed), so the in-order load counter lets each wait cover
    //      only the loads it needs.
    constexpr int MR = kBC / (kGradThreads / 64);           // 4 rows per thread
    constexpr int MU = kBC * 64 / kGradThreads;              // 4 units (d_v <= 64)
    constexpr int MC = kBC * kBC / kGradThreads;             // 2 units
    const int r = tid & 63;
    float fy[MR], fv[MR], fu[MU], fa[MU], fi[MC], fp[MC], fg[MC], fb;
    auto load_chunk = [&](int64_t uu) {
        const int bhl = static_cast<int>(uu / a.NC), tl = static_cast<int>(uu % a.NC) * kBC;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int c = (tid >> 6) + kGradWaves * m;
            const bool in = tl + c < a.T && r < d_v;
            const int64_t g = (int64_t(bhl) * a.T + tl + (in ? c : 0)) * d_v + (in ? r : 0);
            const float y = load_elem<BF16>(a.dy, g), v = load_elem<BF16>(a.v, g);
            fy[m] = in ? y : 0.0f;
            fv[m] = in ? v : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < MU; ++m) {
            const int e = tid + kGradThreads * m;
            const bool in = e < kBC * d_v;
            const float x = a.ws[a.L.uu + uu * kBC * d_v + (in ? e : 0)];
            const float y = a.ws[a.L.aa + uu * kBC * d_v + (in ? e : 0)];
            fu[m] = in ? x : 0.0f;
            fa[m] = in ? y : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            const int e = tid + kGradThreads * m;
            fi[m] = a.ws[a.L.ai + uu * kBC * kBC + e];
            fp[m] = a.ws[a.L.pm + uu * kBC * kBC + e];
            fg[m] = a.ws[a.L.gm + uu * kBC * kBC + e];
        }
        fb = a.ws[a.L.be + uu * kBC + (tid & (kBC - 1))];
    };

    // Chunks u = blockIdx.x + k gridDim.x (the grid holds the workgroups resident at once); the
    // next chunk's operands load while the current one computes.
    int64_t u = blockIdx.x;
    load_chunk(u);
    for (; u < NU; u += gridDim.x) {
        const int64_t u64 = u;
        const int bh = static_cast<int>(u / a.NC), n = static_cast<int>(u % a.NC);
        const int t0 = n * kBC;
        __syncthreads();                                        // the previous chunk's reads are done
        {
            // zero padding: rows past d_v of the transposed tiles, entries past d_v of the row tiles
            for (int e = tid; e < (DV16 - d_v) * CS; e += kGradThreads) {
                dYT[d_v * CS + e] = 0.0f;
                dUT[d_v * CS + e] = 0.0f;
            }
            for (int e = tid; e < kBC * (SV - d_v); e += kGradThreads) {
                const int c = e / (SV - d_v), rr = d_v + e % (SV - d_v);
                dYs[c * SV + rr] = 0.0f;
                Us[c * SV + rr] = 0.0f;
                Ls[c * SV + rr] = 0.0f;
                Vs[c * SV + rr] = 0.0f;
            }
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const int c = (tid >> 6) + kGradWaves * m;
                if (r < d_v) {
                    dYs[c * SV + r] = fy[m];
                    dYT[r * CS + c] = fy[m];
                    Vs[c * SV + r] = fv[m];
                }
            }
#pragma unroll
            for (int m = 0; m < MU; ++m) {
                const int e = tid + kGradThreads * m, rr = e >> 5, c = e & (kBC - 1);
                if (e < kBC * d_v) {
                    Us[c * SV + rr] = fu[m];
                    dUT[rr * CS + c] = fa[m];                  // K dW1^T, P^T dY added below
                }
            }
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const int e = tid + kGradThreads * m, i = e >> 5, j = e & (kBC - 1);
                AiT[j * CS + i] = fi[m];
                PmT[j * CS + i] = fp[m];
                Gm[i * CS + j] = fg[m];
            }
            if (tid < kBC) be[tid] = fb;
        }
        // ---- operands of the D-wide products, per 64-column slice
        const int64_t CD = int64_t(kBC) * D;
        // staging: W0 and dW1 ([d_v][D] rows) as units e = tid + 512 p of (column nn = e % 64, four
        // consecutive d_v indices from 4 (e / 64)): four global loads down the rows (coalesced along
        // D over the lanes) become one 16-byte LDS store of the transposed row.  K and Q are stored
        // transposed ([D][C]): unit e = (column nn = e / 8, chunk rows 4 (e % 8) .. + 3), one 16-byte
        // load and one 16-byte store.
        constexpr int NW = 16 * kSlice / kGradThreads;      // W0 / dW1 units per thread (d_v <= 64)
        constexpr int NK = (kBC / 4) * kSlice / kGradThreads;   // K / Q units per thread
        f32x4 pw[NW], pg[NW], pk[NK], pq[NK];
        auto fetch = [&](int s0) {
#pragma unroll
            for (int p = 0; p < NW; ++p) {
                const int e = tid + kGradThreads * p, k0 = 4 * (e / kSlice), nn = e % kSlice;
                const bool cin = s0 + nn < D;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bool in = cin && k0 + q < d_v;
                    const int64_t o = (u64 * d_v + (in ? k0 + q : 0)) * D + (in ? s0 + nn : 0);
                    const float x = a.ws[a.L.ws + o], y = a.ws[a.L.gs + o];
                    pw[p][q] = in ? x : 0.0f;
                    pg[p][q] = in ? y : 0.0f;
                }
            }
#pragma unroll
            for (int p = 0; p < NK; ++p) {
                const int e = tid + kGradThreads * p, c0 = 4 * (e & 7), nn = e >> 3;
                const bool in = s0 + nn < D;
                const int64_t o = u64 * CD + int64_t(in ? s0 + nn : 0) * kBC + c0;   // [D][C] tiles
                const f32x4 x = *reinterpret_cast<const f32x4*>(a.ws + a.L.kt + o);
                const f32x4 y = *reinterpret_cast<const f32x4*>(a.ws + a.L.qt + o);
                pk[p] = in ? x : zero4();
                pq[p] = in ? y : zero4();
            }
        };
        auto commit = [&]() {
#pragma unroll
            for (int p = 0; p < NW; ++p) {
                const int e = tid + kGradThreads * p, k0 = 4 * (e / kSlice), nn = e % kSlice;
                if (k0 < DV16) {
                    *reinterpret_cast<f32x4*>(W0T + nn * SV + k0) = pw[p];
                    *reinterpret_cast<f32x4*>(G1T + nn * SV + k0) = pg[p];
                }
            }
#pragma unroll
            for (int p = 0; p < NK; ++p) {
                const int e = tid + kGradThreads * p, c0 = 4 * (e & 7), nn = e >> 3;
                *reinterpret_cast<f32x4*>(KT + nn * CS + c0) = pk[p];
                *reinterpret_cast<f32x4*>(QT + nn * CS + c0) = pq[p];
            }
        };
        fetch(0);
        if constexpr (PERSIST)   // the next chunk (this one again past the end: the load counts stay fixed)
            load_chunk(u + gridDim.x < NU ? u + gridDim.x : u);
        __syncthreads();
        // ---- dU = P^T dY + K dW1^T (tiles (it, rt) of dU, stored transposed)
        for (int tau = wv; tau < 2 * NR; tau += kGradWaves) {
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
        for (int tau = wv; tau < 2 * NR; tau += kGradWaves) {
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
        // ---- dP = lower_incl(dY U^T) (and its transpose) on waves 0 .. 3, Z = lam U^T and dG on
        //      waves 4 .. 7: wave w -> tile (w % 2, (w / 2) % 2)
        {
            const bool zw = wv >= 4;
            const int it = wv & 1, jt = (wv >> 1) & 1;
            const float* A = zw ? Ls : dYs;
            f32x4 acc = zero4();
            for (int kb = 0; kb < DV16; kb += 16) {
                const f32x4 bu = *reinterpret_cast<const f32x4*>(Us + (16 * jt + l16) * SV + kb + 4 * g4);
                const f32x4 av = *reinterpret_cast<const f32x4*>(A + (16 * it + l16) * SV + kb + 4 * g4);
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mfma_f32_k4(av[s], bu[s], acc);
            }
            const int j = 16 * jt + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * it + 4 * g4 + e;
                if (zw) {
                    dG[i * CS + j] = j < i ? -be[i] * acc[e] : 0.0f;    // strict lower part for now
                    Zs[i * CS + j] = acc[e];
                } else {
                    const float p = j <= i ? acc[e] : 0.0f;
                    dP[i * CS + j] = p;
                    dPT[j * CS + i] = p;
                }
            }
        }
        __syncthreads();
        // ---- dG's upper part = its transpose; beta partials lam_i.V_i - sum_{j<i} G_ij Z_ij over
        //      the 16 adjacent lanes of row i
        for (int e = tid; e < kBC * kBC; e += kGradThreads) {
            const int i = e >> 5, j = e & (kBC - 1);
            if (j > i) dG[i * CS + j] = dG[j * CS + i];
        }
        {
            static_assert(kGradThreads == 16 * kBC, "16 lanes per chunk row");
            const int i = tid >> 4, p16 = tid & 15;
            float s = 0.0f;
            for (int r = p16; r < d_v; r += 16) s += Ls[i * SV + r] * Vs[i * SV + r];
            for (int j = p16; j < i; j += 16) s -= Gm[i * CS + j] * Zs[i * CS + j];
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            s += __shfl_xor(s, 4);
            s += __shfl_xor(s, 8);
            if (p16 == 0) bpart[i] = s;
        }

        // wave w: column tile w % 4 of the slice, row tile w / 4 of the chunk
        const int rt = wv >> 2;
        float mkp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        const int ncol = 16 * (wv & 3) + l16;                   // the lane's column in the slice
        // ---- D-wide products per 64-column slice
        for (int s0 = 0; s0 < D; s0 += kSlice) {
            __syncthreads();                                    // the previous slice's reads are done
            commit();
            fetch(s0 + kSlice < D ? s0 + kSlice : s0);          // unconditional: the load counts stay fixed
            __syncthreads();
            f32x4 dq = zero4(), mm = zero4(), dk = zero4();
            // k over d_v
            for (int kb = 0; kb < DV16; kb += 16) {
                const f32x4 bw = *reinterpret_cast<const f32x4*>(W0T + ncol * SV + kb + 4 * g4);
                const f32x4 bg = *reinterpret_cast<const f32x4*>(G1T + ncol * SV + kb + 4 * g4);
                const int ro = (16 * rt + l16) * SV + kb + 4 * g4;
                const f32x4 ady = *reinterpret_cast<const f32x4*>(dYs + ro);
                const f32x4 al = *reinterpret_cast<const f32x4*>(Ls + ro);
                const f32x4 au = *reinterpret_cast<const f32x4*>(Us + ro);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    dq = mfma_f32_k4(ady[s], bw[s], dq);
                    mm = mfma_f32_k4(al[s], bw[s], mm);
                    dk = mfma_f32_k4(au[s], bg[s], dk);
                }
            }
            // k over the chunk rows
#pragma unroll
            for (int kb = 0; kb < kBC; kb += 16) {
                const f32x4 bk = *reinterpret_cast<const f32x4*>(KT + ncol * CS + kb + 4 * g4);
                const f32x4 bq = *reinterpret_cast<const f32x4*>(QT + ncol * CS + kb + 4 * g4);
                const int ro = (16 * rt + l16) * CS + kb + 4 * g4;
                const f32x4 ap = *reinterpret_cast<const f32x4*>(dP + ro);
                const f32x4 apt = *reinterpret_cast<const f32x4*>(dPT + ro);
                const f32x4 ag = *reinterpret_cast<const f32x4*>(dG + ro);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    dq = mfma_f32_k4(ap[s], bk[s], dq);
                    dk = mfma_f32_k4(apt[s], bq[s], dk);
                    dk = mfma_f32_k4(ag[s], bk[s], dk);
                }
            }
            // result slot e: row i = 16 rt + 4 g4 + e, column s0 + ncol
            const int col = s0 + ncol;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * rt + 4 * g4 + e;
                const float m = mm[e];
                mkp[e] += m * KT[ncol * CS + i];
                if (col < D) {
                    a.ws[a.L.wy + u64 * CD + int64_t(i) * D + col] = dk[e] - be[i] * m;
                    a.ws[a.L.qp + u64 * CD + int64_t(i) * D + col] = dq[e];
                }
            }
        }
        // M_i . K_i: the 16 lanes of a row group hold its columns; then the four column tiles
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float s = mkp[e];
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            s += __shfl_xor(s, 4);
            s += __shfl_xor(s, 8);
            if (l16 == 0) mkb[(wv & 3) * kBC + 16 * rt + 4 * g4 + e] = s;
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
        if constexpr (!PERSIST) break;
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

// Each wave owns its slices of xs and dr, so their LDS traffic stays inside the wave, whose
// LDS operations complete in order: a wave barrier (which only keeps the compiler from moving
// the reads above the writes) replaces the workgroup barrier.  Every global load of the vector
// (its D entries of dphi, then x) is issued first.
template <bool BF16>
__global__ __launch_bounds__(64 * kDpfpWaves) void bwd_dpfp_kernel(BwdArgs a) {
    constexpr int KP = 6;                                    // D / 64 <= 6 (D <= 384)
    __shared__ float xs_all[kDpfpWaves][128];
    __shared__ float dr_all[kDpfpWaves][64 * KP];
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
    float dph[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int p = lane + 64 * k;
        dph[k] = (live && p < D) ? dphi[p] : 0.0f;
    }
    // lane < 2 d_k holds relu'd entry m = lane (d_k = 16, 32) or entries lane and lane + 64
    // (d_k = 64); kv0 = x[lane % d_k]
    const float kv0 = (live && lane < two) ? load_elem<BF16>(x, vec * d_k + (lane % d_k)) : 0.0f;
    if (lane < two) xs[lane] = lane < d_k ? relu(kv0) : relu(-kv0);
    if (two > 64) xs[lane + 64] = relu(-kv0);
    __builtin_amdgcn_wave_barrier();
    float S = 0.0f, dot = 0.0f;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int p = lane + 64 * k;
        if (p >= D) break;
        const int i = p / two + 1, j = p % two;
        int src = j - i;
        src += src < 0 ? two : 0;
        const float raw = xs[j] * xs[src];
        S += raw;
        dot += dph[k] * raw;
    }
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) {
        S += __shfl_xor(S, mask);
        dot += __shfl_xor(dot, mask);
    }
    const float den = S + kDpfpEps;
    const float dphin = dot / den;                          // dphi . phi
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int p = lane + 64 * k;
        if (p < D) dr[p] = (dph[k] - dphin) / den;
    }
    __builtin_amdgcn_wave_barrier();
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
        const float gk = (kv0 > 0.0f ? dxv[0] : 0.0f) - (kv0 < 0.0f ? dxv[1] : 0.0f);
        store_elem<BF16>(dx_out, vec * d_k + lane, gk);
    }
}

// ------------------------------------------------------------------------------ host


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
    (void)D;
    return 4 * (bwd_prep_region_a(d_k) + bwd_prep_region_b(d_k) + kBC + kBC * d_v);
}
static int lds_grads_bytes(int d_v) {
    const int SV = grads_dvp(d_v), DV16 = grads_dv16(d_v);
    return 4 * (4 * kBC * SV + 2 * DV16 * kCS + 7 * kBC * kCS + 2 * kBC + 4 * kBC +
                2 * kSlice * SV + 2 * kSlice * kCS);
}

template <int NDW, bool BF16>
static hipError_t launch_states(const BwdArgs& a, hipStream_t stream) {
    const int64_t G = int64_t(a.BH) * ((a.d_v + 15) / 16);
    auto k = bwd_states_kernel<BF16, NDW>;
    const int l = 4 * states_lds_floats(a.D);
    hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(k), l);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(2 * G)), dim3(kStThreads), l, stream, a);
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
    switch ((a.D + 127) / 128) {                 // d-tiles per wave
        case 1: e = launch_states<1, BF16>(a, stream); break;
        case 2: e = launch_states<2, BF16>(a, stream); break;
        case 3: e = launch_states<3, BF16>(a, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || NU == 0) return e;
    // chunk gradients: one chunk per workgroup where all fit at once, else the resident
    // workgroups walk the chunks, each loading its next chunk's operands during the current one
    const int lg = lds_grads_bytes(a.d_v);
    auto kc1 = bwd_chunk_grads_kernel<BF16, false>;
    auto kcp = bwd_chunk_grads_kernel<BF16, true>;
    if ((e = ensure_lds_attr(reinterpret_cast<const void*>(kc1), lg)) != hipSuccess) return e;
    if ((e = ensure_lds_attr(reinterpret_cast<const void*>(kcp), lg)) != hipSuccess) return e;
    unsigned cap = 0;
    if ((e = resident_grid(reinterpret_cast<const void*>(kcp), kGradThreads, lg, INT64_MAX, &cap)) != hipSuccess)
        return e;
    if (NU <= int64_t(cap))
        hipLaunchKernelGGL(kc1, dim3(static_cast<unsigned>(NU)), dim3(kGradThreads), lg, stream, a);
    else
        hipLaunchKernelGGL(kcp, dim3(cap), dim3(kGradThreads), lg, stream, a);
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
