// Chunk-parallel causal forward of the fast-weight delta rule with DPFP, for gfx950.
//
// The recurrence ("Fast Weights Transformer" guide, xdnf.cn/news/308600, sections
// "FastWeightsAttention / update formula" and "... / module structure and source walkthrough"):
//     v_bar_t = W_{t-1} f_t,  W_t = W_{t-1} + beta_t (v_t - v_bar_t) f_t^T,  y_t = W_t g_t
// with f_t = phi(k_t), g_t = phi(q_t) (DPFP, section "DPFP / ...") and beta_t = sigmoid(l_t).
// The lucidrains page ("Deep dive into Fast Weight Attention", section 4.2) evaluates such
// layers chunk by chunk, parallel inside a chunk, passing the memory between chunks; the
// chunked algebra used here is derived from the recurrence itself.  For a chunk of C rows
// starting from memory W (d_v x D), with K = [f_t], Q = [g_t], V = [v_t], beta = diag(beta_t):
//     u_t = beta_t (v_t - W f_t - sum_{s<t} (f_s . f_t) u_s)
//  => (I + beta strict_lower(K K^T)) U = beta (V - K W^T)       (unit lower triangular system)
//     Y = Q W^T + lower_incl(Q K^T) U,    W <- W + U^T K.
// This equals the per-step recurrence exactly in exact arithmetic.
//
// Execution (one workgroup of 4 waves per (b, h, slice of d_v)):
//   A  DPFP of the chunk's k and q rows, one row per DK-lane group: lane j holds k_j and gets
//      the rolled operand from lane (j - i) mod d_k with ds_bpermute (sign flip when the roll
//      crosses the [k, -k] seam).  The raw products are written to LDS as K (row-major and a
//      transposed copy) and Q, in the MFMA operand type (bf16 for bf16 inputs, fp32
//      otherwise); the per-row normalisers 1/(sum + eps) are applied to contraction results
//      instead, so every phi entry costs one multiply.
//   B  MFMA contractions over D: G = K K^T and P = Q K^T (lower triangles), and, per wave,
//      the state products K W^T and Q W^T against the fp32 memory held in registers.
//   C  Inverse of each 16x16 diagonal block of I + beta strict_lower(G) (fp32, per-lane
//      forward substitution).
//   D  Block forward substitution for U on the fp32 MFMA (16x16x4), Y = QW^T + P U, and the
//      state update W^T += K^T U accumulated straight into the memory registers.
// The fp32 memory W^T (D x 16 per v-tile) lives in MFMA accumulator registers for the whole
// sequence.  An accumulator tile holds D[4*(l/16) + r][l%16] in lane l, slot r, which is also
// a valid B operand (and the transpose of an A operand) for a product whose contraction runs
// over those 16 rows, as long as the other operand takes its k-slots in the same order; so W,
// U and the intermediate blocks feed the next MFMA with no data movement.
#include "fwa_common.h"
#include "fwa_internal.h"

#include <type_traits>

namespace fwa {


constexpr int kLiStride = 20;   // floats per row of the diagonal-inverse buffer
constexpr int kRedStride = 17;  // floats per row of the cross-wave reduction buffer

template <bool BF16, int C, int NDPM>
__global__ __launch_bounds__(256, 1) void delta_forward_kernel(FwdArgs a) {
    using LT = std::conditional_t<BF16, u16, float>;  // LDS element type of K, Q and P
    constexpr int NT = C / 16;
    constexpr int NGP = NT * (NT + 1);                 // G and P lower-triangle tiles
    constexpr int MAXTW = (NGP + 3) / 4;               // of those, per wave
    extern __shared__ __attribute__((aligned(16))) char smem[];

    LT* Kc = reinterpret_cast<LT*>(smem + a.off_kc);   // [D][kcs]  K transposed
    LT* Kr = reinterpret_cast<LT*>(smem + a.off_kr);   // [C][krs]  K
    LT* Qr = reinterpret_cast<LT*>(smem + a.off_qr);   // [C][krs]  Q
    float* Ls = reinterpret_cast<float*>(smem + a.off_ls);   // [C][lss] beta*strict_lower(G)
    LT* Ps = reinterpret_cast<LT*>(smem + a.off_ps);          // [C][pss] lower_incl(Q K^T)
    float* Li = reinterpret_cast<float*>(smem + a.off_li);    // [C][20]  diagonal inverses
    float* Red = reinterpret_cast<float*>(smem + a.off_red);  // [4][2][C][17] partials
    float* rhok = reinterpret_cast<float*>(smem + a.off_small);
    float* rhoq = rhok + C;
    float* betas = rhoq + C;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int l16 = l & 15, g4 = l >> 4;
    const int d_k = a.d_k, two_dk = 2 * d_k, nu = a.nu;
    const int D = two_dk * nu;
    const int ND = D / 16;
    const int d_v = a.d_v, T = a.T;

    // Workgroup -> (b*H + h, d_v slice r).  When the grid splits evenly over the 8 XCDs,
    // workgroups of one (b, h) are placed on the same XCD so they share its L2 for k and q.
    int L = blockIdx.x;
    const int G = gridDim.x;
    if ((G & 7) == 0 && (a.BH & 7) == 0) L = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int bh = L / a.R, r = L % a.R;

    const bool has_state = w < a.NVT * a.DP;
    const int vt = w % a.NVT, dp = w / a.NVT;
    const int vbase = (r * a.NVT + vt) * 16;
    const int vcol = vbase + l16;
    const int ndp = a.NDP;
    const int dt0 = dp * ndp;

    // ---- memory W^T tiles of this wave: d-tiles dt0 .. dt0+ndp-1 x v-tile vt (fp32)
    f32x4 Wst[NDPM];
#pragma unroll
    for (int i = 0; i < NDPM; ++i) {
        Wst[i] = zero4();
        if (has_state && i < ndp && a.W0) {
            const float* src = a.W0 + (static_cast<int64_t>(bh) * d_v + vcol) * D +
                               16 * (dt0 + i) + 4 * g4;
            const float4 t4 = *reinterpret_cast<const float4*>(src);
            Wst[i] = f32x4{t4.x, t4.y, t4.z, t4.w};
        }
    }

    const int64_t row0 = static_cast<int64_t>(bh) * T;  // first (b, h, t=0) row
    const int nchunks = (T + C - 1) / C;
    const int rpw = 64 / d_k;                             // DPFP rows per wave pass
    const int jl = l % d_k, grp = l / d_k;
    const int gbase = grp * d_k;

    for (int ch = 0; ch < nchunks; ++ch) {
        const int t0 = ch * C;
        const int Cc = min(C, T - t0);

        // ---------------- A: DPFP rows, beta, and this wave's V tile
        for (int p = 0; p < C / (4 * rpw); ++p) {
            const int t = p * 4 * rpw + w * rpw + grp;
            const bool tv = t < Cc;
            const int64_t gi = (row0 + t0 + t) * d_k + jl;
            const float kv = tv ? load_elem<BF16>(a.k, gi) : 0.0f;
            const float qv = tv ? load_elem<BF16>(a.q, gi) : 0.0f;
            const float ka = relu(kv), kb = relu(-kv), qa = relu(qv), qb = relu(-qv);
            float sk = 0.0f, sq = 0.0f;
            for (int i = 1; i <= nu; ++i) {
                // rolled source position m = (j - i) mod 2 d_k: lane (m mod d_k), negated
                // when m falls in the -k half.
                const int m = ((jl - i) % two_dk + two_dk) % two_dk;
                const int srcl = gbase + (m % d_k);
                const bool neg = m >= d_k;
                const float rk = __int_as_float(
                    __builtin_amdgcn_ds_bpermute(srcl * 4, __float_as_int(kv)));
                const float rq = __int_as_float(
                    __builtin_amdgcn_ds_bpermute(srcl * 4, __float_as_int(qv)));
                const float xk = neg ? -rk : rk, xq = neg ? -rq : rq;
                const float pk1 = ka * relu(xk), pk2 = kb * relu(-xk);
                const float pq1 = qa * relu(xq), pq2 = qb * relu(-xq);
                sk += pk1 + pk2;
                sq += pq1 + pq2;
                const int d1 = (i - 1) * two_dk + jl, d2 = d1 + d_k;
                if constexpr (BF16) {
                    Kr[t * a.krs + d1] = f32_to_bf16_bits(pk1);
                    Kr[t * a.krs + d2] = f32_to_bf16_bits(pk2);
                    Kc[d1 * a.kcs + t] = f32_to_bf16_bits(pk1);
                    Kc[d2 * a.kcs + t] = f32_to_bf16_bits(pk2);
                    Qr[t * a.krs + d1] = f32_to_bf16_bits(pq1);
                    Qr[t * a.krs + d2] = f32_to_bf16_bits(pq2);
                } else {
                    Kr[t * a.krs + d1] = pk1;
                    Kr[t * a.krs + d2] = pk2;
                    Kc[d1 * a.kcs + t] = pk1;
                    Kc[d2 * a.kcs + t] = pk2;
                    Qr[t * a.krs + d1] = pq1;
                    Qr[t * a.krs + d2] = pq2;
                }
            }
            for (int off = d_k / 2; off >= 1; off >>= 1) {
                sk += __shfl_xor(sk, off, d_k);
                sq += __shfl_xor(sq, off, d_k);
            }
            if (jl == 0) {
                rhok[t] = 1.0f / (sk + kDpfpEps);
                rhoq[t] = 1.0f / (sq + kDpfpEps);
            }
        }
        if (tid < C) betas[tid] = tid < Cc ? sigmoid_stable(load_elem<BF16>(a.bl, row0 + t0 + tid))
                                           : 0.0f;
        f32x4 Xv[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tt + 4 * g4 + e;
                Xv[tt][e] = (has_state && t < Cc)
                                ? load_elem<BF16>(a.v, (row0 + t0 + t) * d_v + vcol)
                                : 0.0f;
            }
        }
        __syncthreads();

        // ---------------- B: G, P tiles; K W^T and Q W^T against the memory
        f32x4 gp[MAXTW];
#pragma unroll
        for (int j = 0; j < MAXTW; ++j) {
            gp[j] = zero4();
            const int tix = w + 4 * j;
            if (tix < NGP) {
                const bool isP = tix >= NGP / 2;
                int idx = isP ? tix - NGP / 2 : tix;
                int ta = 0;
                while ((ta + 1) * (ta + 2) / 2 <= idx) ++ta;
                const int tb = idx - ta * (ta + 1) / 2;
                const LT* Arow = (isP ? Qr : Kr) + (16 * ta + l16) * a.krs;
                const LT* Brow = Kr + (16 * tb + l16) * a.krs;
                f32x4 acc = zero4();
                if constexpr (BF16) {
                    for (int kk = 0; kk < D / 32; ++kk) {
                        const bf16x8 av = *reinterpret_cast<const bf16x8*>(Arow + 32 * kk + 8 * g4);
                        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(Brow + 32 * kk + 8 * g4);
                        acc = mfma_bf16_k32(av, bv, acc);
                    }
                } else {
                    for (int kk = 0; kk < D / 16; ++kk) {
                        const float4 av = *reinterpret_cast<const float4*>(Arow + 16 * kk + 4 * g4);
                        const float4 bv = *reinterpret_cast<const float4*>(Brow + 16 * kk + 4 * g4);
                        acc = mfma_f32_k4(av.x, bv.x, acc);
                        acc = mfma_f32_k4(av.y, bv.y, acc);
                        acc = mfma_f32_k4(av.z, bv.z, acc);
                        acc = mfma_f32_k4(av.w, bv.w, acc);
                    }
                }
                gp[j] = acc;
            }
        }
        f32x4 S1[NT], QW[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) { S1[tt] = zero4(); QW[tt] = zero4(); }
        if (has_state) {
            if constexpr (BF16) {
#pragma unroll
                for (int i = 0; i < NDPM; i += 2) {
                    if (i < ndp) {
                        const int dcol = 16 * (dt0 + i) + 4 * g4;
                        bf16x8 bw;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            bw[e] = static_cast<__bf16>(Wst[i][e]);
                            bw[4 + e] = static_cast<__bf16>(Wst[i + 1][e]);
                        }
#pragma unroll
                        for (int tt = 0; tt < NT; ++tt) {
                            const LT* kr = Kr + (16 * tt + l16) * a.krs + dcol;
                            const LT* qr = Qr + (16 * tt + l16) * a.krs + dcol;
                            const bf16x4 k0 = *reinterpret_cast<const bf16x4*>(kr);
                            const bf16x4 k1 = *reinterpret_cast<const bf16x4*>(kr + 16);
                            const bf16x4 q0 = *reinterpret_cast<const bf16x4*>(qr);
                            const bf16x4 q1 = *reinterpret_cast<const bf16x4*>(qr + 16);
                            S1[tt] = mfma_bf16_k32(__builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                   bw, S1[tt]);
                            QW[tt] = mfma_bf16_k32(__builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                   bw, QW[tt]);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < NDPM; ++i) {
                    if (i < ndp) {
                        const int dcol = 16 * (dt0 + i) + 4 * g4;
#pragma unroll
                        for (int tt = 0; tt < NT; ++tt) {
                            const float4 kv4 = *reinterpret_cast<const float4*>(
                                Kr + (16 * tt + l16) * a.krs + dcol);
                            const float4 qv4 = *reinterpret_cast<const float4*>(
                                Qr + (16 * tt + l16) * a.krs + dcol);
                            S1[tt] = mfma_f32_k4(kv4.x, Wst[i][0], S1[tt]);
                            S1[tt] = mfma_f32_k4(kv4.y, Wst[i][1], S1[tt]);
                            S1[tt] = mfma_f32_k4(kv4.z, Wst[i][2], S1[tt]);
                            S1[tt] = mfma_f32_k4(kv4.w, Wst[i][3], S1[tt]);
                            QW[tt] = mfma_f32_k4(qv4.x, Wst[i][0], QW[tt]);
                            QW[tt] = mfma_f32_k4(qv4.y, Wst[i][1], QW[tt]);
                            QW[tt] = mfma_f32_k4(qv4.z, Wst[i][2], QW[tt]);
                            QW[tt] = mfma_f32_k4(qv4.w, Wst[i][3], QW[tt]);
                        }
                    }
                }
            }
        }
        __syncthreads();  // K (row-major) and Q are dead from here; their space is reused

        // ---------------- B': scaled G and P to LDS, state partials to the reduction buffer
#pragma unroll
        for (int j = 0; j < MAXTW; ++j) {
            const int tix = w + 4 * j;
            if (tix < NGP) {
                const bool isP = tix >= NGP / 2;
                int idx = isP ? tix - NGP / 2 : tix;
                int ta = 0;
                while ((ta + 1) * (ta + 2) / 2 <= idx) ++ta;
                const int tb = idx - ta * (ta + 1) / 2;
                const int s = 16 * tb + l16;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * ta + 4 * g4 + e;
                    if (isP) {
                        const float val = s <= t ? rhoq[t] * rhok[s] * gp[j][e] : 0.0f;
                        if constexpr (BF16) Ps[t * a.pss + s] = f32_to_bf16_bits(val);
                        else Ps[t * a.pss + s] = val;
                    } else {
                        Ls[t * a.lss + s] = s < t ? betas[t] * rhok[t] * rhok[s] * gp[j][e] : 0.0f;
                    }
                }
            }
        }
        if (has_state && a.DP > 1) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * tt + 4 * g4 + e;
                    Red[((w * 2 + 0) * C + t) * kRedStride + l16] = S1[tt][e];
                    Red[((w * 2 + 1) * C + t) * kRedStride + l16] = QW[tt][e];
                }
            }
        }
        __syncthreads();

        // ---------------- C: diagonal-block inverses; reduce the state partials
        if (tid < C) {
            const int ab = tid >> 4, sc = tid & 15;
            const float* Lb = Ls + (16 * ab) * a.lss + 16 * ab;
            float xcol[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                float acc = 0.0f;
#pragma unroll
                for (int w2 = 0; w2 < u; ++w2) acc += Lb[u * a.lss + w2] * xcol[w2];
                xcol[u] = (u == sc) ? 1.0f : (u < sc ? 0.0f : -acc);
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) Li[(16 * ab + u) * kLiStride + sc] = xcol[u];
        }
        f32x4 X[NT];
        if (has_state) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                if (a.DP > 1) {
                    f32x4 s1 = zero4(), qw = zero4();
                    for (int pp = 0; pp < a.DP; ++pp) {
                        const int ww = vt + a.NVT * pp;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int t = 16 * tt + 4 * g4 + e;
                            s1[e] += Red[((ww * 2 + 0) * C + t) * kRedStride + l16];
                            qw[e] += Red[((ww * 2 + 1) * C + t) * kRedStride + l16];
                        }
                    }
                    S1[tt] = s1;
                    QW[tt] = qw;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * tt + 4 * g4 + e;
                    X[tt][e] = Xv[tt][e] - rhok[t] * S1[tt][e];
                    QW[tt][e] *= rhoq[t];
                }
            }
        }
        __syncthreads();

        // ---------------- D: U by block substitution, Y, and the memory update
        if (has_state) {
            f32x4 U[NT];
#pragma unroll
            for (int ta = 0; ta < NT; ++ta) {
                f32x4 z;
#pragma unroll
                for (int e = 0; e < 4; ++e) z[e] = betas[16 * ta + 4 * g4 + e] * X[ta][e];
                f32x4 acc = zero4();
#pragma unroll
                for (int tb = 0; tb < ta; ++tb) {
                    const float4 l4 = *reinterpret_cast<const float4*>(
                        Ls + (16 * ta + l16) * a.lss + 16 * tb + 4 * g4);
                    acc = mfma_f32_k4(l4.x, U[tb][0], acc);
                    acc = mfma_f32_k4(l4.y, U[tb][1], acc);
                    acc = mfma_f32_k4(l4.z, U[tb][2], acc);
                    acc = mfma_f32_k4(l4.w, U[tb][3], acc);
                }
                z -= acc;
                const float4 i4 = *reinterpret_cast<const float4*>(
                    Li + (16 * ta + l16) * kLiStride + 4 * g4);
                f32x4 u = zero4();
                u = mfma_f32_k4(i4.x, z[0], u);
                u = mfma_f32_k4(i4.y, z[1], u);
                u = mfma_f32_k4(i4.z, z[2], u);
                u = mfma_f32_k4(i4.w, z[3], u);
                U[ta] = u;
            }
            // Y rows of chunk tiles ta = dp, dp + DP, ...
#pragma unroll
            for (int ta = 0; ta < NT; ++ta) {
                if (ta % a.DP != dp) continue;
                f32x4 acc = QW[ta];
                if constexpr (BF16) {
#pragma unroll
                    for (int tb = 0; tb <= ta; tb += 2) {
                        const LT* prow = Ps + (16 * ta + l16) * a.pss + 16 * tb + 4 * g4;
                        const bf16x4 p0 = *reinterpret_cast<const bf16x4*>(prow);
                        bf16x4 p1;
                        bf16x8 bu;
                        if (tb + 1 <= ta) {
                            p1 = *reinterpret_cast<const bf16x4*>(prow + 16);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) p1[e] = static_cast<__bf16>(0.0f);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            bu[e] = static_cast<__bf16>(U[tb][e]);
                            bu[4 + e] = static_cast<__bf16>(tb + 1 <= ta ? U[tb + 1 < NT ? tb + 1 : tb][e] : 0.0f);
                        }
                        acc = mfma_bf16_k32(__builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7),
                                            bu, acc);
                    }
                } else {
#pragma unroll
                    for (int tb = 0; tb <= ta; ++tb) {
                        const float4 p4 = *reinterpret_cast<const float4*>(
                            Ps + (16 * ta + l16) * a.pss + 16 * tb + 4 * g4);
                        acc = mfma_f32_k4(p4.x, U[tb][0], acc);
                        acc = mfma_f32_k4(p4.y, U[tb][1], acc);
                        acc = mfma_f32_k4(p4.z, U[tb][2], acc);
                        acc = mfma_f32_k4(p4.w, U[tb][3], acc);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * ta + 4 * g4 + e;
                    if (t < Cc) store_elem<BF16>(a.y, (row0 + t0 + t) * d_v + vcol, acc[e]);
                }
            }
            // W^T += K^T (rho_k U): rows of U scaled by the key normalisers
#pragma unroll
            for (int tb = 0; tb < NT; ++tb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) U[tb][e] *= rhok[16 * tb + 4 * g4 + e];
            }
            if constexpr (BF16) {
#pragma unroll
                for (int tb = 0; tb < NT; tb += 2) {
                    bf16x8 bu;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bu[e] = static_cast<__bf16>(U[tb][e]);
                        bu[4 + e] = static_cast<__bf16>(tb + 1 < NT ? U[tb + 1 < NT ? tb + 1 : tb][e] : 0.0f);
                    }
#pragma unroll
                    for (int i = 0; i < NDPM; ++i) {
                        if (i < ndp) {
                            const LT* kc = Kc + (16 * (dt0 + i) + l16) * a.kcs + 16 * tb + 4 * g4;
                            const bf16x4 c0 = *reinterpret_cast<const bf16x4*>(kc);
                            bf16x4 c1;
                            if (tb + 1 < NT) {
                                c1 = *reinterpret_cast<const bf16x4*>(kc + 16);
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e) c1[e] = static_cast<__bf16>(0.0f);
                            }
                            Wst[i] = mfma_bf16_k32(__builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                   bu, Wst[i]);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int tb = 0; tb < NT; ++tb) {
#pragma unroll
                    for (int i = 0; i < NDPM; ++i) {
                        if (i < ndp) {
                            const float4 c4 = *reinterpret_cast<const float4*>(
                                Kc + (16 * (dt0 + i) + l16) * a.kcs + 16 * tb + 4 * g4);
                            Wst[i] = mfma_f32_k4(c4.x, U[tb][0], Wst[i]);
                            Wst[i] = mfma_f32_k4(c4.y, U[tb][1], Wst[i]);
                            Wst[i] = mfma_f32_k4(c4.z, U[tb][2], Wst[i]);
                            Wst[i] = mfma_f32_k4(c4.w, U[tb][3], Wst[i]);
                        }
                    }
                }
            }
        }
        __syncthreads();  // every LDS buffer is rewritten by the next chunk
    }

    if (has_state && a.Wf) {
#pragma unroll
        for (int i = 0; i < NDPM; ++i) {
            if (i < ndp) {
                float* dst = a.Wf + (static_cast<int64_t>(bh) * d_v + vcol) * D + 16 * (dt0 + i) +
                             4 * g4;
                *reinterpret_cast<float4*>(dst) = make_float4(Wst[i][0], Wst[i][1], Wst[i][2], Wst[i][3]);
            }
        }
    }
}

// ------------------------------------------------------------------ host-side planning

static int align16(int x) { return (x + 15) & ~15; }


constexpr int kMaxLds = 160 * 1024;

// Chooses the d_v split and the LDS layout; returns false when the shape does not fit.
bool plan_forward(int BH, int d_k, int d_v, int nu, int C, bool bf16, FwdPlan* plan) {
    const int D = 2 * d_k * nu;
    if (D % 32 != 0 || d_v % 16 != 0 || D > 512) return false;
    const int ND = D / 16, NVT_total = d_v / 16;
    const int pair = bf16 ? 2 : 1;
    const int es = bf16 ? 2 : 4;
    // Candidate splits: fewest workgroups per (b, h) that still give >= 256 workgroups.
    int R0 = NVT_total > 4 ? NVT_total / 4 : 1;
    if (NVT_total % R0) return false;
    for (int R = R0; R <= NVT_total; R *= 2) {
        if (NVT_total % R) continue;
        const int NVT = NVT_total / R;
        if (NVT > 4) continue;
        const bool enough = static_cast<int64_t>(BH) * R >= 256 || R == NVT_total;
        if (!enough) continue;
        for (int DP = 4 / NVT; DP >= 1; DP /= 2) {
            if (ND % (DP * pair)) continue;
            const int NDP = ND / DP;
            if (NDP > 32) continue;
            FwdArgs fa = {};
            fa.kcs = C + 4;
            fa.krs = bf16 ? D + 8 : D + 4;
            fa.lss = C + 4;
            fa.pss = C + 4;
            int off = 0;
            fa.off_kc = off;
            off = align16(off + D * fa.kcs * es);
            const int ustart = off;
            fa.off_kr = ustart;
            fa.off_qr = align16(fa.off_kr + C * fa.krs * es);
            const int uend1 = align16(fa.off_qr + C * fa.krs * es);
            fa.off_ls = ustart;
            fa.off_ps = align16(fa.off_ls + C * fa.lss * 4);
            fa.off_li = align16(fa.off_ps + C * fa.pss * es);
            fa.off_red = align16(fa.off_li + C * kLiStride * 4);
            const int uend2 = align16(fa.off_red + (DP > 1 ? 4 * 2 * C * kRedStride * 4 : 0));
            off = uend1 > uend2 ? uend1 : uend2;
            fa.off_small = off;
            off = align16(off + 3 * C * 4);
            if (off > kMaxLds) continue;
            fa.R = R;
            fa.NVT = NVT;
            fa.DP = DP;
            fa.NDP = NDP;
            plan->R = R;
            plan->NVT = NVT;
            plan->DP = DP;
            plan->NDP = NDP;
            plan->NDPM = NDP <= 8 ? 8 : 32;
            plan->args = fa;
            plan->lds_bytes = off;
            return true;
        }
    }
    return false;
}

template <bool BF16, int C, int NDPM>
static hipError_t launch_fwd_t(const FwdPlan& p, int BH, hipStream_t stream) {
    auto kern = delta_forward_kernel<BF16, C, NDPM>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(BH) * p.R)), block(256);
    hipLaunchKernelGGL(kern, grid, block, p.lds_bytes, stream, p.args);
    return hipGetLastError();
}

hipError_t launch_delta_forward(const FwdPlan& plan_in, const void* q, const void* k,
                                const void* v, const void* bl, const float* W0, void* y,
                                float* Wf, int BH, int H, int T, int d_k, int d_v, int nu, int C,
                                bool bf16, hipStream_t stream) {
    FwdPlan p = plan_in;
    FwdArgs& a = p.args;
    a.q = q; a.k = k; a.v = v; a.bl = bl; a.W0 = W0; a.y = y; a.Wf = Wf;
    a.BH = BH; a.H = H; a.T = T; a.d_k = d_k; a.d_v = d_v; a.nu = nu;
#define FWA_FWD_CASE(BF, CC, NM)                                                     \
    if (bf16 == BF && C == CC && p.NDPM == NM) return launch_fwd_t<BF, CC, NM>(p, BH, stream);
    FWA_FWD_CASE(false, 16, 8) FWA_FWD_CASE(false, 16, 32)
    FWA_FWD_CASE(false, 32, 8) FWA_FWD_CASE(false, 32, 32)
    FWA_FWD_CASE(false, 64, 8) FWA_FWD_CASE(false, 64, 32)
    FWA_FWD_CASE(false, 128, 8) FWA_FWD_CASE(false, 128, 32)
    FWA_FWD_CASE(true, 16, 8) FWA_FWD_CASE(true, 16, 32)
    FWA_FWD_CASE(true, 32, 8) FWA_FWD_CASE(true, 32, 32)
    FWA_FWD_CASE(true, 64, 8) FWA_FWD_CASE(true, 64, 32)
    FWA_FWD_CASE(true, 128, 8) FWA_FWD_CASE(true, 128, 32)
#undef FWA_FWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace fwa
