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
#pragma once

#include "fwa_common.h"
#include "fwa_internal.h"

#include <type_traits>

namespace fwa {


constexpr int kLiStride = 20;   // floats per row of the diagonal-inverse buffer

// Sum of v over the d_k-lane group of lane l (d_k in {16, 32, 64}), in every lane of the group:
// rotations inside each 16-lane row (DPP), then the row sums combined with readlane.
__device__ __forceinline__ float row_sum16(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));
    return v;
}

__device__ __forceinline__ float group_sum(float v, int d_k, int l) {
    const float r = row_sum16(v);
    if (d_k == 16) return r;
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 48));
    if (d_k == 32) return l < 32 ? r0 + r1 : r2 + r3;
    return (r0 + r1) + (r2 + r3);
}

// Raw DPFP products of one row (lane jl of a d_k-lane group holds k_jl and q_jl) for every
// shift, written to the row-major K and Q tiles; returns the row sums through sk, sq.  With a
// compile-time NU all rolled operands are fetched (ds_bpermute) before any LDS write, so the
// writes never sit in front of a permute the lane is waiting for.
template <typename LT, int NU>
__device__ __forceinline__ void dpfp_row(float kv, float qv, int nu, int jl, int gbase, int d_k,
                                         LT* krow, LT* qrow, float& sk, float& sq) {
    const int two_dk = 2 * d_k;
    const float ka = relu(kv), kb = relu(-kv), qa = relu(qv), qb = relu(-qv);
    auto emit = [&](int i, float xk, float xq) {
        const float pk1 = ka * relu(xk), pk2 = kb * relu(-xk);
        const float pq1 = qa * relu(xq), pq2 = qb * relu(-xq);
        sk += pk1 + pk2;
        sq += pq1 + pq2;
        const int o1 = (i - 1) * two_dk;
        krow[o1] = from_f32<LT>(pk1);
        krow[o1 + d_k] = from_f32<LT>(pk2);
        qrow[o1] = from_f32<LT>(pq1);
        qrow[o1 + d_k] = from_f32<LT>(pq2);
    };
    // rolled source position m = (j - i) mod 2 d_k (d_k is a power of two): lane (m mod d_k)
    // of the row's group, negated when m falls in the -k half.
    auto fetch = [&](int i, float& xk, float& xq) {
        const int m = (jl - i) & (two_dk - 1);
        const int src4 = (gbase + (m & (d_k - 1))) << 2;
        const float sgn = (m & d_k) ? -1.0f : 1.0f;
        xk = sgn * __int_as_float(__builtin_amdgcn_ds_bpermute(src4, __float_as_int(kv)));
        xq = sgn * __int_as_float(__builtin_amdgcn_ds_bpermute(src4, __float_as_int(qv)));
    };
    if constexpr (NU > 0) {
        float xk[NU], xq[NU];
#pragma unroll
        for (int i = 1; i <= NU; ++i) fetch(i, xk[i - 1], xq[i - 1]);
#pragma unroll
        for (int i = 1; i <= NU; ++i) emit(i, xk[i - 1], xq[i - 1]);
    } else {
        for (int i = 1; i <= nu; ++i) {
            float xk, xq;
            fetch(i, xk, xq);
            emit(i, xk, xq);
        }
    }
}

template <bool BF16, int C, int NDPM>
__global__ __launch_bounds__(256, 1) void delta_forward_kernel(FwdArgs a) {
    using LT = std::conditional_t<BF16, u16, float>;  // LDS element type of K, Q and P
    constexpr int NT = C / 16;
    constexpr int NGP = NT * (NT + 1);                 // G and P lower-triangle tiles
    constexpr int MAXTW = (NGP + 3) / 4;               // of those, per wave
    constexpr int RS = C + 4;                          // row stride of the partials buffer
    extern __shared__ __attribute__((aligned(16))) char smem[];

    LT* Kr = reinterpret_cast<LT*>(smem + a.off_kr);   // [C][krs]  K (lives through D)
    LT* Qr = reinterpret_cast<LT*>(smem + a.off_qr);   // [C][krs]  Q (dead after B)
    using ITs = std::conditional_t<BF16, u16, float>;
    ITs* Xk = reinterpret_cast<ITs*>(smem + a.off_xs);              // [C][d_k] raw k rows
    ITs* Xq = Xk + C * a.d_k;                                       // [C][d_k] raw q rows
    float* Ls = reinterpret_cast<float*>(smem + a.off_ls);   // [C][lss] beta*strict_lower(G)
    LT* Ps = reinterpret_cast<LT*>(smem + a.off_ps);          // [C][pss] lower_incl(Q K^T)
    float* Li = reinterpret_cast<float*>(smem + a.off_li);    // [C][20]  diagonal inverses
    float* Red = reinterpret_cast<float*>(smem + a.off_red);  // [4][2][16][C+4] partials
    float* rhok = reinterpret_cast<float*>(smem + a.off_small);
    float* rhoq = rhok + C;
    float* betas = rhoq + C;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int l16 = l & 15, g4 = l >> 4;
    const int d_k = a.d_k, two_dk = 2 * d_k, nu = a.nu;
    const int D = two_dk * nu;
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
    // Per-(b, h) base pointers; offsets inside one (b, h) fit in 32 bits (checked on the host).
    using IT = std::conditional_t<BF16, u16, float>;  // storage type of q, k, v, beta_logit, y
    const IT* kB = static_cast<const IT*>(a.k) + row0 * d_k;
    const IT* qB = static_cast<const IT*>(a.q) + row0 * d_k;
    const IT* vB = static_cast<const IT*>(a.v) + row0 * d_v;
    const IT* bB = static_cast<const IT*>(a.bl) + row0;
    IT* yB = static_cast<IT*>(a.y) + row0 * d_v;
    const int nchunks = (T + C - 1) / C;
    const int rpw = 64 / d_k;                             // DPFP rows per wave pass
    const int jl = l % d_k, grp = l / d_k;
    const int gbase = grp * d_k;

    // The next chunk's raw inputs are fetched into registers while the current chunk is
    // being computed, so no global-memory latency sits on the serial chain over chunks.
    const int npass = C / (4 * rpw);
    // The next chunk's k and q rows form two contiguous blocks of C*d_k elements; each thread
    // fetches its share as 16-byte units into registers while the current chunk computes.
    // Loads are branch-free: a unit past the sequence end reads unit 0 of the chunk (always in
    // range) and is zeroed when it is staged, so no wait sits next to the loads.
    constexpr int NRM = C / 16;                      // units per thread at d_k = 64, fp32
    const int ubytes = d_k * static_cast<int>(sizeof(IT));  // bytes per row
    const int nunits = C * ubytes / 16;              // 16-byte units per chunk block
    const int nr = (nunits + 255) / 256;
    uint4 kraw[NRM], qraw[NRM];
    IT blpre = IT(0);
    auto prefetch = [&](int chn) {
        const int tn0 = chn * C;
        const int Cn = min(C, T - tn0);
        const char* kc = reinterpret_cast<const char*>(kB + static_cast<int64_t>(tn0) * d_k);
        const char* qc = reinterpret_cast<const char*>(qB + static_cast<int64_t>(tn0) * d_k);
#pragma unroll
        for (int i = 0; i < NRM; ++i) {
            if (i < nr) {
                const int u = tid + 256 * i;
                const bool ok = u < nunits && (u * 16) / ubytes < Cn;
                const int off = ok ? u * 16 : 0;
                kraw[i] = *reinterpret_cast<const uint4*>(kc + off);
                qraw[i] = *reinterpret_cast<const uint4*>(qc + off);
            }
        }
        blpre = bB[tn0 + min(tid, Cn - 1)];
    };
    if (nchunks > 0) prefetch(0);

    for (int ch = 0; ch < nchunks; ++ch) {
        const int t0 = ch * C;
        const int Cc = min(C, T - t0);

        // ---------------- A: DPFP rows, beta, and this wave's V tile (consumed in C)
        f32x4 Xv[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tt + 4 * g4 + e;
                const bool ok = has_state && t < Cc;
                const float vv = to_f32(vB[(t0 + (ok ? t : 0)) * d_v + vcol]);
                Xv[tt][e] = ok ? vv : 0.0f;
            }
        }
        // Stage this chunk's raw rows (zeros past the sequence end) for the DPFP passes.
#pragma unroll
        for (int i = 0; i < NRM; ++i) {
            if (i < nr) {
                const int u = tid + 256 * i;
                if (u < nunits) {
                    const uint32_t m = (u * 16) / ubytes < Cc ? 0xffffffffu : 0u;
                    const uint4 kr4 = kraw[i], qr4 = qraw[i];
                    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Xk) + u * 16) =
                        make_uint4(kr4.x & m, kr4.y & m, kr4.z & m, kr4.w & m);
                    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Xq) + u * 16) =
                        make_uint4(qr4.x & m, qr4.y & m, qr4.z & m, qr4.w & m);
                }
            }
        }
        if (tid < C) betas[tid] = tid < Cc ? sigmoid_stable(to_f32(blpre)) : 0.0f;
        if (ch + 1 < nchunks) prefetch(ch + 1);
        __syncthreads();

        // One row per d_k-lane group and pass; the shift count is a compile-time constant for
        // nu <= 4 so each row's permutes are all issued before its writes.
        auto dpfp_passes = [&](auto nu_tag) {
            constexpr int NU = decltype(nu_tag)::value;
#pragma unroll 4
            for (int p = 0; p < npass; ++p) {
                const int t = p * 4 * rpw + w * rpw + grp;
                const float kv = to_f32(Xk[t * d_k + jl]), qv = to_f32(Xq[t * d_k + jl]);
                float sk = 0.0f, sq = 0.0f;
                dpfp_row<LT, NU>(kv, qv, nu, jl, gbase, d_k, Kr + t * a.krs + jl,
                                 Qr + t * a.krs + jl, sk, sq);
                sk = group_sum(sk, d_k, l);
                sq = group_sum(sq, d_k, l);
                if (jl == 0) {
                    rhok[t] = __builtin_amdgcn_rcpf(sk + kDpfpEps);
                    rhoq[t] = __builtin_amdgcn_rcpf(sq + kDpfpEps);
                }
            }
        };
        switch (nu) {
            case 1: dpfp_passes(std::integral_constant<int, 1>{}); break;
            case 2: dpfp_passes(std::integral_constant<int, 2>{}); break;
            case 3: dpfp_passes(std::integral_constant<int, 3>{}); break;
            case 4: dpfp_passes(std::integral_constant<int, 4>{}); break;
            default: dpfp_passes(std::integral_constant<int, 0>{}); break;
        }
        __syncthreads();

        // ---------------- B: G, P tiles; K W^T and Q W^T against the memory
        // Tiles w, w+4, ... of the list [G tiles (ta >= tb)..., P tiles (ta >= tb)...]; the
        // k-step loop is outside so the wave's independent tiles interleave on the MFMA pipe.
        f32x4 gp[MAXTW];
        const LT* Ap[MAXTW];
        const LT* Bp[MAXTW];
#pragma unroll
        for (int j = 0; j < MAXTW; ++j) {
            gp[j] = zero4();
            const int tix = min(w + 4 * j, NGP - 1);
            const bool isP = tix >= NGP / 2;
            const int idx = isP ? tix - NGP / 2 : tix;
            int ta = 0;
            while ((ta + 1) * (ta + 2) / 2 <= idx) ++ta;
            const int tb = idx - ta * (ta + 1) / 2;
            Ap[j] = (isP ? Qr : Kr) + (16 * ta + l16) * a.krs;
            Bp[j] = Kr + (16 * tb + l16) * a.krs;
        }
        if constexpr (BF16) {
#pragma unroll 2
            for (int kk = 0; kk < D / 32; ++kk) {
#pragma unroll
                for (int j = 0; j < MAXTW; ++j) {
                    if (w + 4 * j < NGP) {
                        const bf16x8 av = *reinterpret_cast<const bf16x8*>(Ap[j] + 32 * kk + 8 * g4);
                        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(Bp[j] + 32 * kk + 8 * g4);
                        gp[j] = mfma_bf16_k32(av, bv, gp[j]);
                    }
                }
            }
        } else {
            for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
                for (int j = 0; j < MAXTW; ++j) {
                    if (w + 4 * j < NGP) {
                        const float4 av = *reinterpret_cast<const float4*>(Ap[j] + 16 * kk + 4 * g4);
                        const float4 bv = *reinterpret_cast<const float4*>(Bp[j] + 16 * kk + 4 * g4);
                        gp[j] = mfma_f32_k4(av.x, bv.x, gp[j]);
                        gp[j] = mfma_f32_k4(av.y, bv.y, gp[j]);
                        gp[j] = mfma_f32_k4(av.z, bv.z, gp[j]);
                        gp[j] = mfma_f32_k4(av.w, bv.w, gp[j]);
                    }
                }
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
        __syncthreads();  // Q is dead from here; its space is reused

        // ---------------- B': scaled G and P to LDS, state partials to the reduction buffer
#pragma unroll
        for (int j = 0; j < MAXTW; ++j) {
            const int tix = w + 4 * j;
            if (tix < NGP) {
                const bool isP = tix >= NGP / 2;
                const int idx = isP ? tix - NGP / 2 : tix;
                int ta = 0;
                while ((ta + 1) * (ta + 2) / 2 <= idx) ++ta;
                const int tb = idx - ta * (ta + 1) / 2;
                const int s = 16 * tb + l16, tr = 16 * ta + 4 * g4;
                const float rks = rhok[s];
                if (isP) {
                    const f32x4 rq = *reinterpret_cast<const f32x4*>(rhoq + tr);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float val = s <= tr + e ? rq[e] * rks * gp[j][e] : 0.0f;
                        Ps[(tr + e) * a.pss + s] = from_f32<LT>(val);
                    }
                } else {
                    const f32x4 rk = *reinterpret_cast<const f32x4*>(rhok + tr);
                    const f32x4 bt = *reinterpret_cast<const f32x4*>(betas + tr);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Ls[(tr + e) * a.lss + s] = s < tr + e ? bt[e] * rk[e] * rks * gp[j][e] : 0.0f;
                }
            }
        }
        if (has_state && a.DP > 1) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                *reinterpret_cast<f32x4*>(Red + ((w * 2 + 0) * 16 + l16) * RS + 16 * tt + 4 * g4) = S1[tt];
                *reinterpret_cast<f32x4*>(Red + ((w * 2 + 1) * 16 + l16) * RS + 16 * tt + 4 * g4) = QW[tt];
            }
        }
        __syncthreads();

        // ---------------- C: diagonal-block inverses; reduce the state partials
        if (tid < C) {
            // Column sc of the inverse of the unit lower 16x16 block ab; each row's dot product
            // is split over four partial sums to keep the dependency chains short.
            const int ab = tid >> 4, sc = tid & 15;
            const float* Lb = Ls + (16 * ab) * a.lss + 16 * ab;
            float xcol[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                f32x4 rw[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    rw[q4] = (4 * q4 < u) ? *reinterpret_cast<const f32x4*>(Lb + u * a.lss + 4 * q4)
                                          : zero4();
                float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int w2 = 0; w2 < u; ++w2) acc[w2 & 3] += rw[w2 >> 2][w2 & 3] * xcol[w2];
                const float tot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
                xcol[u] = (u == sc) ? 1.0f : (u < sc ? 0.0f : -tot);
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
                        s1 += *reinterpret_cast<const f32x4*>(Red + ((ww * 2 + 0) * 16 + l16) * RS + 16 * tt + 4 * g4);
                        qw += *reinterpret_cast<const f32x4*>(Red + ((ww * 2 + 1) * 16 + l16) * RS + 16 * tt + 4 * g4);
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
                    if (t < Cc) yB[(t0 + t) * d_v + vcol] = from_f32<IT>(acc[e]);
                }
            }
            // W^T += K^T (rho_k U): rows of U scaled by the key normalisers
#pragma unroll
            for (int tb = 0; tb < NT; ++tb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) U[tb][e] *= rhok[16 * tb + 4 * g4 + e];
            }
            // A operand K^T[d][t]: lane l16 of group g4 needs K[t][16 dt + l16] for the four
            // rows t = 16 tb + 4 g4 + 0..3 (and the same for tile tb + 1).  For bf16 one
            // ds_read_b64_tr_b16 delivers exactly that from the row-major tile when lane j of
            // the group addresses K[16 tb + 4 g4 + j/4][16 dt + 4 (j%4)].
            if constexpr (BF16) {
#pragma unroll
                for (int tb = 0; tb < NT; tb += 2) {
                    bf16x8 bu;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bu[e] = static_cast<__bf16>(U[tb][e]);
                        bu[4 + e] = static_cast<__bf16>(tb + 1 < NT ? U[tb + 1 < NT ? tb + 1 : tb][e] : 0.0f);
                    }
                    const LT* kt = Kr + (16 * tb + 4 * g4 + (l16 >> 2)) * a.krs + 4 * (l16 & 3);
#pragma unroll
                    for (int i = 0; i < NDPM; ++i) {
                        if (i < ndp) {
                            const LT* kc = kt + 16 * (dt0 + i);
                            const bf16x4 c0 = lds_read_tr_b16x4(kc);
                            bf16x4 c1;
                            if (tb + 1 < NT) {
                                c1 = lds_read_tr_b16x4(kc + 16 * a.krs);
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
                    const LT* kt = Kr + (16 * tb + 4 * g4) * a.krs + l16;
#pragma unroll
                    for (int i = 0; i < NDPM; ++i) {
                        if (i < ndp) {
                            const LT* kc = kt + 16 * (dt0 + i);
                            Wst[i] = mfma_f32_k4(kc[0], U[tb][0], Wst[i]);
                            Wst[i] = mfma_f32_k4(kc[a.krs], U[tb][1], Wst[i]);
                            Wst[i] = mfma_f32_k4(kc[2 * a.krs], U[tb][2], Wst[i]);
                            Wst[i] = mfma_f32_k4(kc[3 * a.krs], U[tb][3], Wst[i]);
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

// Memory-tile capacities (16-row d-tiles of W^T per wave) a kernel is instantiated with; the
// plan picks the smallest capacity that holds a wave's share of D.  Chunks of 128 rows only fit
// the LDS for small D, so they get the small capacities only.
inline int fwd_ndpm_bucket(int ndp, int C) {
    const int caps[] = {2, 4, 8, 12, 16, 24, 32};
    for (int c : caps)
        if (ndp <= c && (C < 128 || c <= 8)) return c;
    return 0;
}

template <bool BF16, int C, int NDPM>
hipError_t launch_fwd_t(const FwdPlan& p, int BH, hipStream_t stream) {
    auto kern = delta_forward_kernel<BF16, C, NDPM>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(BH) * p.R)), block(256);
    hipLaunchKernelGGL(kern, grid, block, p.lds_bytes, stream, p.args);
    return hipGetLastError();
}

template <bool BF16, int C>
hipError_t launch_fwd_dispatch(const FwdPlan& p, int BH, hipStream_t stream) {
    switch (p.NDPM) {
        case 2: return launch_fwd_t<BF16, C, 2>(p, BH, stream);
        case 4: return launch_fwd_t<BF16, C, 4>(p, BH, stream);
        case 8: return launch_fwd_t<BF16, C, 8>(p, BH, stream);
        default: break;
    }
    if constexpr (C < 128) {
        switch (p.NDPM) {
            case 12: return launch_fwd_t<BF16, C, 12>(p, BH, stream);
            case 16: return launch_fwd_t<BF16, C, 16>(p, BH, stream);
            case 24: return launch_fwd_t<BF16, C, 24>(p, BH, stream);
            case 32: return launch_fwd_t<BF16, C, 32>(p, BH, stream);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

// One translation unit per (dtype, chunk) instantiates the capacities above.
hipError_t launch_fwd_f32_c16(const FwdPlan& p, int BH, hipStream_t s);
hipError_t launch_fwd_f32_c32(const FwdPlan& p, int BH, hipStream_t s);
hipError_t launch_fwd_f32_c64(const FwdPlan& p, int BH, hipStream_t s);
hipError_t launch_fwd_f32_c128(const FwdPlan& p, int BH, hipStream_t s);
hipError_t launch_fwd_bf16_c16(const FwdPlan& p, int BH, hipStream_t s);
hipError_t launch_fwd_bf16_c32(const FwdPlan& p, int BH, hipStream_t s);
hipError_t launch_fwd_bf16_c64(const FwdPlan& p, int BH, hipStream_t s);
hipError_t launch_fwd_bf16_c128(const FwdPlan& p, int BH, hipStream_t s);

}  // namespace fwa
