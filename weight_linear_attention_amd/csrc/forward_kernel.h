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

#include "chunk_tile.h"
#include "fwa_internal.h"

#include <type_traits>

namespace fwa {

template <bool BF16, int C, int NDPM>
__global__ __launch_bounds__(256, 1) void delta_forward_kernel(FwdArgs a) {
    using LT = std::conditional_t<BF16, u16, float>;  // LDS element type of K, Q and P
    constexpr int NT = C / 16;
    constexpr int RS = C + 4;                          // row stride of the partials buffer
    extern __shared__ __attribute__((aligned(16))) char smem[];

    LT* Kr = reinterpret_cast<LT*>(smem + a.off_kr);   // [C][krs]  K (lives through D)
    LT* Qr = reinterpret_cast<LT*>(smem + a.off_qr);   // [C][krs]  Q (dead after B)
    using ITs = std::conditional_t<BF16, u16, float>;
    ITs* Xk = reinterpret_cast<ITs*>(smem + a.off_xs);              // [C][d_k] raw k rows
    ITs* Xq = Xk + C * a.d_k;                                       // [C][d_k] raw q rows
    ITs* Xv = Xq + C * a.d_k;                                       // [C][16 NVT] v slice
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
            // internal columns c0 .. c0+3 = positions (o, o + d_k, o + 1, o + d_k + 1)
            const float* src = a.W0 + (static_cast<int64_t>(bh) * d_v + vcol) * D +
                               orig_col(16 * (dt0 + i) + 4 * g4, d_k);
            const float2 lo = *reinterpret_cast<const float2*>(src);
            const float2 hi = *reinterpret_cast<const float2*>(src + d_k);
            Wst[i] = f32x4{lo.x, hi.x, lo.y, hi.y};
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

    // The next chunk's raw inputs are fetched into registers while the current chunk is
    // being computed, so no global-memory latency sits on the serial chain over chunks.
    // The next chunk's k and q rows form two contiguous blocks of C*d_k elements; each thread
    // fetches its share as 16-byte units into registers while the current chunk computes.
    // Loads are branch-free: a unit past the sequence end reads unit 0 of the chunk (always in
    // range) and is zeroed when it is staged, so no wait sits next to the loads.
    constexpr int NRM = C / 16;                      // units per thread at d_k = 64, fp32
    const int ubytes = d_k * static_cast<int>(sizeof(IT));  // bytes per row
    const int nunits = C * ubytes / 16;              // 16-byte units per chunk block
    const int nr = (nunits + 255) / 256;
    uint4 kraw[NRM], qraw[NRM], vraw[NRM];
    IT blpre = IT(0);
    // V rows of this workgroup's d_v slice: VB = 16 * NVT columns, 16-byte units per row.
    const int vbw = r * a.NVT * 16;                  // first column of the slice
    const int vupr = a.NVT * 16 * static_cast<int>(sizeof(IT)) / 16;
    const int nvunits = C * vupr;
    const int nvr = (nvunits + 255) / 256;
    // bytes per row and units per v row are powers of two: row indices by shifts
    const int ush = __builtin_ctz(ubytes) - 4;       // unit u of a k/q block is in row u >> ush
    const int vsh = __builtin_ctz(vupr);             // unit u of the v block: row u >> vsh
    auto prefetch = [&](int chn) {
        const int tn0 = chn * C;
        const int Cn = min(C, T - tn0);
        const char* kc = reinterpret_cast<const char*>(kB + static_cast<int64_t>(tn0) * d_k);
        const char* qc = reinterpret_cast<const char*>(qB + static_cast<int64_t>(tn0) * d_k);
#pragma unroll
        for (int i = 0; i < NRM; ++i) {
            if (i < nr) {
                const int u = tid + 256 * i;
                const bool ok = u < nunits && (u >> ush) < Cn;
                const int off = ok ? u * 16 : 0;
                kraw[i] = *reinterpret_cast<const uint4*>(kc + off);
                qraw[i] = *reinterpret_cast<const uint4*>(qc + off);
            }
            if (i < nvr) {
                const int u = tid + 256 * i;
                const int row = u >> vsh;
                const bool ok = u < nvunits && row < Cn;
                const IT* src = vB + static_cast<int64_t>(tn0 + (ok ? row : 0)) * d_v + vbw +
                                (ok ? (u & (vupr - 1)) : 0) * (16 / static_cast<int>(sizeof(IT)));
                vraw[i] = *reinterpret_cast<const uint4*>(src);
            }
        }
        blpre = bB[tn0 + min(tid, Cn - 1)];
    };
    if (nchunks > 0) prefetch(0);

    for (int ch = 0; ch < nchunks; ++ch) {
        const int t0 = ch * C;
        const int Cc = min(C, T - t0);

        // ---------------- A: DPFP rows, beta, and this wave's V tile (consumed in C)
        // Stage this chunk's raw rows (zeros past the sequence end) for the DPFP passes.
#pragma unroll
        for (int i = 0; i < NRM; ++i) {
            if (i < nr) {
                const int u = tid + 256 * i;
                if (u < nunits) {
                    const uint32_t m = (u >> ush) < Cc ? 0xffffffffu : 0u;
                    const uint4 kr4 = kraw[i], qr4 = qraw[i];
                    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Xk) + u * 16) =
                        make_uint4(kr4.x & m, kr4.y & m, kr4.z & m, kr4.w & m);
                    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Xq) + u * 16) =
                        make_uint4(qr4.x & m, qr4.y & m, qr4.z & m, qr4.w & m);
                }
            }
            if (i < nvr) {
                const int u = tid + 256 * i;
                if (u < nvunits) {
                    const uint32_t m = (u >> vsh) < Cc ? 0xffffffffu : 0u;
                    const uint4 v4 = vraw[i];
                    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Xv) + u * 16) =
                        make_uint4(v4.x & m, v4.y & m, v4.z & m, v4.w & m);
                }
            }
        }
        if (tid < C) betas[tid] = tid < Cc ? sigmoid_stable(to_f32(blpre)) : 0.0f;
        lds_barrier();

        dpfp_chunk<LT, ITs, C>(Xk, Xq, Kr, Qr, a.krs, d_k, nu, w, l);
        lds_barrier();

        // ---------------- B: G, P tiles; K W^T and Q W^T against the memory
        GPTiles<C> gp;
        gp_compute<BF16, C>(gp, Kr, Qr, a.krs, D, w, l16, g4);
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
        gp_write_rho<C>(gp, rhok, rhoq, w, l16, g4);
        lds_barrier();  // Q is dead from here; its space is reused

        // ---------------- B': scaled G and P to LDS, state partials to the reduction buffer
        gp_scale<BF16, C>(gp, rhok, rhoq, betas, Ls, a.lss, Ps, a.pss, w, l16, g4);
        if (has_state && a.DP > 1) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                *reinterpret_cast<f32x4*>(Red + ((w * 2 + 0) * 16 + l16) * RS + 16 * tt + 4 * g4) = S1[tt];
                *reinterpret_cast<f32x4*>(Red + ((w * 2 + 1) * 16 + l16) * RS + 16 * tt + 4 * g4) = QW[tt];
            }
        }
        lds_barrier();

        // ---------------- C: diagonal-block inverses; reduce the state partials
        // (the next chunk's inputs are requested here: their registers are not live in B)
        if (ch + 1 < nchunks) prefetch(ch + 1);
        if (tid < C) diag_inverse(Ls, a.lss, Li, tid);
        f32x4 X[NT];
        if (has_state) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                if (a.DP > 1) {
                    // all (up to 4) partials are read at once; a partial index past DP re-reads
                    // the last wave's and is dropped by the select
                    f32x4 s1 = zero4(), qw = zero4();
#pragma unroll
                    for (int pp = 0; pp < 4; ++pp) {
                        const int ww = min(vt + a.NVT * pp, a.NVT * a.DP - 1);
                        const f32x4 ps = *reinterpret_cast<const f32x4*>(Red + ((ww * 2 + 0) * 16 + l16) * RS + 16 * tt + 4 * g4);
                        const f32x4 pq = *reinterpret_cast<const f32x4*>(Red + ((ww * 2 + 1) * 16 + l16) * RS + 16 * tt + 4 * g4);
                        s1 += pp < a.DP ? ps : zero4();
                        qw += pp < a.DP ? pq : zero4();
                    }
                    S1[tt] = s1;
                    QW[tt] = qw;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * tt + 4 * g4 + e;
                    X[tt][e] = to_f32(Xv[t * (16 * a.NVT) + 16 * vt + l16]) - rhok[t] * S1[tt][e];
                    QW[tt][e] *= rhoq[t];
                }
            }
        }
        lds_barrier();

        // ---------------- D: U by block substitution, Y, and the memory update
        if (has_state) {
            // U = (I + L)^-1 beta X, solved in place
            f32x4 (&U)[NT] = X;
#pragma unroll
            for (int ta = 0; ta < NT; ++ta) {
#pragma unroll
                for (int e = 0; e < 4; ++e) U[ta][e] *= betas[16 * ta + 4 * g4 + e];
            }
            block_solve<NT>(U, Ls, a.lss, Li, l16, g4);
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
        lds_barrier();  // every LDS buffer is rewritten by the next chunk
    }

    if (has_state && a.Wf) {
#pragma unroll
        for (int i = 0; i < NDPM; ++i) {
            if (i < ndp) {
                float* dst = a.Wf + (static_cast<int64_t>(bh) * d_v + vcol) * D +
                             orig_col(16 * (dt0 + i) + 4 * g4, d_k);
                *reinterpret_cast<float2*>(dst) = make_float2(Wst[i][0], Wst[i][2]);
                *reinterpret_cast<float2*>(dst + d_k) = make_float2(Wst[i][1], Wst[i][3]);
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
    hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kern), p.lds_bytes);
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
