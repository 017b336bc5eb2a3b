// Building blocks of the chunked forward kernels, on one chunk of C rows held in LDS:
//   * DPFP of the chunk's k and q rows into raw-product tiles K and Q,
//   * G = K K^T and P = Q K^T (lower triangles, 16x16 MFMA tiles) with the row sums,
//   * the scaled unit lower system L = beta rho_k rho_k^T o strict_lower(G) and
//     P~ = rho_q rho_k^T o lower_incl(P),
//   * inverses of the 16x16 diagonal blocks of I + L, and block forward substitution.
// DPFP follows the "Fast Weights Transformer" guide (xdnf.cn/news/308600), sections "DPFP /
// projection formula and hyper-parameters" and "DPFP / normalisation": x = relu([k, -k]); the
// block of shift i (1..nu) holds x_j * x_{(j - i) mod 2 d_k}; phi = raw / (sum(raw) + 1e-6).
// The tiles hold the raw products; the normalisers rho = 1 / (row sum + eps) are applied to
// contraction results.
#pragma once

#include "fwa_common.h"

#include <type_traits>

namespace fwa {

constexpr int kLiStride = 20;   // floats per row of the diagonal-inverse buffer

// K and Q tiles store their D columns in an internal order that puts the two halves of a
// shift block next to each other: internal column 2 ((i-1) d_k + j) + h holds DPFP position
// (i-1) 2 d_k + h d_k + j (h = 0: relu(k_j) * ..., h = 1: relu(-k_j) * ...).  Inner products
// over D do not depend on the order; the memory W^T uses the same order internally and is
// mapped back at load/store.  The two halves of a position are adjacent, so a run of 8 positions
// is 16 consecutive columns (two 16-byte stores for bf16).
__device__ __forceinline__ int orig_col(int c, int d_k) {
    const int m = c >> 1;
    return (m / d_k) * 2 * d_k + (c & 1) * d_k + (m % d_k);
}

__device__ __forceinline__ float relu_f(float x) { return fmaxf(x, 0.0f); }

// Eight consecutive staged inputs (bf16 or fp32) as fp32.  `p` is 16-byte aligned.
__device__ __forceinline__ void load8_f32(const u16* p, float (&v)[8]) {
    const uint4 r = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(w[e] << 16);
        v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8_f32(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Sixteen consecutive tile columns from fp32 values (16-byte stores; `p` 32-byte aligned).
__device__ __forceinline__ void store16(u16* p, const float (&f)[16]) {
    uint4* q = reinterpret_cast<uint4*>(p);
    q[0] = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    q[1] = make_uint4(pack_bf16x2(f[8], f[9]), pack_bf16x2(f[10], f[11]),
                      pack_bf16x2(f[12], f[13]), pack_bf16x2(f[14], f[15]));
}
__device__ __forceinline__ void store16(float* p, const float (&f)[16]) {
    float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) q[e] = make_float4(f[4 * e], f[4 * e + 1], f[4 * e + 2], f[4 * e + 3]);
}

// One DPFP task: the 8 positions j0 .. j0+7 of one staged row (a = k[j0 .. j0+7]) for every
// shift, written as 16 consecutive internal columns per shift.  The rolled operand of position
// j for shift i is relu([k,-k]) at (j - i) mod 2 d_k, which is +-k[(j - i) mod d_k], negated
// when j < i (the index wraps into the [-k] half).  pv = k over the 8 positions before j0
// (cyclically), so window index 8 + e - i of [pv, a] is k[(j0 + e - i) mod d_k] for every
// shift up to 4 (d_k = 16: the window is the whole row, so the index is cyclic).
// Both factors of a product are non-negative parts of k: the positive and negative parts of the
// window are taken once per task, and each product is then a single multiply (relu(a) relu(x)
// equals relu(relu(a) x), so the values are the same as relu of the product).
// With `wraps` false the caller has already negated pv for the group at position 0 (so the
// wrapped operands need no swap here).
template <typename LT, int NU>
__device__ __forceinline__ float dpfp_task_w(const float (&a)[8], const float (&pv)[8], int j0,
                                             int d_k, LT* out, bool wraps) {
    static_assert(NU >= 1 && NU <= 4, "window indices 8 - NU .. 15");
    float P[16], N[16];
#pragma unroll
    for (int m = 8 - NU; m < 16; ++m) {
        const float r = m >= 8 ? a[m - 8] : pv[m];
        P[m] = relu_f(r);
        N[m] = P[m] - r;                 // relu(-r), exactly
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 1; i <= NU; ++i) {
        float f[16];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int m = 8 + e - i;
            const float xp = (e < i && wraps) ? N[m] : P[m];
            const float xn = (e < i && wraps) ? P[m] : N[m];
            f[2 * e] = P[8 + e] * xp;
            f[2 * e + 1] = N[8 + e] * xn;
            sum += f[2 * e] + f[2 * e + 1];
        }
        store16(out + 2 * ((i - 1) * d_k + j0), f);
    }
    return sum;
}
template <typename LT, int NU>
__device__ __forceinline__ float dpfp_task(const float (&a)[8], const float (&pv)[8], int j0,
                                           int d_k, LT* out) {
    return dpfp_task_w<LT, NU>(a, pv, j0, d_k, out, j0 == 0);   // positions e < i of group 0 wrap
}

// Any nu (runtime shift count): the rolled operands are read from the staged row per shift.
template <typename LT, typename IT>
__device__ __forceinline__ float dpfp_task_any(const float (&a)[8], const IT* row, int j0,
                                               int d_k, int nu, LT* out) {
    float sum = 0.0f;
    for (int i = 1; i <= nu; ++i) {
        float f[16];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float r = to_f32(row[(j0 + e - i + 2 * d_k) & (d_k - 1)]);
            const float x = (j0 + e < i) ? -r : r;
            f[2 * e] = relu_f(relu_f(a[e]) * x);
            f[2 * e + 1] = relu_f(-(relu_f(-a[e]) * x));
            sum += f[2 * e] + f[2 * e + 1];
        }
        store16(out + 2 * ((i - 1) * d_k + j0), f);
    }
    return sum;
}

// DPFP of the C staged raw rows Xk, Xq ([C][d_k], input storage type) into the tiles Kr, Qr
// ([C][krs], internal column order).  A task is (tile, row, group of 8 positions); the NTH
// threads take 2 C d_k / 8 tasks, two per pass with both tasks' loads issued first.  Each
// task reads its row through two 16-byte LDS loads and writes 16-byte LDS stores; no lane
// exchanges.  The shift count is a compile-time constant for nu <= 4.
// With rhok / rhoq given, the row normalisers rho = 1 / (row sum + eps) are formed as well: a
// row's d_k / 8 tasks sit in adjacent lanes of one pass, so their fp32 sums reduce by lane
// shuffles and the row's first task writes rho[t].
// NTH threads take part (64 w + l < NTH); WITH_Q = false forms the K tile only (Xq, Qr unused).
template <typename LT, typename IT, int C, int NTH = 256, bool WITH_Q = true>
__device__ __forceinline__ void dpfp_chunk(const IT* Xk, const IT* Xq, LT* Kr, LT* Qr, int krs,
                                           int d_k, int nu, int w, int l,
                                           float* rhok = nullptr, float* rhoq = nullptr) {
    const int tid = 64 * w + l;
    const int lg = __builtin_ctz(d_k >> 3);           // log2(groups per row)
    const int gm = (d_k >> 3) - 1;
    const int ntask = (WITH_Q ? 2 : 1) * C * (d_k >> 3);
    auto locate = [&](int tau, const IT*& row, LT*& out, int& j0, int& jp) {
        const int jg = tau & gm;
        const int rt = tau >> lg;                      // 0 .. 2C-1: K rows, then Q rows
        const bool isq = rt >= C;
        const int t = isq ? rt - C : rt;
        row = (isq ? Xq : Xk) + t * d_k;
        out = (isq ? Qr : Kr) + t * krs;
        j0 = 8 * jg;
        jp = 8 * ((jg + gm) & gm);
    };
    auto run = [&](auto nu_tag) {
        constexpr int NU = decltype(nu_tag)::value;
        for (int tau = tid; tau < ntask; tau += 2 * NTH) {
            // two tasks per pass (the second clamps to the first when past the end: it then
            // rewrites identical values)
            const int tau2 = tau + NTH < ntask ? tau + NTH : tau;
            const IT *r1, *r2;
            LT *o1, *o2;
            int j1, p1, j2, p2;
            locate(tau, r1, o1, j1, p1);
            locate(tau2, r2, o2, j2, p2);
            float a1[8], v1[8], a2[8], v2[8];
            load8_f32(r1 + j1, a1);
            load8_f32(r2 + j2, a2);
            float s1, s2 = 0.0f;
            // ntask and NTH are multiples of 64, so `two` is uniform over each wave
            const bool two = tau2 != tau;
            if constexpr (NU > 0) {
                load8_f32(r1 + p1, v1);
                load8_f32(r2 + p2, v2);
                s1 = dpfp_task<LT, NU>(a1, v1, j1, d_k, o1);
                if (two) s2 = dpfp_task<LT, NU>(a2, v2, j2, d_k, o2);
            } else {
                s1 = dpfp_task_any<LT, IT>(a1, r1, j1, d_k, nu, o1);
                if (two) s2 = dpfp_task_any<LT, IT>(a2, r2, j2, d_k, nu, o2);
            }
            if (rhok != nullptr) {
                // sums over aligned groups of 2, 4 or 8 lanes by DPP (no LDS traffic, so no
                // wait on the task stores): lane ^ 1, lane ^ 2, then the mirror inside 8 lanes
                s1 += dpp_f32<0xB1>(s1);
                s2 += dpp_f32<0xB1>(s2);
                if (gm >= 3) {
                    s1 += dpp_f32<0x4E>(s1);
                    s2 += dpp_f32<0x4E>(s2);
                }
                if (gm >= 7) {
                    s1 += dpp_f32<0x141>(s1);
                    s2 += dpp_f32<0x141>(s2);
                }
                if ((tau & gm) == 0) {
                    const int rt1 = tau >> lg, rt2 = tau2 >> lg;
                    (rt1 >= C ? rhoq + (rt1 - C) : rhok + rt1)[0] = __builtin_amdgcn_rcpf(s1 + kDpfpEps);
                    if (two) (rt2 >= C ? rhoq + (rt2 - C) : rhok + rt2)[0] = __builtin_amdgcn_rcpf(s2 + kDpfpEps);
                }
            }
        }
    };
    switch (nu) {
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        case 4: run(std::integral_constant<int, 4>{}); break;
        default: run(std::integral_constant<int, 0>{}); break;
    }
}

// G = K K^T and P = Q K^T lower triangles in 16x16 tiles.  Work is split in units: one of G or
// P for the tile rows {q, NT-1-q}; unit u goes to wave u % 4.  Inside a unit the row operands
// are loaded once per k-step and reused by every tile of the two rows, and the tiles are
// independent accumulators that interleave on the MFMA pipe.  a[ui][tb] holds tile (ra, tb),
// b[ui][tb] tile (rb, tb) (static register indices); sa / sb are the row sums of the unit's
// rows, computed as the same operands times a ones matrix.
// NW waves share the units: unit u goes to wave u % NW.
template <int C, int NW = 4>
struct GPTiles {
    static constexpr int NT = C / 16;
    static constexpr int NQ = (NT + 1) / 2;            // tile-row pairs {q, NT-1-q}
    static constexpr int UPW = (2 * NQ + NW - 1) / NW; // units per wave
    f32x4 a[UPW][NT], b[UPW][NT], sa[UPW], sb[UPW];
};

// One unit: tile rows RA = Q and RB = NT-1-Q of X (K or Q) against the K rows, with the row
// sums of the two rows.  The rows are compile-time constants, so every tile condition folds away.
template <bool BF16, int C, int Q, bool ROWSUMS>
__device__ __forceinline__ void gp_unit(f32x4 (&ta)[C / 16], f32x4 (&tb_)[C / 16], f32x4& sa,
                                        f32x4& sb, const void* Xv, const void* Kv, int krs,
                                        int D, int l16, int g4) {
    using LT = std::conditional_t<BF16, u16, float>;
    constexpr int NT = C / 16, RA = Q, RB = NT - 1 - Q;   // RB >= RA
    const LT* X = static_cast<const LT*>(Xv);
    const LT* Kr = static_cast<const LT*>(Kv);
    const LT* Xa = X + (16 * RA + l16) * krs;
    const LT* Xb = X + (16 * RB + l16) * krs;
    const LT* Kb = Kr + l16 * krs;
    if constexpr (BF16) {
        bf16x8 ones;
#pragma unroll
        for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);
#pragma unroll 2
        for (int kk = 0; kk < D / 32; ++kk) {
            const int c0 = 32 * kk + 8 * g4;
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(Xa + c0);
            const bf16x8 vb = *reinterpret_cast<const bf16x8*>(Xb + c0);
            bf16x8 kv8[RB + 1];
#pragma unroll
            for (int tb = 0; tb <= RB; ++tb) kv8[tb] = *reinterpret_cast<const bf16x8*>(Kb + 16 * tb * krs + c0);
            if constexpr (ROWSUMS) {
                sa = mfma_bf16_k32(va, ones, sa);
                if (RB != RA) sb = mfma_bf16_k32(vb, ones, sb);
            }
#pragma unroll
            for (int tb = 0; tb <= RB; ++tb) {
                if (tb <= RA) ta[tb] = mfma_bf16_k32(va, kv8[tb], ta[tb]);
                if (RB != RA) tb_[tb] = mfma_bf16_k32(vb, kv8[tb], tb_[tb]);
            }
        }
    } else if constexpr (!ROWSUMS) {
        // fp32 tiles on the bf16 MFMA: each operand split on the fly into bf16 hi + lo
        // (x = hi + lo to about 2^-16); hi hi + hi lo + lo hi per 32-deep k-step (48 cycles of
        // MFMA against 256 for the eight fp32 16x16x4 products)
        auto split8 = [](const float* p, bf16x8& hi, bf16x8& lo) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
            f32x4 r0, r1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hi[e] = static_cast<__bf16>(x0[e]);
                hi[4 + e] = static_cast<__bf16>(x1[e]);
                r0[e] = x0[e] - static_cast<float>(hi[e]);
                r1[e] = x1[e] - static_cast<float>(hi[4 + e]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo[e] = static_cast<__bf16>(r0[e]);
                lo[4 + e] = static_cast<__bf16>(r1[e]);
            }
        };
        for (int kk = 0; kk < D / 32; ++kk) {
            const int c0 = 32 * kk + 8 * g4;
            bf16x8 ah, al, bh, bl;
            split8(Xa + c0, ah, al);
            split8(Xb + c0, bh, bl);
#pragma unroll
            for (int tb = 0; tb <= RB; ++tb) {
                bf16x8 kh, kl;
                split8(Kb + 16 * tb * krs + c0, kh, kl);
                if (tb <= RA) {
                    ta[tb] = mfma_bf16_k32(ah, kh, ta[tb]);
                    ta[tb] = mfma_bf16_k32(ah, kl, ta[tb]);
                    ta[tb] = mfma_bf16_k32(al, kh, ta[tb]);
                }
                if (RB != RA) {
                    tb_[tb] = mfma_bf16_k32(bh, kh, tb_[tb]);
                    tb_[tb] = mfma_bf16_k32(bh, kl, tb_[tb]);
                    tb_[tb] = mfma_bf16_k32(bl, kh, tb_[tb]);
                }
            }
        }
    } else {
#pragma unroll 2
        for (int kk = 0; kk < D / 16; ++kk) {
            const int c0 = 16 * kk + 4 * g4;
            const f32x4 va = *reinterpret_cast<const f32x4*>(Xa + c0);
            const f32x4 vb = *reinterpret_cast<const f32x4*>(Xb + c0);
            f32x4 k4[RB + 1];
#pragma unroll
            for (int tb = 0; tb <= RB; ++tb) k4[tb] = *reinterpret_cast<const f32x4*>(Kb + 16 * tb * krs + c0);
            // consecutive MFMAs write different accumulators
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (ROWSUMS) {
                    sa = mfma_f32_k4(va[e], 1.0f, sa);
                    if (RB != RA) sb = mfma_f32_k4(vb[e], 1.0f, sb);
                }
#pragma unroll
                for (int tb = 0; tb <= RB; ++tb) {
                    if (tb <= RA) ta[tb] = mfma_f32_k4(va[e], k4[tb][e], ta[tb]);
                    if (RB != RA) tb_[tb] = mfma_f32_k4(vb[e], k4[tb][e], tb_[tb]);
                }
            }
        }
    }
}

template <int C, int NW>
__device__ __forceinline__ void gp_zero(GPTiles<C, NW>& gp) {
    using GP = GPTiles<C, NW>;
#pragma unroll
    for (int ui = 0; ui < GP::UPW; ++ui) {
        gp.sa[ui] = gp.sb[ui] = zero4();
#pragma unroll
        for (int tb = 0; tb < GP::NT; ++tb) gp.a[ui][tb] = gp.b[ui][tb] = zero4();
    }
}

// Adds the products over D columns of the K and Q tiles (row stride krs) to the wave's units;
// the tiles may be a slice of the columns, so several calls accumulate the full inner product.
// ROWSUMS: the row sums (sa, sb) as the operands times a ones matrix; without it the caller
// has formed the normalisers elsewhere (dpfp_chunk with rho outputs).
template <bool BF16, int C, bool ROWSUMS = true, int NW = 4>
__device__ __forceinline__ void gp_accumulate(GPTiles<C, NW>& gp, const void* Kv, const void* Qv,
                                              int krs, int D, int w, int l16, int g4) {
    using GP = GPTiles<C, NW>;
    constexpr int NQ = GP::NQ, UPW = GP::UPW;
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
        const int u = w + NW * ui;
        if (u < 2 * NQ) {
            const bool isP = u >= NQ;
            const int q = isP ? u - NQ : u;
            const void* X = isP ? Qv : Kv;
            // q is uniform over the wave: one branch selects the unit's instantiation
            switch (q) {
                case 0: gp_unit<BF16, C, 0, ROWSUMS>(gp.a[ui], gp.b[ui], gp.sa[ui], gp.sb[ui], X, Kv, krs, D, l16, g4); break;
                case 1: if constexpr (NQ > 1) gp_unit<BF16, C, (NQ > 1 ? 1 : 0), ROWSUMS>(gp.a[ui], gp.b[ui], gp.sa[ui], gp.sb[ui], X, Kv, krs, D, l16, g4); break;
                case 2: if constexpr (NQ > 2) gp_unit<BF16, C, (NQ > 2 ? 2 : 0), ROWSUMS>(gp.a[ui], gp.b[ui], gp.sa[ui], gp.sb[ui], X, Kv, krs, D, l16, g4); break;
                case 3: if constexpr (NQ > 3) gp_unit<BF16, C, (NQ > 3 ? 3 : 0), ROWSUMS>(gp.a[ui], gp.b[ui], gp.sa[ui], gp.sb[ui], X, Kv, krs, D, l16, g4); break;
                default: break;
            }
        }
    }
}

template <bool BF16, int C, bool ROWSUMS = true, int NW = 4>
__device__ __forceinline__ void gp_compute(GPTiles<C, NW>& gp, const void* Kv, const void* Qv,
                                           int krs, int D, int w, int l16, int g4) {
    gp_zero(gp);
    gp_accumulate<BF16, C, ROWSUMS, NW>(gp, Kv, Qv, krs, D, w, l16, g4);
}

// Normalisers 1 / (row sum + eps) of the unit's rows (G units: K rows, P units: Q rows).
template <int C, int NW>
__device__ __forceinline__ void gp_write_rho(const GPTiles<C, NW>& gp, float* rhok, float* rhoq,
                                             int w, int l16, int g4) {
    using GP = GPTiles<C, NW>;
    constexpr int NT = GP::NT, NQ = GP::NQ, UPW = GP::UPW;
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
        const int u = w + NW * ui;
        if (u < 2 * NQ && l16 == 0) {
            const bool isP = u >= NQ;
            const int q = isP ? u - NQ : u;
            const int ra = q, rb = NT - 1 - q;
            float* rho = isP ? rhoq : rhok;
            f32x4 r0, r1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r0[e] = __builtin_amdgcn_rcpf(gp.sa[ui][e] + kDpfpEps);
                r1[e] = __builtin_amdgcn_rcpf(gp.sb[ui][e] + kDpfpEps);
            }
            *reinterpret_cast<f32x4*>(rho + 16 * ra + 4 * g4) = r0;
            if (rb != ra) *reinterpret_cast<f32x4*>(rho + 16 * rb + 4 * g4) = r1;
        }
    }
}

// Scaling of one unit's tiles (rows RA = Q and RB = NT-1-Q), see gp_scale.
template <bool BF16, int C, int Q>
__device__ __forceinline__ void gp_scale_unit(const f32x4 (&ta_)[C / 16], const f32x4 (&tb_)[C / 16],
                                              bool isP, const float* rhok, const float* rhoq,
                                              const float* betas, float* Ls, int lss, void* Pv,
                                              int pss, int l16, int g4) {
    using LT = std::conditional_t<BF16, u16, float>;
    constexpr int NT = C / 16, RA = Q, RB = NT - 1 - Q;
    LT* Ps = static_cast<LT*>(Pv);
#pragma unroll
    for (int k2 = 0; k2 < 2 * NT; ++k2) {
        // k2 < NT: tile (RA, k2); k2 >= NT: tile (RB, k2 - NT)
        const bool rowa = k2 < NT;
        const int ta = rowa ? RA : RB;
        const int tb = rowa ? k2 : k2 - NT;
        if (tb > ta || (!rowa && RB == RA)) continue;
        const f32x4 acc = rowa ? ta_[k2 % NT] : tb_[k2 % NT];
        const int s = 16 * tb + l16, tr = 16 * ta + 4 * g4;
        const float rks = rhok[s];
        if (isP) {
            const f32x4 rq = *reinterpret_cast<const f32x4*>(rhoq + tr);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float val = s <= tr + e ? rq[e] * rks * acc[e] : 0.0f;
                Ps[(tr + e) * pss + s] = from_f32<LT>(val);
            }
        } else {
            const f32x4 rk = *reinterpret_cast<const f32x4*>(rhok + tr);
            const f32x4 bt = *reinterpret_cast<const f32x4*>(betas + tr);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Ls[(tr + e) * lss + s] = s < tr + e ? bt[e] * rk[e] * rks * acc[e] : 0.0f;
        }
    }
}

// Writes Ls = beta_t rho_t rho_s G[t][s] (s < t, fp32) and Ps = rho_q,t rho_k,s P[t][s]
// (s <= t, operand type) for the tiles of this wave's units; tiles above the diagonal are not
// written.
template <bool BF16, int C, int NW>
__device__ __forceinline__ void gp_scale(const GPTiles<C, NW>& gp, const float* rhok,
                                         const float* rhoq, const float* betas, float* Ls,
                                         int lss, void* Pv, int pss, int w, int l16, int g4) {
    using GP = GPTiles<C, NW>;
    constexpr int NQ = GP::NQ, UPW = GP::UPW;
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
        const int u = w + NW * ui;
        if (u < 2 * NQ) {
            const bool isP = u >= NQ;
            const int q = isP ? u - NQ : u;
            switch (q) {
                case 0: gp_scale_unit<BF16, C, 0>(gp.a[ui], gp.b[ui], isP, rhok, rhoq, betas, Ls, lss, Pv, pss, l16, g4); break;
                case 1: if constexpr (NQ > 1) gp_scale_unit<BF16, C, (NQ > 1 ? 1 : 0)>(gp.a[ui], gp.b[ui], isP, rhok, rhoq, betas, Ls, lss, Pv, pss, l16, g4); break;
                case 2: if constexpr (NQ > 2) gp_scale_unit<BF16, C, (NQ > 2 ? 2 : 0)>(gp.a[ui], gp.b[ui], isP, rhok, rhoq, betas, Ls, lss, Pv, pss, l16, g4); break;
                case 3: if constexpr (NQ > 3) gp_scale_unit<BF16, C, (NQ > 3 ? 3 : 0)>(gp.a[ui], gp.b[ui], isP, rhok, rhoq, betas, Ls, lss, Pv, pss, l16, g4); break;
                default: break;
            }
        }
    }
}

// Column sc = idx % 16 of the inverse of the unit lower 16x16 diagonal block ab = idx / 16 of
// I + L (L strictly lower, in Ls), written to Li[16 ab + row][sc].  Each row's dot product is
// split over four partial sums to keep the dependency chains short.
__device__ __forceinline__ void diag_inverse(const float* Ls, int lss, float* Li, int idx) {
    const int ab = idx >> 4, sc = idx & 15;
    const float* Lb = Ls + (16 * ab) * lss + 16 * ab;
    float xcol[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        f32x4 rw[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            rw[q4] = (4 * q4 < u) ? *reinterpret_cast<const f32x4*>(Lb + u * lss + 4 * q4) : zero4();
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int w2 = 0; w2 < u; ++w2) acc[w2 & 3] += rw[w2 >> 2][w2 & 3] * xcol[w2];
        const float tot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        xcol[u] = (u == sc) ? 1.0f : (u < sc ? 0.0f : -tot);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) Li[(16 * ab + u) * kLiStride + sc] = xcol[u];
}

// Solves (I + L) X = Z for one 16-column tile by block forward substitution on the fp32 MFMA,
// in place (ZX holds Z on entry and X on return):
// X[ta] = Li[ta] (Z[ta] - sum_{tb < ta} L[ta][tb] X[tb]).  Z and X are in accumulator layout
// (lane l, slot e holds row 16 ta + 4 (l / 16) + e, column l % 16), so X[tb] is directly the
// B operand of the next products.
template <int NT>
__device__ __forceinline__ void block_solve(f32x4 (&ZX)[NT], const float* Ls, int lss,
                                            const float* Li, int l16, int g4) {
#pragma unroll
    for (int ta = 0; ta < NT; ++ta) {
        f32x4 acc = zero4();
#pragma unroll
        for (int tb = 0; tb < ta; ++tb) {
            const float4 l4 = *reinterpret_cast<const float4*>(Ls + (16 * ta + l16) * lss + 16 * tb + 4 * g4);
            acc = mfma_f32_k4(l4.x, ZX[tb][0], acc);
            acc = mfma_f32_k4(l4.y, ZX[tb][1], acc);
            acc = mfma_f32_k4(l4.z, ZX[tb][2], acc);
            acc = mfma_f32_k4(l4.w, ZX[tb][3], acc);
        }
        const f32x4 z = ZX[ta] - acc;
        const float4 i4 = *reinterpret_cast<const float4*>(Li + (16 * ta + l16) * kLiStride + 4 * g4);
        f32x4 x = zero4();
        x = mfma_f32_k4(i4.x, z[0], x);
        x = mfma_f32_k4(i4.y, z[1], x);
        x = mfma_f32_k4(i4.z, z[2], x);
        x = mfma_f32_k4(i4.w, z[3], x);
        ZX[ta] = x;
    }
}

}  // namespace fwa
