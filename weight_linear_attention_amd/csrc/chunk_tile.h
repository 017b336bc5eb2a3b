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

// Roll constants of one lane for shifts 1..4: the ds_bpermute byte address of the source lane
// and the sign mask.  For shift i the rolled operand of position j is relu([k,-k]) at
// m = (j - i) mod 2 d_k, i.e. lane (m mod d_k) of the row's group, negated when m >= d_k.
struct RollConst {
    int src4[4];
    uint32_t smask[4];
};

__device__ __forceinline__ RollConst roll_consts(int jl, int gbase, int d_k) {
    RollConst rc;
#pragma unroll
    for (int i = 1; i <= 4; ++i) {
        const int m = (jl - i) & (2 * d_k - 1);
        rc.src4[i - 1] = (gbase + (m & (d_k - 1))) << 2;
        rc.smask[i - 1] = (m & d_k) ? 0x80000000u : 0u;
    }
    return rc;
}

__device__ __forceinline__ float flip(float x, uint32_t mask) {
    return __uint_as_float(__float_as_uint(x) ^ mask);
}

// K and Q tiles store their D columns in an internal order that puts the two halves of a
// shift block next to each other: internal column 2 ((i-1) d_k + j) + h holds DPFP position
// (i-1) 2 d_k + h d_k + j (h = 0: relu(k_j) * ..., h = 1: relu(-k_j) * ...).  Inner products
// over D do not depend on the order; the memory W^T uses the same order internally and is
// mapped back at load/store.  So a lane writes both halves of its position with one store.
__device__ __forceinline__ int orig_col(int c, int d_k) {
    const int m = c >> 1;
    return (m / d_k) * 2 * d_k + (c & 1) * d_k + (m % d_k);
}

__device__ __forceinline__ float relu_f(float x) { return fmaxf(x, 0.0f); }

template <typename LT>
__device__ __forceinline__ void store_pair(LT* p, float lo, float hi) {
    if constexpr (sizeof(LT) == 2) *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(lo, hi);
    else *reinterpret_cast<float2*>(p) = make_float2(lo, hi);
}

// Raw DPFP products of R rows for NU shifts (lane jl of a DK-lane group holds k_jl and q_jl
// of its row), written as (h = 0, h = 1) pairs to the row-major K and Q tiles.  All loads and
// permutes of the R rows are issued before the first LDS write.
template <typename LT, int NU, int R>
__device__ __forceinline__ void dpfp_rows(const float (&kv)[R], const float (&qv)[R],
                                          const RollConst& rc, int d_k, LT* const (&krow)[R],
                                          LT* const (&qrow)[R]) {
    float xk[R][NU], xq[R][NU];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            xk[r][i] = flip(__int_as_float(__builtin_amdgcn_ds_bpermute(rc.src4[i], __float_as_int(kv[r]))),
                            rc.smask[i]);
            xq[r][i] = flip(__int_as_float(__builtin_amdgcn_ds_bpermute(rc.src4[i], __float_as_int(qv[r]))),
                            rc.smask[i]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float ka = relu_f(kv[r]), kb = relu_f(-kv[r]), qa = relu_f(qv[r]), qb = relu_f(-qv[r]);
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            // ka, kb >= 0, so ka * relu(x) = relu(ka * x) and kb * relu(-x) = relu(-(kb * x))
            store_pair(krow[r] + 2 * i * d_k, relu_f(ka * xk[r][i]), relu_f(-(kb * xk[r][i])));
            store_pair(qrow[r] + 2 * i * d_k, relu_f(qa * xq[r][i]), relu_f(-(qb * xq[r][i])));
        }
    }
}

// Any nu (slow path, one row): the permute address and sign are computed per shift.
template <typename LT>
__device__ __forceinline__ void dpfp_row_any(float kv, float qv, int nu, int jl, int gbase,
                                             int d_k, LT* krow, LT* qrow) {
    const int two_dk = 2 * d_k;
    const float ka = relu_f(kv), kb = relu_f(-kv), qa = relu_f(qv), qb = relu_f(-qv);
    for (int i = 1; i <= nu; ++i) {
        const int m = (jl - i) & (two_dk - 1);
        const int src4 = (gbase + (m & (d_k - 1))) << 2;
        const uint32_t sm = (m & d_k) ? 0x80000000u : 0u;
        const float xk = flip(__int_as_float(__builtin_amdgcn_ds_bpermute(src4, __float_as_int(kv))), sm);
        const float xq = flip(__int_as_float(__builtin_amdgcn_ds_bpermute(src4, __float_as_int(qv))), sm);
        store_pair(krow + 2 * (i - 1) * d_k, relu_f(ka * xk), relu_f(-(kb * xk)));
        store_pair(qrow + 2 * (i - 1) * d_k, relu_f(qa * xq), relu_f(-(qb * xq)));
    }
}

// DPFP of the C staged raw rows Xk, Xq ([C][d_k], input storage type) into the tiles Kr, Qr
// ([C][krs], internal column order).  One row per d_k-lane group and pass, two passes per
// iteration; the shift count is a compile-time constant on the fast path (nu <= 4).
template <typename LT, typename IT, int C>
__device__ __forceinline__ void dpfp_chunk(const IT* Xk, const IT* Xq, LT* Kr, LT* Qr, int krs,
                                           int d_k, int nu, int w, int l) {
    const int rpw = 64 / d_k;                 // rows per wave pass
    const int jl = l % d_k, grp = l / d_k;
    const int gbase = grp * d_k;
    const int npass = C / (4 * rpw);
    auto passes = [&](auto nu_tag) {
        constexpr int NU = decltype(nu_tag)::value;
        const RollConst rc = roll_consts(jl, gbase, d_k);
        for (int p = 0; p < npass; p += 2) {
            const bool two = p + 1 < npass;
            const int t0r = p * 4 * rpw + w * rpw + grp;
            const int t1r = two ? t0r + 4 * rpw : t0r;
            const float kv[2] = {to_f32(Xk[t0r * d_k + jl]), to_f32(Xk[t1r * d_k + jl])};
            const float qv[2] = {to_f32(Xq[t0r * d_k + jl]), to_f32(Xq[t1r * d_k + jl])};
            LT* const krow[2] = {Kr + t0r * krs + 2 * jl, Kr + t1r * krs + 2 * jl};
            LT* const qrow[2] = {Qr + t0r * krs + 2 * jl, Qr + t1r * krs + 2 * jl};
            dpfp_rows<LT, NU, 2>(kv, qv, rc, d_k, krow, qrow);
        }
    };
    auto passes_any = [&]() {
        for (int p = 0; p < npass; ++p) {
            const int t = p * 4 * rpw + w * rpw + grp;
            const float kv = to_f32(Xk[t * d_k + jl]), qv = to_f32(Xq[t * d_k + jl]);
            dpfp_row_any<LT>(kv, qv, nu, jl, gbase, d_k, Kr + t * krs + 2 * jl,
                             Qr + t * krs + 2 * jl);
        }
    };
    switch (nu) {
        case 1: passes(std::integral_constant<int, 1>{}); break;
        case 2: passes(std::integral_constant<int, 2>{}); break;
        case 3: passes(std::integral_constant<int, 3>{}); break;
        case 4: passes(std::integral_constant<int, 4>{}); break;
        default: passes_any(); break;
    }
}

// G = K K^T and P = Q K^T lower triangles in 16x16 tiles.  Work is split in units: one of G or
// P for the tile rows {q, NT-1-q}; unit u goes to wave u % 4.  Inside a unit the row operands
// are loaded once per k-step and reused by every tile of the two rows, and the tiles are
// independent accumulators that interleave on the MFMA pipe.  a[ui][tb] holds tile (ra, tb),
// b[ui][tb] tile (rb, tb) (static register indices); sa / sb are the row sums of the unit's
// rows, computed as the same operands times a ones matrix.
template <int C>
struct GPTiles {
    static constexpr int NT = C / 16;
    static constexpr int NQ = (NT + 1) / 2;            // tile-row pairs {q, NT-1-q}
    static constexpr int UPW = (2 * NQ + 3) / 4;       // units per wave
    f32x4 a[UPW][NT], b[UPW][NT], sa[UPW], sb[UPW];
};

// One unit: tile rows RA = Q and RB = NT-1-Q of X (K or Q) against the K rows, with the row
// sums of the two rows.  The rows are compile-time constants, so every tile condition folds away.
template <bool BF16, int C, int Q>
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
            sa = mfma_bf16_k32(va, ones, sa);
            if (RB != RA) sb = mfma_bf16_k32(vb, ones, sb);
#pragma unroll
            for (int tb = 0; tb <= RB; ++tb) {
                if (tb <= RA) ta[tb] = mfma_bf16_k32(va, kv8[tb], ta[tb]);
                if (RB != RA) tb_[tb] = mfma_bf16_k32(vb, kv8[tb], tb_[tb]);
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
                sa = mfma_f32_k4(va[e], 1.0f, sa);
                if (RB != RA) sb = mfma_f32_k4(vb[e], 1.0f, sb);
#pragma unroll
                for (int tb = 0; tb <= RB; ++tb) {
                    if (tb <= RA) ta[tb] = mfma_f32_k4(va[e], k4[tb][e], ta[tb]);
                    if (RB != RA) tb_[tb] = mfma_f32_k4(vb[e], k4[tb][e], tb_[tb]);
                }
            }
        }
    }
}

template <bool BF16, int C>
__device__ __forceinline__ void gp_compute(GPTiles<C>& gp, const void* Kv, const void* Qv,
                                           int krs, int D, int w, int l16, int g4) {
    using GP = GPTiles<C>;
    constexpr int NT = GP::NT, NQ = GP::NQ, UPW = GP::UPW;
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
        gp.sa[ui] = gp.sb[ui] = zero4();
#pragma unroll
        for (int tb = 0; tb < NT; ++tb) gp.a[ui][tb] = gp.b[ui][tb] = zero4();
    }
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
        const int u = w + 4 * ui;
        if (u < 2 * NQ) {
            const bool isP = u >= NQ;
            const int q = isP ? u - NQ : u;
            const void* X = isP ? Qv : Kv;
            // q is uniform over the wave: one branch selects the unit's instantiation
            switch (q) {
                case 0: gp_unit<BF16, C, 0>(gp.a[ui], gp.b[ui], gp.sa[ui], gp.sb[ui], X, Kv, krs, D, l16, g4); break;
                case 1: if constexpr (NQ > 1) gp_unit<BF16, C, (NQ > 1 ? 1 : 0)>(gp.a[ui], gp.b[ui], gp.sa[ui], gp.sb[ui], X, Kv, krs, D, l16, g4); break;
                case 2: if constexpr (NQ > 2) gp_unit<BF16, C, (NQ > 2 ? 2 : 0)>(gp.a[ui], gp.b[ui], gp.sa[ui], gp.sb[ui], X, Kv, krs, D, l16, g4); break;
                case 3: if constexpr (NQ > 3) gp_unit<BF16, C, (NQ > 3 ? 3 : 0)>(gp.a[ui], gp.b[ui], gp.sa[ui], gp.sb[ui], X, Kv, krs, D, l16, g4); break;
                default: break;
            }
        }
    }
}

// Normalisers 1 / (row sum + eps) of the unit's rows (G units: K rows, P units: Q rows).
template <int C>
__device__ __forceinline__ void gp_write_rho(const GPTiles<C>& gp, float* rhok, float* rhoq,
                                             int w, int l16, int g4) {
    using GP = GPTiles<C>;
    constexpr int NT = GP::NT, NQ = GP::NQ, UPW = GP::UPW;
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
        const int u = w + 4 * ui;
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
template <bool BF16, int C>
__device__ __forceinline__ void gp_scale(const GPTiles<C>& gp, const float* rhok,
                                         const float* rhoq, const float* betas, float* Ls,
                                         int lss, void* Pv, int pss, int w, int l16, int g4) {
    using GP = GPTiles<C>;
    constexpr int NQ = GP::NQ, UPW = GP::UPW;
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
        const int u = w + 4 * ui;
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
