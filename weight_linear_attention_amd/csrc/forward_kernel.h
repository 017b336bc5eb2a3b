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

template <bool BF16, int C, int NDPM>
__global__ __launch_bounds__(256, 1) void delta_forward_kernel(FwdArgs a) {
    using LT = std::conditional_t<BF16, u16, float>;  // LDS element type of K, Q and P
    constexpr int NT = C / 16;
    constexpr int NQ = (NT + 1) / 2;                   // tile-row pairs {q, NT-1-q}
    constexpr int UPW = (2 * NQ + 3) / 4;              // G/P units per wave
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
    uint4 kraw[NRM], qraw[NRM], vraw[NRM];
    IT blpre = IT(0);
    // V rows of this workgroup's d_v slice: VB = 16 * NVT columns, 16-byte units per row.
    const int vbw = r * a.NVT * 16;                  // first column of the slice
    const int vupr = a.NVT * 16 * static_cast<int>(sizeof(IT)) / 16;
    const int nvunits = C * vupr;
    const int nvr = (nvunits + 255) / 256;
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
            if (i < nvr) {
                const int u = tid + 256 * i;
                const int row = u / vupr;
                const bool ok = u < nvunits && row < Cn;
                const IT* src = vB + static_cast<int64_t>(tn0 + (ok ? row : 0)) * d_v + vbw +
                                (ok ? (u % vupr) : 0) * (16 / static_cast<int>(sizeof(IT)));
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
                    const uint32_t m = (u * 16) / ubytes < Cc ? 0xffffffffu : 0u;
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
                    const uint32_t m = u / vupr < Cc ? 0xffffffffu : 0u;
                    const uint4 v4 = vraw[i];
                    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Xv) + u * 16) =
                        make_uint4(v4.x & m, v4.y & m, v4.z & m, v4.w & m);
                }
            }
        }
        if (tid < C) betas[tid] = tid < Cc ? sigmoid_stable(to_f32(blpre)) : 0.0f;
        __syncthreads();

        // One row per d_k-lane group and pass, two passes per iteration; the shift count is
        // a compile-time constant on the fast path (nu <= 4).  Row sums come from the MFMA
        // pipe in phase B.
        auto dpfp_passes = [&](auto nu_tag) {
            constexpr int NU = decltype(nu_tag)::value;
            const RollConst rc = roll_consts(jl, gbase, d_k);
            for (int p = 0; p < npass; p += 2) {
                const bool two = p + 1 < npass;
                const int t0r = p * 4 * rpw + w * rpw + grp;
                const int t1r = two ? t0r + 4 * rpw : t0r;
                const float kv[2] = {to_f32(Xk[t0r * d_k + jl]), to_f32(Xk[t1r * d_k + jl])};
                const float qv[2] = {to_f32(Xq[t0r * d_k + jl]), to_f32(Xq[t1r * d_k + jl])};
                LT* const krow[2] = {Kr + t0r * a.krs + 2 * jl, Kr + t1r * a.krs + 2 * jl};
                LT* const qrow[2] = {Qr + t0r * a.krs + 2 * jl, Qr + t1r * a.krs + 2 * jl};
                dpfp_rows<LT, NU, 2>(kv, qv, rc, d_k, krow, qrow);
            }
        };
        auto dpfp_passes_any = [&]() {
            for (int p = 0; p < npass; ++p) {
                const int t = p * 4 * rpw + w * rpw + grp;
                const float kv = to_f32(Xk[t * d_k + jl]), qv = to_f32(Xq[t * d_k + jl]);
                dpfp_row_any<LT>(kv, qv, nu, jl, gbase, d_k, Kr + t * a.krs + 2 * jl,
                                 Qr + t * a.krs + 2 * jl);
            }
        };
        switch (nu) {
            case 1: dpfp_passes(std::integral_constant<int, 1>{}); break;
            case 2: dpfp_passes(std::integral_constant<int, 2>{}); break;
            case 3: dpfp_passes(std::integral_constant<int, 3>{}); break;
            case 4: dpfp_passes(std::integral_constant<int, 4>{}); break;
            default: dpfp_passes_any(); break;
        }
        __syncthreads();

        // ---------------- B: G, P tiles; K W^T and Q W^T against the memory
        // G = K K^T and P = Q K^T lower triangles in 16x16 tiles.  Work is split in units: one
        // of G or P for the tile rows {q, NT-1-q}; unit u goes to wave u % 4.  Inside a unit the
        // row operands are loaded once per k-step and reused by every tile of the two rows,
        // and the tiles are independent accumulators that interleave on the MFMA pipe.
        // gpa[ui][tb]: tile (ra, tb); gpb[ui][tb]: tile (rb, tb) (static register indices)
        // sa/sb: row sums of the unit's rows (the same operands times a ones matrix).
        f32x4 gpa[UPW][NT], gpb[UPW][NT], sa[UPW], sb[UPW];
#pragma unroll
        for (int ui = 0; ui < UPW; ++ui) {
            sa[ui] = sb[ui] = zero4();
#pragma unroll
            for (int tb = 0; tb < NT; ++tb) gpa[ui][tb] = gpb[ui][tb] = zero4();
        }
#pragma unroll
        for (int ui = 0; ui < UPW; ++ui) {
            const int u = w + 4 * ui;
            if (u < 2 * NQ) {
                const bool isP = u >= NQ;
                const int q = isP ? u - NQ : u;
                const int ra = q, rb = NT - 1 - q;       // rb >= ra
                const LT* Xa = (isP ? Qr : Kr) + (16 * ra + l16) * a.krs;
                const LT* Xb = (isP ? Qr : Kr) + (16 * rb + l16) * a.krs;
                const LT* Kb = Kr + l16 * a.krs;
                if constexpr (BF16) {
                    bf16x8 ones;
#pragma unroll
                    for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);
#pragma unroll 2
                    for (int kk = 0; kk < D / 32; ++kk) {
                        const int c0 = 32 * kk + 8 * g4;
                        const bf16x8 va = *reinterpret_cast<const bf16x8*>(Xa + c0);
                        const bf16x8 vb = *reinterpret_cast<const bf16x8*>(Xb + c0);
                        sa[ui] = mfma_bf16_k32(va, ones, sa[ui]);
                        if (rb != ra) sb[ui] = mfma_bf16_k32(vb, ones, sb[ui]);
#pragma unroll
                        for (int tb = 0; tb < NT; ++tb) {
                            if (tb <= rb) {
                                const bf16x8 kv8 = *reinterpret_cast<const bf16x8*>(Kb + 16 * tb * a.krs + c0);
                                if (tb <= ra) gpa[ui][tb] = mfma_bf16_k32(va, kv8, gpa[ui][tb]);
                                if (rb != ra) gpb[ui][tb] = mfma_bf16_k32(vb, kv8, gpb[ui][tb]);
                            }
                        }
                    }
                } else {
#pragma unroll 2
                    for (int kk = 0; kk < D / 16; ++kk) {
                        const int c0 = 16 * kk + 4 * g4;
                        const float4 va = *reinterpret_cast<const float4*>(Xa + c0);
                        const float4 vb = *reinterpret_cast<const float4*>(Xb + c0);
                        sa[ui] = mfma_f32_k4(va.x, 1.0f, sa[ui]);
                        sa[ui] = mfma_f32_k4(va.y, 1.0f, sa[ui]);
                        sa[ui] = mfma_f32_k4(va.z, 1.0f, sa[ui]);
                        sa[ui] = mfma_f32_k4(va.w, 1.0f, sa[ui]);
                        if (rb != ra) {
                            sb[ui] = mfma_f32_k4(vb.x, 1.0f, sb[ui]);
                            sb[ui] = mfma_f32_k4(vb.y, 1.0f, sb[ui]);
                            sb[ui] = mfma_f32_k4(vb.z, 1.0f, sb[ui]);
                            sb[ui] = mfma_f32_k4(vb.w, 1.0f, sb[ui]);
                        }
#pragma unroll
                        for (int tb = 0; tb < NT; ++tb) {
                            if (tb <= rb) {
                                const float4 k4 = *reinterpret_cast<const float4*>(Kb + 16 * tb * a.krs + c0);
                                if (tb <= ra) {
                                    f32x4& g = gpa[ui][tb];
                                    g = mfma_f32_k4(va.x, k4.x, g);
                                    g = mfma_f32_k4(va.y, k4.y, g);
                                    g = mfma_f32_k4(va.z, k4.z, g);
                                    g = mfma_f32_k4(va.w, k4.w, g);
                                }
                                if (rb != ra) {
                                    f32x4& g = gpb[ui][tb];
                                    g = mfma_f32_k4(vb.x, k4.x, g);
                                    g = mfma_f32_k4(vb.y, k4.y, g);
                                    g = mfma_f32_k4(vb.z, k4.z, g);
                                    g = mfma_f32_k4(vb.w, k4.w, g);
                                }
                            }
                        }
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
        // normalisers 1/(S + eps) of the unit's rows (G units: K rows, P units: Q rows)
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
                    r0[e] = __builtin_amdgcn_rcpf(sa[ui][e] + kDpfpEps);
                    r1[e] = __builtin_amdgcn_rcpf(sb[ui][e] + kDpfpEps);
                }
                *reinterpret_cast<f32x4*>(rho + 16 * ra + 4 * g4) = r0;
                if (rb != ra) *reinterpret_cast<f32x4*>(rho + 16 * rb + 4 * g4) = r1;
            }
        }
        __syncthreads();  // Q is dead from here; its space is reused

        // ---------------- B': scaled G and P to LDS, state partials to the reduction buffer
#pragma unroll
        for (int ui = 0; ui < UPW; ++ui) {
            const int u = w + 4 * ui;
            if (u < 2 * NQ) {
                const bool isP = u >= NQ;
                const int q = isP ? u - NQ : u;
                const int ra = q, rb = NT - 1 - q;
#pragma unroll
                for (int k2 = 0; k2 < 2 * NT; ++k2) {
                    // k2 < NT: tile (ra, k2) from gpa; k2 >= NT: tile (rb, k2 - NT) from gpb
                    const bool rowa = k2 < NT;
                    const int ta = rowa ? ra : rb;
                    const int tb = rowa ? k2 : k2 - NT;
                    if (tb > ta || (!rowa && rb == ra)) continue;
                    const f32x4 acc = rowa ? gpa[ui][k2 % NT] : gpb[ui][k2 % NT];
                    const int s = 16 * tb + l16, tr = 16 * ta + 4 * g4;
                    const float rks = rhok[s];
                    if (isP) {
                        const f32x4 rq = *reinterpret_cast<const f32x4*>(rhoq + tr);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float val = s <= tr + e ? rq[e] * rks * acc[e] : 0.0f;
                            Ps[(tr + e) * a.pss + s] = from_f32<LT>(val);
                        }
                    } else {
                        const f32x4 rk = *reinterpret_cast<const f32x4*>(rhok + tr);
                        const f32x4 bt = *reinterpret_cast<const f32x4*>(betas + tr);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            Ls[(tr + e) * a.lss + s] = s < tr + e ? bt[e] * rk[e] * rks * acc[e] : 0.0f;
                    }
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
        // (the next chunk's inputs are requested here: their registers are not live in B)
        if (ch + 1 < nchunks) prefetch(ch + 1);
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
                    X[tt][e] = to_f32(Xv[t * (16 * a.NVT) + 16 * vt + l16]) - rhok[t] * S1[tt][e];
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
