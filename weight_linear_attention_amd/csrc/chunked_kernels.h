// Chunked forward of the fast-weight delta rule: chunk-parallel preparation and the serial pass
// of the memory over the chunks, which forms the outputs as it goes for the shapes its staged
// and direct kernels take; elsewhere a third, chunk-parallel launch forms them.
//
// The recurrence ("Fast Weights Transformer" guide, xdnf.cn/news/308600, sections
// "FastWeightsAttention / update formula" and "... / module structure and source walkthrough"):
//     v_bar_t = W_{t-1} f_t,  W_t = W_{t-1} + beta_t (v_t - v_bar_t) f_t^T,  y_t = W_t g_t,
// f = phi(k), g = phi(q) (DPFP), beta_t = sigmoid(l_t).  The lucidrains page ("Deep dive into
// Fast Weight Attention", section 4.2) runs such layers chunk by chunk, parallel inside a chunk,
// passing the memory from chunk to chunk; the algebra below is derived from the recurrence.
// For a chunk of C rows starting from memory W (d_v x D), with raw DPFP product tiles K, Q,
// normalisers rho_k, rho_q (phi = rho * raw), K~ = diag(rho_k) K, Q~ = diag(rho_q) Q and
// L = diag(beta) strict_lower(K~ K~^T):
//     (I + L) U = diag(beta) (V - K~ W^T)
//  => U = U_y - W_y W^T  with  W_y = (I + L)^-1 diag(beta) K~,  U_y = (I + L)^-1 diag(beta) V
//     Y = Q~ W^T + P~ U  with  P~ = lower_incl(Q~ K~^T),        W^T <- W^T + K~^T U.
// W_y, U_y, P~ do not depend on the memory, so every chunk prepares them at once (prep);
// only U = U_y - W_y W^T and the update K~^T U stay on the serial chain (chain), and Y follows
// from the chunk-start memory and U of each chunk (in the chain, or in the output launch).
//
// Workspace blocks.  Every operand the chain and output kernels read is stored as 1 KiB blocks
// in the exact register layout of one MFMA operand (64 lanes x 16 bytes), so each wave loads a
// block with one fully coalesced 16-byte load per lane.  With pair = 2 for bf16 (16x16x32 MFMA,
// the two halves of a lane's 8 slots cover two 16-wide k-tiles) and 1 for fp32 (16x16x4, a
// lane's 4 slots feed four MFMAs):
//   A operand (rows m, k-tiles):   lane l, half h, slot e = X[16 m + l % 16][16 (pair j + h) + 4 (l / 16) + e]
//   B operand (k-tiles, cols n):   lane l, half h, slot e = X[16 (pair j + h) + 4 (l / 16) + e][16 n + l % 16]
// An fp32 accumulator tile (lane l, slot e = D[4 (l / 16) + e][l % 16]) is a B block with
// pair = 1 as it stands.
#pragma once

#include "chunk_tile.h"
#include "fwa_internal.h"

#include <cstdlib>
#include <type_traits>

namespace fwa {

template <bool BF16>
struct ChunkTypes {
    using LT = std::conditional_t<BF16, u16, float>;   // operand storage (and input) type
    static constexpr int pair = BF16 ? 2 : 1;
    static constexpr int es = BF16 ? 2 : 4;
};

__device__ __forceinline__ f32x4 as_f32x4(uint4 v) { return __builtin_bit_cast(f32x4, v); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 pack_bf16x8(const f32x4& lo, const f32x4& hi) {
    return make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                      pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]));
}

// The residuals x - bf16(x) of eight fp32 values, rounded to bf16: with pack_bf16x8 (the
// rounded values) a hi + lo pair whose sum carries each value to about 2^-16 relative.
__device__ __forceinline__ uint4 bf16_lo_part(const f32x4& x0, const f32x4& x1) {
    f32x4 r0, r1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r0[e] = x0[e] - static_cast<float>(static_cast<__bf16>(x0[e]));
        r1[e] = x1[e] - static_cast<float>(static_cast<__bf16>(x1[e]));
    }
    return pack_bf16x8(r0, r1);
}

// Split fp32 operand format.  An fp32 operand block pair (k-blocks 2 j', 2 j' + 1 of 16 each,
// lane l slot e) is stored instead as a bf16 hi block and a lo block, each in the register layout
// of one 32-deep bf16 MFMA operand: slot (h, e) of the hi block holds bf16(x) for k-block
// 2 j' + h, slot e, and the lo block bf16(x - bf16(x)).  The sum carries x to about 2^-16
// relative, and three bf16 MFMAs (hi hi + hi lo + lo hi; the lo lo term is below the split's own
// error) replace eight fp32 ones: a 32-deep k-step costs 48 cycles instead of 256.  A writer of
// one fp32 tile (4 values per lane) fills 8 bytes of each block at offset 8 (k-block & 1).
__device__ __forceinline__ uint2 pack_bf16x4(const f32x4& x) {
    return make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}
__device__ __forceinline__ uint2 bf16_lo_part4(const f32x4& x) {
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = x[e] - static_cast<float>(static_cast<__bf16>(x[e]));
    return pack_bf16x4(r);
}
// Lane l's 16 bytes of split block pair (hi at `pair_lane`, lo 1 KiB after it) for k-block kb.
__device__ __forceinline__ void store_split(char* pair_lane, int kb, const f32x4& x) {
    *reinterpret_cast<uint2*>(pair_lane + 8 * (kb & 1)) = pack_bf16x4(x);
    *reinterpret_cast<uint2*>(pair_lane + 1024 + 8 * (kb & 1)) = bf16_lo_part4(x);
}
// The same for a B-operand pair whose two blocks are not adjacent (hi and lo lane pointers).
__device__ __forceinline__ void store_split2(char* hi_lane, char* lo_lane, int kb, const f32x4& x) {
    *reinterpret_cast<uint2*>(hi_lane + 8 * (kb & 1)) = pack_bf16x4(x);
    *reinterpret_cast<uint2*>(lo_lane + 8 * (kb & 1)) = bf16_lo_part4(x);
}
__device__ __forceinline__ f32x4 mfma_split(const uint4& ah, const uint4& al, const uint4& bh,
                                            const uint4& bl, f32x4 acc) {
    acc = mfma_bf16_k32(as_bf16x8(ah), as_bf16x8(bh), acc);
    acc = mfma_bf16_k32(as_bf16x8(ah), as_bf16x8(bl), acc);
    return mfma_bf16_k32(as_bf16x8(al), as_bf16x8(bh), acc);
}

// Byte address of lane l's 16 bytes in block `blk` of the region at `base`.
__device__ __forceinline__ char* blk_ptr(char* base, int64_t blk, int l) {
    return base + (blk * 64 + l) * 16;
}
__device__ __forceinline__ const char* blk_ptr(const char* base, int64_t blk, int l) {
    return base + (blk * 64 + l) * 16;
}

// Block-lower-triangular operand matrices of a chunk (A'' hi, lo and P~ as 16-row x 32-column
// A-operand blocks (ta, j)) in the order that leaves out the blocks above the diagonal: block
// (ta, j) exists for 2 j <= ta, row tile by row tile, so row tile ta starts after
// sum_{r < ta} (r / 2 + 1) blocks.  C = 64 keeps 6 of 8 blocks, C = 128 20 of 32.
__host__ __device__ constexpr int tri_nblocks(int C) {
    return (C / 32) * (C / 32 + 1);
}
__device__ __forceinline__ int tri_blk(int ta, int j) {
    const int hf = ta >> 1;
    return hf * (hf + 1) + (ta & 1) * (hf + 1) + j;
}

// ------------------------------------------------------------------------------------------
// prep, one chunk (b, h, n) per workgroup pass.  DPFP, G and P with the normalisers, L and its
// diagonal-block inverses, the block inverse A = (I + L)^-1, U_y by block substitution and
// W_y^T = K^T (A diag(beta rho_k))^T on the MFMA; writes
//   WyA (A blocks of W_y, C x D), KtA (A blocks of K^T, D x C, raw products),
//   QA (A blocks of Q, raw), PA (A blocks of P~, zero above the diagonal),
//   Uy (fp32 accumulator tiles of U_y), RK, RQ (rho_k, rho_q).
// Eight waves (two per SIMD), so one wave's LDS and MFMA latencies overlap the other's work.
// G/P, its scaling and the block inverse keep one unit or block column per wave (waves 0-3);
// DPFP, the write-outs and the U_y / W_y GEMMs spread over all eight.
constexpr int kPrepThreads = 512, kPrepWaves = kPrepThreads / 64;

// LITE (bf16 only, for the streaming forward): stage k, q and beta only; write PA, RK, RQ and
// A'' = A diag(beta) as hi and lo A-operand blocks (AH, AL); no K^T, Q, W_y or U_y.
// Raw rows of one chunk in registers: 16-byte units e = tid + kPrepThreads i of the k, q and v
// rows (d_k, d_v <= 128) and the chunk's beta logit of row tid.
template <bool BF16, int C>
struct PrepStage {
    static constexpr int NU16 = (C * 128 * (BF16 ? 2 : 4) / 16 + kPrepThreads - 1) / kPrepThreads;
    uint4 k[NU16], q[NU16], v[NU16];
    float bl;
};

// Issue the loads of chunk `blk`'s raw rows into `st`.  A unit past the sequence end reads the
// chunk's first unit (always in range); staging zeroes it.
template <bool BF16, int C, bool LITE, int ROLE = 0>
__device__ __forceinline__ void prep_stage_load(const ChunkArgs& a, int64_t blk, PrepStage<BF16, C>& st) {
    using LT = typename ChunkTypes<BF16>::LT;
    const int tid = threadIdx.x, d_k = a.d_k, d_v = a.d_v, T = a.T;
    const BhIndex bi = xcd_local(blk, a.BH, a.NC);
    const int t0 = static_cast<int>(bi.i) * C, Cc = min(C, T - t0);
    const int64_t row0 = static_cast<int64_t>(bi.bh) * T + t0;
    const char* kc = reinterpret_cast<const char*>(static_cast<const LT*>(a.k) + row0 * d_k);
    const char* qc = reinterpret_cast<const char*>(static_cast<const LT*>(a.q) + row0 * d_k);
    const char* vc = reinterpret_cast<const char*>(static_cast<const LT*>(a.v) + row0 * d_v);
    const int kb = d_k * static_cast<int>(sizeof(LT)), vb = d_v * static_cast<int>(sizeof(LT));
#pragma unroll
    for (int i = 0; i < PrepStage<BF16, C>::NU16; ++i) {
        const int e = tid + kPrepThreads * i;
        if (kPrepThreads * i < C * kb / 16) {              // uniform over the workgroup
            const int ek = e < C * kb / 16 && (e * 16) / kb < Cc ? e * 16 : 0;
            st.k[i] = *reinterpret_cast<const uint4*>(kc + ek);
            if constexpr (ROLE != 1) st.q[i] = *reinterpret_cast<const uint4*>(qc + ek);
        }
        if (!LITE && ROLE != 2 && kPrepThreads * i < C * vb / 16) {
            const int ev = e < C * vb / 16 && (e * 16) / vb < Cc ? e * 16 : 0;
            st.v[i] = *reinterpret_cast<const uint4*>(vc + ev);
        }
    }
    st.bl = to_f32(static_cast<const LT*>(a.bl)[row0 + (tid < Cc ? tid : 0)]);
}

// ROLE 0 forms everything; with two workgroups per chunk, ROLE 1 (the K side) forms K's DPFP,
// G, L, A, U_y, W_y, K^T and rho_k, and ROLE 2 (the Q side) forms K's and Q's DPFP, P, P~, Q and
// rho_q.
template <bool BF16, int C, bool LITE, bool PERSIST, int ROLE = 0>
__device__ __forceinline__ void prep_chunk(const ChunkArgs& a, int64_t blk, int64_t blk_next,
                                           PrepStage<BF16, C>& st) {
    using LT = typename ChunkTypes<BF16>::LT;
    constexpr int pair = ChunkTypes<BF16>::pair;
    constexpr int NT = C / 16, NTB = NT / pair;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    LT* Kr = reinterpret_cast<LT*>(smem + a.l_kr);        // [C][krs] K raw products
    LT* Qr = reinterpret_cast<LT*>(smem + a.l_qr);        // [C][krs] Q, then A' (below)
    LT* Xk = reinterpret_cast<LT*>(smem + a.l_x);         // [C][d_k] raw k rows (staging)
    LT* Xq = Xk + C * a.d_k;                              // [C][d_k] raw q rows (staging)
    float* Ls = reinterpret_cast<float*>(smem + a.l_ls);  // [C][lss] L (over the staging)
    LT* Ps = reinterpret_cast<LT*>(smem + a.l_ps);        // [C][pss] P~
    float* Li = reinterpret_cast<float*>(smem + a.l_li);  // [C][20] diagonal-block inverses
    LT* Xv = reinterpret_cast<LT*>(smem + a.l_xv);        // [C][d_v] raw v rows
    float* rhok = reinterpret_cast<float*>(smem + a.l_small);
    float* rhoq = rhok + C;
    float* betas = rhoq + C;

    // In the chunk loop the lane index passes through an empty asm statement in every chunk, so
    // the per-lane address arithmetic below is recomputed per chunk instead of hoisted out of
    // the loop (where it would stay live across the whole body).
    int tid_opaque = static_cast<int>(threadIdx.x);
    if constexpr (PERSIST) __asm__ volatile("" : "+v"(tid_opaque));
    const int tid = tid_opaque, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = l & 15, g4 = l >> 4;
    const int d_k = a.d_k, d_v = a.d_v, D = a.D, T = a.T, krs = a.krs;
    const int ND = D / 16, NDB = ND / pair, NVT = d_v / 16;
    const BhIndex bi = xcd_local(blk, a.BH, a.NC);
    const int bh = bi.bh, n = static_cast<int>(bi.i);
    const int64_t u = static_cast<int64_t>(bh) * a.NC + n;    // unit (b, h, chunk n)
    const int t0 = n * C, Cc = min(C, T - t0);

    // ---- stage the chunk's raw k, q, v rows (zeros past the sequence end) and beta from the
    //      registers loaded earlier, then issue the next chunk's loads into them
    {
        const int kb = d_k * static_cast<int>(sizeof(LT)), vb = d_v * static_cast<int>(sizeof(LT));
        auto masked = [](uint4 x, uint32_t m) { return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m); };
#pragma unroll
        for (int i = 0; i < PrepStage<BF16, C>::NU16; ++i) {
            const int e = tid + kPrepThreads * i;
            const uint32_t mk = (e * 16) / kb < Cc ? 0xffffffffu : 0u;
            if (e < C * kb / 16) {
                reinterpret_cast<uint4*>(Xk)[e] = masked(st.k[i], mk);
                if constexpr (ROLE != 1) reinterpret_cast<uint4*>(Xq)[e] = masked(st.q[i], mk);
            }
            if constexpr (!LITE && ROLE != 2) {
                const uint32_t mv = (e * 16) / vb < Cc ? 0xffffffffu : 0u;
                if (e < C * vb / 16) reinterpret_cast<uint4*>(Xv)[e] = masked(st.v[i], mv);
            }
        }
        if (tid < C) betas[tid] = tid < Cc ? sigmoid_stable(st.bl) : 0.0f;
        if (blk_next != blk) prep_stage_load<BF16, C, LITE, ROLE>(a, blk_next, st);
    }
    lds_barrier();

    dpfp_chunk<LT, LT, C, kPrepThreads, ROLE != 1>(Xk, Xq, Kr, Qr, krs, d_k, a.nu, w, l, rhok, rhoq);
    lds_barrier();

    if constexpr (ROLE != 0) {
        // one side's two units (G: K rows; P: Q rows), each over four quarters of D on the eight
        // waves; the quarters are added through LDS (over the staging rows, dead since DPFP)
        using GP = GPTiles<C>;
        static_assert(GP::NQ == 2, "two units per side (chunk 64)");
        const int wu = w & 1, quarter = w >> 1, Dq = D / 4;
        const int unit = (ROLE == 2 ? GP::NQ : 0) + wu;
        const int ra = wu, rb = GP::NT - 1 - wu;
        GP gp;
        gp_compute<BF16, C, false>(gp, Kr + quarter * Dq, Qr + quarter * Dq, krs, Dq, unit, l16, g4);
        f32x4* part = reinterpret_cast<f32x4*>(smem + a.l_x);
        if (quarter > 0) {
            f32x4* up = part + static_cast<int64_t>(wu * 3 + quarter - 1) * (GP::NT + 1) * 64 + l;
#pragma unroll
            for (int tb = 0; tb < GP::NT; ++tb) {
                if (tb <= ra) up[tb * 64] = gp.a[0][tb];
                if (tb <= rb) up[(ra + 1 + tb) * 64] = gp.b[0][tb];
            }
        }
        lds_barrier();
        if (quarter == 0) {
#pragma unroll
            for (int qq = 0; qq < 3; ++qq) {
                const f32x4* up = part + static_cast<int64_t>(wu * 3 + qq) * (GP::NT + 1) * 64 + l;
#pragma unroll
                for (int tb = 0; tb < GP::NT; ++tb) {
                    if (tb <= ra) gp.a[0][tb] += up[tb * 64];
                    if (tb <= rb) gp.b[0][tb] += up[(ra + 1 + tb) * 64];
                }
            }
        }
        lds_barrier();   // the staging rows are dead (L and P~ go over them)
        if (quarter == 0) gp_scale<BF16, C>(gp, rhok, rhoq, betas, Ls, a.lss, Ps, a.pss, unit, l16, g4);
    } else {
        // G/P has 2 NQ <= 4 units (one per wave of 0-3); waves 4-7 take the second half of D for
        // the same units, and the halves are added through LDS (over the staging rows, dead
        // since DPFP).  Each half must be whole k-steps (32 columns bf16, 16 fp32).
        using GP = GPTiles<C>;
        constexpr int NUNITS = 2 * GP::NQ;
        const bool ksplit = NUNITS <= 4 && D % 64 == 0;
        const int half = ksplit ? (w >> 2) : 0;
        const int wu = ksplit ? (w & 3) : w;             // the unit this wave computes (if < NUNITS)
        const int Dw = ksplit ? D / 2 : D;
        GP gp;
        gp_compute<BF16, C, false>(gp, Kr + half * Dw, Qr + half * Dw, krs, Dw, wu, l16, g4);
        if (ksplit) {
            // the unit's tiles (ra, 0..ra) then (rb, 0..rb): NT + 1 slots of 1 KiB per unit
            f32x4* part = reinterpret_cast<f32x4*>(smem + a.l_x);
            const int q = wu < GP::NQ ? wu : wu - GP::NQ;
            const int ra = q, rb = GP::NT - 1 - q;
            f32x4* up = part + static_cast<int64_t>(wu) * (GP::NT + 1) * 64 + l;
            if (w >= 4 && wu < NUNITS) {
#pragma unroll
                for (int tb = 0; tb < GP::NT; ++tb) {
                    if (tb <= ra) up[tb * 64] = gp.a[0][tb];
                    if (tb <= rb) up[(ra + 1 + tb) * 64] = gp.b[0][tb];
                }
            }
            lds_barrier();
            if (w < 4 && wu < NUNITS) {
#pragma unroll
                for (int tb = 0; tb < GP::NT; ++tb) {
                    if (tb <= ra) gp.a[0][tb] += up[tb * 64];
                    if (tb <= rb) gp.b[0][tb] += up[(ra + 1 + tb) * 64];
                }
            }
        }
        lds_barrier();   // the staging rows are dead (L and P~ go over them)
        gp_scale<BF16, C>(gp, rhok, rhoq, betas, Ls, a.lss, Ps, a.pss, w, l16, g4);
    }
    lds_barrier();

    char* ws = a.ws;
    // P~ write-out, run by the waves the A phase leaves idle (A does not touch P~); the K^T
    // blocks are written by the W_y product below, which loads them as its operands anyway
    auto write_pa = [&](int e0, int estep) {
        // PA: blocks (ta, j), j < NTB; tiles above the diagonal are zero
        char* pa = ws + a.o_pa + u * (static_cast<int64_t>(C) * C * sizeof(LT));
        for (int e = e0; e < NT * NTB * 64; e += estep) {
            const int blk = e >> 6, lam = e & 63, ta = blk / NTB, j = blk % NTB;
            const LT* src = Ps + (16 * ta + (lam & 15)) * a.pss + 16 * pair * j + 4 * (lam >> 4);
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if constexpr (BF16) {
                if (2 * j <= ta) {
                    const uint2 lo = *reinterpret_cast<const uint2*>(src);
                    val.x = lo.x;
                    val.y = lo.y;
                }
                if (2 * j + 1 <= ta) {
                    const uint2 hi = *reinterpret_cast<const uint2*>(src + 16);
                    val.z = hi.x;
                    val.w = hi.y;
                }
            } else {
                if (j <= ta) val = *reinterpret_cast<const uint4*>(src);
                if (a.split) {
                    store_split(pa + ((static_cast<int64_t>(blk - (j & 1)) * 64) + lam) * 16, j, as_f32x4(val));
                    continue;
                }
            }
            *reinterpret_cast<uint4*>(pa + static_cast<int64_t>(e) * 16) = val;
        }
    };

    // QA: blocks (tt, j), j < NDB
    auto write_qa = [&](int e0, int estep) {
        char* qa = ws + a.o_qa + u * (static_cast<int64_t>(C) * D * sizeof(LT));
        for (int e = e0; e < NT * NDB * 64; e += estep) {
            const int blk = e >> 6, lam = e & 63, tt = blk / NDB, j = blk % NDB;
            const LT* src = Qr + (16 * tt + (lam & 15)) * krs + 16 * pair * j + 4 * (lam >> 4);
            uint4 val;
            if constexpr (BF16) {
                const uint2 lo = *reinterpret_cast<const uint2*>(src);
                const uint2 hi = *reinterpret_cast<const uint2*>(src + 16);
                val = make_uint4(lo.x, lo.y, hi.x, hi.y);
            } else {
                val = *reinterpret_cast<const uint4*>(src);
                if (a.split) {
                    store_split(qa + ((static_cast<int64_t>(blk - (j & 1)) * 64) + lam) * 16, j, as_f32x4(val));
                    continue;
                }
            }
            *reinterpret_cast<uint4*>(qa + static_cast<int64_t>(e) * 16) = val;
        }
    };

    if constexpr (ROLE == 2) {
        // the Q side ends here: Q, P~ and rho_q go out
        write_qa(tid, kPrepThreads);
        write_pa(tid, kPrepThreads);
        if (tid < C) reinterpret_cast<float*>(ws + a.o_rq)[u * C + tid] = rhoq[tid];
        return;
    }

    // ---- diagonal-block inverses (the first C threads); write-out of the Q blocks by the other
    //      waves, and of the normalisers
    static_assert(C <= 64, "the inverses take wave 0 alone");
    if (tid < C) diag_inverse(Ls, a.lss, Li, tid);
    if (!LITE && ROLE == 0 && w > 0) write_qa(tid - 64, kPrepThreads - 64);
    if (tid < C) {
        reinterpret_cast<float*>(ws + a.o_rk)[u * C + tid] = rhok[tid];
        if constexpr (ROLE == 0) reinterpret_cast<float*>(ws + a.o_rq)[u * C + tid] = rhoq[tid];
    }
    lds_barrier();   // Li complete; Q is dead (its space holds A')

    // ---- A = (I + L)^-1 by block columns (column block tb = w per wave), stored twice with
    //      its columns scaled: A' = A diag(beta rho_k) and A'' = A diag(beta), each as fp32 or
    //      as a bf16 hi + lo pair whose sum carries the fp32 value to about 2^-17.
    float* Af = reinterpret_cast<float*>(smem + a.l_qr);           // fp32: A' [C][aps]
    float* Bf = Af + C * a.aps;                                      //       A''
    u16* Ah = reinterpret_cast<u16*>(smem + a.l_qr);                // bf16: A' hi, lo
    u16* Al = Ah + C * a.aps;
    u16* Bh = Al + C * a.aps;                                        //       A'' hi, lo
    u16* Bl = Bh + C * a.aps;
    const int aps = a.aps;
    static_assert(NT < kPrepWaves, "waves left over for the write-outs");
    if (ROLE == 0 && w >= NT) write_pa(tid - 64 * NT, kPrepThreads - 64 * NT);
    if (w < NT) {
        const int tb = w;
        const float bsc = betas[16 * tb + l16];
        const float csc = bsc * rhok[16 * tb + l16];
        f32x4 Ab[NT];
#pragma unroll
        for (int ta = 0; ta < NT; ++ta) {
            f32x4 val = zero4();
            if (ta == tb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = Li[(16 * ta + 4 * g4 + e) * kLiStride + l16];
            } else if (ta > tb) {
                // A[ta][tb] = -Li[ta] sum_{tc = tb}^{ta-1} L[ta][tc] A[tc][tb]
                f32x4 acc = zero4();
#pragma unroll
                for (int tc = 0; tc < NT; ++tc) {
                    if (tc >= tb && tc < ta) {
                        const float4 l4 = *reinterpret_cast<const float4*>(
                            Ls + (16 * ta + l16) * a.lss + 16 * tc + 4 * g4);
                        acc = mfma_f32_k4(l4.x, Ab[tc][0], acc);
                        acc = mfma_f32_k4(l4.y, Ab[tc][1], acc);
                        acc = mfma_f32_k4(l4.z, Ab[tc][2], acc);
                        acc = mfma_f32_k4(l4.w, Ab[tc][3], acc);
                    }
                }
                const float4 i4 = *reinterpret_cast<const float4*>(Li + (16 * ta + l16) * kLiStride + 4 * g4);
                val = mfma_f32_k4(i4.x, acc[0], val);
                val = mfma_f32_k4(i4.y, acc[1], val);
                val = mfma_f32_k4(i4.z, acc[2], val);
                val = mfma_f32_k4(i4.w, acc[3], val);
                val = -val;
            }
            Ab[ta] = val;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int at = (16 * ta + 4 * g4 + e) * aps + 16 * tb + l16;
                const float x = val[e] * csc, y = val[e] * bsc;
                if constexpr (BF16) {
                    const u16 xh = f32_to_bf16_bits(x), yh = f32_to_bf16_bits(y);
                    Ah[at] = xh;
                    Al[at] = f32_to_bf16_bits(x - bf16_bits_to_f32(xh));
                    Bh[at] = yh;
                    Bl[at] = f32_to_bf16_bits(y - bf16_bits_to_f32(yh));
                } else {
                    Af[at] = x;
                    Bf[at] = y;
                }
            }
        }
    }
    lds_barrier();

    if constexpr (LITE) {
        static_assert(BF16, "the compact mode serves the bf16 streaming forward");
        // AH, AL: A-operand blocks (ta, j), j < NTB, of A'' hi and lo (slot (h, e) of lane l =
        // A''[16 ta + l % 16][16 (2 j + h) + 4 (l / 16) + e]); blocks above the diagonal are zero
        char* ah = ws + a.o_ah + u * (static_cast<int64_t>(C) * C * 2);
        char* al = ws + a.o_al + u * (static_cast<int64_t>(C) * C * 2);
        for (int e = tid; e < NT * NTB * 64; e += kPrepThreads) {
            const int blk = e >> 6, lam = e & 63, ta = blk / NTB, j = blk % NTB;
            const int at = (16 * ta + (lam & 15)) * aps + 32 * j + 4 * (lam >> 4);
            const uint2 h0 = *reinterpret_cast<const uint2*>(Bh + at);
            const uint2 h1 = *reinterpret_cast<const uint2*>(Bh + at + 16);
            const uint2 l0 = *reinterpret_cast<const uint2*>(Bl + at);
            const uint2 l1 = *reinterpret_cast<const uint2*>(Bl + at + 16);
            *reinterpret_cast<uint4*>(ah + static_cast<int64_t>(e) * 16) = make_uint4(h0.x, h0.y, h1.x, h1.y);
            *reinterpret_cast<uint4*>(al + static_cast<int64_t>(e) * 16) = make_uint4(l0.x, l0.y, l1.x, l1.y);
        }
        return;
    }

    // ---- U_y = A'' V as accumulator tiles (t-tile, v-tile), one v-tile per wave and pass
    char* uy = ws + a.o_uy + u * (static_cast<int64_t>(C) * d_v * 4);
    for (int vt = w; vt < NVT; vt += kPrepWaves) {
        f32x4 acc[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) acc[tt] = zero4();
        if constexpr (BF16) {
            // k-slot (h, e) of lane group g is row s = 32 kb + 16 h + 4 g + e; V by transpose reads
#pragma unroll
            for (int kb = 0; kb < C / 32; ++kb) {
                const LT* vp = Xv + (32 * kb + 4 * g4 + (l16 >> 2)) * d_v + 16 * vt + 4 * (l16 & 3);
                const bf16x4 c0 = lds_read_tr_b16x4(vp);
                const bf16x4 c1 = lds_read_tr_b16x4(vp + 16 * d_v);
                const bf16x8 bv = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    if (32 * kb <= 16 * tt + 15) {
                        const int ho = (16 * tt + l16) * aps + 32 * kb + 4 * g4;
                        const bf16x8 ah = __builtin_shufflevector(lds_read_b64_single(Bh, ho),
                                                                  lds_read_b64_single(Bh, ho + 16),
                                                                  0, 1, 2, 3, 4, 5, 6, 7);
                        const bf16x8 al = __builtin_shufflevector(lds_read_b64_single(Bl, ho),
                                                                  lds_read_b64_single(Bl, ho + 16),
                                                                  0, 1, 2, 3, 4, 5, 6, 7);
                        acc[tt] = mfma_bf16_k32(ah, bv, acc[tt]);
                        acc[tt] = mfma_bf16_k32(al, bv, acc[tt]);
                    }
                }
            }
        } else {
            // fp32 operands split into bf16 hi + lo, three MFMAs per 32-row k-step; k-slot
            // (h, e) of lane group g is row s = 32 kb + 16 h + 4 g + e
#pragma unroll
            for (int kb = 0; kb < C / 32; ++kb) {
                f32x4 v0, v1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v0[e] = to_f32(Xv[(32 * kb + 4 * g4 + e) * d_v + 16 * vt + l16]);
                    v1[e] = to_f32(Xv[(32 * kb + 16 + 4 * g4 + e) * d_v + 16 * vt + l16]);
                }
                const uint4 bh = pack_bf16x8(v0, v1), bl = bf16_lo_part(v0, v1);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    if (32 * kb <= 16 * tt + 15) {
                        const float* ap = Bf + (16 * tt + l16) * aps + 32 * kb + 4 * g4;
                        const f32x4 a0 = *reinterpret_cast<const f32x4*>(ap);
                        const f32x4 a1 = *reinterpret_cast<const f32x4*>(ap + 16);
                        acc[tt] = mfma_split(pack_bf16x8(a0, a1), bf16_lo_part(a0, a1), bh, bl, acc[tt]);
                    }
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
            *reinterpret_cast<f32x4*>(blk_ptr(uy, tt * NVT + vt, l)) = acc[tt];
    }

    // ---- W_y^T = K^T A'^T as accumulator tiles (d-tile, t-tile), which are the WyA blocks:
    //      lane l, slot e of tile (dt, tt) holds W_y[16 tt + l % 16][16 dt + 4 (l / 16) + e].
    char* wy = ws + a.o_wy + u * (static_cast<int64_t>(C) * D * sizeof(LT));
    char* kt = ws + a.o_kt + u * (static_cast<int64_t>(C) * D * sizeof(LT));   // KtA blocks
    if constexpr (BF16) {
        // k-slot (h, e) of lane group g is row s = 32 kb + 16 h + 4 g + e of the chunk; the K^T
        // operand comes from the row-major K tile by two LDS transpose reads.
        for (int j = w; j < NDB; j += kPrepWaves) {
            f32x4 acc[2][NT];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) acc[h][tt] = zero4();
#pragma unroll
            for (int kb = 0; kb < C / 32; ++kb) {
                bf16x8 ka[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const LT* kp = Kr + (32 * kb + 4 * g4 + (l16 >> 2)) * krs + 16 * (2 * j + h) + 4 * (l16 & 3);
                    const bf16x4 c0 = lds_read_tr_b16x4(kp);
                    const bf16x4 c1 = lds_read_tr_b16x4(kp + 16 * krs);
                    ka[h] = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
                    // the same operand is the KtA block (d-tile 2 j + h, k-block kb)
                    *reinterpret_cast<uint4*>(blk_ptr(kt, static_cast<int64_t>(2 * j + h) * NTB + kb, l)) =
                        __builtin_bit_cast(uint4, ka[h]);
                }
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    if (32 * kb <= 16 * tt + 15) {
                        const int ho = (16 * tt + l16) * aps + 32 * kb + 4 * g4;
                        const bf16x4 h0 = lds_read_b64_single(Ah, ho);
                        const bf16x4 h1 = lds_read_b64_single(Ah, ho + 16);
                        const bf16x4 o0 = lds_read_b64_single(Al, ho);
                        const bf16x4 o1 = lds_read_b64_single(Al, ho + 16);
                        const bf16x8 bh = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
                        const bf16x8 bl = __builtin_shufflevector(o0, o1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            acc[h][tt] = mfma_bf16_k32(ka[h], bh, acc[h][tt]);
                            acc[h][tt] = mfma_bf16_k32(ka[h], bl, acc[h][tt]);
                        }
                    }
                }
            }
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
                *reinterpret_cast<uint4*>(blk_ptr(wy, tt * NDB + j, l)) = pack_bf16x8(acc[0][tt], acc[1][tt]);
        }
    } else {
        // fp32 operands split into bf16 hi + lo, three MFMAs per 32-row k-step; k-slot (h, e)
        // of lane group g is row s = 32 kb + 16 h + 4 g + e, so the K^T operand halves are the
        // KtA blocks (dt, 2 kb + h) as they stand.
        for (int dt = w; dt < ND; dt += kPrepWaves) {
            f32x4 acc[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) acc[tt] = zero4();
#pragma unroll
            for (int kb = 0; kb < C / 32; ++kb) {
                f32x4 k0, k1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    k0[e] = to_f32(Kr[(32 * kb + 4 * g4 + e) * krs + 16 * dt + l16]);
                    k1[e] = to_f32(Kr[(32 * kb + 16 + 4 * g4 + e) * krs + 16 * dt + l16]);
                }
                const uint4 kh = pack_bf16x8(k0, k1), kl = bf16_lo_part(k0, k1);
                if (a.split) {
                    // the split pair of KtA blocks (dt, 2 kb), (dt, 2 kb + 1), of K~^T =
                    // K^T diag(rho_k): the staged chain then updates with U itself
                    const f32x4 r0 = *reinterpret_cast<const f32x4*>(rhok + 32 * kb + 4 * g4);
                    const f32x4 r1 = *reinterpret_cast<const f32x4*>(rhok + 32 * kb + 16 + 4 * g4);
                    const f32x4 s0 = k0 * r0, s1 = k1 * r1;
                    char* kp = blk_ptr(kt, static_cast<int64_t>(dt) * NTB + 2 * kb, l);
                    *reinterpret_cast<uint4*>(kp) = pack_bf16x8(s0, s1);
                    *reinterpret_cast<uint4*>(kp + 1024) = bf16_lo_part(s0, s1);
                } else {
                    *reinterpret_cast<f32x4*>(blk_ptr(kt, static_cast<int64_t>(dt) * NTB + 2 * kb, l)) = k0;
                    *reinterpret_cast<f32x4*>(blk_ptr(kt, static_cast<int64_t>(dt) * NTB + 2 * kb + 1, l)) = k1;
                }
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    if (32 * kb <= 16 * tt + 15) {
                        const float* bp = Af + (16 * tt + l16) * aps + 32 * kb + 4 * g4;
                        const f32x4 b0 = *reinterpret_cast<const f32x4*>(bp);
                        const f32x4 b1 = *reinterpret_cast<const f32x4*>(bp + 16);
                        acc[tt] = mfma_split(kh, kl, pack_bf16x8(b0, b1), bf16_lo_part(b0, b1), acc[tt]);
                    }
                }
            }
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                if (a.split) store_split(blk_ptr(wy, tt * NDB + (dt & ~1), l), dt, acc[tt]);
                else *reinterpret_cast<f32x4*>(blk_ptr(wy, tt * NDB + dt, l)) = acc[tt];
            }
        }
    }
}

// The prep kernel.  One workgroup per chunk; or, with PERSIST, where there are more chunks than
// workgroups fit at once, each workgroup takes chunks blockIdx.x, + gridDim.x, ... (the launch
// sizes the grid to the resident workgroups, a multiple of 8, so every chunk a workgroup takes
// keeps its XCD) and the next chunk's raw rows load into registers while the current one is
// processed.
template <bool BF16, int C, bool LITE = false, bool PERSIST = false>
__global__ __launch_bounds__(kPrepThreads, 1) void delta_prep_kernel(ChunkArgs a) {
    PrepStage<BF16, C> st;
    if constexpr (!PERSIST) {
        prep_stage_load<BF16, C, LITE>(a, blockIdx.x, st);
        prep_chunk<BF16, C, LITE, false>(a, blockIdx.x, blockIdx.x, st);
    } else {
        const int64_t total = static_cast<int64_t>(a.BH) * a.NC;
        int64_t blk = blockIdx.x;
        if (blk < total) prep_stage_load<BF16, C, LITE>(a, blk, st);
        for (; blk < total; blk += gridDim.x) {
            const int64_t nxt = blk + gridDim.x < total ? blk + gridDim.x : blk;
            prep_chunk<BF16, C, LITE, true>(a, blk, nxt, st);
            lds_barrier();                 // LDS of this chunk is dead before the next staging
        }
    }
}

// The prep as two workgroups per chunk (chunk 64, where twice the chunks fit on the GPU at
// once): workgroups [0, BH NC) take the K side of chunk blockIdx.x, workgroups [BH NC, 2 BH NC)
// the Q side of chunk blockIdx.x - BH NC.
template <bool BF16, int C>
__global__ __launch_bounds__(kPrepThreads, 1) void delta_prep_split_kernel(ChunkArgs a) {
    const int64_t total = static_cast<int64_t>(a.BH) * a.NC;
    PrepStage<BF16, C> st;
    if (static_cast<int64_t>(blockIdx.x) < total) {
        prep_stage_load<BF16, C, false, 1>(a, blockIdx.x, st);
        prep_chunk<BF16, C, false, false, 1>(a, blockIdx.x, blockIdx.x, st);
    } else {
        const int64_t blk = blockIdx.x - total;
        prep_stage_load<BF16, C, false, 2>(a, blk, st);
        prep_chunk<BF16, C, false, false, 2>(a, blk, blk, st);
    }
}

// ------------------------------------------------------------------------------------------
// chain: one workgroup of DP waves per (b, h, 16-column v-tile r); wave w holds the fp32 memory
// tiles W^T[16 (dt0 + i) .. +16][v-tile r], i < NDP (dt0 = w NDP), in MFMA accumulators.  Per
// chunk: store the chunk-start memory (Wn, B blocks); S = W_y W^T, partial over the wave's
// d-tiles, summed over the waves through LDS; U = U_y - S (stored as Un, B blocks);
// W^T += K^T (rho_k o U).
// The next chunk's operand blocks are loaded into registers right after each set's last use.
// The loop body has no data-dependent branches around memory operations (the last chunk's
// prefetch re-reads that chunk; every wave stores the full U tile it computed, identical
// across waves), so the compiler's wait counters stay exact and every wait covers just the
// loads it needs, never the prefetch in flight.
template <bool BF16, int C, int NDP, int DP>
__global__ __launch_bounds__(64 * DP, 1) void delta_chain_kernel(ChunkArgs a) {
    using LT = typename ChunkTypes<BF16>::LT;
    constexpr int pair = ChunkTypes<BF16>::pair;
    constexpr int NT = C / 16, NTB = NT / pair, NDPB = NDP / pair;
    static_assert(NDP % pair == 0, "bf16 waves hold whole d-tile pairs");
    // partial S of each wave, double-buffered: [2][DP][NT] tiles of 64 lanes
    extern __shared__ __attribute__((aligned(16))) char smem[];
    f32x4* Red = reinterpret_cast<f32x4*>(smem);

    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = l & 15, g4 = l >> 4;
    const int d_k = a.d_k, D = a.D, NC = a.NC;
    const int ND = D / 16, NDB = ND / pair, NVT = a.d_v / 16;
    const BhIndex bi = xcd_local(blockIdx.x, a.BH, NVT);      // workgroup -> (b, h, v-tile r)
    const int bh = bi.bh, r = static_cast<int>(bi.i);
    const int dt0 = w * NDP;
    const int vcol = 16 * r + l16;

    f32x4 Wst[NDP];
#pragma unroll
    for (int i = 0; i < NDP; ++i) {
        Wst[i] = zero4();
        if (a.W0) {
            // internal columns c0 .. c0+3 = positions (o, o + d_k, o + 1, o + d_k + 1)
            const float* src = a.W0 + (static_cast<int64_t>(bh) * a.d_v + vcol) * D +
                               orig_col(16 * (dt0 + i) + 4 * g4, d_k);
            const float2 lo = *reinterpret_cast<const float2*>(src);
            const float2 hi = *reinterpret_cast<const float2*>(src + d_k);
            Wst[i] = f32x4{lo.x, hi.x, lo.y, hi.y};
        }
    }

    const int64_t szCD = static_cast<int64_t>(C) * D * sizeof(LT);
    const int64_t szUy = static_cast<int64_t>(C) * a.d_v * 4;
    const int64_t szWn = static_cast<int64_t>(D) * a.d_v * sizeof(LT);
    const int64_t szUn = static_cast<int64_t>(C) * a.d_v * sizeof(LT);
    // Per-lane base addresses of this workgroup's blocks; chunk uu adds uu * region size.
    const char* wyB = a.ws + a.o_wy + (static_cast<int64_t>(dt0 / pair) * 64 + l) * 16;
    const char* ktB = a.ws + a.o_kt + (static_cast<int64_t>(dt0) * NTB * 64 + l) * 16;
    const char* uyB = a.ws + a.o_uy + (static_cast<int64_t>(r) * 64 + l) * 16;
    const float* rkB = reinterpret_cast<const float*>(a.ws + a.o_rk) + 4 * g4;
    char* wnB = a.ws + a.o_wn + ((static_cast<int64_t>(dt0 / pair) * NVT + r) * 64 + l) * 16;
    char* unB = a.ws + a.o_un + (static_cast<int64_t>(r) * 64 + l) * 16;

    uint4 wy[NT][NDPB];     // WyA blocks (tt, dt0 / pair + i)
    uint4 kt[NDP][NTB];     // KtA blocks (dt0 + i, j)
    f32x4 uy[NT];           // U_y tiles (tt, r)
    f32x4 rk[NT];           // rho_k of rows 16 tt + 4 g4 + e
    auto load_wy = [&](int64_t uu) {
        const char* p = wyB + uu * szCD;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int i = 0; i < NDPB; ++i)
                wy[tt][i] = *reinterpret_cast<const uint4*>(p + (static_cast<int64_t>(tt) * NDB + i) * 1024);
    };
    auto load_uy = [&](int64_t uu) {
        const char* p = uyB + uu * szUy;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            uy[tt] = *reinterpret_cast<const f32x4*>(p + static_cast<int64_t>(tt) * NVT * 1024);
            rk[tt] = *reinterpret_cast<const f32x4*>(rkB + uu * C + 16 * tt);
        }
    };
    auto load_kt = [&](int64_t uu) {
        const char* p = ktB + uu * szCD;
#pragma unroll
        for (int i = 0; i < NDP; ++i)
#pragma unroll
            for (int j = 0; j < NTB; ++j)
                kt[i][j] = *reinterpret_cast<const uint4*>(p + (static_cast<int64_t>(i) * NTB + j) * 1024);
    };
    const int64_t u0 = static_cast<int64_t>(bh) * NC;
    const int64_t ulast = u0 + NC - 1;
    if (NC > 0) {
        load_wy(u0);
        load_uy(u0);
        load_kt(u0);
    }

    for (int n = 0; n < NC; ++n) {
        const int64_t uu = u0 + n;
        const int64_t un = uu + 1 <= ulast ? uu + 1 : ulast;  // next chunk (clamped)
        const int buf = n & 1;
        // chunk-start memory for the output kernel
#pragma unroll
        for (int i = 0; i < NDPB; ++i) {
            uint4 val;
            if constexpr (BF16) val = pack_bf16x8(Wst[2 * i], Wst[2 * i + 1]);
            else val = __builtin_bit_cast(uint4, Wst[i]);
            *reinterpret_cast<uint4*>(wnB + uu * szWn + static_cast<int64_t>(i) * NVT * 1024) = val;
        }
        // S = W_y W^T over this wave's d-tiles
        f32x4 S[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) S[tt] = zero4();
#pragma unroll
        for (int i = 0; i < NDPB; ++i) {
            if constexpr (BF16) {
                const uint4 bw = pack_bf16x8(Wst[2 * i], Wst[2 * i + 1]);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
                    S[tt] = mfma_bf16_k32(as_bf16x8(wy[tt][i]), as_bf16x8(bw), S[tt]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt)
                        S[tt] = mfma_f32_k4(as_f32x4(wy[tt][i])[e], Wst[i][e], S[tt]);
            }
        }
        load_wy(un);
        if constexpr (DP > 1) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) Red[((buf * DP + w) * NT + tt) * 64 + l] = S[tt];
            lds_barrier();
            f32x4 part[DP][NT];
#pragma unroll
            for (int pp = 0; pp < DP; ++pp)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) part[pp][tt] = Red[((buf * DP + pp) * NT + tt) * 64 + l];
            // all partial reads go out together, ahead of their uses (one LDS round trip)
            __builtin_amdgcn_sched_group_barrier(0x100, DP * NT, 0);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x4 s2 = part[0][tt];
#pragma unroll
                for (int pp = 1; pp < DP; ++pp) s2 += part[pp][tt];
                S[tt] = s2;
            }
        }
        f32x4 U[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) U[tt] = uy[tt] - S[tt];
        // U for the output kernel (B blocks (j, r)); every wave holds the same U
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
            uint4 val;
            if constexpr (BF16) val = pack_bf16x8(U[2 * j], U[2 * j + 1]);
            else val = __builtin_bit_cast(uint4, U[j]);
            *reinterpret_cast<uint4*>(unB + uu * szUn + static_cast<int64_t>(j) * NVT * 1024) = val;
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) U[tt] *= rk[tt];
        load_uy(un);
        // W^T += K^T (rho_k o U); fp32 sums even and odd t-tiles in separate accumulators so
        // that consecutive MFMAs are independent
        if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < NTB; ++j) {
                const uint4 bu = pack_bf16x8(U[2 * j], U[2 * j + 1]);
#pragma unroll
                for (int i = 0; i < NDP; ++i) Wst[i] = mfma_bf16_k32(as_bf16x8(kt[i][j]), as_bf16x8(bu), Wst[i]);
            }
        } else {
            f32x4 odd[NDP];
#pragma unroll
            for (int i = 0; i < NDP; ++i) odd[i] = zero4();
#pragma unroll
            for (int j = 0; j < NTB; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int i = 0; i < NDP; ++i) {
                        f32x4& dst = (j & 1) ? odd[i] : Wst[i];
                        dst = mfma_f32_k4(as_f32x4(kt[i][j])[e], U[j][e], dst);
                    }
#pragma unroll
            for (int i = 0; i < NDP; ++i) Wst[i] += odd[i];
        }
        load_kt(un);
    }

    if (a.Wf) {
#pragma unroll
        for (int i = 0; i < NDP; ++i) {
            float* dst = a.Wf + (static_cast<int64_t>(bh) * a.d_v + vcol) * D +
                         orig_col(16 * (dt0 + i) + 4 * g4, d_k);
            *reinterpret_cast<float2*>(dst) = make_float2(Wst[i][0], Wst[i][2]);
            *reinterpret_cast<float2*>(dst + d_k) = make_float2(Wst[i][1], Wst[i][3]);
        }
    }
}

// ------------------------------------------------------------------------------------------
// chain, staged: the same recurrence with the operand fetch taken off the waves that run the
// MFMAs.  One workgroup of 8 waves per (b, h, v-tile r): compute waves 0..3 and loader waves
// 4..7 (loader 4 + w shares a SIMD with compute wave w and fetches its blocks).  Loaders copy the
// next chunk's blocks straight into LDS with global_load_lds (lane i's 16 bytes land at the
// block base + 16 i, the operand layout) into a two-slot ring.  Compute wave w:
//   * owns row tile t = w of S = W_y W^T (GEMM1) over all of D, reading W^T from an LDS copy
//     that every wave refreshes with its d-tiles at the top of the chunk;
//   * forms U = U_y - S for its rows and publishes rho_k o U in LDS;
//   * owns d-tiles dt0 = w NDP .. +NDP of the memory for the update W^T += K^T (rho_k o U).
// Two barriers per chunk: B1 after the W^T copy is written (and, for the loaders, after the
// slot they refill has been read), B2 after rho_k o U is written.  Each LDS buffer is written
// only after the barrier that follows its last read, so the W^T copy and U need one buffer
// each and the operand ring two slots.
constexpr int kChainWaves = 4;

template <bool BF16, int C, int NDP>
struct StagedLayout {
    static constexpr int pair = BF16 ? 2 : 1;
    static constexpr int NT = C / 16, NTB = NT / pair;
    static constexpr int ND = kChainWaves * NDP, NDB = ND / pair;
    static constexpr int PW = NDB + NDP * NTB + 1;             // blocks per compute wave and slot
    static constexpr int SLOT = (kChainWaves * PW + 1) * 1024;  // + rho_k (C floats)
    static constexpr int XOFF = 2 * SLOT;                       // W^T copy: NDB blocks
    static constexpr int UOFF = XOFF + NDB * 1024;              // rho_k o U: NT fp32 tiles
    static constexpr int BYTES = UOFF + NT * 1024;
};

template <bool BF16, int C, int NDP>
__global__ __launch_bounds__(512, 1) void delta_chain_staged_kernel(ChunkArgs a) {
    using LT = typename ChunkTypes<BF16>::LT;
    using SL = StagedLayout<BF16, C, NDP>;
    constexpr int pair = SL::pair, NT = SL::NT, NTB = SL::NTB, NDB = SL::NDB;
    constexpr int NDPB = NDP / pair;
    static_assert(NDP % pair == 0, "bf16 waves hold whole d-tile pairs");
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, l = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool loader = wave >= kChainWaves;
    const int w = loader ? wave - kChainWaves : wave;    // the compute wave served or run
    const int l16 = l & 15, g4 = l >> 4;
    const int d_k = a.d_k, D = a.D, NC = a.NC, NVT = a.d_v / 16;
    const BhIndex bi = xcd_local(blockIdx.x, a.BH, NVT);
    const int bh = bi.bh, r = static_cast<int>(bi.i);
    const int dt0 = w * NDP;
    const int vcol = 16 * r + l16;
    const int64_t u0 = static_cast<int64_t>(bh) * NC;
    const int64_t szCD = static_cast<int64_t>(C) * D * sizeof(LT);
    char* X = smem + SL::XOFF;
    char* Ub = smem + SL::UOFF;
    auto lane16 = [&](char* base, int blk) { return base + blk * 1024 + l * 16; };

    // ---- loader: chunk uu's blocks for compute wave w into ring slot `slot`
    auto issue_loads = [&](int64_t uu, int slot) {
        char* sw = smem + slot * SL::SLOT + w * SL::PW * 1024;
        const char* wy = a.ws + a.o_wy + uu * szCD + (static_cast<int64_t>(w) * NDB * 64 + l) * 16;
        const char* kt = a.ws + a.o_kt + uu * szCD + (static_cast<int64_t>(dt0) * NTB * 64 + l) * 16;
        typedef __attribute__((address_space(1))) const void* gptr;
        typedef __attribute__((address_space(3))) void* lptr;
        if (w < NT) {
#pragma unroll
            for (int j = 0; j < NDB; ++j)
                __builtin_amdgcn_global_load_lds((gptr)(wy + j * 1024), (lptr)(sw + j * 1024), 16, 0, 0);
            const char* uy = a.ws + a.o_uy + uu * (static_cast<int64_t>(C) * a.d_v * 4) +
                             ((static_cast<int64_t>(w) * NVT + r) * 64 + l) * 16;
            __builtin_amdgcn_global_load_lds((gptr)uy, (lptr)(sw + (SL::PW - 1) * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int b = 0; b < NDP * NTB; ++b)
            __builtin_amdgcn_global_load_lds((gptr)(kt + b * 1024), (lptr)(sw + (NDB + b) * 1024), 16, 0, 0);
        if (w == 0 && l < C) {
            const float* rk = reinterpret_cast<const float*>(a.ws + a.o_rk) + uu * C + l;
            __builtin_amdgcn_global_load_lds((gptr)rk, (lptr)(smem + slot * SL::SLOT + kChainWaves * SL::PW * 1024), 4, 0, 0);
        }
    };
    constexpr int kWaitVm0 = 0x0F70;   // s_waitcnt vmcnt(0), other counters unconstrained

    if (loader) {
        // Loader loop: the same barrier sequence as the compute loop (one before it, B1 and B2 per
        // chunk).  After B1(n) the slot of chunk n - 1 is free; chunk n + 1 goes there and is
        // complete before this wave arrives at B1(n + 1).
        // A loader publishes LDS only through its LDS-DMA loads, which it waits for explicitly
        // (vmcnt) before B1; its barriers are bare so that B2 does not wait for the loads just
        // issued.
        auto bare_barrier = []() {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        if (NC > 0) {
            issue_loads(u0, 0);
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
        }
        bare_barrier();
        for (int n = 0; n < NC; ++n) {
            bare_barrier();                                          // B1
            if (n + 1 < NC) issue_loads(u0 + n + 1, (n & 1) ^ 1);
            bare_barrier();                                          // B2
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
        }
        return;
    }

    f32x4 Wst[NDP];
#pragma unroll
    for (int i = 0; i < NDP; ++i) {
        Wst[i] = zero4();
        if (a.W0) {
            // internal columns c0 .. c0+3 = positions (o, o + d_k, o + 1, o + d_k + 1)
            const float* src = a.W0 + (static_cast<int64_t>(bh) * a.d_v + vcol) * D +
                               orig_col(16 * (dt0 + i) + 4 * g4, d_k);
            const float2 lo = *reinterpret_cast<const float2*>(src);
            const float2 hi = *reinterpret_cast<const float2*>(src + d_k);
            Wst[i] = f32x4{lo.x, hi.x, lo.y, hi.y};
        }
    }
    lds_barrier();

    const int64_t szWn = static_cast<int64_t>(D) * a.d_v * sizeof(LT);
    const int64_t szUn = static_cast<int64_t>(C) * a.d_v * sizeof(LT);
    // fp32 (split format): the outputs of the chunk are formed here, Y = rho_q o (Q W^T) + P~ U
    // for row tile w, from the Q and P~ blocks (registers, fetched a chunk ahead) and the W^T
    // copy and U the chain already holds in LDS; no chunk-start memories or U go to the
    // workspace and no output kernel runs.
    constexpr bool FUSE_Y = !BF16;
    constexpr int NQB = FUSE_Y ? NDB : 1, NPB = FUSE_Y ? NT : 1;
    uint4 qy[NQB], py[NPB];
    f32x4 rqv = zero4(), qacc = zero4();
    auto load_q = [&](int64_t uu) {
        if (!FUSE_Y || w >= NT) return;
        const char* qa = a.ws + a.o_qa + uu * (static_cast<int64_t>(C) * D * 4);
#pragma unroll
        for (int j = 0; j < NQB; ++j) qy[j] = *reinterpret_cast<const uint4*>(blk_ptr(qa, w * NDB + j, l));
    };
    auto load_p = [&](int64_t uu) {
        if (!FUSE_Y || w >= NT) return;
        const char* pa = a.ws + a.o_pa + uu * (static_cast<int64_t>(C) * C * 4);
#pragma unroll
        for (int j = 0; j < NPB; ++j) py[j] = *reinterpret_cast<const uint4*>(blk_ptr(pa, w * NT + j, l));
        rqv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.ws + a.o_rq) + uu * C + 16 * w + 4 * g4);
    };
    // y of this (b, h), columns 16 r + l16, as a buffer whose range check drops rows past T
    const __amdgpu_buffer_rsrc_t yrsrc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<float*>(a.y) + static_cast<int64_t>(bh) * a.T * a.d_v, static_cast<short>(0),
        a.T * a.d_v * 4, 0x00020000);
    if (NC > 0) {
        load_q(u0);
        load_p(u0);
    }
    for (int n = 0; n < NC; ++n) {
        const int64_t uu = u0 + n;
        const int64_t unext = n + 1 < NC ? uu + 1 : uu;
        const int slot = n & 1;
        char* sw = smem + slot * SL::SLOT + w * SL::PW * 1024;
        // chunk-start memory: the LDS copy for GEMM1 and (bf16) the Wn blocks for the output kernel
        char* wn = a.ws + a.o_wn + uu * szWn;
#pragma unroll
        for (int i = 0; i < NDPB; ++i) {
            uint4 val;
            if constexpr (BF16) val = pack_bf16x8(Wst[2 * i], Wst[2 * i + 1]);
            else val = __builtin_bit_cast(uint4, Wst[i]);
            const int jb = dt0 / pair + i;
            if constexpr (BF16) {
                *reinterpret_cast<uint4*>(lane16(X, jb)) = val;
                *reinterpret_cast<uint4*>(blk_ptr(wn, static_cast<int64_t>(jb) * NVT + r, l)) = val;
            } else {
                store_split(lane16(X, jb & ~1), jb, Wst[i]);          // split format for GEMM1
            }
        }
        lds_barrier();                                               // B1
        if (w < NT) {
            // S = W_y W^T for row tile w, two accumulators over alternating k-blocks
            f32x4 s0 = zero4(), s1 = zero4();
            if constexpr (BF16) {
#pragma unroll
                for (int j = 0; j < NDB; ++j) {
                    const uint4 av = *reinterpret_cast<const uint4*>(lane16(sw, j));
                    const uint4 bv = *reinterpret_cast<const uint4*>(lane16(X, j));
                    f32x4& acc = (j & 1) ? s1 : s0;
                    acc = mfma_bf16_k32(as_bf16x8(av), as_bf16x8(bv), acc);
                }
            } else {
                // fp32 operands in the split format: one 32-deep k-step per block pair
                static_assert(NDB % 2 == 0, "fp32 k-blocks pair up");
#pragma unroll
                for (int j = 0; j < NDB; j += 2) {
                    f32x4& acc = (j & 2) ? s1 : s0;
                    const uint4 xh = *reinterpret_cast<const uint4*>(lane16(X, j));
                    const uint4 xl = *reinterpret_cast<const uint4*>(lane16(X, j + 1));
                    acc = mfma_split(*reinterpret_cast<const uint4*>(lane16(sw, j)),
                                     *reinterpret_cast<const uint4*>(lane16(sw, j + 1)), xh, xl, acc);
                    qacc = mfma_split(qy[j], qy[j + 1], xh, xl, qacc);   // Q W^T, same W^T blocks
                }
                load_q(unext);
            }
            const f32x4 uyv = *reinterpret_cast<const f32x4*>(lane16(sw, SL::PW - 1));
            const f32x4 U = uyv - (s0 + s1);
            if constexpr (BF16) {
                // U for the output kernel: B blocks (j, r); tile w is half h = w & 1 of pair
                // block w / 2 (slots 4 h .. 4 h + 3 of every lane)
                char* un = a.ws + a.o_un + uu * szUn;
                *reinterpret_cast<uint2*>(blk_ptr(un, static_cast<int64_t>(w >> 1) * NVT + r, l) + 8 * (w & 1)) =
                    make_uint2(pack_bf16x2(U[0], U[1]), pack_bf16x2(U[2], U[3]));
                const float* rk = reinterpret_cast<const float*>(smem + slot * SL::SLOT + kChainWaves * SL::PW * 1024);
                const f32x4 rkv = *reinterpret_cast<const f32x4*>(rk + 16 * w + 4 * g4);
                *reinterpret_cast<f32x4*>(lane16(Ub, w)) = U * rkv;
            } else {
                // U itself in the split format: the K^T blocks carry rho_k (K~^T)
                store_split(lane16(Ub, w & ~1), w, U);
            }
        }
        lds_barrier();                                               // B2
        if (FUSE_Y && w < NT) {
            // Y for row tile w = rho_q o (Q W^T) + P~ U (P~ zero above the diagonal)
            f32x4 yacc = qacc * rqv;
            qacc = zero4();
#pragma unroll
            for (int j = 0; j < NPB; j += 2) {
                if (j > w) break;
                yacc = mfma_split(py[j], py[j + 1], *reinterpret_cast<const uint4*>(lane16(Ub, j)),
                                  *reinterpret_cast<const uint4*>(lane16(Ub, j + 1)), yacc);
            }
            load_p(unext);
            const int t0 = n * C;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yacc[e]), yrsrc,
                                                      ((t0 + 16 * w + 4 * g4 + e) * a.d_v + vcol) * 4, 0, 0);
        }
        // W^T += K^T (rho_k o U) for this wave's d-tiles
        f32x4 odd[NDP];
#pragma unroll
        for (int i = 0; i < NDP; ++i) odd[i] = zero4();
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
            if constexpr (BF16) {
                const f32x4 u0v = *reinterpret_cast<const f32x4*>(lane16(Ub, 2 * j));
                const f32x4 u1v = *reinterpret_cast<const f32x4*>(lane16(Ub, 2 * j + 1));
                const uint4 bu = pack_bf16x8(u0v, u1v);
#pragma unroll
                for (int i = 0; i < NDP; ++i) {
                    const uint4 av = *reinterpret_cast<const uint4*>(lane16(sw, NDB + i * NTB + j));
                    f32x4& dst = (j & 1) ? odd[i] : Wst[i];
                    dst = mfma_bf16_k32(as_bf16x8(av), as_bf16x8(bu), dst);
                }
            } else if ((j & 1) == 0) {
                // fp32 operands in the split format: K^T and rho_k o U block pairs (j, j + 1)
                static_assert(NTB % 2 == 0, "fp32 k-blocks pair up");
                const uint4 uh = *reinterpret_cast<const uint4*>(lane16(Ub, j));
                const uint4 ul = *reinterpret_cast<const uint4*>(lane16(Ub, j + 1));
#pragma unroll
                for (int i = 0; i < NDP; ++i) {
                    f32x4& dst = (j & 2) ? odd[i] : Wst[i];
                    dst = mfma_split(*reinterpret_cast<const uint4*>(lane16(sw, NDB + i * NTB + j)),
                                     *reinterpret_cast<const uint4*>(lane16(sw, NDB + i * NTB + j + 1)),
                                     uh, ul, dst);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NDP; ++i) Wst[i] += odd[i];
    }

    if (a.Wf) {
#pragma unroll
        for (int i = 0; i < NDP; ++i) {
            float* dst = a.Wf + (static_cast<int64_t>(bh) * a.d_v + vcol) * D +
                         orig_col(16 * (dt0 + i) + 4 * g4, d_k);
            *reinterpret_cast<float2*>(dst) = make_float2(Wst[i][0], Wst[i][2]);
            *reinterpret_cast<float2*>(dst + d_k) = make_float2(Wst[i][1], Wst[i][3]);
        }
    }
}

// ------------------------------------------------------------------------------------------
// chain, direct: the staged kernel's decomposition (chain wave w owns row tile w of
// S = W_y W^T over all of D and d-tiles w NDP .. +NDP of the memory) with no loader waves: each
// wave loads its own operand blocks (W_y row tile, K^T d-tiles, U_y tile, rho_k) into registers
// two chunks ahead, into one of two register sets, right after their last use.  LDS carries only
// what the waves share: the W^T copy (GEMM1's B operand) and rho_k o U (the update's B
// operand), about a third of the staged kernel's LDS traffic.  Chunks go in pairs, one per
// register set, so every register index is static; the loop body has no branches around memory
// operations (prefetches past the last chunk re-read it), so every wait covers only the loads
// it needs.
// The outputs are formed by a second group of NT waves next to the chain, off its dependency
// chain: output wave NT + t accumulates Q W^T for row tile t from the W^T copy while the chain
// waves form S, and after the second barrier adds P~ U from U (kept in LDS as well) and scales by
// rho_q; Q, P~ and rho_q travel in its own register sets, and y goes out through a range-checked
// buffer store.  No chunk-start memories or U go to the workspace and no output kernel runs.
template <bool BF16, int C, int NDP>
__global__ __launch_bounds__(128 * kChainWaves, 1) void delta_chain_direct_kernel(ChunkArgs a) {
    using LT = typename ChunkTypes<BF16>::LT;
    constexpr int pair = BF16 ? 2 : 1, NT = C / 16, NTB = NT / pair;
    constexpr int ND = kChainWaves * NDP, NDB = ND / pair, NDPB = NDP / pair;
    static_assert(NT == kChainWaves, "one row tile of S per chain wave");
    static_assert(NDP % pair == 0, "bf16 waves hold whole d-tile pairs");
    __shared__ __attribute__((aligned(1024))) char X[NDB * 1024];   // W^T copy
    __shared__ __attribute__((aligned(1024))) char Ub[NT * 1024];   // rho_k o U, fp32 tiles
    __shared__ __attribute__((aligned(1024))) char Uo[NT * 1024];   // U, fp32 tiles
    static_assert(BF16, "the direct chain serves bf16 inputs");

    const int tid = threadIdx.x, l = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool outw = wave >= NT;                 // output waves NT .. 2 NT - 1
    const int w = outw ? wave - NT : wave;        // the wave's row tile
    const int l16 = l & 15, g4 = l >> 4;
    const int d_k = a.d_k, D = a.D, NC = a.NC, NVT = a.d_v / 16;
    const BhIndex bi = xcd_local(blockIdx.x, a.BH, NVT);
    const int bh = bi.bh, r = static_cast<int>(bi.i);
    const int dt0 = w * NDP;
    const int vcol = 16 * r + l16;
    const int64_t u0 = static_cast<int64_t>(bh) * NC;
    const int64_t ulast = u0 + NC - 1;
    const int64_t szCD = static_cast<int64_t>(C) * D * sizeof(LT);
    const int64_t szUy = static_cast<int64_t>(C) * a.d_v * 4;
    auto lane16 = [&](char* base, int blk) { return base + blk * 1024 + l * 16; };
    auto clampu = [&](int64_t uu) { return uu <= ulast ? uu : ulast; };

    if (!outw) {
        const char* wyB = a.ws + a.o_wy + (static_cast<int64_t>(w) * NDB * 64 + l) * 16;
        const char* ktB = a.ws + a.o_kt + (static_cast<int64_t>(dt0) * NTB * 64 + l) * 16;
        const char* uyB = a.ws + a.o_uy + ((static_cast<int64_t>(w) * NVT + r) * 64 + l) * 16;
        const float* rkB = reinterpret_cast<const float*>(a.ws + a.o_rk) + 16 * w + 4 * g4;
        uint4 wy[2][NDB];          // W_y blocks of row tile w, per register set
        uint4 kt[2][NDP * NTB];    // K^T blocks of d-tiles dt0 ..
        f32x4 uy[2], rk[2];        // U_y tile (w, r) and rho_k of its rows
        auto load_wy = [&](int set, int64_t uu) {
#pragma unroll
            for (int j = 0; j < NDB; ++j) wy[set][j] = *reinterpret_cast<const uint4*>(wyB + uu * szCD + j * 1024);
        };
        auto load_kt = [&](int set, int64_t uu) {
#pragma unroll
            for (int b = 0; b < NDP * NTB; ++b) kt[set][b] = *reinterpret_cast<const uint4*>(ktB + uu * szCD + b * 1024);
        };
        auto load_uy = [&](int set, int64_t uu) {
            uy[set] = *reinterpret_cast<const f32x4*>(uyB + uu * szUy);
            rk[set] = *reinterpret_cast<const f32x4*>(rkB + uu * C);
        };
        f32x4 Wst[NDP];
#pragma unroll
        for (int i = 0; i < NDP; ++i) {
            Wst[i] = zero4();
            if (a.W0) {
                // internal columns c0 .. c0+3 = positions (o, o + d_k, o + 1, o + d_k + 1)
                const float* src = a.W0 + (static_cast<int64_t>(bh) * a.d_v + vcol) * D +
                                   orig_col(16 * (dt0 + i) + 4 * g4, d_k);
                const float2 lo = *reinterpret_cast<const float2*>(src);
                const float2 hi = *reinterpret_cast<const float2*>(src + d_k);
                Wst[i] = f32x4{lo.x, hi.x, lo.y, hi.y};
            }
        }
        // One chunk with register set SET; its operands are replaced by those of chunk uu + 2.
        auto chunk = [&](int64_t uu, auto set_tag) {
            constexpr int SET = decltype(set_tag)::value;
            const int64_t ua = clampu(uu + 2);
            // chunk-start memory: the LDS copy for GEMM1 and Q W^T
#pragma unroll
            for (int i = 0; i < NDPB; ++i)
                *reinterpret_cast<uint4*>(lane16(X, dt0 / pair + i)) = pack_bf16x8(Wst[2 * i], Wst[2 * i + 1]);
            lds_barrier();                                           // B1: W^T copy complete
            // S = W_y W^T for row tile w, two accumulators over alternating k-blocks
            f32x4 s0 = zero4(), s1 = zero4();
#pragma unroll
            for (int j = 0; j < NDB; ++j) {
                const bf16x8 bv = as_bf16x8(*reinterpret_cast<const uint4*>(lane16(X, j)));
                f32x4& acc = (j & 1) ? s1 : s0;
                acc = mfma_bf16_k32(as_bf16x8(wy[SET][j]), bv, acc);
            }
            load_wy(SET, ua);
            const f32x4 U = uy[SET] - (s0 + s1);
            *reinterpret_cast<f32x4*>(lane16(Ub, w)) = U * rk[SET];
            *reinterpret_cast<f32x4*>(lane16(Uo, w)) = U;
            load_uy(SET, ua);
            lds_barrier();                                           // B2: U and rho_k o U complete
            // W^T += K^T (rho_k o U) for this wave's d-tiles
            f32x4 odd[NDP];
#pragma unroll
            for (int i = 0; i < NDP; ++i) odd[i] = zero4();
#pragma unroll
            for (int j = 0; j < NTB; ++j) {
                const f32x4 u0v = *reinterpret_cast<const f32x4*>(lane16(Ub, 2 * j));
                const f32x4 u1v = *reinterpret_cast<const f32x4*>(lane16(Ub, 2 * j + 1));
                const uint4 bu = pack_bf16x8(u0v, u1v);
#pragma unroll
                for (int i = 0; i < NDP; ++i) {
                    f32x4& dst = (j & 1) ? odd[i] : Wst[i];
                    dst = mfma_bf16_k32(as_bf16x8(kt[SET][i * NTB + j]), as_bf16x8(bu), dst);
                }
            }
            load_kt(SET, ua);
#pragma unroll
            for (int i = 0; i < NDP; ++i) Wst[i] += odd[i];
        };
        if (NC > 0) {
            load_wy(0, u0);
            load_uy(0, u0);
            load_kt(0, u0);
            load_wy(1, clampu(u0 + 1));
            load_uy(1, clampu(u0 + 1));
            load_kt(1, clampu(u0 + 1));
        }
        int n = 0;
        for (; n + 1 < NC; n += 2) {
            chunk(u0 + n, std::integral_constant<int, 0>());
            chunk(u0 + n + 1, std::integral_constant<int, 1>());
        }
        if (n < NC) chunk(u0 + n, std::integral_constant<int, 0>());
        if (a.Wf) {
#pragma unroll
            for (int i = 0; i < NDP; ++i) {
                float* dst = a.Wf + (static_cast<int64_t>(bh) * a.d_v + vcol) * D +
                             orig_col(16 * (dt0 + i) + 4 * g4, d_k);
                *reinterpret_cast<float2*>(dst) = make_float2(Wst[i][0], Wst[i][2]);
                *reinterpret_cast<float2*>(dst + d_k) = make_float2(Wst[i][1], Wst[i][3]);
            }
        }
        return;
    }

    // ---- output waves: Q blocks and P~ blocks of row tile w, rho_q of its rows
    uint4 qy[2][NDB], py[2][NTB];
    f32x4 rq[2];
    const char* qaB = a.ws + a.o_qa + (static_cast<int64_t>(w) * NDB * 64 + l) * 16;
    const char* paB = a.ws + a.o_pa + (static_cast<int64_t>(w) * NTB * 64 + l) * 16;
    const float* rqB = reinterpret_cast<const float*>(a.ws + a.o_rq) + 16 * w + 4 * g4;
    const int64_t szCC = static_cast<int64_t>(C) * C * sizeof(LT);
    auto load_qp = [&](int set, int64_t uu) {
#pragma unroll
        for (int j = 0; j < NDB; ++j) qy[set][j] = *reinterpret_cast<const uint4*>(qaB + uu * szCD + j * 1024);
#pragma unroll
        for (int j = 0; j < NTB; ++j) py[set][j] = *reinterpret_cast<const uint4*>(paB + uu * szCC + j * 1024);
        rq[set] = *reinterpret_cast<const f32x4*>(rqB + uu * C);
    };
    // y of this (b, h), columns 16 r + l16, as a buffer whose range check drops rows past T
    const __amdgpu_buffer_rsrc_t yrsrc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<LT*>(a.y) + static_cast<int64_t>(bh) * a.T * a.d_v, static_cast<short>(0),
        a.T * a.d_v * static_cast<int>(sizeof(LT)), 0x00020000);
    auto chunk = [&](int64_t uu, auto set_tag) {
        constexpr int SET = decltype(set_tag)::value;
        const int64_t ua = clampu(uu + 2);
        lds_barrier();                                               // B1: W^T copy complete
        f32x4 q0 = zero4(), q1 = zero4();
#pragma unroll
        for (int j = 0; j < NDB; ++j) {
            const bf16x8 bv = as_bf16x8(*reinterpret_cast<const uint4*>(lane16(X, j)));
            f32x4& qacc = (j & 1) ? q1 : q0;
            qacc = mfma_bf16_k32(as_bf16x8(qy[SET][j]), bv, qacc);
        }
        lds_barrier();                                               // B2: U complete
        // Y for row tile w = rho_q o (Q W^T) + P~ U (P~ zero above the diagonal)
        f32x4 y = (q0 + q1) * rq[SET];
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
            if (2 * j > w) break;
            const uint4 ub = pack_bf16x8(*reinterpret_cast<const f32x4*>(lane16(Uo, 2 * j)),
                                         *reinterpret_cast<const f32x4*>(lane16(Uo, 2 * j + 1)));
            y = mfma_bf16_k32(as_bf16x8(py[SET][j]), as_bf16x8(ub), y);
        }
        const int t0 = static_cast<int>(uu - u0) * C;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(y[e]), yrsrc,
                                                  ((t0 + 16 * w + 4 * g4 + e) * a.d_v + vcol) * 2, 0, 0);
        load_qp(SET, ua);
    };
    if (NC > 0) {
        load_qp(0, u0);
        load_qp(1, clampu(u0 + 1));
    }
    int n = 0;
    for (; n + 1 < NC; n += 2) {
        chunk(u0 + n, std::integral_constant<int, 0>());
        chunk(u0 + n + 1, std::integral_constant<int, 1>());
    }
    if (n < NC) chunk(u0 + n, std::integral_constant<int, 0>());
}

// ------------------------------------------------------------------------------------------
// output: one wave per output tile (chunk u, row tile tt, v-tile vt), four tiles per workgroup:
//   Y = rho_q o (Q W_n^T) + P~ U_n.
template <bool BF16, int C>
__global__ __launch_bounds__(256) void delta_output_kernel(ChunkArgs a) {
    using LT = typename ChunkTypes<BF16>::LT;
    constexpr int pair = ChunkTypes<BF16>::pair;
    constexpr int NT = C / 16;
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = l & 15, g4 = l >> 4;
    const int D = a.D, d_v = a.d_v, T = a.T;
    const int ND = D / 16, NDB = ND / pair, NVT = d_v / 16, NTB = NT / pair;
    const int ntile = NT * NVT;
    const int wgs = (ntile + 3) / 4;                      // workgroups per chunk
    const BhIndex bi = xcd_local(blockIdx.x, a.BH, static_cast<int64_t>(a.NC) * wgs);
    const int bh = bi.bh, n = static_cast<int>(bi.i / wgs);
    const int64_t u = static_cast<int64_t>(bh) * a.NC + n;
    const int tile = static_cast<int>(bi.i % wgs) * 4 + w;
    if (tile >= ntile) return;                            // no barrier in this kernel
    const int tt = tile / NVT, vt = tile % NVT;
    const int t0 = n * C, Cc = min(C, T - t0);

    const char* ws = a.ws;
    const char* qa = ws + a.o_qa + u * (static_cast<int64_t>(C) * D * sizeof(LT));
    const char* wn = ws + a.o_wn + u * (static_cast<int64_t>(D) * d_v * sizeof(LT));
    const char* pa = ws + a.o_pa + u * (static_cast<int64_t>(C) * C * sizeof(LT));
    const char* un = ws + a.o_un + u * (static_cast<int64_t>(C) * d_v * sizeof(LT));
    const f32x4 rq = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(ws + a.o_rq) +
                                                     u * C + 16 * tt + 4 * g4);
    f32x4 acc = zero4();
    if (!BF16 && a.split) {
        // fp32 operands in the split bf16 hi + lo format: block pairs (j, j + 1)
        auto ld = [&](const char* base, int64_t blk) { return *reinterpret_cast<const uint4*>(blk_ptr(base, blk, l)); };
#pragma unroll 2
        for (int j = 0; j < NDB; j += 2)
            acc = mfma_split(ld(qa, tt * NDB + j), ld(qa, tt * NDB + j + 1), ld(wn, j * NVT + vt),
                             ld(wn, (j + 1) * NVT + vt), acc);
        acc *= rq;
        for (int j = 0; j < NT && j <= tt; j += 2)
            acc = mfma_split(ld(pa, tt * NT + j), ld(pa, tt * NT + j + 1), ld(un, j * NVT + vt),
                             ld(un, (j + 1) * NVT + vt), acc);
    } else {
#pragma unroll 4
    for (int j = 0; j < NDB; ++j) {
        const uint4 av = *reinterpret_cast<const uint4*>(blk_ptr(qa, tt * NDB + j, l));
        const uint4 bv = *reinterpret_cast<const uint4*>(blk_ptr(wn, j * NVT + vt, l));
        if constexpr (BF16) {
            acc = mfma_bf16_k32(as_bf16x8(av), as_bf16x8(bv), acc);
        } else {
            const f32x4 af = as_f32x4(av), bf = as_f32x4(bv);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = mfma_f32_k4(af[e], bf[e], acc);
        }
    }
    acc *= rq;
    for (int j = 0; j < NTB && pair * j <= tt; ++j) {
        const uint4 av = *reinterpret_cast<const uint4*>(blk_ptr(pa, tt * NTB + j, l));
        const uint4 bv = *reinterpret_cast<const uint4*>(blk_ptr(un, j * NVT + vt, l));
        if constexpr (BF16) {
            acc = mfma_bf16_k32(as_bf16x8(av), as_bf16x8(bv), acc);
        } else {
            const f32x4 af = as_f32x4(av), bf = as_f32x4(bv);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = mfma_f32_k4(af[e], bf[e], acc);
        }
    }
    }
    LT* yB = static_cast<LT*>(a.y) + (static_cast<int64_t>(bh) * T + t0) * d_v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = 16 * tt + 4 * g4 + e;
        if (t < Cc) yB[static_cast<int64_t>(t) * d_v + 16 * vt + l16] = from_f32<LT>(acc[e]);
    }
}

// (d-tiles per wave, waves) pairs of the chain kernel that plans use: fp32 waves hold 1 or 2
// d-tiles, bf16 waves 2 or 4.
inline bool chain_config_ok(bool bf16, int ndp, int dp) {
    const bool waves = dp == 1 || dp == 2 || dp == 3 || dp == 4 || dp == 6 || dp == 8;
    return waves && (bf16 ? (ndp == 2 || ndp == 4) : (ndp == 1 || ndp == 2));
}

template <bool BF16, int C, int NDP>
hipError_t launch_chain_ndp(const ChunkArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.BH) * (a.d_v / 16)));
    const unsigned red = a.DP > 1 ? 2u * a.DP * (C / 16) * 1024u : 0u;
    switch (a.DP) {
        case 1: hipLaunchKernelGGL((delta_chain_kernel<BF16, C, NDP, 1>), grid, dim3(64), red, stream, a); break;
        case 2: hipLaunchKernelGGL((delta_chain_kernel<BF16, C, NDP, 2>), grid, dim3(128), red, stream, a); break;
        case 3: hipLaunchKernelGGL((delta_chain_kernel<BF16, C, NDP, 3>), grid, dim3(192), red, stream, a); break;
        case 4: hipLaunchKernelGGL((delta_chain_kernel<BF16, C, NDP, 4>), grid, dim3(256), red, stream, a); break;
        case 6: hipLaunchKernelGGL((delta_chain_kernel<BF16, C, NDP, 6>), grid, dim3(384), red, stream, a); break;
        case 8: hipLaunchKernelGGL((delta_chain_kernel<BF16, C, NDP, 8>), grid, dim3(512), red, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Staged chain kernel: (d-tiles per compute wave) instantiated per dtype, and its LDS bytes
// (0 when the shape has no staged instantiation).
inline int staged_chain_lds(bool bf16, int C, int ndp) {
    const int ok = bf16 ? (ndp == 2 || ndp == 4) : (ndp == 1 || ndp == 2);
    if (!ok || (C != 32 && C != 64)) return 0;
    const int pair = bf16 ? 2 : 1, NT = C / 16, NTB = NT / pair, ND = kChainWaves * ndp;
    const int NDB = ND / pair, PW = NDB + ndp * NTB + 1;
    return 2 * (kChainWaves * PW + 1) * 1024 + NDB * 1024 + NT * 1024;
}

template <bool BF16, int C, int NDP>
hipError_t launch_chain_staged(const ChunkPlan& p, hipStream_t stream) {
    auto kern = delta_chain_staged_kernel<BF16, C, NDP>;
    static_assert(StagedLayout<BF16, C, NDP>::BYTES > 0, "layout");
    hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kern), p.lds_chain);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.args.BH) * (p.args.d_v / 16)));
    hipLaunchKernelGGL(kern, grid, dim3(64 * 2 * kChainWaves), p.lds_chain, stream, p.args);
    return hipGetLastError();
}

template <bool BF16, int C>
hipError_t launch_chunked_t(const ChunkPlan& p, hipStream_t stream) {
    const ChunkArgs& a = p.args;
    const int64_t NU = static_cast<int64_t>(a.BH) * a.NC;
    if (NU > 0) {
        // two workgroups per chunk (K side, Q side) where twice the chunks fit at once (chunk
        // 64, D a multiple of 128 so that quarters of D are whole k-steps, and room for the
        // quarter partials over the staging rows)
        hipError_t e;
        bool launched = false;
        if constexpr (C == 64) {
            auto preps = delta_prep_split_kernel<BF16, C>;
            const bool allowed = a.D % 128 == 0 &&
                                 a.l_xv - a.l_x >= 6 * (C / 16 + 1) * 1024;
            if (allowed) {
                if ((e = ensure_lds_attr(reinterpret_cast<const void*>(preps), p.lds_prep)) != hipSuccess) return e;
                unsigned caps = 0;
                e = resident_grid(reinterpret_cast<const void*>(preps), kPrepThreads, p.lds_prep, INT64_MAX, &caps);
                if (e != hipSuccess) return e;
                if (2 * NU <= static_cast<int64_t>(caps)) {
                    hipLaunchKernelGGL(preps, dim3(static_cast<unsigned>(2 * NU)), dim3(kPrepThreads), p.lds_prep, stream, a);
                    launched = true;
                }
            }
        }
        if (!launched) {
        // the persistent form where more chunks than fit at once and it keeps as many
        // workgroups resident as the one-chunk form, else one workgroup per chunk
        auto prep1 = delta_prep_kernel<BF16, C, false, false>;
        auto prepp = delta_prep_kernel<BF16, C, false, true>;
        e = ensure_lds_attr(reinterpret_cast<const void*>(prepp), p.lds_prep);
        if (e != hipSuccess) return e;
        if ((e = ensure_lds_attr(reinterpret_cast<const void*>(prep1), p.lds_prep)) != hipSuccess) return e;
        unsigned grid = 0, cap1 = 0;
        e = resident_grid(reinterpret_cast<const void*>(prepp), kPrepThreads, p.lds_prep, NU, &grid);
        if (e != hipSuccess) return e;
        e = resident_grid(reinterpret_cast<const void*>(prep1), kPrepThreads, p.lds_prep, INT64_MAX, &cap1);
        if (e != hipSuccess) return e;
        if (static_cast<int64_t>(grid) < NU && grid >= cap1) {
            hipLaunchKernelGGL(prepp, dim3(grid), dim3(kPrepThreads), p.lds_prep, stream, a);
        } else {
            hipLaunchKernelGGL(prep1, dim3(static_cast<unsigned>(NU)), dim3(kPrepThreads), p.lds_prep, stream, a);
        }
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipError_t e;
    bool direct = false;
    if constexpr (BF16 && C == 64) {
        // bf16: the direct chain (two chunks of register lookahead, outputs formed in the chain)
        // over the staged one
        if (p.direct) {
            const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.BH) * (a.d_v / 16)));
            if (p.staged_ndp == 2)
                hipLaunchKernelGGL((delta_chain_direct_kernel<BF16, C, 2>), grid, dim3(128 * kChainWaves), 0, stream, a);
            else
                hipLaunchKernelGGL((delta_chain_direct_kernel<BF16, C, 4>), grid, dim3(128 * kChainWaves), 0, stream, a);
            direct = true;
        }
    }
    if (direct) {
        e = hipGetLastError();
    } else if (p.staged_ndp > 0) {
        if constexpr (BF16) e = p.staged_ndp == 2 ? launch_chain_staged<BF16, C, 2>(p, stream)
                                                  : launch_chain_staged<BF16, C, 4>(p, stream);
        else e = p.staged_ndp == 1 ? launch_chain_staged<BF16, C, 1>(p, stream)
                                   : launch_chain_staged<BF16, C, 2>(p, stream);
    } else if constexpr (BF16) e = a.NDP == 2 ? launch_chain_ndp<BF16, C, 2>(a, stream)
                                       : (a.NDP == 4 ? launch_chain_ndp<BF16, C, 4>(a, stream) : hipErrorInvalidValue);
    else e = a.NDP == 1 ? launch_chain_ndp<BF16, C, 1>(a, stream)
                        : (a.NDP == 2 ? launch_chain_ndp<BF16, C, 2>(a, stream) : hipErrorInvalidValue);
    if (e != hipSuccess) return e;
    // the fp32 staged chain and the bf16 direct chain form the outputs themselves
    const bool outputs_done = p.chain_outputs;
    if (NU > 0 && !outputs_done) {
        const int ntile = (C / 16) * (a.d_v / 16);
        const int64_t grid = NU * ((ntile + 3) / 4);
        hipLaunchKernelGGL((delta_output_kernel<BF16, C>), dim3(static_cast<unsigned>(grid)),
                           dim3(256), 0, stream, a);
        e = hipGetLastError();
    }
    return e;
}

hipError_t launch_chunked_f32_c32(const ChunkPlan& p, hipStream_t s);
hipError_t launch_chunked_f32_c64(const ChunkPlan& p, hipStream_t s);
hipError_t launch_chunked_bf16_c32(const ChunkPlan& p, hipStream_t s);
hipError_t launch_chunked_bf16_c64(const ChunkPlan& p, hipStream_t s);

}  // namespace fwa
