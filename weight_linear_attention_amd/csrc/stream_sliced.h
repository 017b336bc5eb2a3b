// Shift-sliced streaming forward (bf16, d_k = 64): the compact preparation and the serial pass
// over chunks with the K and Q tiles built one DPFP shift block at a time, so the on-chip
// working set no longer grows with D.  This is what lets a chunk of 128 rows run at D = 384.
//
// The recurrence ("Fast Weights Transformer" guide, xdnf.cn/news/308600, sections
// "FastWeightsAttention / update formula" and "... / module structure and source walkthrough")
// is evaluated chunk by chunk with the chunked algebra derived from it.  For a chunk of C rows
// starting from memory W (d_v x D), with raw DPFP tiles K, Q, normalisers rho_k, rho_q, beta =
// sigmoid(beta_logit) and L = diag(beta) strict_lower(K~ K~^T) (K~ = diag(rho_k) K):
//     A'' = (I + L)^-1 diag(beta),   P~ = lower_incl(Q~ K~^T)                (prep, all chunks)
//     X = K W^T,  U = A'' (V - rho_k o X),  Y = rho_q o (Q W^T) + P~ U,
//     W^T += K^T (rho_k o U)                                                 (stream, serial)
//
// Shift slices.  The DPFP columns of shift i (1..nu) are one block of 2 d_k = 128 internal
// columns (the two halves of a position side by side, as in the full tiles), built from the
// staged raw rows by per-lane tasks: (row, 8 positions) -> 16 columns, with the rolled partner
// taken from a 16-entry window [8 positions before, the 8 positions] of the row, so no lane
// exchange is needed.  Every contraction over D is a sum of per-slice contractions:
//   prep:   G += K_i K_i^T and P += Q_i K_i^T, accumulated in MFMA registers over the slices;
//   stream: X += K_i W_i^T and Q W^T += Q_i W_i^T over the slices, then the memory update
//           W_i^T += K_i^T (rho_k o U) with each K_i built again (the update needs U, which
//           needs all of X first).  DPFP is cheap VALU work next to keeping C x D tiles.
// LDS holds one K and one Q slice (C x 136 bf16 each), never the full C x D tiles.
#pragma once

#include "chunk_tile.h"
#include "chunked_kernels.h"
#include "stream_kernel.h"

namespace fwa {

constexpr int kSliceDk = 64;                 // d_k of the sliced kernels: one shift = 128 columns
constexpr int kSliceCols = 2 * kSliceDk;
constexpr int kSliceThreads = 512;

// One DPFP task restricted to shift I: positions j0 .. j0+7 of a staged row (a = k[j0..j0+7],
// pv = the 8 positions before j0, cyclically), written as 16 consecutive slice columns at
// out + 2 j0.  Position j's partner is relu([k, -k]) at (j - I) mod 2 d_k = +-k[(j - I) mod d_k],
// negated when j < I (the index wraps into the [-k] half); window index 8 + e - I of [pv, a]
// holds k[(j0 + e - I) mod d_k] for 1 <= I <= 8.  Returns the task's sum of products.
template <int I>
__device__ __forceinline__ float dpfp_task_shift(const float (&a)[8], const float (&pv)[8], int j0,
                                                 u16* out) {
    static_assert(I >= 1 && I <= 8, "the window holds rolls of at most 8 positions");
    // positive and negative parts of window indices 8 - I .. 15 of [pv, a]; a product of two
    // such parts is a single multiply
    float P[16], N[16], f[16], sum = 0.0f;
#pragma unroll
    for (int m = 8 - I; m < 16; ++m) {
        const float r = m >= 8 ? a[m - 8] : pv[m];
        P[m] = relu_f(r);
        N[m] = P[m] - r;                 // relu(-r), exactly
    }
    const bool wraps = j0 == 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int m = 8 - I + e;                                 // compile-time window index
        const float xp = (e < I && wraps) ? N[m] : P[m];
        const float xn = (e < I && wraps) ? P[m] : N[m];
        f[2 * e] = P[8 + e] * xp;
        f[2 * e + 1] = N[8 + e] * xn;
        sum += f[2 * e] + f[2 * e + 1];
    }
    store16(out + 2 * j0, f);
    return sum;
}

// The shift-I slices of the C staged rows Xk (and Xq) ([C][64] bf16) into Ks (and Qs)
// ([C][ss] bf16), by NTH threads.  Task tau = tid + NTH p (p < NP) is (row tau / 8, group tau % 8); K rows come
// first, then Q rows.  A row's eight tasks sit in eight adjacent lanes, and each thread keeps
// the same tasks for every shift, so sums[p] accumulates the row partial sums over the slices.
template <int C, int NTH, bool WITH_Q, int I, int NP>
__device__ __forceinline__ void dpfp_slice(const u16* Xk, const u16* Xq, u16* Ks, u16* Qs, int ss,
                                           int tid, float (&sums)[NP]) {
    static_assert(NP * NTH == (WITH_Q ? 2 : 1) * C * (kSliceDk / 8), "task split");
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int tau = tid + NTH * p;
        const int jg = tau & 7, rt = tau >> 3;
        const bool isq = WITH_Q && rt >= C;                      // uniform per wave
        const int t = isq ? rt - C : rt;
        const u16* row = (isq ? Xq : Xk) + t * kSliceDk;
        u16* out = (isq ? Qs : Ks) + t * ss;
        float a[8], pv[8];
        load8_f32(row + 8 * jg, a);
        load8_f32(row + 8 * ((jg + 7) & 7), pv);
        sums[p] += dpfp_task_shift<I>(a, pv, 8 * jg, out);
    }
}

template <int C, int NTH, bool WITH_Q, int NP>
__device__ __forceinline__ void dpfp_slice_any(int i, const u16* Xk, const u16* Xq, u16* Ks,
                                               u16* Qs, int ss, int tid, float (&sums)[NP]) {
    switch (i) {
        case 1: dpfp_slice<C, NTH, WITH_Q, 1>(Xk, Xq, Ks, Qs, ss, tid, sums); break;
        case 2: dpfp_slice<C, NTH, WITH_Q, 2>(Xk, Xq, Ks, Qs, ss, tid, sums); break;
        case 3: dpfp_slice<C, NTH, WITH_Q, 3>(Xk, Xq, Ks, Qs, ss, tid, sums); break;
        default: dpfp_slice<C, NTH, WITH_Q, 4>(Xk, Xq, Ks, Qs, ss, tid, sums); break;
    }
}

// ------------------------------------------------------------------------------------------
// G = K K^T and P = Q K^T at chunk 64 with the DPFP operands built in registers.  The MFMA A
// operand of row r and the B operand of column r (16x16x32 bf16) hold the same eight values per
// lane: slot 2 f + h of lane (l16, g4) in k-step kk of shift block i is internal column
// (i - 1) 2 d_k + 2 (16 kk + 4 g4 + f) + h of row r.  Each lane builds them from a window of
// its staged raw row, positions p0 - 4 .. p0 + 3 (p0 = 16 kk + 4 g4), so no feature tile goes
// through LDS: the window is read once per k-step and serves every shift.  The staged rows are
// kRawRow bf16 apart (136 bytes: the 16 rows a wave reads at once fall in distinct banks).
constexpr int kRawRow = kSliceDk + 4;

// The window's k values as fp32 positive and negative parts.  For the window starting at
// position 0, the four entries before it wrap into the [-k] half: their signs are flipped in
// the packed words before unpacking, which swaps their parts.
struct DpfpWin {
    float P[8], N[8];
};
__device__ __forceinline__ DpfpWin dpfp_window(const u16* row, int p0) {
    const uint2 lo = *reinterpret_cast<const uint2*>(row + ((p0 + kSliceDk - 4) & (kSliceDk - 1)));
    const uint2 hi = *reinterpret_cast<const uint2*>(row + p0);
    const uint32_t sg = p0 == 0 ? 0x80008000u : 0u;
    const uint32_t wd[4] = {lo.x ^ sg, lo.y ^ sg, hi.x, hi.y};
    DpfpWin wn;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float r = (e & 1) ? __uint_as_float(wd[e >> 1] & 0xffff0000u) : __uint_as_float(wd[e >> 1] << 16);
        wn.P[e] = relu_f(r);
        wn.N[e] = wn.P[e] - r;                 // relu(-r), exactly
    }
    return wn;
}

// The operand of shift I: slot 2 f + h = position p0 + f, half h (h = 0: relu(k_j) times the
// rolled factor, h = 1: relu(-k_j) times it); with SUM, the fp32 products are added to *sum.
template <int I, bool SUM>
__device__ __forceinline__ bf16x8 dpfp_operand(const DpfpWin& wn, float& sum) {
    bf16x8 o;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int m = 4 + f - I;
        const float a = wn.P[4 + f] * wn.P[m], b = wn.N[4 + f] * wn.N[m];
        o[2 * f] = static_cast<__bf16>(a);
        o[2 * f + 1] = static_cast<__bf16>(b);
        if constexpr (SUM) sum += a + b;
    }
    return o;
}

// The tiles of tile-row pair Q (rows RA = Q, RB = 3 - Q) of both G = K K^T and P = Q K^T,
// with the row sums of K rows and Q rows RA, RB: ga / gb tiles (RA, tb) / (RB, tb) of G,
// pa / pb those of P, sums kA, kB, qA, qB.
struct GPPair {
    f32x4 ga[4], gb[4], pa[4], pb[4];
    float kA, kB, qA, qB;
};

// One k-step of shift I: the A operands of K and Q rows RA, RB, then the K rows 0 .. RB as B
// operands one at a time (rows RA and RB are the A operands already built).
template <int Q, int I>
__device__ __forceinline__ void gp_pair_step(GPPair& g, const DpfpWin& ka, const DpfpWin& kb,
                                             const DpfpWin& qa, const DpfpWin& qb,
                                             const u16* Xk, int p0, int l16) {
    constexpr int RA = Q, RB = 3 - Q;
    const bf16x8 vka = dpfp_operand<I, true>(ka, g.kA);
    const bf16x8 vkb = dpfp_operand<I, true>(kb, g.kB);
    const bf16x8 vqa = dpfp_operand<I, true>(qa, g.qA);
    const bf16x8 vqb = dpfp_operand<I, true>(qb, g.qB);
    float dummy = 0.0f;
#pragma unroll
    for (int tb = 0; tb <= RB; ++tb) {
        bf16x8 kv;
        if (tb == RA) kv = vka;
        else if (tb == RB) kv = vkb;
        else kv = dpfp_operand<I, false>(dpfp_window(Xk + (16 * tb + l16) * kRawRow, p0), dummy);
        if (tb <= RA) {
            g.ga[tb] = mfma_bf16_k32(vka, kv, g.ga[tb]);
            g.pa[tb] = mfma_bf16_k32(vqa, kv, g.pa[tb]);
        }
        g.gb[tb] = mfma_bf16_k32(vkb, kv, g.gb[tb]);
        g.pb[tb] = mfma_bf16_k32(vqb, kv, g.pb[tb]);
    }
}

// Pair Q over the k-steps kk0, kk0 + 1 of every shift block (half of D); the sums cover this
// lane's positions 4 g4 .. + 3 of every 16 in those k-steps.
template <int Q, int NU>
__device__ __forceinline__ void gp_pair_half(GPPair& g, const u16* Xk, const u16* Xq, int kk0,
                                             int l16, int g4) {
    static_assert(NU >= 1 && NU <= 4, "window entries 4 + f - i stay in 0 .. 7");
    constexpr int RA = Q, RB = 3 - Q;
#pragma unroll 1
    for (int kk = kk0; kk < kk0 + 2; ++kk) {
        const int p0 = 16 * kk + 4 * g4;
        const DpfpWin ka = dpfp_window(Xk + (16 * RA + l16) * kRawRow, p0);
        const DpfpWin kb = dpfp_window(Xk + (16 * RB + l16) * kRawRow, p0);
        const DpfpWin qa = dpfp_window(Xq + (16 * RA + l16) * kRawRow, p0);
        const DpfpWin qb = dpfp_window(Xq + (16 * RB + l16) * kRawRow, p0);
        gp_pair_step<Q, 1>(g, ka, kb, qa, qb, Xk, p0, l16);
        if constexpr (NU >= 2) gp_pair_step<Q, 2>(g, ka, kb, qa, qb, Xk, p0, l16);
        if constexpr (NU >= 3) gp_pair_step<Q, 3>(g, ka, kb, qa, qb, Xk, p0, l16);
        if constexpr (NU >= 4) gp_pair_step<Q, 4>(g, ka, kb, qa, qb, Xk, p0, l16);
    }
}

// Chunk 64, four waves: wave w takes pair q = w % 2 over half h = w / 2 of the k-steps.  The
// two waves of a pair then swap halves through LDS at `part` (dead space of the phase): the
// h = 0 wave completes the pair's G tiles and K normalisers, the h = 1 wave its P tiles and Q
// normalisers (1 / (row sum + eps)).  The caller scales the completed tiles (G in ga / gb of
// the h = 0 waves, P in pa / pb of the h = 1 waves).
template <int NU>
__device__ __forceinline__ void gp_raw_c64(GPPair& g, const u16* Xk, const u16* Xq, f32x4* part,
                                           float* rhok, float* rhoq, int w, int l, int l16, int g4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) g.ga[t] = g.gb[t] = g.pa[t] = g.pb[t] = zero4();
    g.kA = g.kB = g.qA = g.qB = 0.0f;
    const int q = w & 1, h = w >> 1;
    if (q == 0) gp_pair_half<0, NU>(g, Xk, Xq, 2 * h, l16, g4);
    else gp_pair_half<1, NU>(g, Xk, Xq, 2 * h, l16, g4);
    // the four lanes l16 + 16 g4 of a row hold its shares
    float s[4] = {g.kA, g.kB, g.qA, g.qB};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s[i] += __shfl_xor(s[i], 16);
        s[i] += __shfl_xor(s[i], 32);
    }
    // slot (q, h): the half that wave (q, 1 - h) completes, 8 tiles (32 KB for the four slots)
    // and its 2 row sums (2 KB after the tiles)
    f32x4* mine = part + (q * 2 + h) * 8 * 64 + l;
    f32x4* other = part + (q * 2 + 1 - h) * 8 * 64 + l;
    float2* sums = reinterpret_cast<float2*>(part + 4 * 8 * 64);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        mine[t * 64] = h == 0 ? g.pa[t] : g.ga[t];
        mine[(4 + t) * 64] = h == 0 ? g.pb[t] : g.gb[t];
    }
    sums[(q * 2 + h) * 64 + l] = h == 0 ? make_float2(s[2], s[3]) : make_float2(s[0], s[1]);
    lds_barrier();
    const float2 o = sums[(q * 2 + 1 - h) * 64 + l];
    if (h == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            g.ga[t] += other[t * 64];
            g.gb[t] += other[(4 + t) * 64];
        }
        if (g4 == 0) {
            rhok[16 * q + l16] = __builtin_amdgcn_rcpf(s[0] + o.x + kDpfpEps);
            rhok[16 * (3 - q) + l16] = __builtin_amdgcn_rcpf(s[1] + o.y + kDpfpEps);
        }
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            g.pa[t] += other[t * 64];
            g.pb[t] += other[(4 + t) * 64];
        }
        if (g4 == 0) {
            rhoq[16 * q + l16] = __builtin_amdgcn_rcpf(s[2] + o.x + kDpfpEps);
            rhoq[16 * (3 - q) + l16] = __builtin_amdgcn_rcpf(s[3] + o.y + kDpfpEps);
        }
    }
}

// A 16x16 fp32 tile in accumulator layout (lane (l16, g4), slot e: row 4 g4 + e, column l16)
// transposed into row layout (lane (l16, g4), slot e: row l16, column 4 g4 + e) on the MFMA:
// the tile fed as the A operand of the four k-steps of a 16x16x4 product reads as its transpose,
// and the B operand is the identity (id[s] = 1 where 4 g4 + s == l16), so each output is one
// exact product with 1.
__device__ __forceinline__ f32x4 tile_to_rows(const f32x4& x, const float (&id)[4]) {
    f32x4 t = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) t = mfma_f32_k4(x[s], id[s], t);
    return t;
}

// ------------------------------------------------------------------------------------------
// prep (compact, sliced): one workgroup of NTH / 64 waves per chunk (b, h, n): 4 at chunk 64,
// 8 at chunk 128 (one wave per 16-column block of A).  Writes, per chunk, the
// A-operand blocks of A'' = (I + L)^-1 diag(beta) as a bf16 hi + lo pair (AH, AL; the pair's sum
// carries the fp32 value to about 2^-17), the A-operand blocks of P~ (PA, zero above the
// diagonal) and the normalisers rho_k, rho_q (RK, RQ).
// LDS: phase 1 holds the raw k, q rows and one K and one Q slice; phase 2 (over it) L (fp32),
// the diagonal-block inverses, and P~ followed by A'' hi / lo over it.
// Raw k and q rows of one chunk in registers (16-byte units tid + NTH p) and its beta logit of
// row tid.
template <int C, int NTH>
struct SlicedStage {
    static constexpr int NPU = C * 8 / NTH;
    uint4 k[NPU], q[NPU];
    float bl;
};

// Issue the loads of chunk `blk`'s raw rows into `st`; a unit past the sequence end reads the
// chunk's first unit (always in range), and staging zeroes it.
template <int C, int NTH>
__device__ __forceinline__ void sliced_stage_load(const ChunkArgs& a, int64_t blk, SlicedStage<C, NTH>& st) {
    const int tid = threadIdx.x, T = a.T;
    const BhIndex bi = xcd_local(blk, a.BH, a.NC);
    const int t0 = static_cast<int>(bi.i) * C, Cc = min(C, T - t0);
    const int64_t row0 = static_cast<int64_t>(bi.bh) * T + t0;
    const uint4* kc = reinterpret_cast<const uint4*>(static_cast<const u16*>(a.k) + row0 * kSliceDk);
    const uint4* qc = reinterpret_cast<const uint4*>(static_cast<const u16*>(a.q) + row0 * kSliceDk);
#pragma unroll
    for (int p = 0; p < SlicedStage<C, NTH>::NPU; ++p) {
        const int e = tid + NTH * p;                   // 16-byte unit, row e / 8
        const int ee = (e >> 3) < Cc ? e : 0;
        st.k[p] = kc[ee];
        st.q[p] = qc[ee];
    }
    st.bl = bf16_bits_to_f32(static_cast<const u16*>(a.bl)[row0 + (tid < Cc ? tid : 0)]);
}

template <int C, int NU, int NTH, bool PERSIST>
__device__ __forceinline__ void prep_sliced_chunk(const ChunkArgs& a, int64_t blk, int64_t blk_next,
                                                  SlicedStage<C, NTH>& st) {
    constexpr int NT = C / 16, NTB = NT / 2, NW = NTH / 64;
    static_assert(NW >= NT, "one wave per block column of A");
    constexpr int NP = 2 * C * (kSliceDk / 8) / NTH;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // raw k and q rows: [C][XS]; at chunk 64 the rows are padded for the register-built
    // operands' window reads
    constexpr bool RAWGP = C == 64 && NW == 4;
    constexpr int XS = RAWGP ? kRawRow : kSliceDk;
    u16* Xk = reinterpret_cast<u16*>(smem + a.l_x);
    u16* Xq = Xk + C * XS;
    u16* Ks = reinterpret_cast<u16*>(smem + a.l_kr);          // [C][ss] K slice
    u16* Qs = reinterpret_cast<u16*>(smem + a.l_qr);          // [C][ss] Q slice
    float* Ls = reinterpret_cast<float*>(smem + a.l_ls);      // [C][lss] L      (phase 2)
    float* Li = reinterpret_cast<float*>(smem + a.l_li);      // [C][20] inverses (phase 2)
    u16* Ps = reinterpret_cast<u16*>(smem + a.l_ps);          // [C][pss] P~     (phase 2)
    u16* Bh = reinterpret_cast<u16*>(smem + a.l_ps);          // [C][aps] A'' hi, lo (over P~)
    u16* Bl = Bh + C * a.aps;
    float* rhok = reinterpret_cast<float*>(smem + a.l_small);
    float* rhoq = rhok + C;
    float* betas = rhoq + C;

    // In the chunk loop the lane index passes through an empty asm statement in every chunk, so
    // the per-lane address arithmetic is recomputed per chunk instead of hoisted out of the loop.
    int tid_opaque = static_cast<int>(threadIdx.x);
    if constexpr (PERSIST) __asm__ volatile("" : "+v"(tid_opaque));
    const int tid = tid_opaque, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = l & 15, g4 = l >> 4;
    const int T = a.T, ss = a.ss, aps = a.aps;
    const BhIndex bi = xcd_local(blk, a.BH, a.NC);
    const int bh = bi.bh, n = static_cast<int>(bi.i);
    const int64_t u = static_cast<int64_t>(bh) * a.NC + n;
    const int t0 = n * C, Cc = min(C, T - t0);

    // ---- stage the chunk's raw k and q rows (zeros past the sequence end) and beta from the
    //      registers loaded earlier, then issue the next chunk's loads into them
    {
#pragma unroll
        for (int p = 0; p < SlicedStage<C, NTH>::NPU; ++p) {
            const int e = tid + NTH * p;               // 16-byte unit, row e / 8
            const uint32_t m = (e >> 3) < Cc ? 0xffffffffu : 0u;
            const uint4 kv = make_uint4(st.k[p].x & m, st.k[p].y & m, st.k[p].z & m, st.k[p].w & m);
            const uint4 qv = make_uint4(st.q[p].x & m, st.q[p].y & m, st.q[p].z & m, st.q[p].w & m);
            if constexpr (XS == kSliceDk) {
                reinterpret_cast<uint4*>(Xk)[e] = kv;
                reinterpret_cast<uint4*>(Xq)[e] = qv;
            } else {
                // 8-byte aligned rows: two 8-byte stores per unit
                const int o = (e >> 3) * XS + 8 * (e & 7);
                *reinterpret_cast<uint2*>(Xk + o) = make_uint2(kv.x, kv.y);
                *reinterpret_cast<uint2*>(Xk + o + 4) = make_uint2(kv.z, kv.w);
                *reinterpret_cast<uint2*>(Xq + o) = make_uint2(qv.x, qv.y);
                *reinterpret_cast<uint2*>(Xq + o + 4) = make_uint2(qv.z, qv.w);
            }
        }
        if (tid < C) betas[tid] = tid < Cc ? sigmoid_stable(st.bl) : 0.0f;
        if (blk_next != blk) sliced_stage_load<C, NTH>(a, blk_next, st);
    }
    lds_barrier();

    // ---- G = K K^T and P = Q K^T over D, and the normalisers
    GPTiles<C, NW> gp;
    GPPair gpp;
    if constexpr (RAWGP) {
        // operands built in registers from the raw rows; partial tiles over the K and Q
        // slices' space (34 KB, dead at chunk 64)
        gp_raw_c64<NU>(gpp, Xk, Xq, reinterpret_cast<f32x4*>(Ks), rhok, rhoq, w, l, l16, g4);
    } else {
        gp_zero(gp);
        // shift slices through LDS; row sums from the DPFP tasks
        float sums[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) sums[p] = 0.0f;
        // a rolled loop: unrolled, the compiler keeps every slice's task inputs in registers
#pragma unroll 1
        for (int s = 0; s < NU; ++s) {
            dpfp_slice_any<C, NTH, true>(s + 1, Xk, Xq, Ks, Qs, ss, tid, sums);
            lds_barrier();
            gp_accumulate<true, C, false, NW>(gp, Ks, Qs, ss, kSliceCols, w, l16, g4);
            lds_barrier();
        }
        // row sums over the row's eight adjacent lanes (lane ^ 1, lane ^ 2, then the mirror
        // inside 8 lanes); the row's first lane writes rho = 1 / (sum + eps)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float s = sums[p];
            s += dpp_f32<0xB1>(s);
            s += dpp_f32<0x4E>(s);
            s += dpp_f32<0x141>(s);
            const int tau = tid + NTH * p, rt = tau >> 3;
            if ((tau & 7) == 0) (rt >= C ? rhoq + (rt - C) : rhok + rt)[0] = __builtin_amdgcn_rcpf(s + kDpfpEps);
        }
    }
    lds_barrier();

    if constexpr (RAWGP) {
        // waves 0, 1 hold G of pairs 0, 1; waves 2, 3 P of pairs 0, 1
        switch (w) {
            case 0: gp_scale_unit<true, C, 0>(gpp.ga, gpp.gb, false, rhok, rhoq, betas, Ls, a.lss, Ps, a.pss, l16, g4); break;
            case 1: gp_scale_unit<true, C, 1>(gpp.ga, gpp.gb, false, rhok, rhoq, betas, Ls, a.lss, Ps, a.pss, l16, g4); break;
            case 2: gp_scale_unit<true, C, 0>(gpp.pa, gpp.pb, true, rhok, rhoq, betas, Ls, a.lss, Ps, a.pss, l16, g4); break;
            default: gp_scale_unit<true, C, 1>(gpp.pa, gpp.pb, true, rhok, rhoq, betas, Ls, a.lss, Ps, a.pss, l16, g4); break;
        }
    } else {
        gp_scale<true, C>(gp, rhok, rhoq, betas, Ls, a.lss, Ps, a.pss, w, l16, g4);
    }
    lds_barrier();

    // ---- diagonal-block inverses; write-out of the P~ blocks (those on or below the diagonal,
    //      in tri_blk order) and the normalisers
    if (tid < C) diag_inverse(Ls, a.lss, Li, tid);
    {
        char* pa = a.ws + a.o_pa + u * (static_cast<int64_t>(tri_nblocks(C)) * 1024);
        for (int e = tid; e < NT * NTB * 64; e += NTH) {
            const int blk = e >> 6, lam = e & 63, ta = blk / NTB, j = blk % NTB;
            if (2 * j > ta) continue;                    // uniform over the wave
            const u16* src = Ps + (16 * ta + (lam & 15)) * a.pss + 32 * j + 4 * (lam >> 4);
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
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
            *reinterpret_cast<uint4*>(blk_ptr(pa, tri_blk(ta, j), lam)) = val;
        }
        if (tid < C) {
            reinterpret_cast<float*>(a.ws + a.o_rk)[u * C + tid] = rhok[tid];
            reinterpret_cast<float*>(a.ws + a.o_rq)[u * C + tid] = rhoq[tid];
        }
    }
    lds_barrier();   // Li complete; P~ is dead (its space holds A'')

    // ---- A = (I + L)^-1 by block columns (column block tb = w), stored as A'' = A diag(beta)
    //      in bf16 hi + lo:  A[ta][tb] = -Li[ta] sum_{tb <= tc < ta} L[ta][tc] A[tc][tb].  At
    //      chunk 64 each block goes to row layout on the MFMA and straight into its A-operand
    //      blocks in the workspace (half tb & 1 of block (ta, tb / 2); a block on the diagonal
    //      with even ta also writes its zero half); otherwise through LDS (Bh, Bl).
    char* ahg = a.ws + a.o_ah + u * (static_cast<int64_t>(tri_nblocks(C)) * 1024);
    char* alg = a.ws + a.o_al + u * (static_cast<int64_t>(tri_nblocks(C)) * 1024);
    float id[4];                                       // identity B operands of tile_to_rows
#pragma unroll
    for (int s = 0; s < 4; ++s) id[s] = 4 * g4 + s == l16 ? 1.0f : 0.0f;
    if (w < NT) {
        const int tb = w;
        const float bsc = betas[16 * tb + l16];
        const f32x4 bsr = *reinterpret_cast<const f32x4*>(betas + 16 * tb + 4 * g4);
        f32x4 Ab[NT];
#pragma unroll
        for (int ta = 0; ta < NT; ++ta) {
            f32x4 val = zero4();
            if (ta == tb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = Li[(16 * ta + 4 * g4 + e) * kLiStride + l16];
            } else if (ta > tb) {
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
            if constexpr (RAWGP) {
                if (ta >= tb) {
                    const f32x4 y = tile_to_rows(val, id) * bsr;
                    const uint2 hi = pack_bf16x4(y), lo = bf16_lo_part4(y);
                    const int64_t off = (static_cast<int64_t>(tri_blk(ta, tb >> 1)) * 64 + l) * 16;
                    if (ta == tb && (tb & 1) == 0) {
                        *reinterpret_cast<uint4*>(ahg + off) = make_uint4(hi.x, hi.y, 0u, 0u);
                        *reinterpret_cast<uint4*>(alg + off) = make_uint4(lo.x, lo.y, 0u, 0u);
                    } else {
                        *reinterpret_cast<uint2*>(ahg + off + 8 * (tb & 1)) = hi;
                        *reinterpret_cast<uint2*>(alg + off + 8 * (tb & 1)) = lo;
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int at = (16 * ta + 4 * g4 + e) * aps + 16 * tb + l16;
                    const float y = val[e] * bsc;
                    const u16 yh = f32_to_bf16_bits(y);
                    Bh[at] = yh;
                    Bl[at] = f32_to_bf16_bits(y - bf16_bits_to_f32(yh));
                }
            }
        }
    }
    if constexpr (RAWGP) return;
    lds_barrier();

    // ---- AH, AL: A-operand blocks (ta, j) of A'' hi and lo (slot (h, e) of lane l =
    //      A''[16 ta + l % 16][16 (2 j + h) + 4 (l / 16) + e]), those on or below the diagonal
    //      in tri_blk order
    {
        char* ah = ahg;
        char* al = alg;
        for (int e = tid; e < NT * NTB * 64; e += NTH) {
            const int blk = e >> 6, lam = e & 63, ta = blk / NTB, j = blk % NTB;
            if (2 * j > ta) continue;                    // uniform over the wave
            const int at = (16 * ta + (lam & 15)) * aps + 32 * j + 4 * (lam >> 4);
            const uint2 h0 = *reinterpret_cast<const uint2*>(Bh + at);
            const uint2 h1 = *reinterpret_cast<const uint2*>(Bh + at + 16);
            const uint2 l0 = *reinterpret_cast<const uint2*>(Bl + at);
            const uint2 l1 = *reinterpret_cast<const uint2*>(Bl + at + 16);
            const int tb = tri_blk(ta, j);
            *reinterpret_cast<uint4*>(blk_ptr(ah, tb, lam)) = make_uint4(h0.x, h0.y, h1.x, h1.y);
            *reinterpret_cast<uint4*>(blk_ptr(al, tb, lam)) = make_uint4(l0.x, l0.y, l1.x, l1.y);
        }
    }
}

// The sliced prep kernel: one workgroup per chunk, or, with PERSIST (more chunks than fit at
// once), a grid of the resident workgroups (a multiple of 8) that walks the chunks with the grid
// as stride, loading the next chunk's raw rows while the current one is processed.
template <int C, int NU, int NTH = kSliceThreads, bool PERSIST = false>
__global__ __launch_bounds__(NTH, (C == 64 && !PERSIST) ? 3 : 1) void delta_prep_sliced_kernel(ChunkArgs a) {
    SlicedStage<C, NTH> st;
    if constexpr (!PERSIST) {
        sliced_stage_load<C, NTH>(a, blockIdx.x, st);
        prep_sliced_chunk<C, NU, NTH, false>(a, blockIdx.x, blockIdx.x, st);
    } else {
        const int64_t total = static_cast<int64_t>(a.BH) * a.NC;
        int64_t blk = blockIdx.x;
        if (blk < total) sliced_stage_load<C, NTH>(a, blk, st);
        for (; blk < total; blk += gridDim.x) {
            const int64_t nxt = blk + gridDim.x < total ? blk + gridDim.x : blk;
            prep_sliced_chunk<C, NU, NTH, true>(a, blk, nxt, st);
            lds_barrier();                 // LDS of this chunk is dead before the next staging
        }
    }
}

// ------------------------------------------------------------------------------------------
// stream (sliced): one workgroup of NW = C / 16 waves per (b, h, 16 NCT columns of d_v), serial
// over the chunks: chunk 128 with 8 waves and 32 columns, or chunk 64 with 4 waves and 16
// columns (67.5 KB of LDS at D = 384, so two workgroups share a CU and overlap their phases).
// The fp32 memory W^T (D x 16 NCT) lives in MFMA accumulators: wave w holds d-tiles
// w + NW r (r < 8 / NW) of every shift slice s (global d-tile 8 s + w + NW r), all column
// tiles.  Wave w owns row tile w of X, Q W^T, U and Y.  Per chunk:
//   B  for each slice s: build K_s, Q_s; X += K_s W_s^T, Q W^T += Q_s W_s^T (bf16 W^T copy in
//      LDS, refreshed at the top of the chunk); then Z = V - rho_k o X (fp32, over the Q slice)
//   C  U = A'' Z (A'' and Z as bf16 hi + lo pairs, 3 MFMAs per k-step), over the Q slice
//   D  Y = rho_q o (Q W^T) + P~ U (bf16 rows to LDS); for each slice s: build K_s again and
//      W_s^T += K_s^T (rho_k o U), K_s^T read by LDS transpose reads; then the next chunk's raw
//      rows, loaded into registers at the top of the chunk, go to the raw slot.
//   After the last barrier every thread stores 8 NCT bytes of the chunk's y with a buffer
//   store whose range check drops rows past the sequence end.
// Every wave issues the same global loads and stores in every chunk with no branch around
// them, so the compiler's in-order wait counts stay exact.  Per thread, every chunk moves 32
// bytes of raw k and q rows, 8 NCT bytes of v and 8 NCT bytes of y for either shape.
template <int C, int NU, int NCT>
__global__ __launch_bounds__(4 * C, 512 / (4 * C)) void delta_stream_sliced_kernel(ChunkArgs a) {
    constexpr int NW = C / 16, NTH = 64 * NW, NT = C / 16, NTB = NT / 2;
    constexpr int NR = 8 / NW;                               // d-tiles per wave and slice
    constexpr int NPK = C * (kSliceDk / 8) / NTH;            // K-only DPFP tasks per thread
    constexpr int NPQ = 2 * NPK;                             // K and Q
    constexpr int RU = C * kSliceDk / 8 / NTH;               // 16-byte raw k units per thread
    constexpr int CW = 16 * NCT;                             // columns of the workgroup
    static_assert(NW == 4 || NW == 8, "chunk 64 or 128");
    static_assert(C * CW * 2 == NTH * 8 * NCT, "8 NCT bytes of v and y per thread");
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    using VU = std::conditional_t<NCT == 1, uint2, uint4>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = l & 15, g4 = l >> 4;
    const int d_v = a.d_v, D = a.D, T = a.T, NC = a.NC, ss = a.ss;
    const BhIndex bi = xcd_local(blockIdx.x, a.BH, d_v / CW);
    const int bh = bi.bh, cp = static_cast<int>(bi.i);
    const int col0 = CW * cp;

    u16* Ks = reinterpret_cast<u16*>(smem + a.s_k);
    u16* Qs = reinterpret_cast<u16*>(smem + a.s_q);
    char* WT = smem + a.s_wt;                       // B blocks (jb, ct) of W^T, bf16
    float* Zb = reinterpret_cast<float*>(smem + a.s_z);   // over the Q slice
    float* Ub = reinterpret_cast<float*>(smem + a.s_u);   // over the Q slice
    u16* Yb = reinterpret_cast<u16*>(smem + a.s_y);       // [C][CW] bf16
    char* sb = smem + a.s_raw;
    const u16* Xk = reinterpret_cast<const u16*>(sb);
    const u16* Xq = reinterpret_cast<const u16*>(sb + a.s_qoff);
    const u16* Xv = reinterpret_cast<const u16*>(sb + a.s_voff);   // [C][CW]
    auto tile = [&](float* base, int r, int c) { return reinterpret_cast<f32x4*>(base + ((r * NCT + c) * 64 + l) * 4); };
    auto wblk = [&](int jb, int ct) { return WT + ((jb * NCT + ct) * 64 + l) * 16; };

    // ---- memory tiles: d-tile 8 s + w + NW r, column tile ct
    f32x4 Wst[NU][NR][NCT];
#pragma unroll
    for (int s = 0; s < NU; ++s)
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                Wst[s][r][ct] = zero4();
                if (a.W0) {
                    // internal columns c0 .. c0+3 = positions (o, o + d_k, o + 1, o + d_k + 1)
                    const float* src = a.W0 + (static_cast<int64_t>(bh) * d_v + col0 + 16 * ct + l16) * D +
                                       orig_col(16 * (8 * s + w + NW * r) + 4 * g4, kSliceDk);
                    const float2 lo = *reinterpret_cast<const float2*>(src);
                    const float2 hi = *reinterpret_cast<const float2*>(src + kSliceDk);
                    Wst[s][r][ct] = f32x4{lo.x, hi.x, lo.y, hi.y};
                }
            }

    // ---- raw inputs of a chunk: k and q rows ([C][64] bf16, RU 16-byte units per thread) and
    //      the workgroup's CW v columns ([C][CW], 8 NCT bytes per thread).  A unit past the
    //      sequence end reads unit 0 of the chunk (in range) and is zeroed by its mask.
    const int64_t row0 = static_cast<int64_t>(bh) * T;
    const uint4* kB = reinterpret_cast<const uint4*>(static_cast<const u16*>(a.k) + row0 * kSliceDk);
    const uint4* qB = reinterpret_cast<const uint4*>(static_cast<const u16*>(a.q) + row0 * kSliceDk);
    const u16* vB = static_cast<const u16*>(a.v) + row0 * d_v + col0;
    constexpr int VPR = CW / (4 * NCT);                      // v units per row (4 NCT columns each)
    uint4 rk[RU], rq[RU];
    VU rv;
    uint32_t mk[RU], mv = 0u;
    auto load_raw = [&](int n) {
        const int t0 = n * C, Cn = min(C, T - t0);
#pragma unroll
        for (int p = 0; p < RU; ++p) {
            const int e = tid + NTH * p;
            const bool ok = (e >> 3) < Cn;
            const int64_t o = static_cast<int64_t>(t0) * 8 + (ok ? e : 0);
            rk[p] = kB[o];
            rq[p] = qB[o];
            mk[p] = ok ? 0xffffffffu : 0u;
        }
        const bool okv = tid / VPR < Cn;
        rv = *reinterpret_cast<const VU*>(vB + static_cast<int64_t>(t0 + (okv ? tid / VPR : 0)) * d_v +
                                          (okv ? 4 * NCT * (tid % VPR) : 0));
        mv = okv ? 0xffffffffu : 0u;
    };
    auto store_raw = [&]() {
#pragma unroll
        for (int p = 0; p < RU; ++p) {
            const int e = tid + NTH * p;
            const uint32_t m = mk[p];
            reinterpret_cast<uint4*>(sb)[e] = make_uint4(rk[p].x & m, rk[p].y & m, rk[p].z & m, rk[p].w & m);
            reinterpret_cast<uint4*>(sb + a.s_qoff)[e] = make_uint4(rq[p].x & m, rq[p].y & m, rq[p].z & m, rq[p].w & m);
        }
        if constexpr (NCT == 1)
            reinterpret_cast<uint2*>(sb + a.s_voff)[tid] = make_uint2(rv.x & mv, rv.y & mv);
        else
            reinterpret_cast<uint4*>(sb + a.s_voff)[tid] = make_uint4(rv.x & mv, rv.y & mv, rv.z & mv, rv.w & mv);
    };

    // ---- per-chunk results of the prep kernel: A'' blocks (w, j) hi and lo, P~ blocks (w, j),
    //      rho_k of every row tile and rho_q of row tile w (accumulator row order).  Blocks
    //      above the diagonal are not stored: their loads re-read the row tile's last block and
    //      go unused (every wave issues the same loads in every chunk)
    uint4 ah[NTB], al[NTB], pa[NTB];
    f32x4 rka[NT], rqv;
    auto load_ws = [&](int n) {
        const int64_t u = static_cast<int64_t>(bh) * NC + n;
        const char* ahp = a.ws + a.o_ah + u * (tri_nblocks(C) * 1024);
        const char* alp = a.ws + a.o_al + u * (tri_nblocks(C) * 1024);
        const char* pap = a.ws + a.o_pa + u * (tri_nblocks(C) * 1024);
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
            const int tb = tri_blk(w, min(j, w >> 1));
            ah[j] = *reinterpret_cast<const uint4*>(blk_ptr(ahp, tb, l));
            al[j] = *reinterpret_cast<const uint4*>(blk_ptr(alp, tb, l));
            pa[j] = *reinterpret_cast<const uint4*>(blk_ptr(pap, tb, l));
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
            rka[tt] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.ws + a.o_rk) + u * C + 16 * tt + 4 * g4);
        rqv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.ws + a.o_rq) + u * C + 16 * w + 4 * g4);
    };

    if (NC > 0) {
        load_raw(0);
        store_raw();
    }
    lds_barrier();

    // y of this workgroup's columns as a buffer: offsets from (b, h, t = 0, col0); the range ends
    // where row T would begin, so rows past the sequence end are dropped by the hardware
    const __amdgpu_buffer_rsrc_t yrsrc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<u16*>(a.y) + row0 * d_v + col0, static_cast<short>(0),
        static_cast<int>((static_cast<uint32_t>(T) * d_v - col0) * 2u), kBufferWord3);
    float unused_q[NPQ], unused_k[NPK];   // the serial pass takes rho from the prep; the task
                                          // sums written here are dead and compiled away
    for (int n = 0; n < NC; ++n) {
        const int t0 = n * C;
        const int nn = n + 1 < NC ? n + 1 : n;          // the last chunk re-reads itself
        load_ws(n);
        load_raw(nn);

        // ---- W^T copy (bf16 B blocks): wave w writes its d-tiles
#pragma unroll
        for (int s = 0; s < NU; ++s)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int dt = 8 * s + w + NW * r;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    *reinterpret_cast<uint2*>(wblk(dt >> 1, ct) + 8 * (dt & 1)) =
                        make_uint2(pack_bf16x2(Wst[s][r][ct][0], Wst[s][r][ct][1]),
                                   pack_bf16x2(Wst[s][r][ct][2], Wst[s][r][ct][3]));
            }

        // ---- B: X = K W^T and Q W^T for row tile w, slice by slice
        f32x4 xacc[NCT], qacc[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) xacc[ct] = qacc[ct] = zero4();
        const int ro = (16 * w + l16) * ss + 4 * g4;
        const u16* kr = Ks;
        const u16* qr = Qs;
        auto opnd = [&](const u16* r, int kk) {
            const bf16x4 x0 = lds_read_b64_single(r, ro + 32 * kk);
            const bf16x4 x1 = lds_read_b64_single(r, ro + 32 * kk + 16);
            return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
#pragma unroll
        for (int s = 0; s < NU; ++s) {
            dpfp_slice_any<C, NTH, true>(s + 1, Xk, Xq, Ks, Qs, ss, tid, unused_q);
            lds_barrier();
#pragma unroll
            for (int kk = 0; kk < kSliceCols / 32; ++kk) {
                const int jb = (kSliceCols / 32) * s + kk;
                const bf16x8 ak = opnd(kr, kk), aq = opnd(qr, kk);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const bf16x8 wb = as_bf16x8(*reinterpret_cast<const uint4*>(wblk(jb, ct)));
                    xacc[ct] = mfma_bf16_k32(ak, wb, xacc[ct]);
                    qacc[ct] = mfma_bf16_k32(aq, wb, qacc[ct]);
                }
            }
            lds_barrier();
        }
        {
            // Z = V - rho_k o X (rows 16 w + 4 g4 + e, columns 16 ct + l16), over the Q slice
            const f32x4 rkc = rka[w];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    xacc[ct][e] = bf16_bits_to_f32(Xv[(16 * w + 4 * g4 + e) * CW + 16 * ct + l16]) - rkc[e] * xacc[ct][e];
                *tile(Zb, w, ct) = xacc[ct];
                qacc[ct] *= rqv;
            }
        }
        lds_barrier();

        // ---- C: U tiles (w, ct) = A'' Z
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 uacc = zero4();
#pragma unroll
            for (int j = 0; j < NTB; ++j) {
                if (2 * j > w) break;                            // A'' is zero above the diagonal
                const f32x4 z0 = *tile(Zb, 2 * j, ct), z1 = *tile(Zb, 2 * j + 1, ct);
                const bf16x8 zh = as_bf16x8(pack_bf16x8(z0, z1));
                const bf16x8 zl = as_bf16x8(bf16_lo_part(z0, z1));
                uacc = mfma_bf16_k32(as_bf16x8(ah[j]), zh, uacc);
                uacc = mfma_bf16_k32(as_bf16x8(ah[j]), zl, uacc);
                uacc = mfma_bf16_k32(as_bf16x8(al[j]), zh, uacc);
            }
            *tile(Ub, w, ct) = uacc;
        }
        lds_barrier();

        // ---- D: Y tiles (w, ct), then the memory update slice by slice
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 y = qacc[ct];
#pragma unroll
            for (int j = 0; j < NTB; ++j) {
                if (2 * j > w) break;
                const bf16x8 ub = as_bf16x8(pack_bf16x8(*tile(Ub, 2 * j, ct), *tile(Ub, 2 * j + 1, ct)));
                y = mfma_bf16_k32(as_bf16x8(pa[j]), ub, y);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Yb[(16 * w + 4 * g4 + e) * CW + 16 * ct + l16] = f32_to_bf16_bits(y[e]);
        }
        // B operands rho_k o U of rows 32 j .. 32 j + 31 (tiles 2 j, 2 j + 1)
        bf16x8 ubk[NTB][NCT];
#pragma unroll
        for (int j = 0; j < NTB; ++j)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                ubk[j][ct] = as_bf16x8(pack_bf16x8(*tile(Ub, 2 * j, ct) * rka[2 * j], *tile(Ub, 2 * j + 1, ct) * rka[2 * j + 1]));
#pragma unroll
        for (int s = 0; s < NU; ++s) {
            // K_s again (the previous K slice is dead: its last reads were in phase B)
            dpfp_slice_any<C, NTH, false>(s + 1, Xk, nullptr, Ks, nullptr, ss, tid, unused_k);
            lds_barrier();
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const u16* kt = Ks + (4 * g4 + (l16 >> 2)) * ss + 16 * (w + NW * r) + 4 * (l16 & 3);
#pragma unroll
                for (int j = 0; j < NTB; ++j) {
                    const u16* kc = kt + 32 * j * ss;
                    const bf16x4 c0 = lds_read_tr_b16x4(kc);
                    const bf16x4 c1 = lds_read_tr_b16x4(kc + 16 * ss);
                    const bf16x8 kta = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) Wst[s][r][ct] = mfma_bf16_k32(kta, ubk[j][ct], Wst[s][r][ct]);
                }
            }
            if (s + 1 < NU) lds_barrier();                       // compile-time condition
        }
        // the raw slot's last reads were the K builds above, each followed by a barrier
        store_raw();
        lds_barrier();
        // y rows of the chunk: 8 NCT bytes per thread; rows past the sequence end fall outside
        // the buffer's range and are dropped
        {
            const int t = tid / VPR, c4 = 4 * NCT * (tid % VPR);
            const VU v4 = *reinterpret_cast<const VU*>(Yb + t * CW + c4);
            if constexpr (NCT == 1)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{v4.x, v4.y}, yrsrc, ((t0 + t) * d_v + c4) * 2, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{v4.x, v4.y, v4.z, v4.w}, yrsrc,
                                                       ((t0 + t) * d_v + c4) * 2, 0, 0);
        }
    }

    if (a.Wf) {
#pragma unroll
        for (int s = 0; s < NU; ++s)
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    float* dst = a.Wf + (static_cast<int64_t>(bh) * d_v + col0 + 16 * ct + l16) * D +
                                 orig_col(16 * (8 * s + w + NW * r) + 4 * g4, kSliceDk);
                    *reinterpret_cast<float2*>(dst) = make_float2(Wst[s][r][ct][0], Wst[s][r][ct][2]);
                    *reinterpret_cast<float2*>(dst + kSliceDk) = make_float2(Wst[s][r][ct][1], Wst[s][r][ct][3]);
                }
    }
}

}  // namespace fwa
