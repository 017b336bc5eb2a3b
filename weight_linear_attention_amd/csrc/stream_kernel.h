// Streaming forward of the fast-weight delta rule for bf16 inputs: the serial pass over the
// chunks without the D-wide workspace of the chunked path.
//
// The recurrence ("Fast Weights Transformer" guide, xdnf.cn/news/308600, sections
// "FastWeightsAttention / update formula" and "... / module structure and source walkthrough")
// is evaluated chunk by chunk with the chunked algebra derived from it: for a chunk of C rows
// starting from memory W (d_v x D), with raw DPFP tiles K, Q, normalisers rho_k, rho_q and
// A'' = (I + L)^-1 diag(beta) (L = diag(beta) strict_lower(K~ K~^T)):
//     X = K W^T,   U = A'' (V - rho_k o X),   Y = rho_q o (Q W^T) + P~ U,   W^T += K^T (rho_k o U).
// A'', P~ and the normalisers do not depend on the memory; the prep kernel (compact mode) forms
// them for all chunks at once, about 24.5 KB per chunk.  This kernel runs the memory-dependent
// part: one workgroup of 8 waves per (b, h, 32 columns of d_v), the fp32 memory W^T (D x 32)
// in MFMA accumulators, ND / 8 d-tiles per wave x 2 column tiles.  Per chunk:
//   A  K and Q tiles from the raw rows (DPFP tasks over all 512 threads); each wave writes its
//      memory tiles as bf16 halves of the B-operand blocks of W^T (the LDS copy the products
//      read).
//   Wave w owns tile (row tile w % 4, column tile w / 4) of X, Q W^T, U and Y:
//   B  X = K W^T and Q W^T over all of D (one W^T block per k-step feeds both products); Z =
//      V - rho_k o X to LDS (split once into bf16 hi and lo B blocks), rho_q o Q W^T kept in
//      registers.
//   C  U = A'' Z (A'' and Z as bf16 hi + lo pairs, 3 MFMAs per k-step).
//   D  Y = rho_q o (Q W^T) + P~ U, as bf16 rows in LDS (over Z); the wave's memory tiles +=
//      K^T (rho_k o U), K^T read from the K tile by LDS
//      transpose reads; the next chunk's raw k, q, v (loaded at the top of the chunk, after
//      this chunk's A'', P~ and normalisers) go to the raw slot, dead since phase B.
//   After the last barrier every thread stores 8 bytes of the chunk's y with a buffer store
//   whose range check drops rows past the sequence end.
// Four LDS-only barriers per chunk.  Every wave issues the same global loads and stores in
// every chunk with no branch around them, so the compiler's in-order wait counts stay exact:
// a wait for data loaded earlier never waits for the y stores issued after it.
#pragma once

#include "chunk_tile.h"
#include "chunked_kernels.h"

namespace fwa {

constexpr int kStreamWaves = 8;
// Word 3 of a raw buffer resource on gfx9-family GPUs: 32-bit data format (a zero format
// disables the access); the hardware drops accesses at or past the range in word 2.
constexpr int kBufferWord3 = 0x00020000;

template <int C, int NDW>
__global__ __launch_bounds__(512, 1) void delta_stream_kernel(ChunkArgs a) {
    static_assert(C == 64, "row tiles map one-to-one onto waves 0-3 and 4-7");
    constexpr int NT = C / 16, NTB = NT / 2;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = l & 15, g4 = l >> 4;
    const int d_k = a.d_k, d_v = a.d_v, D = a.D, T = a.T, NC = a.NC, krs = a.krs;
    const int NP = d_v / 32;
    const BhIndex bi = xcd_local(blockIdx.x, a.BH, NP);
    const int bh = bi.bh, cp = static_cast<int>(bi.i);
    const int col0 = 32 * cp;
    const int rt = w & 3, ct = w >> 2;         // the wave's (row tile, column tile) of X, Q W^T,
                                               // U and Y

    u16* Kt = reinterpret_cast<u16*>(smem + a.s_k);
    u16* Qt = reinterpret_cast<u16*>(smem + a.s_q);
    char* WT = smem + a.s_wt;                  // B blocks (jb, ct) of W^T, bf16
    char* Zc = smem + a.s_z;                   // Z as bf16 hi, then lo at + 4 KiB: B blocks of
                                               // 32 rows (row pair j, column tile c)
    float* Ub = reinterpret_cast<float*>(smem + a.s_u);
    char* sb = smem + a.s_raw;                 // raw k rows, q rows, v columns of one chunk
    auto tile = [&](float* base, int r, int c) { return reinterpret_cast<f32x4*>(base + ((r * 2 + c) * 64 + l) * 4); };

    // ---- memory tiles: d-tile w + 8 s, column tile ct
    f32x4 Wst[NDW][2];
#pragma unroll
    for (int s = 0; s < NDW; ++s)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            Wst[s][ct] = zero4();
            if (a.W0) {
                // internal columns c0 .. c0+3 = positions (o, o + d_k, o + 1, o + d_k + 1)
                const float* src = a.W0 + (static_cast<int64_t>(bh) * d_v + col0 + 16 * ct + l16) * D +
                                   orig_col(16 * (w + 8 * s) + 4 * g4, d_k);
                const float2 lo = *reinterpret_cast<const float2*>(src);
                const float2 hi = *reinterpret_cast<const float2*>(src + d_k);
                Wst[s][ct] = f32x4{lo.x, hi.x, lo.y, hi.y};
            }
        }

    // ---- raw inputs of a chunk: k and q rows (bf16 [C][d_k]) and the workgroup's 32 v columns
    //      ([C][32]); registers at the top of the previous chunk, the LDS slot in its phase D
    const int64_t row0 = static_cast<int64_t>(bh) * T;
    const u16* kB = static_cast<const u16*>(a.k) + row0 * d_k;
    const u16* qB = static_cast<const u16*>(a.q) + row0 * d_k;
    const u16* vB = static_cast<const u16*>(a.v) + row0 * d_v + col0;
    const int kunits = C * d_k / 8;            // 16-byte units of the k (and q) block: <= 512
    const int ush = __builtin_ctz(d_k) - 3;    // unit u lies in row u >> ush
    // Loads are branch-free: a unit past the sequence end reads unit 0 of the chunk (always in
    // range) and is zeroed by its mask when it is written to LDS, so no wait follows the loads.
    uint4 rk, rq, rv;
    uint32_t mk = 0u, mv = 0u;
    auto load_raw = [&](int n) {
        const int t0 = n * C, Cn = min(C, T - t0);
        const bool okk = tid < kunits && (tid >> ush) < Cn;
        const int64_t ko = static_cast<int64_t>(t0) * d_k + (okk ? tid * 8 : 0);
        rk = *reinterpret_cast<const uint4*>(kB + ko);
        rq = *reinterpret_cast<const uint4*>(qB + ko);
        const bool okv = tid < 4 * C && (tid >> 2) < Cn;
        rv = *reinterpret_cast<const uint4*>(vB + static_cast<int64_t>(t0 + (okv ? tid >> 2 : 0)) * d_v +
                                             (okv ? 8 * (tid & 3) : 0));
        mk = okk ? 0xffffffffu : 0u;
        mv = okv ? 0xffffffffu : 0u;
    };
    auto store_raw = [&]() {
        rk = make_uint4(rk.x & mk, rk.y & mk, rk.z & mk, rk.w & mk);
        rq = make_uint4(rq.x & mk, rq.y & mk, rq.z & mk, rq.w & mk);
        rv = make_uint4(rv.x & mv, rv.y & mv, rv.z & mv, rv.w & mv);
        if (tid < kunits) {
            reinterpret_cast<uint4*>(sb)[tid] = rk;
            reinterpret_cast<uint4*>(sb + a.s_qoff)[tid] = rq;
        }
        if (tid < 4 * C) reinterpret_cast<uint4*>(sb + a.s_voff)[tid] = rv;
    };

    // ---- per-chunk results of the prep kernel: A'' blocks (rt, j) hi and lo, P~ blocks
    //      (rt, j) (Y waves), rho_k of every row tile and rho_q of row tile rt (accumulator row
    //      order)
    uint4 ah[NTB], al[NTB], pa[NTB];
    f32x4 rka[NT], rqv;
    auto load_ws = [&](int n) {
        const int64_t u = static_cast<int64_t>(bh) * NC + n;
        const char* ahp = a.ws + a.o_ah + u * (C * C * 2);
        const char* alp = a.ws + a.o_al + u * (C * C * 2);
        const char* pap = a.ws + a.o_pa + u * (C * C * 2);
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
            ah[j] = *reinterpret_cast<const uint4*>(blk_ptr(ahp, rt * NTB + j, l));
            al[j] = *reinterpret_cast<const uint4*>(blk_ptr(alp, rt * NTB + j, l));
            pa[j] = *reinterpret_cast<const uint4*>(blk_ptr(pap, rt * NTB + j, l));
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
            rka[tt] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.ws + a.o_rk) + u * C + 16 * tt + 4 * g4);
        rqv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.ws + a.o_rq) + u * C + 16 * rt + 4 * g4);
    };

    if (NC > 0) {
        load_raw(0);
        store_raw();
    }
    lds_barrier();

    // y of this workgroup's columns as a buffer: offsets from (b, h, t = 0, col0); the range ends
    // where row T would begin, so rows past the sequence end are dropped by the hardware
    u16* Yb = reinterpret_cast<u16*>(smem + a.s_z);          // [C][32] bf16, over Z
    const __amdgpu_buffer_rsrc_t yrsrc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<u16*>(a.y) + row0 * d_v + col0, static_cast<short>(0),
        static_cast<int>((static_cast<uint32_t>(T) * d_v - col0) * 2u), kBufferWord3);
    for (int n = 0; n < NC; ++n) {
        const int t0 = n * C;
        const int nn = n + 1 < NC ? n + 1 : n;          // the last chunk re-reads itself
        // this chunk's prep results (first used in phase B), then the next chunk's raw rows
        load_ws(n);
        load_raw(nn);
        const f32x4 rkc = rka[rt];

        // ---- A: K and Q tiles, W^T copy
        dpfp_chunk<u16, u16, C, 512, true>(reinterpret_cast<const u16*>(sb),
                                           reinterpret_cast<const u16*>(sb + a.s_qoff), Kt, Qt,
                                           krs, d_k, a.nu, w, l);
#pragma unroll
        for (int s = 0; s < NDW; ++s) {
            const int dt = w + 8 * s;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                *reinterpret_cast<uint2*>(WT + (((dt >> 1) * 2 + ct) * 64 + l) * 16 + 8 * (dt & 1)) =
                    make_uint2(pack_bf16x2(Wst[s][ct][0], Wst[s][ct][1]), pack_bf16x2(Wst[s][ct][2], Wst[s][ct][3]));
        }
        lds_barrier();                                           // B1

        // ---- B: X = K W^T and Q W^T for tile (rt, ct)
        f32x4 xacc = zero4(), qacc = zero4();
        {
            constexpr int NDB = 4 * NDW;                           // D / 32 k-steps
            const int ro = (16 * rt + l16) * krs + 4 * g4;
            const u16* kr = Kt;
            const u16* qr = Qt;
            auto opnd = [&](const u16* r, int jb) {
                const bf16x4 x0 = lds_read_b64_single(r, ro + 32 * jb);
                const bf16x4 x1 = lds_read_b64_single(r, ro + 32 * jb + 16);
                return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
            };
            auto wblk = [&](int jb) {
                return as_bf16x8(*reinterpret_cast<const uint4*>(WT + ((jb * 2 + ct) * 64 + l) * 16));
            };
            // fully unrolled: the scheduler issues the LDS reads several k-steps ahead; two
            // accumulators per product keep consecutive MFMAs independent
            f32x4 xacc1 = zero4(), qacc1 = zero4();
#pragma unroll
            for (int jb = 0; jb < NDB; jb += 2) {
                const bf16x8 w0 = wblk(jb), w1 = wblk(jb + 1);
                xacc = mfma_bf16_k32(opnd(kr, jb), w0, xacc);
                qacc = mfma_bf16_k32(opnd(qr, jb), w0, qacc);
                xacc1 = mfma_bf16_k32(opnd(kr, jb + 1), w1, xacc1);
                qacc1 = mfma_bf16_k32(opnd(qr, jb + 1), w1, qacc1);
            }
            xacc += xacc1;
            qacc += qacc1;
        }
        {
            // Z = V - rho_k o X (rows 16 rt + 4 g4 + e, columns 16 ct + l16)
            const u16* vs = reinterpret_cast<const u16*>(sb + a.s_voff);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                xacc[e] = bf16_bits_to_f32(vs[(16 * rt + 4 * g4 + e) * 32 + 16 * ct + l16]) - rkc[e] * xacc[e];
            // split once, by the wave that forms the tile, into the hi and lo blocks U = A'' Z reads
            char* const zd = Zc + (((rt >> 1) * 2 + ct) * 64 + l) * 16 + 8 * (rt & 1);
            *reinterpret_cast<uint2*>(zd) = pack_bf16x4(xacc);
            *reinterpret_cast<uint2*>(zd + 4096) = bf16_lo_part4(xacc);
            qacc *= rqv;
        }
        lds_barrier();                                           // B2

        // ---- C: U tile (rt, ct) = A'' Z
        {
            f32x4 u = zero4();
#pragma unroll
            for (int j = 0; j < NTB; ++j) {
                if (2 * j > rt) break;                            // A'' is zero above the diagonal
                const char* zs = Zc + ((j * 2 + ct) * 64 + l) * 16;
                const bf16x8 zh = as_bf16x8(*reinterpret_cast<const uint4*>(zs));
                const bf16x8 zl = as_bf16x8(*reinterpret_cast<const uint4*>(zs + 4096));
                u = mfma_bf16_k32(as_bf16x8(ah[j]), zh, u);
                u = mfma_bf16_k32(as_bf16x8(ah[j]), zl, u);
                u = mfma_bf16_k32(as_bf16x8(al[j]), zh, u);
            }
            *tile(Ub, rt, ct) = u;
        }
        lds_barrier();                                           // B3

        // ---- D: Y tile (rt, ct), memory update, next chunk's raw inputs
        {
            f32x4 y = qacc;
#pragma unroll
            for (int j = 0; j < NTB; ++j) {
                if (2 * j > rt) break;
                const bf16x8 ub = as_bf16x8(pack_bf16x8(*tile(Ub, 2 * j, ct), *tile(Ub, 2 * j + 1, ct)));
                y = mfma_bf16_k32(as_bf16x8(pa[j]), ub, y);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Yb[(16 * rt + 4 * g4 + e) * 32 + 16 * ct + l16] = f32_to_bf16_bits(y[e]);
        }
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
            // B operand rho_k o U of rows 32 j .. 32 j + 31 (tiles 2 j, 2 j + 1)
            const bf16x8 ub0 = as_bf16x8(pack_bf16x8(*tile(Ub, 2 * j, 0) * rka[2 * j], *tile(Ub, 2 * j + 1, 0) * rka[2 * j + 1]));
            const bf16x8 ub1 = as_bf16x8(pack_bf16x8(*tile(Ub, 2 * j, 1) * rka[2 * j], *tile(Ub, 2 * j + 1, 1) * rka[2 * j + 1]));
            const u16* kt = Kt + (32 * j + 4 * g4 + (l16 >> 2)) * krs + 4 * (l16 & 3);
#pragma unroll
            for (int s = 0; s < NDW; ++s) {
                const u16* kc = kt + 16 * (w + 8 * s);
                const bf16x4 c0 = lds_read_tr_b16x4(kc);
                const bf16x4 c1 = lds_read_tr_b16x4(kc + 16 * krs);
                const bf16x8 kta = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
                Wst[s][0] = mfma_bf16_k32(kta, ub0, Wst[s][0]);
                Wst[s][1] = mfma_bf16_k32(kta, ub1, Wst[s][1]);
            }
        }
        store_raw();
        lds_barrier();                                           // B4
        // y rows of the chunk: 8 bytes per thread; rows past the sequence end fall outside the
        // buffer's range and are dropped
        {
            const int t = tid >> 3, c4 = 4 * (tid & 7);
            const uint2 v2 = *reinterpret_cast<const uint2*>(Yb + t * 32 + c4);
            typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{v2.x, v2.y}, yrsrc,
                                                  ((t0 + t) * d_v + c4) * 2, 0, 0);
        }
    }

    if (a.Wf) {
#pragma unroll
        for (int s = 0; s < NDW; ++s)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                float* dst = a.Wf + (static_cast<int64_t>(bh) * d_v + col0 + 16 * ct + l16) * D +
                             orig_col(16 * (w + 8 * s) + 4 * g4, d_k);
                *reinterpret_cast<float2*>(dst) = make_float2(Wst[s][ct][0], Wst[s][ct][2]);
                *reinterpret_cast<float2*>(dst + d_k) = make_float2(Wst[s][ct][1], Wst[s][ct][3]);
            }
    }
}

// Pipelined serial pass for d_k = 64, nu <= 3 (D = 128 nu): the same chunk algebra as
// delta_stream_kernel, with the DPFP work taken off the serial critical path.
//   * Q is never stored: each wave builds its A operands of Q in registers from the raw q rows
//     (lane l16 of a row tile, positions j0 .. j0+3 of one shift block per 32-deep k-step) and
//     forms a partial Q W^T over half of the k-steps, for both column tiles; the two waves of a
//     row tile swap the halves they do not own through LDS.
//   * K is double-buffered: the K tile of chunk n + 1 is built in phase C of chunk n, where the
//     SIMDs otherwise wait on the short U products and the barrier, instead of in a phase of
//     its own.  (Built in phase B, between the X and Q W^T products, or in phase D beside the
//     memory update, it measured slower.)  Its 8 preceding positions per task come from the
//     neighbouring lane by DPP.  The prep results of chunk n + 1 are loaded as soon as chunk
//     n's are dead (after the memory update), a whole chunk ahead of their use.
//   * The W^T copy is written in the canonical B-operand layout (lane L, slot s = k-row
//     8 (L / 16) + s of the block, column L % 16), so the K operand of X = K W^T is one 16-byte
//     LDS read per k-step, and the register-built Q operand uses the same k order.
//   * U and rho_k o U are stored once, by the wave that forms the U tile, as the packed bf16 B
//     blocks that Y and the memory update read (one 16-byte read per block and k-step).
// Wave w owns row tile rt = w % 4 and column tile / Q half h = w / 4.  Per chunk:
//   B  X = K W^T for tile (rt, h) over all of D; partial Q W^T over k-steps 4 p + 2 h + e
//      (both column tiles); Z = V - rho_k o X to LDS (split into the bf16 hi and lo blocks
//      that the U product reads), the partner's partial to LDS.
//   C  U tile (rt, h) = A'' Z, stored as U and rho_k o U blocks; Q W^T tile (rt, h) = own +
//      partner partial, times rho_q; the next chunk's K tile (one DPFP task per thread) and
//      v columns.
//   D  Y tile (rt, h) = rho_q o Q W^T + P~ U; the memory tiles += K^T (rho_k o U); the W^T
//      copy.
// Three LDS-only barriers per chunk.  Global loads are issued by every lane in every chunk with
// clamped addresses (masked after arrival), so the compiler's in-order wait counts stay exact.
template <int NU>
__global__ __launch_bounds__(512, 1) void delta_stream_pipe_kernel(ChunkArgs a) {
    constexpr int C = 64, DK = 64, NDW = NU, NTB = 2;
    static_assert(NU >= 1 && NU <= 3, "window index 4 + f - i stays in 0 .. 7");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = l & 15, g4 = l >> 4;
    const int d_v = a.d_v, D = a.D, T = a.T, NC = a.NC;
    constexpr int krs = 2 * DK * NU + 16;       // K row stride (bf16), as the planner sets it
    const int NP = d_v / 32;
    const BhIndex bi = xcd_local(blockIdx.x, a.BH, NP);
    const int bh = bi.bh, col0 = 32 * static_cast<int>(bi.i);
    const int rt = w & 3, h = w >> 2;

    u16* const Kb0 = reinterpret_cast<u16*>(smem + a.s_k);
    u16* const Kb1 = reinterpret_cast<u16*>(smem + a.s_q);
    char* const WT = smem + a.s_wt;
    char* const Zc = smem + a.s_z;                                 // Z as bf16 hi, then lo at
                                                                   // + 4 KiB: B blocks as U's
    char* const Ub = smem + a.s_u;                                 // U, then rho_k o U at + 4 KiB:
                                                                   // bf16 B blocks of 32 rows
    float* const Xq = reinterpret_cast<float*>(smem + a.s_raw);    // Q W^T partials exchanged
    u16* const Yb = reinterpret_cast<u16*>(smem + a.s_y);          // [C][32] bf16
    u16* const Vr = reinterpret_cast<u16*>(smem + a.s_voff);       // [C][32] bf16
    auto tile = [&](float* base, int r, int c) { return reinterpret_cast<f32x4*>(base + ((r * 2 + c) * 64 + l) * 4); };
    // B block (row pair j, column tile c) of a bf16 U-type operand: lane l's 16 bytes hold its
    // four values of row tile 2 j, then its four of row tile 2 j + 1
    auto ublk = [&](int off, int j, int c) {
        return as_bf16x8(*reinterpret_cast<const uint4*>(Ub + off + ((j * 2 + c) * 64 + l) * 16));
    };
    auto put_ublk = [&](int off, const f32x4& x) {
        *reinterpret_cast<uint2*>(Ub + off + (((rt >> 1) * 2 + h) * 64 + l) * 16 + 8 * (rt & 1)) = pack_bf16x4(x);
    };
    // Z tile (rt, h), split once by the wave that forms it into the hi and lo blocks U = A'' Z reads
    auto put_zblk = [&](const f32x4& x) {
        char* const d = Zc + (((rt >> 1) * 2 + h) * 64 + l) * 16 + 8 * (rt & 1);
        *reinterpret_cast<uint2*>(d) = pack_bf16x4(x);
        *reinterpret_cast<uint2*>(d + 4096) = bf16_lo_part4(x);
    };
    auto zblk = [&](int off, int j) {
        return as_bf16x8(*reinterpret_cast<const uint4*>(Zc + off + ((j * 2 + h) * 64 + l) * 16));
    };

    // ---- memory tiles: d-tile w + 8 s, column tile c (rows d = 16 dt + 4 g4 + e, column l16)
    f32x4 Wst[NDW][2];
#pragma unroll
    for (int s = 0; s < NDW; ++s)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            Wst[s][c] = zero4();
            if (a.W0) {
                const float* src = a.W0 + (static_cast<int64_t>(bh) * d_v + col0 + 16 * c + l16) * D +
                                   orig_col(16 * (w + 8 * s) + 4 * g4, DK);
                const float2 lo = *reinterpret_cast<const float2*>(src);
                const float2 hi = *reinterpret_cast<const float2*>(src + DK);
                Wst[s][c] = f32x4{lo.x, hi.x, lo.y, hi.y};
            }
        }
    // the memory tiles as bf16 B blocks of W^T: block jb = dt / 2, lane 16 (2 (dt & 1) + g4 / 2)
    // + l16, slots 4 (g4 & 1) .. + 3
    auto write_wt = [&]() {
#pragma unroll
        for (int s = 0; s < NDW; ++s) {
            const int dt = w + 8 * s;
            const int lp = 16 * (2 * (dt & 1) + (g4 >> 1)) + l16;
#pragma unroll
            for (int c = 0; c < 2; ++c)
                *reinterpret_cast<uint2*>(WT + (((dt >> 1) * 2 + c) * 64 + lp) * 16 + 8 * (g4 & 1)) =
                    make_uint2(pack_bf16x2(Wst[s][c][0], Wst[s][c][1]), pack_bf16x2(Wst[s][c][2], Wst[s][c][3]));
        }
    };
    auto wblk = [&](int jb, int c) {
        return as_bf16x8(*reinterpret_cast<const uint4*>(WT + ((jb * 2 + c) * 64 + l) * 16));
    };

    // ---- raw inputs.  K task of this thread: row tid / 8, positions 8 (tid % 8) .. + 7 and the
    //      8 positions before them (cyclically: the previous lane's 8 of the same row, taken
    //      by DPP when the tile is built); the v columns as before; the Q windows of the
    //      wave's row tile: q[j0 - 4 .. j0 + 3] for j0 = 16 (2 h + e) + 4 g4, e = 0, 1
    const int64_t row0 = static_cast<int64_t>(bh) * T;
    const u16* kB = static_cast<const u16*>(a.k) + row0 * DK;
    const u16* qB = static_cast<const u16*>(a.q) + row0 * DK;
    const u16* vB = static_cast<const u16*>(a.v) + row0 * d_v + col0;
    const int ktr = tid >> 3, kjg = tid & 7;
    // k rows and v columns of this (b, h) as buffers whose range check returns zeros past the
    // sequence end (the planner keeps their byte sizes below 2^32)
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u16*>(kB), static_cast<short>(0), static_cast<int>(static_cast<uint32_t>(T) * DK * 2u),
        kBufferWord3);
    const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u16*>(vB), static_cast<short>(0),
        static_cast<int>((static_cast<uint32_t>(T) * d_v - col0) * 2u), kBufferWord3);
    uint4 ka, rv;
    auto load_k = [&](int n) {
        const uint32_t t0 = static_cast<uint32_t>(n) * C;
        const u32x4 k4 = __builtin_amdgcn_raw_buffer_load_b128(
            krsrc, static_cast<int>(((t0 + ktr) * DK + 8 * kjg) * 2u), 0, 0);
        ka = make_uint4(k4.x, k4.y, k4.z, k4.w);
        // threads past the chunk's v units read past the buffer (zeros, no memory traffic)
        const uint32_t vo = tid < 4 * C ? ((t0 + (tid >> 2)) * d_v + 8 * (tid & 3)) * 2u : 0xfffffff0u;
        const u32x4 v4 = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, static_cast<int>(vo), 0, 0);
        rv = make_uint4(v4.x, v4.y, v4.z, v4.w);
    };
    // q rows likewise (rows past the end read zeros; their y rows are dropped at the store)
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u16*>(qB), static_cast<short>(0), static_cast<int>(static_cast<uint32_t>(T) * DK * 2u),
        kBufferWord3);
    uint2 qlo[2], qhi[2];
    auto load_q = [&](int n) {
        const uint32_t r0 = (static_cast<uint32_t>(n) * C + 16 * rt + l16) * DK;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint32_t j0 = 16 * (2 * h + e) + 4 * g4;
            const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(
                qrsrc, static_cast<int>((r0 + ((j0 + DK - 4) & (DK - 1))) * 2u), 0, 0);
            const u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(qrsrc, static_cast<int>((r0 + j0) * 2u), 0, 0);
            qlo[e] = make_uint2(lo.x, lo.y);
            qhi[e] = make_uint2(hi.x, hi.y);
        }
    };
    // the next chunk's K tile: one DPFP task per thread (rows past the end zero: their k loads
    // return zeros)
    auto build_k = [&](u16* Kn) {
        const uint32_t ak[4] = {ka.x, ka.y, ka.z, ka.w};
        // a row's eight tasks sit in eight aligned lanes: lane kjg - 1 (kjg >= 1, DPP row_shr:1)
        // or kjg + 7 (kjg == 0, row_shl:7) holds the positions before this task's
        const uint32_t a4[4] = {ka.x, ka.y, ka.z, ka.w};
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t prev = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(a4[e]), 0x111, 0xF, 0xF, false));
            const uint32_t wrap = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(a4[e]), 0x107, 0xF, 0xF, false));
            // the positions before 0 wrap into the [-k] half: their signs flip here
            pk[e] = kjg == 0 ? wrap ^ 0x80008000u : prev;
        }
        float a8[8], p8[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a8[2 * e] = __uint_as_float(ak[e] << 16);
            a8[2 * e + 1] = __uint_as_float(ak[e] & 0xffff0000u);
            p8[2 * e] = __uint_as_float(pk[e] << 16);
            p8[2 * e + 1] = __uint_as_float(pk[e] & 0xffff0000u);
        }
        dpfp_task_w<u16, NU>(a8, p8, 8 * kjg, DK, Kn + ktr * krs, false);
    };
    auto store_v = [&]() {
        if (tid < 4 * C)
            reinterpret_cast<uint4*>(Vr)[tid] = rv;
    };

    // ---- per-chunk results of the prep kernel (as in delta_stream_kernel)
    uint4 ah[NTB], al[NTB], pa[NTB];
    f32x4 rkc, rqv;
    // (the A'' and P~ blocks are stored on and below the diagonal only, in tri_blk order; the
    // loads of a block above it re-read the row tile's last block and go unused)
    // the prep results of this (b, h) as buffers: each lane's offsets are fixed, the chunk's
    // offset is uniform (no range check: every chunk index is below NC)
    const int64_t ub0 = static_cast<int64_t>(bh) * NC;
    constexpr uint32_t szT = tri_nblocks(C) * 1024;
    auto ws_rsrc = [&](int64_t off) {
        return __builtin_amdgcn_make_buffer_rsrc(a.ws + off, static_cast<short>(0), -1, kBufferWord3);
    };
    const __amdgpu_buffer_rsrc_t ahr = ws_rsrc(a.o_ah + ub0 * szT), alr = ws_rsrc(a.o_al + ub0 * szT),
                                 par = ws_rsrc(a.o_pa + ub0 * szT);
    const __amdgpu_buffer_rsrc_t rkr = ws_rsrc(a.o_rk + ub0 * C * 4), rqr = ws_rsrc(a.o_rq + ub0 * C * 4);
    int blo[NTB];
#pragma unroll
    for (int j = 0; j < NTB; ++j) blo[j] = (tri_blk(rt, min(j, rt >> 1)) * 64 + l) * 16;
    const int rlo = (16 * rt + 4 * g4) * 4;
    auto load_ws = [&](int n) {
        const int so = static_cast<int>(static_cast<uint32_t>(n) * szT);
        const int sr = static_cast<int>(static_cast<uint32_t>(n) * C * 4u);
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(ahr, blo[j], so, 0);
            const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(alr, blo[j], so, 0);
            const u32x4 z = __builtin_amdgcn_raw_buffer_load_b128(par, blo[j], so, 0);
            ah[j] = make_uint4(x.x, x.y, x.z, x.w);
            al[j] = make_uint4(y.x, y.y, y.z, y.w);
            pa[j] = make_uint4(z.x, z.y, z.z, z.w);
        }
        rkc = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rkr, rlo, sr, 0));
        rqv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rqr, rlo, sr, 0));
    };

    if (NC > 0) {
        load_k(0);
        load_q(0);
        load_ws(0);
        write_wt();
        build_k(Kb0);
        store_v();
        load_k(NC > 1 ? 1 : 0);
    }
    lds_barrier();

    const __amdgpu_buffer_rsrc_t yrsrc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<u16*>(a.y) + row0 * d_v + col0, static_cast<short>(0),
        static_cast<int>((static_cast<uint32_t>(T) * d_v - col0) * 2u), kBufferWord3);
    // One chunk; ODD (chunk parity) picks the K buffers, so that the loop below, two chunks per
    // iteration, addresses them with fixed offsets.
    auto chunk = [&](int n, auto odd_tag) {
        constexpr bool ODD = decltype(odd_tag)::value;
        const int t0 = n * C;
        const int nn = n + 1 < NC ? n + 1 : n;
        const int n2 = n + 2 < NC ? n + 2 : NC - 1;
        const u16* Kc = ODD ? Kb1 : Kb0;
        u16* Kn = ODD ? Kb0 : Kb1;

        // ---- B: X tile (rt, h), partial Q W^T (rt, both), Z
        f32x4 xa = zero4(), xb = zero4(), qo = zero4(), qx = zero4();
        {
            // window values as fp32 positive / negative parts; for the lane whose window starts
            // at position 0 the four values before it wrap into the [-k] half: their signs are
            // flipped before unpacking, which swaps their parts
            float Pw[2][8], Nw[2][8];
            const uint32_t sg = (h == 0 && g4 == 0) ? 0x80008000u : 0u;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t se = e == 0 ? sg : 0u;
                const uint32_t wd[4] = {qlo[e].x ^ se, qlo[e].y ^ se, qhi[e].x, qhi[e].y};
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const float r = (m & 1) ? __uint_as_float(wd[m >> 1] & 0xffff0000u)
                                            : __uint_as_float(wd[m >> 1] << 16);
                    Pw[e][m] = relu_f(r);
                    Nw[e][m] = Pw[e][m] - r;
                }
            }
            const u16* kr = Kc + (16 * rt + l16) * krs + 8 * g4;
#pragma unroll
            for (int p = 0; p < NU; ++p)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int jo = 4 * p + 2 * h + e, jx = 4 * p + 2 - 2 * h + e;
                    const bf16x8 k_o = as_bf16x8(*reinterpret_cast<const uint4*>(kr + 32 * jo));
                    const bf16x8 k_x = as_bf16x8(*reinterpret_cast<const uint4*>(kr + 32 * jx));
                    const bf16x8 w_oh = wblk(jo, h), w_xh = wblk(jx, h), w_oo = wblk(jo, 1 - h);
                    // A operand of Q for k-step jo: slot 2 f + s = position j0 + f of shift p + 1,
                    // half s (s = 0: relu(q_j) times the rolled factor, s = 1: relu(-q_j) times it)
                    bf16x8 qa;
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        const int m = 4 + f - (p + 1);
                        qa[2 * f] = static_cast<__bf16>(Pw[e][4 + f] * Pw[e][m]);
                        qa[2 * f + 1] = static_cast<__bf16>(Nw[e][4 + f] * Nw[e][m]);
                    }
                    xa = mfma_bf16_k32(k_o, w_oh, xa);
                    xb = mfma_bf16_k32(k_x, w_xh, xb);
                    qo = mfma_bf16_k32(qa, w_oh, qo);
                    qx = mfma_bf16_k32(qa, w_oo, qx);
                }
        }
        load_q(nn);
        xa += xb;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            xa[e] = bf16_bits_to_f32(Vr[(16 * rt + 4 * g4 + e) * 32 + 16 * h + l16]) - rkc[e] * xa[e];
        put_zblk(xa);
        *tile(Xq, rt, 1 - h) = qx;
        lds_barrier();                                           // B2

        // ---- C: U tile (rt, h) = A'' Z; the full Q W^T tile
        f32x4 qacc;
        {
            f32x4 u = zero4();
#pragma unroll
            for (int j = 0; j < NTB; ++j) {
                if (2 * j > rt) break;                            // A'' is zero above the diagonal
                const bf16x8 zh = zblk(0, j), zl = zblk(4096, j);
                u = mfma_bf16_k32(as_bf16x8(ah[j]), zh, u);
                u = mfma_bf16_k32(as_bf16x8(ah[j]), zl, u);
                u = mfma_bf16_k32(as_bf16x8(al[j]), zh, u);
            }
            // U for Y and rho_k o U for the memory update, stored once as the bf16 operands
            // both take (so no wave needs the other row tiles' rho_k)
            put_ublk(0, u);
            put_ublk(4096, u * rkc);
            qacc = (qo + *tile(Xq, rt, h)) * rqv;
        }
        // the next chunk's K tile and v columns (buffers last read in the previous chunk and in
        // phase B), then the loads of the chunk after it
        build_k(Kn);
        store_v();
        load_k(n2);
        lds_barrier();                                           // B3

        // ---- D: Y tile (rt, h), memory update, W^T copy
        {
            f32x4 y = qacc;
#pragma unroll
            for (int j = 0; j < NTB; ++j) {
                if (2 * j > rt) break;
                y = mfma_bf16_k32(as_bf16x8(pa[j]), ublk(0, j, h), y);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Yb[(16 * rt + 4 * g4 + e) * 32 + 16 * h + l16] = f32_to_bf16_bits(y[e]);
        }
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
            const bf16x8 ub0 = ublk(4096, j, 0), ub1 = ublk(4096, j, 1);
            const u16* kt = Kc + (32 * j + 4 * g4 + (l16 >> 2)) * krs + 4 * (l16 & 3);
#pragma unroll
            for (int s = 0; s < NDW; ++s) {
                const u16* kc = kt + 16 * (w + 8 * s);
                const bf16x4 c0 = lds_read_tr_b16x4(kc);
                const bf16x4 c1 = lds_read_tr_b16x4(kc + 16 * krs);
                const bf16x8 kta = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
                Wst[s][0] = mfma_bf16_k32(kta, ub0, Wst[s][0]);
                Wst[s][1] = mfma_bf16_k32(kta, ub1, Wst[s][1]);
            }
        }
        load_ws(nn);            // this chunk's prep results are dead from here on
        write_wt();
        lds_barrier();                                           // B4
        {
            const int t = tid >> 3, c4 = 4 * (tid & 7);
            const uint2 v2 = *reinterpret_cast<const uint2*>(Yb + t * 32 + c4);
            typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2{v2.x, v2.y}, yrsrc, static_cast<int>((static_cast<uint32_t>(t0 + t) * d_v + c4) * 2u), 0, 0);
        }
    };
    int n = 0;
    for (; n + 1 < NC; n += 2) {
        chunk(n, std::false_type());
        chunk(n + 1, std::true_type());
    }
    if (n < NC) chunk(n, std::false_type());

    if (a.Wf) {
#pragma unroll
        for (int s = 0; s < NDW; ++s)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float* dst = a.Wf + (static_cast<int64_t>(bh) * d_v + col0 + 16 * c + l16) * D +
                             orig_col(16 * (w + 8 * s) + 4 * g4, DK);
                *reinterpret_cast<float2*>(dst) = make_float2(Wst[s][c][0], Wst[s][c][2]);
                *reinterpret_cast<float2*>(dst + DK) = make_float2(Wst[s][c][1], Wst[s][c][3]);
            }
    }
}

hipError_t launch_stream_c64(const StreamPlan& p, hipStream_t s);

}  // namespace fwa
