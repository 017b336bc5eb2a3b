// Streaming forward, producer / consumer form (bf16, d_k = 64, chunk 64, 32 columns of d_v per
// workgroup): the serial pass over the chunks with the DPFP work of one step overlapped with the
// MFMA work of the previous one.
//
// Same algebra as the other serial kernels (the chunked form of the recurrence of the "Fast
// Weights Transformer" guide, xdnf.cn/news/308600, sections "FastWeightsAttention / update
// formula" and "... / module structure and source walkthrough"): per chunk of C rows from memory
// W, X = K W^T, U = A'' (V - rho_k o X), Y = rho_q o (Q W^T) + P~ U, W^T += K^T (rho_k o U), with
// A'', P~ and the normalisers from the prep kernel.
//
// Eight waves: waves 0-3 produce, waves 4-7 consume.  The DPFP features are built one shift
// block of 128 columns ("slice") at a time, as in the other sliced kernels: per chunk the items
// B_0 .. B_{nu-1} (K and Q slices, for X and Q W^T) then D_0 .. D_{nu-1} (K slices again, for the
// update, which needs U and so all of X first), alternating between two LDS slots.  Time runs in
// steps that end in one workgroup barrier; in each step the producers build one item while the
// consumers run the products on the item built in the step before.  A chunk takes 2 nu + 1 steps:
//   producer step t:  t < nu: build B_t;  t = nu: move the next chunk's raw rows (loaded into
//                     registers at t = 0) into the other raw slot;  t > nu: build D_{t-nu-1}.
//   consumer step tau = t + 1 (one step behind):  tau <= nu: X, Q W^T += B_{tau-1} (and at
//                     tau = nu, Z = V - rho_k o X to LDS);  tau = nu + 1: U = A'' Z;
//                     tau = nu + 2: Y to LDS and the update with D_0;  tau > nu + 2: the update
//                     with D_{tau-nu-2}; at tau = 2 nu + 1 the refreshed bf16 W^T copy.
// Item i of a chunk is built in step p(i) and read in step p(i) + 1; the item after next in the
// same slot is built no earlier than p(i) + 2, so one barrier per step orders every slot reuse
// (the D items are built one step after the B items end for exactly this).
// The consumer waves own row tile c = w - 4 of X, Q W^T, U and Y (both 16-column tiles) and
// d-tiles c and c + 4 of every slice of the fp32 memory W^T, in MFMA accumulators.
#pragma once

#include "stream_sliced.h"

namespace fwa {

template <int NU>
__global__ __launch_bounds__(512, 1) void delta_stream_pc_kernel(ChunkArgs a) {
    constexpr int C = 64, NT = C / 16, NTB = NT / 2, NCT = 2, CW = 32, NR = 2;
    constexpr int PTH = 256;                                   // producer threads
    constexpr int SPC = 2 * NU + 1;                            // steps per chunk
    constexpr int RAWB = 2 * C * kSliceDk * 2 + C * CW * 2;    // one raw slot: k, q rows, v columns
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = w < 4;
    const int c = w & 3;                                       // consumer row tile / producer index
    const int ptid = tid & (PTH - 1);
    const int l16 = l & 15, g4 = l >> 4;
    const int d_v = a.d_v, D = a.D, T = a.T, NC = a.NC, ss = a.ss;
    const BhIndex bi = xcd_local(blockIdx.x, a.BH, d_v / CW);
    const int bh = bi.bh, cp = static_cast<int>(bi.i);
    const int col0 = CW * cp;
    const int slb = C * ss * 2;                                // bytes of one K (or Q) slice

    char* WT = smem + a.s_wt;
    float* Zb = reinterpret_cast<float*>(smem + a.s_z);
    float* Ub = reinterpret_cast<float*>(smem + a.s_u);
    u16* Yb = reinterpret_cast<u16*>(smem + a.s_y);           // [C][CW] bf16
    auto raw = [&](int slot) { return smem + a.s_raw + slot * RAWB; };
    auto kslice = [&](int slot) { return reinterpret_cast<u16*>(smem + a.s_k + slot * 2 * slb); };
    auto qslice = [&](int slot) { return reinterpret_cast<u16*>(smem + a.s_k + slot * 2 * slb + slb); };
    auto tile = [&](float* base, int r, int ct) { return reinterpret_cast<f32x4*>(base + ((r * NCT + ct) * 64 + l) * 4); };
    auto wblk = [&](int jb, int ct) { return WT + ((jb * NCT + ct) * 64 + l) * 16; };
    const int64_t row0 = static_cast<int64_t>(bh) * T;

    // ---- producer state: the next chunk's raw rows in registers (two 16-byte k and q units and
    //      one v unit per producer thread); a unit past the sequence end reads unit 0 of the chunk
    //      and is zeroed by its mask
    const uint4* kB = reinterpret_cast<const uint4*>(static_cast<const u16*>(a.k) + row0 * kSliceDk);
    const uint4* qB = reinterpret_cast<const uint4*>(static_cast<const u16*>(a.q) + row0 * kSliceDk);
    const u16* vB = static_cast<const u16*>(a.v) + row0 * d_v + col0;
    uint4 rk[2], rq[2], rv;
    uint32_t mk[2], mv = 0u;
    auto load_raw = [&](int n) {
        const int t0 = n * C, Cn = min(C, T - t0);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int e = ptid + PTH * p;
            const bool ok = (e >> 3) < Cn;
            const int64_t o = static_cast<int64_t>(t0) * 8 + (ok ? e : 0);
            rk[p] = kB[o];
            rq[p] = qB[o];
            mk[p] = ok ? 0xffffffffu : 0u;
        }
        const bool okv = (ptid >> 2) < Cn;
        rv = *reinterpret_cast<const uint4*>(vB + static_cast<int64_t>(t0 + (okv ? ptid >> 2 : 0)) * d_v +
                                             (okv ? 8 * (ptid & 3) : 0));
        mv = okv ? 0xffffffffu : 0u;
    };
    auto store_raw = [&](int slot) {
        char* sb = raw(slot);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int e = ptid + PTH * p;
            const uint32_t m = mk[p];
            reinterpret_cast<uint4*>(sb)[e] = make_uint4(rk[p].x & m, rk[p].y & m, rk[p].z & m, rk[p].w & m);
            reinterpret_cast<uint4*>(sb + C * kSliceDk * 2)[e] =
                make_uint4(rq[p].x & m, rq[p].y & m, rq[p].z & m, rq[p].w & m);
        }
        reinterpret_cast<uint4*>(sb + 2 * C * kSliceDk * 2)[ptid] = make_uint4(rv.x & mv, rv.y & mv, rv.z & mv, rv.w & mv);
    };

    // ---- consumer state
    f32x4 Wst[NU][NR][NCT];
    f32x4 xacc[NCT], qacc[NCT];
    uint4 ah[NTB], al[NTB], pa[NTB];
    f32x4 rka[NT], rqv;
    bf16x8 ubk[NTB][NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) xacc[ct] = qacc[ct] = zero4();
    auto load_ws = [&](int n) {
        const int64_t u = static_cast<int64_t>(bh) * NC + n;
        const char* ahp = a.ws + a.o_ah + u * (C * C * 2);
        const char* alp = a.ws + a.o_al + u * (C * C * 2);
        const char* pap = a.ws + a.o_pa + u * (C * C * 2);
#pragma unroll
        for (int j = 0; j < NTB; ++j) {
            ah[j] = *reinterpret_cast<const uint4*>(blk_ptr(ahp, c * NTB + j, l));
            al[j] = *reinterpret_cast<const uint4*>(blk_ptr(alp, c * NTB + j, l));
            pa[j] = *reinterpret_cast<const uint4*>(blk_ptr(pap, c * NTB + j, l));
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
            rka[tt] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.ws + a.o_rk) + u * C + 16 * tt + 4 * g4);
        rqv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.ws + a.o_rq) + u * C + 16 * c + 4 * g4);
    };
    auto write_wt = [&]() {
#pragma unroll
        for (int s = 0; s < NU; ++s)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int dt = 8 * s + c + 4 * r;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    *reinterpret_cast<uint2*>(wblk(dt >> 1, ct) + 8 * (dt & 1)) =
                        make_uint2(pack_bf16x2(Wst[s][r][ct][0], Wst[s][r][ct][1]),
                                   pack_bf16x2(Wst[s][r][ct][2], Wst[s][r][ct][3]));
            }
    };
    // y rows of chunk n from Yb: 16 bytes per consumer thread; the buffer's range ends where row
    // T would begin, so rows past the sequence end are dropped
    const __amdgpu_buffer_rsrc_t yrsrc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<u16*>(a.y) + row0 * d_v + col0, static_cast<short>(0), (T * d_v - col0) * 2,
        kBufferWord3);
    auto store_y = [&](int n) {
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        const int t = ptid >> 2, c8 = 8 * (ptid & 3);
        const uint4 v4 = *reinterpret_cast<const uint4*>(Yb + t * CW + c8);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{v4.x, v4.y, v4.z, v4.w}, yrsrc,
                                               ((n * C + t) * d_v + c8) * 2, 0, 0);
    };

    // The two roles run separate loops with the same barrier sequence (one after the prologue,
    // one per step), so each loop's registers hold only its own role's state.
    float unused_q[4], unused_k[2];   // DPFP task sums: dead here (rho comes from the prep)
    const int nsteps = SPC * NC + (NC > 0 ? 1 : 0);
    if (producer) {
        if (NC > 0) {
            load_raw(0);
            store_raw(0);
        }
        lds_barrier();
        for (int g = 0; g < nsteps; ++g) {
            const int n = g / SPC, t = g - (g / SPC) * SPC;
            if (n < NC) {
                const u16* Xk = reinterpret_cast<const u16*>(raw(n & 1));
                const u16* Xq = Xk + C * kSliceDk;
                if (t == 0) load_raw(n + 1 < NC ? n + 1 : n);
                if (t < NU) {
                    dpfp_slice_any<C, PTH, true>(t + 1, Xk, Xq, kslice(t & 1), qslice(t & 1), ss, ptid, unused_q);
                } else if (t == NU) {
                    store_raw((n + 1) & 1);        // the last chunk rewrites its own rows' twin slot
                } else {
                    const int j = t - NU - 1;
                    dpfp_slice_any<C, PTH, false>(j + 1, Xk, nullptr, kslice((NU + j) & 1), nullptr, ss, ptid, unused_k);
                }
            }
            lds_barrier();
        }
        return;
    }

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
                                       orig_col(16 * (8 * s + c + 4 * r) + 4 * g4, kSliceDk);
                    const float2 lo = *reinterpret_cast<const float2*>(src);
                    const float2 hi = *reinterpret_cast<const float2*>(src + kSliceDk);
                    Wst[s][r][ct] = f32x4{lo.x, hi.x, lo.y, hi.y};
                }
            }
    write_wt();
    lds_barrier();
    for (int g = 1; g < nsteps; ++g) {
        lds_barrier();   // end of step g - 1 (the producers' first item)
        const int n = (g - 1) / SPC, tau = g - (g - 1) / SPC * SPC;   // 1 .. SPC
        if (tau == 1) {
            load_ws(n);
            if (n >= 1) store_y(n - 1);
        }
        if (tau <= NU) {
            // X and Q W^T over slice tau - 1 (k-steps of 32 columns)
            const int s = tau - 1, slot = s & 1;
            const u16* kr = kslice(slot) + (16 * c + l16) * ss + 4 * g4;
            const u16* qr = qslice(slot) + (16 * c + l16) * ss + 4 * g4;
#pragma unroll
            for (int kk = 0; kk < kSliceCols / 32; ++kk) {
                const bf16x4 k0 = *reinterpret_cast<const bf16x4*>(kr + 32 * kk);
                const bf16x4 k1 = *reinterpret_cast<const bf16x4*>(kr + 32 * kk + 16);
                const bf16x4 q0 = *reinterpret_cast<const bf16x4*>(qr + 32 * kk);
                const bf16x4 q1 = *reinterpret_cast<const bf16x4*>(qr + 32 * kk + 16);
                const bf16x8 ak = __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7);
                const bf16x8 aq = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
                const int jb = (kSliceCols / 32) * s + kk;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const bf16x8 wb = as_bf16x8(*reinterpret_cast<const uint4*>(wblk(jb, ct)));
                    xacc[ct] = mfma_bf16_k32(ak, wb, xacc[ct]);
                    qacc[ct] = mfma_bf16_k32(aq, wb, qacc[ct]);
                }
            }
            if (tau == NU) {
                // Z = V - rho_k o X (rows 16 c + 4 g4 + e, columns 16 ct + l16)
                const u16* Xv = reinterpret_cast<const u16*>(raw(n & 1) + 2 * C * kSliceDk * 2);
                const f32x4 rkc = rka[c];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    f32x4 z;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        z[e] = bf16_bits_to_f32(Xv[(16 * c + 4 * g4 + e) * CW + 16 * ct + l16]) - rkc[e] * xacc[ct][e];
                    *tile(Zb, c, ct) = z;
                    qacc[ct] *= rqv;
                    xacc[ct] = zero4();
                }
            }
        } else if (tau == NU + 1) {
            // U tiles (c, ct) = A'' Z
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 uacc = zero4();
#pragma unroll
                for (int j = 0; j < NTB; ++j) {
                    if (2 * j > c) break;                          // A'' is zero above the diagonal
                    const f32x4 z0 = *tile(Zb, 2 * j, ct), z1 = *tile(Zb, 2 * j + 1, ct);
                    const bf16x8 zh = as_bf16x8(pack_bf16x8(z0, z1));
                    const bf16x8 zl = as_bf16x8(bf16_lo_part(z0, z1));
                    uacc = mfma_bf16_k32(as_bf16x8(ah[j]), zh, uacc);
                    uacc = mfma_bf16_k32(as_bf16x8(ah[j]), zl, uacc);
                    uacc = mfma_bf16_k32(as_bf16x8(al[j]), zh, uacc);
                }
                *tile(Ub, c, ct) = uacc;
            }
        } else {
            const int j = tau - NU - 2;                                // D_j, 0 .. NU-1
            if (j == 0) {
                // Y tiles (c, ct) = rho_q o (Q W^T) + P~ U, and the update's B operands
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    f32x4 y = qacc[ct];
#pragma unroll
                    for (int jj = 0; jj < NTB; ++jj) {
                        if (2 * jj > c) break;
                        const bf16x8 ub = as_bf16x8(pack_bf16x8(*tile(Ub, 2 * jj, ct), *tile(Ub, 2 * jj + 1, ct)));
                        y = mfma_bf16_k32(as_bf16x8(pa[jj]), ub, y);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) Yb[(16 * c + 4 * g4 + e) * CW + 16 * ct + l16] = f32_to_bf16_bits(y[e]);
                    qacc[ct] = zero4();
                }
#pragma unroll
                for (int jj = 0; jj < NTB; ++jj)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        ubk[jj][ct] = as_bf16x8(pack_bf16x8(*tile(Ub, 2 * jj, ct) * rka[2 * jj],
                                                            *tile(Ub, 2 * jj + 1, ct) * rka[2 * jj + 1]));
            }
            // W_j^T += K_j^T (rho_k o U) for this wave's d-tiles c, c + 4 of slice j
            const u16* ks = kslice((NU + j) & 1);
#pragma unroll
            for (int s = 0; s < NU; ++s) {
                if (s != j) continue;                              // static register indices
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const u16* kt = ks + (4 * g4 + (l16 >> 2)) * ss + 16 * (c + 4 * r) + 4 * (l16 & 3);
#pragma unroll
                    for (int jj = 0; jj < NTB; ++jj) {
                        const u16* kc = kt + 32 * jj * ss;
                        const bf16x4 c0 = lds_read_tr_b16x4(kc);
                        const bf16x4 c1 = lds_read_tr_b16x4(kc + 16 * ss);
                        const bf16x8 kta = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) Wst[s][r][ct] = mfma_bf16_k32(kta, ubk[jj][ct], Wst[s][r][ct]);
                    }
                }
            }
            if (j == NU - 1) write_wt();                           // the next chunk's W^T copy
        }
    }
    if (nsteps > 0) {
        lds_barrier();   // end of the last step (the producers' barrier count: 1 + nsteps)
        store_y(NC - 1);
    }

    if (a.Wf) {
#pragma unroll
        for (int s = 0; s < NU; ++s)
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    float* dst = a.Wf + (static_cast<int64_t>(bh) * d_v + col0 + 16 * ct + l16) * D +
                                 orig_col(16 * (8 * s + c + 4 * r) + 4 * g4, kSliceDk);
                    *reinterpret_cast<float2*>(dst) = make_float2(Wst[s][r][ct][0], Wst[s][r][ct][2]);
                    *reinterpret_cast<float2*>(dst + kSliceDk) = make_float2(Wst[s][r][ct][1], Wst[s][r][ct][3]);
                }
    }
}

}  // namespace fwa
