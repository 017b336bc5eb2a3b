// Sum-update linear attention with the z normaliser ("Fast Weights Transformer" guide,
// xdnf.cn/news/308600, section "Background / fast computation form of linear self-attention"):
//   W_t = W_{t-1} + v_t phi(k_t)^T,  z_t = z_{t-1} + phi(k_t),  y_t = W_t phi(q_t) / (z_t . phi(q_t))
// with phi = DPFP, and y_t = 0 where the denominator is exactly 0.
//
// For a chunk of C rows with normalised features K, Q (C x D) starting from W0, z0, and
// M = lower_incl(Q K^T):
//   Y = (Q W0^T + M V) / (Q z0 + M 1)   (row-wise),   W1 = W0 + V^T K,   z1 = z0 + K^T 1.
// Launches:
//   1. sum_prep  per chunk: K, Q, and the chunk-local parts M V and M 1            (parallel)
//   2. sum_scan  per (b, h, 16 rows of W), chunks in order: W^T in fp32 MFMA accumulators
//      split over the 4 waves by d-tiles; Q W^T, Q z, y, then W^T += K^T V, z += K^T 1 (serial)
//   3. sum_zfinal per (b, h): z_final from z0 and the chunks' key sums (where it is asked for)
// The memory's recurrence is a plain sum, so where fewer than 256 serial workgroups would cover
// the sequences, each sequence is cut into NB blocks of LC chunks: a launch before the scan
// forms the sums of K^T V and of the key sums over SP parts of every block but the last in
// parallel (sum_blocksum), and block b's scan starts from W0 + the parts of blocks 0 .. b - 1
// (W0 itself copied into the workspace by that launch, since W_final may be W0).
// Arithmetic is fp32 (the vector ALU and the fp32 MFMA); chunks of 32 rows.
#include "chunk_f32.h"
#include "fwa_internal.h"

namespace fwa {

constexpr int kSumThreads = 256;

struct SumLayout {
    int64_t kt, qt, nm, dn, ks;   // K, Q [C][D]; M V [C][d_v]; M 1 [C]; K^T 1 [D] (per chunk)
    int64_t wc, bs, zb;           // with NB > 1: W0 copy [BH][d_v][D]; sums of K^T V over the
    int64_t end;                  // block parts [NB-1][SP][BH][d_v][D] and of K^T 1 [..][BH][D]
};

// Blocks per sequence: enough (b, h, 16-column) scan workgroups to cover the 256 CUs, at most
// one per chunk.  *LC = chunks per block; the count returned is the number of non-empty blocks.
static int sum_blocks(int BH, int NC, int d_v, int* LC) {
    const int64_t wgs = int64_t(BH) * ((d_v + 15) / 16);
    int nb = 1;
    if (NC > 1 && wgs < 256) nb = static_cast<int>(256 / wgs < NC ? 256 / wgs : NC);
    *LC = NC > 0 ? (NC + nb - 1) / nb : 1;
    return NC > 0 ? (NC + *LC - 1) / *LC : 1;
}
// Parts per block for the block sums: about 2048 sum workgroups (eight per CU, so that their
// load latency hides behind each other's products), each over at least four chunks (a scan
// workgroup adds up the parts of every block before its own).
static int sum_parts(int BH, int NB, int LC, int d_v) {
    if (NB <= 1) return 1;
    const int64_t wgs = int64_t(BH) * (NB - 1) * ((d_v + 15) / 16);
    int64_t sp = 2048 / wgs;
    if (sp > LC / 4) sp = LC / 4;
    return static_cast<int>(sp < 1 ? 1 : sp);
}

static SumLayout sum_layout(int64_t BH, int NC, int D, int d_v, int NB, int SP) {
    const int64_t NU = BH * NC;
    SumLayout L;
    int64_t o = 0;
    L.kt = o; o += NU * kBC * D;
    L.qt = o; o += NU * kBC * D;
    L.nm = o; o += NU * kBC * d_v;
    L.dn = o; o += NU * kBC;
    L.ks = o; o += NU * D;
    L.wc = o; o += NB > 1 ? BH * d_v * D : 0;
    L.bs = o; o += NB > 1 ? int64_t(NB - 1) * SP * BH * d_v * D : 0;
    L.zb = o; o += NB > 1 ? int64_t(NB - 1) * SP * BH * D : 0;
    L.end = o;
    return L;
}

struct SumArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* W0;
    const float* z0;
    void* y;
    float* Wf;
    float* zf;
    float* ws;
    int BH, T, NC, d_k, d_v, nu, D;
    int NB, LC, SP;               // blocks per sequence, chunks per block (NB = 1: one scan),
                                  // parts per block for the block sums
    SumLayout L;
};

// LDS: x rows of k and q (C x 2 d_k each), one shift slice of K and of Q (C x (2 d_k + 4)),
// M (C x (C + 4)), V: 78 KB at d_k = 64 and d_v = 64, so two workgroups share a CU.
// The row sums of the raw features come first (a pass of products without stores); then, one
// shift i at a time, the slice's normalised features (columns (i - 1) 2 d_k .. + 2 d_k - 1)
// go to LDS, to the workspace (16-byte stores) and into M = lower_incl(Q K^T) (fp32 MFMA
// accumulators of waves 0-2) and the key sums (wave 3).
template <bool BF16>
__global__ __launch_bounds__(kSumThreads, 2) void sum_prep_kernel(SumArgs a) {
    extern __shared__ float lds[];
    const int D = a.D, d_k = a.d_k, d_v = a.d_v, two = 2 * d_k;
    const int u = blockIdx.x;
    const int bh = u / a.NC, n = u % a.NC;
    const int t0 = n * kBC;
    const int tid = threadIdx.x;
    const int rows = a.T - t0 < kBC ? a.T - t0 : kBC;
    const int wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    constexpr int CS = kBC + 4;       // 16-byte rows for the MFMA operand reads
    const int SS = two + 4;           // slice row stride
    float* xk = lds;
    float* xq = xk + kBC * two;
    float* Ks = xq + kBC * two;
    float* Qs = Ks + kBC * SS;
    float* Mm = Qs + kBC * SS;
    float* Vs = Mm + kBC * CS;
    load_chunk_inputs<BF16, kSumThreads, 128>(a.k, a.q, a.v, xk, xq, Vs, int64_t(bh) * a.T, rows,
                                              t0, d_k, d_v, tid);
    __syncthreads();
    // row sums: row c = tid / 8, entries p = tid % 8 + 8 m of every shift (the eight threads of
    // a row are adjacent lanes)
    const int c = tid >> 3, s0 = tid & 7;
    const float* xrk = xk + c * two;
    const float* xrq = xq + c * two;
    float sk = 0.0f, sq = 0.0f;
    for (int i = 1; i <= a.nu; ++i)
        for (int jj = s0; jj < two; jj += 8) {
            int src = jj - i;
            src += (src < 0) ? two : 0;
            sk += xrk[jj] * xrk[src];
            sq += xrq[jj] * xrq[src];
        }
    sk = sum8_dpp(sk);
    sq = sum8_dpp(sq);
    const float ik = 1.0f / (sk + kDpfpEps), iq = 1.0f / (sq + kDpfpEps);
    const int64_t CD = int64_t(kBC) * D;
    float* gK = a.ws + a.L.kt + int64_t(u) * CD;
    float* gQ = a.ws + a.L.qt + int64_t(u) * CD;
    float* gks = a.ws + a.L.ks + int64_t(u) * D;
    // waves 0-2: tiles (0,0), (1,0), (1,1) of M
    const int it = wv == 0 ? 0 : 1, jt = wv == 2 ? 1 : 0;
    f32x4 acc = zero4();
    for (int i = 1; i <= a.nu; ++i) {
        for (int jj = s0; jj < two; jj += 8) {
            int src = jj - i;
            src += (src < 0) ? two : 0;
            Ks[c * SS + jj] = xrk[jj] * xrk[src] * ik;
            Qs[c * SS + jj] = xrq[jj] * xrq[src] * iq;
        }
        __syncthreads();
        // the slice to the workspace: 16-byte units e = (row, 4 columns)
        const int col0 = (i - 1) * two, q4 = two / 4;
        for (int e = tid; e < kBC * q4; e += kSumThreads) {
            const int r = e / q4, cc = 4 * (e - r * q4);
            *reinterpret_cast<f32x4*>(gK + r * D + col0 + cc) = *reinterpret_cast<const f32x4*>(Ks + r * SS + cc);
            *reinterpret_cast<f32x4*>(gQ + r * D + col0 + cc) = *reinterpret_cast<const f32x4*>(Qs + r * SS + cc);
        }
        if (wv < 3) {
            for (int kb = 0; kb < two; kb += 16) {
                const f32x4 av = *reinterpret_cast<const f32x4*>(Qs + (16 * it + l16) * SS + kb + 4 * g4);
                const f32x4 bv = *reinterpret_cast<const f32x4*>(Ks + (16 * jt + l16) * SS + kb + 4 * g4);
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mfma_f32_k4(av[s], bv[s], acc);
            }
        } else {
            for (int f = lane; f < two; f += 64) {
                float ssum = 0.0f;
#pragma unroll 8
                for (int r = 0; r < kBC; ++r) ssum += Ks[r * SS + f];
                gks[col0 + f] = ssum;
            }
        }
        __syncthreads();                                 // the slice is dead
    }
    if (wv < 3) {
        const int colm = 16 * jt + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * it + 4 * g4 + e;
            Mm[row * CS + colm] = colm <= row ? acc[e] : 0.0f;
        }
    } else {
        for (int e = lane; e < 256; e += 64) Mm[(e >> 4) * CS + 16 + (e & 15)] = 0.0f;
    }
    __syncthreads();
    // M V ([c][r]) on the fp32 MFMA: tiles (it, rt), wave w takes w + 4 q
    float* gN = a.ws + a.L.nm + int64_t(u) * kBC * d_v;
    for (int tau = wv; tau < 2 * ((d_v + 15) / 16); tau += 4) {
        const int it2 = tau & 1, rt = tau >> 1;
        const int r = 16 * rt + l16;
        f32x4 acc2 = zero4();
#pragma unroll
        for (int kb = 0; kb < kBC; kb += 16) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(Mm + (16 * it2 + l16) * CS + kb + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc2 = mfma_f32_k4(av[s], r < d_v ? Vs[(kb + 4 * g4 + s) * d_v + r] : 0.0f, acc2);
        }
        if (r < d_v) {
#pragma unroll
            for (int e = 0; e < 4; ++e) gN[(16 * it2 + 4 * g4 + e) * d_v + r] = acc2[e];
        }
    }
    if (tid < kBC) {
        float sm = 0.0f;
        for (int j2 = 0; j2 <= tid; ++j2) sm += Mm[tid * CS + j2];
        a.ws[a.L.dn + int64_t(u) * kBC + tid] = sm;
    }
}

// z_final = z0 + the chunks' column sums of K, one thread per entry (each reads its z0 entry
// before writing its z_final entry, so z_final may be z0).
// Eight independent partial sums keep eight loads in flight per thread.
__global__ __launch_bounds__(256) void sum_zfinal_kernel(SumArgs a) {
    const int bh = blockIdx.x;
    for (int p = threadIdx.x; p < a.D; p += 256) {
        const float* ks = a.ws + a.L.ks + int64_t(bh) * a.NC * a.D + p;
        float zp[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        int n = 0;
        for (; n + 8 <= a.NC; n += 8)
#pragma unroll
            for (int i = 0; i < 8; ++i) zp[i] += ks[int64_t(n + i) * a.D];
        for (; n < a.NC; ++n) zp[0] += ks[int64_t(n) * a.D];
        const float z = a.z0 ? a.z0[int64_t(bh) * a.D + p] : 0.0f;
        a.zf[int64_t(bh) * a.D + p] = z + (((zp[0] + zp[1]) + (zp[2] + zp[3])) + ((zp[4] + zp[5]) + (zp[6] + zp[7])));
    }
}

// Blocked scan, first launch: per (b, h, block blk < NB - 1, part sp, 16 columns) the sum of
// K^T V over the part's chunks (fp32 MFMA; the same accumulator layout as the scan's memory
// tiles: wave w holds d-tiles w + 4 q, lane group g supplies rows 4 g + s of each 16-row step
// to sub-step s), and, in its first column group, the part's sum of the key sums.  A chunk's
// operands (NDW x 8 values of K and 8 of V per lane) load a chunk ahead of its products.  The
// workgroups of block NB - 1 (part 0) copy W0 (zeros where there is none) into the workspace.
template <bool BF16, int NDW>
__global__ __launch_bounds__(256) void sum_blocksum_kernel(SumArgs a) {
    const int D = a.D, d_v = a.d_v, NDT = D / 16;
    const int cgroups = (d_v + 15) / 16;
    // the column groups of one (b, h, block, part) share an XCD (and its L2 copy of K)
    const BhIndex xi = xcd_local(blockIdx.x, a.BH * a.NB * a.SP, cgroups);
    const int cg = static_cast<int>(xi.i);
    int rest = xi.bh;
    const int sp = rest % a.SP;
    rest /= a.SP;
    const int blk = rest % a.NB, bh = rest / a.NB;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int col = 16 * cg + l16;
    const bool cok = col < d_v;
    if (blk == a.NB - 1) {
        if (sp != 0) return;
#pragma unroll
        for (int q = 0; q < NDW; ++q) {
            const int dt = wv + 4 * q;
            if (!cok || dt >= NDT) continue;
            const int64_t o = (int64_t(bh) * d_v + col) * D + 16 * dt + 4 * g4;
            *reinterpret_cast<f32x4*>(a.ws + a.L.wc + o) =
                a.W0 ? *reinterpret_cast<const f32x4*>(a.W0 + o) : zero4();
        }
        return;
    }
    // this part's chunks
    const int b0 = blk * a.LC, b1 = min(a.NC, b0 + a.LC);
    const int per = (b1 - b0 + a.SP - 1) / a.SP;
    const int c0 = min(b1, b0 + sp * per), c1 = min(b1, c0 + per);
    const int64_t part = (int64_t(blk) * a.SP + sp) * a.BH + bh;
    if (cg == 0) {
        for (int p = tid; p < D; p += 256) {
            float zp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            int c = c0;
            for (; c + 4 <= c1; c += 4)
#pragma unroll
                for (int i = 0; i < 4; ++i) zp[i] += a.ws[a.L.ks + (int64_t(bh) * a.NC + c + i) * D + p];
            for (; c < c1; ++c) zp[0] += a.ws[a.L.ks + (int64_t(bh) * a.NC + c) * D + p];
            a.ws[a.L.zb + part * D + p] = (zp[0] + zp[1]) + (zp[2] + zp[3]);
        }
    }
    f32x4 acc[NDW];
#pragma unroll
    for (int q = 0; q < NDW; ++q) acc[q] = zero4();
    float kv[NDW][8], vv[8];
    auto fetch = [&](int c) {
        const float* Kc = a.ws + a.L.kt + (int64_t(bh) * a.NC + c) * (kBC * D);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 16 * (i >> 2) + 4 * g4 + (i & 3), t = c * kBC + r;
            vv[i] = (cok && t < a.T) ? load_elem<BF16>(a.v, (int64_t(bh) * a.T + t) * d_v + col) : 0.0f;
#pragma unroll
            for (int q = 0; q < NDW; ++q) {
                const int dt = wv + 4 * q < NDT ? wv + 4 * q : 0;
                kv[q][i] = Kc[r * D + 16 * dt + l16];
            }
        }
    };
    if (c0 < c1) fetch(c0);
    for (int c = c0; c < c1; ++c) {
        float kc[NDW][8], vc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            vc[i] = vv[i];
#pragma unroll
            for (int q = 0; q < NDW; ++q) kc[q][i] = kv[q][i];
        }
        if (c + 1 < c1) fetch(c + 1);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int q = 0; q < NDW; ++q) acc[q] = mfma_f32_k4(kc[q][i], vc[i], acc[q]);
    }
#pragma unroll
    for (int q = 0; q < NDW; ++q) {
        const int dt = wv + 4 * q;
        if (cok && dt < NDT)
            *reinterpret_cast<f32x4*>(a.ws + a.L.bs + (part * d_v + col) * D + 16 * dt + 4 * g4) = acc[q];
    }
}

// One workgroup of 4 waves per (b, h, 16 columns of W = 16 rows of the memory), chunks in
// order.  The memory W^T (D x 16) lives in fp32 MFMA accumulators, wave w holding d-tiles
// w + 4 q (rows d = 16 dt + 4 (l / 16) + e, column l % 16 of lane l, slot e), which is exactly
// the B operand of a 16x16x4 product over those d (lane group g supplies k = 4 g + s to
// sub-step s).  Per chunk:
//   1. each wave forms its part of Q W^T over its d-tiles (two 16-row tiles) and of Q z (z, the
//      same for every column, sits in LDS), into LDS;
//   2. waves 0 and 1 sum the four parts of row tile 0 and 1 and write y = (Q W^T + M V) /
//      (Q z + M 1) (0 where the denominator is exactly 0);
//   3. each wave adds K^T V to its d-tiles and K^T 1 to its entries of z (K and V staged
//      transposed, so every operand read is one 16-byte read per lane).
// The next chunk's K and Q tiles, V columns and chunk-local parts load into registers while
// the current chunk computes.
template <bool BF16, int NDW>
__global__ __launch_bounds__(256) void sum_scan_kernel(SumArgs a) {
    extern __shared__ float lds[];
    const int D = a.D, d_v = a.d_v, NDT = a.D / 16;
    const int cgroups = (d_v + 15) / 16;
    // the column groups of one (b, h, block) share an XCD (and its L2 copy of the chunk's tiles)
    const BhIndex xi = xcd_local(blockIdx.x, a.BH * a.NB, cgroups);
    const int rest = xi.bh, col0 = static_cast<int>(xi.i) * 16;
    const int blk = rest % a.NB, bh = rest / a.NB;
    const int c0 = blk * a.LC, c1 = min(a.NC, c0 + a.LC);   // this workgroup's chunks
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int col = col0 + l16;
    const bool cok = col < d_v;
    const int SDQ = D + 4;                    // row stride of the staged tiles
    constexpr int VS = kBC + 4;               // row stride of V^T
    float* Qt = lds;                          // [C][SDQ]
    float* KT = Qt + kBC * SDQ;               // [D][VS]: K^T
    float* Vt = KT + D * VS;                  // [16][VS]: V^T of the chunk's 16 columns
    float* zs = Vt + 16 * VS;                 // [D]
    f32x4* red = reinterpret_cast<f32x4*>(zs + D);   // [4 waves][2 row tiles][64 lanes]
    float* qzr = reinterpret_cast<float*>(red + 4 * 2 * 64);   // [4][C]

    // memory tiles and z at the block's start: W0 and z0 (one block), else the workspace's W0
    // copy plus the sums of the blocks before this one
    f32x4 W[NDW];
#pragma unroll
    for (int q = 0; q < NDW; ++q) {
        const int dt = wv + 4 * q;
        W[q] = zero4();
        if (!cok || dt >= NDT) continue;
        const int64_t o = (int64_t(bh) * d_v + col) * D + 16 * dt + 4 * g4;
        if (a.NB == 1) {
            if (a.W0) W[q] = *reinterpret_cast<const f32x4*>(a.W0 + o);
        } else {
            // four independent sums keep four loads in flight
            const float* src = a.ws + a.L.bs + o;
            const int64_t stride = int64_t(a.BH) * d_v * D;
            f32x4 s4[4] = {zero4(), zero4(), zero4(), zero4()};
            int b = 0;
            for (; b + 4 <= blk * a.SP; b += 4)
#pragma unroll
                for (int i = 0; i < 4; ++i) s4[i] += *reinterpret_cast<const f32x4*>(src + (b + i) * stride);
            for (; b < blk * a.SP; ++b) s4[0] += *reinterpret_cast<const f32x4*>(src + b * stride);
            W[q] = *reinterpret_cast<const f32x4*>(a.ws + a.L.wc + o) + ((s4[0] + s4[1]) + (s4[2] + s4[3]));
        }
    }
    for (int d = tid; d < D; d += 256) {
        float z = a.z0 ? a.z0[int64_t(bh) * D + d] : 0.0f;
        for (int b = 0; b < blk * a.SP; ++b) z += a.ws[a.L.zb + (int64_t(b) * a.BH + bh) * D + d];
        zs[d] = z;
    }

    // staging units: Q as 16-byte units u = tid + 256 m of the [C][D] tile (row u / (D / 4));
    // K^T as units (column d = u % D, rows 4 (u / D) .. + 3), four loads down a column of K
    // (coalesced along D over the lanes) and one 16-byte store.  The LDS offsets are fixed, so
    // they are computed once.
    const int units = kBC * D / 4;
    constexpr int NUM = 2 * NDW;              // D / 32 <= 2 NDW units per thread and tile
    int loff[NUM], koff[NUM], kgo[NUM];
#pragma unroll
    for (int m = 0; m < NUM; ++m) {
        const int uu = tid + 256 * m;
        const int c = uu / (D / 4), c4 = uu - c * (D / 4);
        loff[m] = uu < units ? c * SDQ + 4 * c4 : -1;
        const int kc = uu / D, kd = uu - kc * D;
        koff[m] = kd * VS + 4 * kc;
        kgo[m] = 4 * kc * D + kd;
    }
    const int64_t CD = int64_t(kBC) * D;
    f32x4 pq[NUM], pk[NUM];
    float pv[2], pnm[4], pdn[4];
    auto fetch = [&](int n) {
        const int64_t uf = int64_t(bh) * a.NC + n;
        const f32x4* gq = reinterpret_cast<const f32x4*>(a.ws + a.L.qt + uf * CD);
        const float* gk = a.ws + a.L.kt + uf * CD;
#pragma unroll
        for (int m = 0; m < NUM; ++m) {
            const int uu = tid + 256 * m;
            pq[m] = uu < units ? gq[uu] : zero4();
            pk[m] = zero4();
            if (uu < units) {
#pragma unroll
                for (int q = 0; q < 4; ++q) pk[m][q] = gk[kgo[m] + q * D];
            }
        }
        // V^T: element e = tid + 256 m2 -> (c = e / 16, column e % 16)
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
            const int e = tid + 256 * m2, c = e >> 4, cc = col0 + (e & 15);
            const int t = n * kBC + c;
            pv[m2] = (t < a.T && cc < d_v) ? load_elem<BF16>(a.v, (int64_t(bh) * a.T + t) * d_v + cc) : 0.0f;
        }
        // chunk-local parts of the rows this lane writes (row tile wv, waves 0 and 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = 16 * (wv & 1) + 4 * g4 + e;
            pnm[e] = cok ? a.ws[a.L.nm + (uf * kBC + c) * d_v + col] : 0.0f;
            pdn[e] = a.ws[a.L.dn + uf * kBC + c];
        }
    };
    if (c0 < c1) fetch(c0);
    for (int n = c0; n < c1; ++n) {
        const int t0 = n * kBC;
        __syncthreads();                      // the previous chunk's tile reads are done
#pragma unroll
        for (int m = 0; m < NUM; ++m)
            if (loff[m] >= 0) {
                *reinterpret_cast<f32x4*>(Qt + loff[m]) = pq[m];
                *reinterpret_cast<f32x4*>(KT + koff[m]) = pk[m];
            }
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
            const int e = tid + 256 * m2;
            Vt[(e & 15) * VS + (e >> 4)] = pv[m2];
        }
        float nm[4], dn[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            nm[e] = pnm[e];
            dn[e] = pdn[e];
        }
        __syncthreads();
        if (n + 1 < c1) fetch(n + 1);
        // ---- 1. parts of Q W^T (MFMA) and Q z (lane -> row c = lane % 32, half of each d-tile)
        f32x4 P0 = zero4(), P1 = zero4();
        float qz = 0.0f;
        const int cz = lane & 31, hz = lane >> 5;
#pragma unroll
        for (int q = 0; q < NDW; ++q) {
            const int dt = wv + 4 * q;
            if (dt >= NDT) continue;
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(Qt + l16 * SDQ + 16 * dt + 4 * g4);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(Qt + (16 + l16) * SDQ + 16 * dt + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                P0 = mfma_f32_k4(a0[s], W[q][s], P0);
                P1 = mfma_f32_k4(a1[s], W[q][s], P1);
            }
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                const int d = 16 * dt + 8 * hz + dd;
                qz += Qt[cz * SDQ + d] * zs[d];
            }
        }
        qz += __shfl_xor(qz, 32);
        red[(wv * 2 + 0) * 64 + lane] = P0;
        red[(wv * 2 + 1) * 64 + lane] = P1;
        if (lane < kBC) qzr[wv * kBC + lane] = qz;
        __syncthreads();
        // ---- 2. y rows of row tile wv (waves 0, 1)
        if (wv < 2) {
            const int rt = wv;
            const f32x4 num = (red[(0 * 2 + rt) * 64 + lane] + red[(1 * 2 + rt) * 64 + lane]) +
                              (red[(2 * 2 + rt) * 64 + lane] + red[(3 * 2 + rt) * 64 + lane]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * rt + 4 * g4 + e;
                const float den = (qzr[c] + qzr[kBC + c]) + (qzr[2 * kBC + c] + qzr[3 * kBC + c]) + dn[e];
                const float nv = num[e] + nm[e];
                if (cok && t0 + c < a.T)
                    store_elem<BF16>(a.y, (int64_t(bh) * a.T + t0 + c) * d_v + col,
                                     den != 0.0f ? nv / den : 0.0f);
            }
        }
        // ---- 3. W^T += K^T V and z += K^T 1 on this wave's d-tiles
#pragma unroll
        for (int q = 0; q < NDW; ++q) {
            const int dt = wv + 4 * q;
            if (dt >= NDT) continue;
            const float* kr = KT + (16 * dt + l16) * VS;
#pragma unroll
            for (int kb = 0; kb < kBC; kb += 16) {
                const f32x4 bv = *reinterpret_cast<const f32x4*>(Vt + l16 * VS + kb + 4 * g4);
                const f32x4 av = *reinterpret_cast<const f32x4*>(kr + kb + 4 * g4);
#pragma unroll
                for (int s = 0; s < 4; ++s) W[q] = mfma_f32_k4(av[s], bv[s], W[q]);
            }
            const f32x4 z0v = *reinterpret_cast<const f32x4*>(kr + 8 * g4);
            const f32x4 z1v = *reinterpret_cast<const f32x4*>(kr + 8 * g4 + 4);
            float zp = (z0v[0] + z0v[1]) + (z0v[2] + z0v[3]) + (z1v[0] + z1v[1]) + (z1v[2] + z1v[3]);
            zp += __shfl_xor(zp, 16);
            zp += __shfl_xor(zp, 32);
            if (g4 == 0) zs[16 * dt + l16] += zp;
        }
    }
    if (a.Wf && cok && blk == a.NB - 1) {
#pragma unroll
        for (int q = 0; q < NDW; ++q) {
            const int dt = wv + 4 * q;
            if (dt < NDT)
                *reinterpret_cast<f32x4*>(a.Wf + (int64_t(bh) * d_v + col) * D + 16 * dt + 4 * g4) = W[q];
        }
    }
}

bool plan_sum_forward(int BH, int T, int d_k, int d_v, int nu, int64_t* ws_bytes) {
    const int D = 2 * d_k * nu;
    if (d_k != 16 && d_k != 32 && d_k != 64) return false;
    if (d_v < 1 || d_v > 128 || D > 384) return false;
    const int NC = (T + kBC - 1) / kBC;
    int LC;
    const int NB = sum_blocks(BH, NC, d_v, &LC);
    *ws_bytes = sum_layout(BH, NC, D, d_v, NB, sum_parts(BH, NB, LC, d_v)).end * 4;
    return true;
}

template <int NDW, bool BF16>
static hipError_t launch_scan(const SumArgs& a, hipStream_t stream) {
    const int cgroups = (a.d_v + 15) / 16;
    auto kern = sum_scan_kernel<BF16, NDW>;
    const int lds = 4 * (kBC * (a.D + 4) + a.D * (kBC + 4) + 16 * (kBC + 4) + a.D + 4 * 2 * 64 * 4 +
                         4 * kBC);
    hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kern), lds);
    if (e != hipSuccess) return e;
    if (a.NB > 1) {
        auto bk = sum_blocksum_kernel<BF16, NDW>;
        hipLaunchKernelGGL(bk, dim3(static_cast<unsigned>(int64_t(a.BH) * a.NB * a.SP * cgroups)),
                           dim3(256), 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(int64_t(a.BH) * a.NB * cgroups)), dim3(256),
                       lds, stream, a);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_sum_t(const SumArgs& a, hipStream_t stream) {
    const int64_t NU = int64_t(a.BH) * a.NC;
    hipError_t e;
    if (NU > 0) {
        const int lp = 4 * (2 * kBC * 2 * a.d_k + 2 * kBC * (2 * a.d_k + 4) + kBC * (kBC + 4) +
                            kBC * a.d_v);
        auto kp = sum_prep_kernel<BF16>;
        if ((e = ensure_lds_attr(reinterpret_cast<const void*>(kp), lp)) != hipSuccess) return e;
        hipLaunchKernelGGL(kp, dim3(static_cast<unsigned>(NU)), dim3(kSumThreads), lp, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    switch ((a.D / 16 + 3) / 4) {
        case 1: e = launch_scan<1, BF16>(a, stream); break;
        case 2: e = launch_scan<2, BF16>(a, stream); break;
        case 3: e = launch_scan<3, BF16>(a, stream); break;
        case 4: e = launch_scan<4, BF16>(a, stream); break;
        case 5: e = launch_scan<5, BF16>(a, stream); break;
        case 6: e = launch_scan<6, BF16>(a, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || !a.zf) return e;
    hipLaunchKernelGGL(sum_zfinal_kernel, dim3(static_cast<unsigned>(a.BH)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_sum_forward(const void* q, const void* k, const void* v, const float* W0,
                              const float* z0, void* y, float* Wf, float* zf, int BH, int T,
                              int d_k, int d_v, int nu, bool bf16, void* workspace,
                              hipStream_t stream) {
    SumArgs a;
    a.q = q; a.k = k; a.v = v; a.W0 = W0; a.z0 = z0; a.y = y; a.Wf = Wf; a.zf = zf;
    a.ws = static_cast<float*>(workspace);
    a.BH = BH; a.T = T; a.NC = (T + kBC - 1) / kBC; a.d_k = d_k; a.d_v = d_v; a.nu = nu;
    a.D = 2 * d_k * nu;
    a.NB = sum_blocks(BH, a.NC, d_v, &a.LC);
    a.SP = sum_parts(BH, a.NB, a.LC, d_v);
    a.L = sum_layout(BH, a.NC, a.D, d_v, a.NB, a.SP);
    return bf16 ? launch_sum_t<true>(a, stream) : launch_sum_t<false>(a, stream);
}

}  // namespace fwa
