// Sum-update linear attention with the z normaliser ("Fast Weights Transformer" guide,
// xdnf.cn/news/308600, section "Background / fast computation form of linear self-attention"):
//   W_t = W_{t-1} + v_t phi(k_t)^T,  z_t = z_{t-1} + phi(k_t),  y_t = W_t phi(q_t) / (z_t . phi(q_t))
// with phi = DPFP, and y_t = 0 where the denominator is exactly 0.
//
// For a chunk of C rows with normalised features K, Q (C x D) starting from W0, z0, and
// M = lower_incl(Q K^T):
//   Y = (Q W0^T + M V) / (Q z0 + M 1)   (row-wise),   W1 = W0 + V^T K,   z1 = z0 + K^T 1.
// Three launches:
//   1. sum_prep  per chunk: K, Q, and the chunk-local parts M V and M 1            (parallel)
//   2. sum_scan  per (b, h, 8 rows of W), chunks in order: row r of W moves on its own
//      (w <- w + K^T V[:, r]); each wave also carries z (the same for every row), so it forms
//      y[:, r] itself                                                                (serial)
//   3. sum_zfinal per (b, h): z_final from z0 and the chunks' key sums (where it is asked for)
// Arithmetic is fp32 on the vector ALU; chunks of 32 rows.
#include "chunk_f32.h"
#include "fwa_internal.h"

namespace fwa {

constexpr int kSumThreads = 256;

struct SumLayout {
    int64_t kt, qt, nm, dn, ks, end;   // K, Q [C][D]; M V [C][d_v]; M 1 [C]; K^T 1 [D] (per chunk)
};

static SumLayout sum_layout(int64_t NU, int D, int d_v) {
    SumLayout L;
    int64_t o = 0;
    L.kt = o; o += NU * kBC * D;
    L.qt = o; o += NU * kBC * D;
    L.nm = o; o += NU * kBC * d_v;
    L.dn = o; o += NU * kBC;
    L.ks = o; o += NU * D;
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
    SumLayout L;
};

// LDS: x rows of k and q (C x 2 d_k each), K and Q (C x SD, SD = D + 8), M (C x (C + 1)), V.
template <bool BF16>
__global__ __launch_bounds__(kSumThreads) void sum_prep_kernel(SumArgs a) {
    extern __shared__ float lds[];
    const int D = a.D, d_k = a.d_k, d_v = a.d_v, two = 2 * d_k;
    const int u = blockIdx.x;
    const int bh = u / a.NC, n = u % a.NC;
    const int t0 = n * kBC;
    const int tid = threadIdx.x;
    const int rows = a.T - t0 < kBC ? a.T - t0 : kBC;
    const int wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    constexpr int CS = kBC + 4;       // 16-byte rows for the MFMA operand reads
    const int SD = tile_stride(D);
    float* xk = lds;
    float* xq = xk + kBC * two;
    float* Kt = xq + kBC * two;
    float* Qt = Kt + kBC * SD;
    float* Mm = Qt + kBC * SD;
    float* Vs = Mm + kBC * CS;
    load_relu_rows<BF16>(a.k, xk, int64_t(bh) * a.T, rows, t0, d_k, tid, kSumThreads);
    load_relu_rows<BF16>(a.q, xq, int64_t(bh) * a.T, rows, t0, d_k, tid, kSumThreads);
    for (int c = wv; c < kBC; c += kSumThreads / 64)
        for (int r = lane; r < d_v; r += 64)
            Vs[c * d_v + r] = c < rows ? load_elem<BF16>(a.v, (int64_t(bh) * a.T + t0 + c) * d_v + r) : 0.0f;
    dpfp_tiles(xk, xq, Kt, Qt, D, d_k, tid);
    const int64_t CD = int64_t(kBC) * D;
    float* gK = a.ws + a.L.kt + int64_t(u) * CD;
    float* gQ = a.ws + a.L.qt + int64_t(u) * CD;
    for (int c = wv; c < kBC; c += kSumThreads / 64)
        for (int p = lane; p < D; p += 64) {
            gK[c * D + p] = Kt[c * SD + p];
            gQ[c * D + p] = Qt[c * SD + p];
        }
    // M = lower_incl(Q K^T) on the fp32 MFMA: wave w < 3 takes tile (0,0), (1,0), (1,1); wave 3
    // zeroes tile (0, 1).  Lane group g supplies k = 4 g + s to sub-step s of a 16-deep block.
    if (wv < 3) {
        const int it = wv == 0 ? 0 : 1, jt = wv == 2 ? 1 : 0;
        f32x4 acc = zero4();
        for (int kb = 0; kb < D; kb += 16) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(Qt + (16 * it + l16) * SD + kb + 4 * g4);
            const f32x4 bv = *reinterpret_cast<const f32x4*>(Kt + (16 * jt + l16) * SD + kb + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma_f32_k4(av[s], bv[s], acc);
        }
        const int col = 16 * jt + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * it + 4 * g4 + e;
            Mm[row * CS + col] = col <= row ? acc[e] : 0.0f;
        }
    } else {
        for (int e = lane; e < 256; e += 64) Mm[(e >> 4) * CS + 16 + (e & 15)] = 0.0f;
    }
    __syncthreads();
    // M V ([c][r]) on the fp32 MFMA: tiles (it, rt), wave w takes w + 4 q
    float* gN = a.ws + a.L.nm + int64_t(u) * kBC * d_v;
    for (int tau = wv; tau < 2 * ((d_v + 15) / 16); tau += 4) {
        const int it = tau & 1, rt = tau >> 1;
        const int r = 16 * rt + l16;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < kBC; kb += 16) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(Mm + (16 * it + l16) * CS + kb + 4 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = mfma_f32_k4(av[s], r < d_v ? Vs[(kb + 4 * g4 + s) * d_v + r] : 0.0f, acc);
        }
        if (r < d_v) {
#pragma unroll
            for (int e = 0; e < 4; ++e) gN[(16 * it + 4 * g4 + e) * d_v + r] = acc[e];
        }
    }
    if (tid < kBC) {
        float s = 0.0f;
        for (int j = 0; j <= tid; ++j) s += Mm[tid * CS + j];
        a.ws[a.L.dn + int64_t(u) * kBC + tid] = s;
    }
    for (int p = tid; p < D; p += kSumThreads) {
        float s = 0.0f;
        for (int c = 0; c < kBC; ++c) s += Kt[c * SD + p];
        a.ws[a.L.ks + int64_t(u) * D + p] = s;
    }
}

// z_final = z0 + the chunks' column sums of K, one thread per entry (each reads its z0 entry
// before writing its z_final entry, so z_final may be z0).
__global__ __launch_bounds__(256) void sum_zfinal_kernel(SumArgs a) {
    const int bh = blockIdx.x;
    for (int p = threadIdx.x; p < a.D; p += 256) {
        float z = a.z0 ? a.z0[int64_t(bh) * a.D + p] : 0.0f;
        for (int n = 0; n < a.NC; ++n) z += a.ws[a.L.ks + (int64_t(bh) * a.NC + n) * a.D + p];
        a.zf[int64_t(bh) * a.D + p] = z;
    }
}

// Lane l holds w[l + 64 m] (row r of W) and zz[l + 64 m] (z), m < NPL.  The next chunk's K
// and Q tiles load into registers while the current chunk computes.
template <bool BF16, int NPL>
__global__ __launch_bounds__(64 * kRowWaves) void sum_scan_kernel(SumArgs a) {
    extern __shared__ float lds[];
    const int D = a.D, d_v = a.d_v;
    const int rgroups = (d_v + kRowWaves - 1) / kRowWaves;
    const int bh = blockIdx.x / rgroups;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = (blockIdx.x % rgroups) * kRowWaves + wave;
    const bool live = r < d_v;
    constexpr int SDP = 64 * NPL;     // padded LDS row stride of the staged tiles
    float* Kt = lds;                  // [C][SDP]
    float* Qt = Kt + kBC * SDP;
    int slot[NPL];
    tile_slots<NPL>(slot, D, tid);
    zero_tile_pads<NPL>(Kt, D, tid);
    zero_tile_pads<NPL>(Qt, D, tid);
    float w[NPL], zz[NPL];
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
        const int p = lane + 64 * m;
        w[m] = (live && a.W0 && p < D) ? a.W0[(int64_t(bh) * d_v + r) * D + p] : 0.0f;
        zz[m] = (a.z0 && p < D) ? a.z0[int64_t(bh) * D + p] : 0.0f;
    }
    const int64_t CD = int64_t(kBC) * D;
    const int n_tile = kBC * D;
    f32x4 rk[NPL], rq[NPL];
    float v_next = 0.0f, nm_next = 0.0f, dn_next = 0.0f;
    // v[t, r] in lane t - t0; the chunk-local parts of row lane >> 1
#define FWA_SUM_FETCH(nn)                                                                       \
    do {                                                                                       \
        const int64_t uf = int64_t(bh) * a.NC + (nn);                                          \
        prefetch_tile<NPL>(rk, a.ws + a.L.kt + uf * CD, n_tile, tid);                          \
        prefetch_tile<NPL>(rq, a.ws + a.L.qt + uf * CD, n_tile, tid);                          \
        const int tf = (nn) * kBC + lane;                                                      \
        v_next = (live && lane < kBC && tf < a.T)                                             \
                     ? load_elem<BF16>(a.v, (int64_t(bh) * a.T + tf) * d_v + r) : 0.0f;       \
        nm_next = live ? a.ws[a.L.nm + (uf * kBC + (lane >> 1)) * d_v + r] : 0.0f;            \
        dn_next = a.ws[a.L.dn + uf * kBC + (lane >> 1)];                                       \
    } while (0)
    if (a.NC > 0) FWA_SUM_FETCH(0);
    for (int n = 0; n < a.NC; ++n) {
        const int t0 = n * kBC;
        lds_barrier();
        commit_tile<NPL>(Kt, rk, slot);
        commit_tile<NPL>(Qt, rq, slot);
        const float vc = v_next, nm = nm_next, dn = dn_next;
        lds_barrier();
        if (n + 1 < a.NC) FWA_SUM_FETCH(n + 1);
        float pn[kBC], pd[kBC];
#pragma unroll
        for (int c = 0; c < kBC; ++c) {
            float sn = 0.0f, sd = 0.0f;
#pragma unroll
            for (int m = 0; m < NPL; ++m) {
                const float qv = Qt[c * SDP + lane + 64 * m];
                sn += qv * w[m];
                sd += qv * zz[m];
            }
            pn[c] = sn;
            pd[c] = sd;
        }
        const float qw = wave_reduce_scatter32(pn);           // (Q w)[lane >> 1]
        const float qz = wave_reduce_scatter32(pd);           // (Q z)[lane >> 1]
        const int c = lane >> 1;
        if (live && (lane & 1) == 0 && t0 + c < a.T) {
            const float num = qw + nm, den = qz + dn;
            store_elem<BF16>(a.y, (int64_t(bh) * a.T + t0 + c) * d_v + r, den != 0.0f ? num / den : 0.0f);
        }
#pragma unroll
        for (int cc = 0; cc < kBC; ++cc) {
            const float vv = lane_value(vc, cc);
#pragma unroll
            for (int m = 0; m < NPL; ++m) {
                const float kv = Kt[cc * SDP + lane + 64 * m];
                w[m] += vv * kv;
                zz[m] += kv;
            }
        }
    }
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
        const int p = lane + 64 * m;
        if (p < D && live && a.Wf) a.Wf[(int64_t(bh) * d_v + r) * D + p] = w[m];
    }
#undef FWA_SUM_FETCH
}

bool plan_sum_forward(int BH, int T, int d_k, int d_v, int nu, int64_t* ws_bytes) {
    const int D = 2 * d_k * nu;
    if (d_k != 16 && d_k != 32 && d_k != 64) return false;
    if (d_v < 1 || d_v > 128 || D > 384) return false;
    const int NC = (T + kBC - 1) / kBC;
    *ws_bytes = sum_layout(int64_t(BH) * NC, D, d_v).end * 4;
    return true;
}

template <int NPL, bool BF16>
static hipError_t launch_scan(const SumArgs& a, hipStream_t stream) {
    const int rgroups = (a.d_v + kRowWaves - 1) / kRowWaves;
    auto kern = sum_scan_kernel<BF16, NPL>;
    const int lds = 4 * 2 * kBC * 64 * NPL;
    hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kern), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(int64_t(a.BH) * rgroups)),
                       dim3(64 * kRowWaves), lds, stream, a);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_sum_t(const SumArgs& a, hipStream_t stream) {
    const int64_t NU = int64_t(a.BH) * a.NC;
    hipError_t e;
    if (NU > 0) {
        const int lp = 4 * (2 * kBC * 2 * a.d_k + 2 * kBC * tile_stride(a.D) + kBC * (kBC + 4) +
                            kBC * a.d_v);
        auto kp = sum_prep_kernel<BF16>;
        if ((e = ensure_lds_attr(reinterpret_cast<const void*>(kp), lp)) != hipSuccess) return e;
        hipLaunchKernelGGL(kp, dim3(static_cast<unsigned>(NU)), dim3(kSumThreads), lp, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    switch ((a.D + 63) / 64) {
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
    a.L = sum_layout(int64_t(BH) * a.NC, a.D, d_v);
    return bf16 ? launch_sum_t<true>(a, stream) : launch_sum_t<false>(a, stream);
}

}  // namespace fwa
