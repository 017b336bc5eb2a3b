// The linear maps around the layer ("Fast Weights Transformer" guide, xdnf.cn/news/308600,
// section "FastWeightsAttention / module structure and source walkthrough"): the bias-free
// query, key, value and interpolation-weight projections of x, written straight into the
// head-split [B, H, T, d] layout the layer reads, and the output map (with bias) of the heads'
// concatenated outputs, read straight from [B, H, T, d_v] and added to a residual.
//
// Both are C[M x N] = A[M x K] B^T with B an [N x K] weight (out = x W^T).  A workgroup of 4
// waves computes a (16 MI) x (16 NJ) tile of C (MI x NJ sub-tiles of 16 x 16) with the k range
// split over its waves in 32-deep steps (step s to wave s % 4), so a token-wise decode (M = the
// number of sequences, a few hundred) still spreads over a few hundred workgroups; each wave
// issues the next pair of steps' loads before the current pair's products.  The four partial
// tiles are summed through LDS, each wave then finishing its sub-tiles.  bf16 operands use
// v_mfma_f32_16x16x32_bf16 directly.  fp32 operands use the same product on a split: each run
// of 8 values becomes bf16 hi + lo (x = hi + lo to about 2^-16), and hi hi + hi lo + lo hi
// carries a product to about 2^-16 relative (the lo lo term is below the split's own error),
// three 16-cycle products where the fp32 MFMA needs eight 32-cycle ones per 32-deep step.  In
// both, lane l supplies row l % 16 of A and of B^T over a run of 8 consecutive k (contiguous in
// x, y and the weights).
#include "fwa_common.h"
#include "fwa_internal.h"

namespace fwa {

struct LinArgs {
    const void* A;       // x [M, K] (projection) or y [B, H, T, d_v] (output map)
    const void* Bw;      // weight [N, K]
    const void* bias;    // [N] or null (output map)
    const void* res;     // [M, N] or null (output map)
    void* out;           // [M, N] (output map)
    void* q;             // projection outputs
    void* k;
    void* v;
    void* bl;
    int M, N, K, T, H, d_k, d_v;
    int mblk0;           // first row block of this launch (grids are at most 65535 tall)
};

enum { kLinProject = 0, kLinOutput = 1 };

// Element offset of A[m][kk] (the first of a run of consecutive kk within one head).
template <int MODE>
// `mb`, `mt` are m / T and m % T (row m = token t of sequence b); 32-bit divisions, as
// M = B T fits an int.
__device__ __forceinline__ int64_t a_offset(const LinArgs& a, int64_t m, int mb, int mt, int kk) {
    if constexpr (MODE == kLinProject) return m * a.K + kk;
    const int hh = static_cast<int>(static_cast<unsigned>(kk) / static_cast<unsigned>(a.d_v));
    return ((int64_t(mb) * a.H + hh) * a.T + mt) * a.d_v + (kk - hh * a.d_v);
}

template <bool BF16, int MODE, int MI, int NJ>
__global__ __launch_bounds__(256) void linear_kernel(LinArgs a) {
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int NL = BF16 ? 1 : 2;             // 16-byte loads per operand row and k-step
    constexpr int NS = MI * NJ;                  // 16 x 16 sub-tiles per workgroup
    static_assert(NS <= 8, "at most two sub-tiles per wave in the epilogue");
    __shared__ f32x4 part[4][NS][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t mt0 = (int64_t(a.mblk0) + blockIdx.y) * (16 * MI);
    const int nt0 = blockIdx.x * (16 * NJ);
    const int li = lane & 15, lg = lane >> 4;
    // the lane's rows (sub-tile rows i < MI) and columns (sub-tile columns j < NJ)
    int64_t mi[MI];
    int mb[MI], mtt[MI];
    bool mok[MI], nok[NJ];
    const char* Bb[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        mi[i] = mt0 + 16 * i + li;
        mok[i] = mi[i] < a.M;
        const unsigned mu = mok[i] ? static_cast<unsigned>(mi[i]) : 0u;
        mb[i] = static_cast<int>(mu / static_cast<unsigned>(a.T));
        mtt[i] = static_cast<int>(mu) - mb[i] * a.T;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int nj = nt0 + 16 * j + li;
        nok[j] = nj < a.N;
        Bb[j] = static_cast<const char*>(a.Bw) + (nok[j] ? int64_t(nj) * a.K * ES : 0);
    }
    const char* Ab = static_cast<const char*>(a.A);
    // k-step s: the lane's k run kk = 32 s + 8 lg .. + 7 (one head's columns in the output
    // map, as d_v is a multiple of 8); a run past K (or a row past M / N) reads as zero
    uint4 ra0[MI][NL], rb0[NJ][NL], ra1[MI][NL], rb1[NJ][NL];
    auto load = [&](int st, uint4 (&xa)[MI][NL], uint4 (&xb)[NJ][NL]) {
        const int kk = 32 * st + 8 * lg;
        const bool kok = kk < a.K;
#pragma unroll
        for (int h = 0; h < NL; ++h) {
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                xa[i][h] = make_uint4(0u, 0u, 0u, 0u);
                if (mok[i] && kok)
                    xa[i][h] = *reinterpret_cast<const uint4*>(Ab + (a_offset<MODE>(a, mi[i], mb[i], mtt[i], kk) + 4 * h) * ES);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                xb[j][h] = make_uint4(0u, 0u, 0u, 0u);
                if (nok[j] && kok) xb[j][h] = *reinterpret_cast<const uint4*>(Bb[j] + int64_t(kk + 4 * h) * ES);
            }
        }
    };
    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = zero4();
    // bf16: one 16x16x32 product per sub-tile and k-step.  fp32: each 8-value run split into
    // bf16 hi + lo (x = hi + lo to about 2^-16), hi hi + hi lo + lo hi per sub-tile (the lo lo
    // term is below the split's own error)
    auto split8 = [](const uint4 (&x)[NL], bf16x8& hi, bf16x8& lo) {
        const f32x4 x0 = __builtin_bit_cast(f32x4, x[0]), x1 = __builtin_bit_cast(f32x4, x[NL - 1]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hi[e] = static_cast<__bf16>(x0[e]);
            hi[4 + e] = static_cast<__bf16>(x1[e]);
            lo[e] = static_cast<__bf16>(x0[e] - static_cast<float>(hi[e]));
            lo[4 + e] = static_cast<__bf16>(x1[e] - static_cast<float>(hi[4 + e]));
        }
    };
    auto products = [&](const uint4 (&xa)[MI][NL], const uint4 (&xb)[NJ][NL]) {
        if constexpr (BF16) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, xa[i][0]), __builtin_bit_cast(bf16x8, xb[j][0]), acc[i][j]);
        } else {
            bf16x8 ah[MI], al[MI], bh[NJ], bl[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i) split8(xa[i], ah[i], al[i]);
#pragma unroll
            for (int j = 0; j < NJ; ++j) split8(xb[j], bh[j], bl[j]);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    acc[i][j] = mfma_bf16_k32(ah[i], bh[j], acc[i][j]);
                    acc[i][j] = mfma_bf16_k32(ah[i], bl[j], acc[i][j]);
                    acc[i][j] = mfma_bf16_k32(al[i], bh[j], acc[i][j]);
                }
        }
    };
    // this wave's k-steps wave, wave + 4, ...: two register sets, the next pair's loads issued
    // before the current pair's products
    const int stages = (a.K + 31) / 32;
    int st = wave;
    if (st < stages) load(st, ra0, rb0);
    if (st + 4 < stages) load(st + 4, ra1, rb1);
    for (; st < stages; st += 8) {
        products(ra0, rb0);
        if (st + 8 < stages) load(st + 8, ra0, rb0);
        if (st + 4 >= stages) break;
        products(ra1, rb1);
        if (st + 12 < stages) load(st + 12, ra1, rb1);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) part[wave][NJ * i + j][lane] = acc[i][j];
    __syncthreads();
    // wave w sums and writes sub-tiles w and w + 4 (sub-tile s = (s / NJ, s % NJ))
#pragma unroll
    for (int s = wave; s < NS; s += 4) {
    const int si = s / NJ, sj = s % NJ;
    f32x4 sacc = (part[0][s][lane] + part[1][s][lane]) + (part[2][s][lane] + part[3][s][lane]);
    const int64_t m0 = mt0 + 16 * si;
    const int n = nt0 + 16 * sj + li;
    if (n >= a.N) continue;
    // result slot r: row m0 + 4 lg + r, column n
    if constexpr (MODE == kLinProject) {
        // the column's destination: q, k, v (head hh, column c) or the beta logit of head hh
        const int nq = a.H * a.d_k, nv = a.H * a.d_v;
        void* dst;
        int hh, c, dw;
        if (n < 2 * nq) {
            const int cn = n < nq ? n : n - nq;
            dst = n < nq ? a.q : a.k;
            hh = static_cast<int>(static_cast<unsigned>(cn) / static_cast<unsigned>(a.d_k));
            c = cn - hh * a.d_k;
            dw = a.d_k;
        } else if (n < 2 * nq + nv) {
            const int cn = n - 2 * nq;
            dst = a.v;
            hh = static_cast<int>(static_cast<unsigned>(cn) / static_cast<unsigned>(a.d_v));
            c = cn - hh * a.d_v;
            dw = a.d_v;
        } else {
            dst = a.bl;
            hh = n - 2 * nq - nv;
            c = 0;
            dw = 1;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t mr = m0 + 4 * lg + r;
            if (mr >= a.M) continue;
            const int b = static_cast<int>(static_cast<unsigned>(mr) / static_cast<unsigned>(a.T));
            const int tt = static_cast<int>(mr) - b * a.T;
            store_elem<BF16>(dst, ((int64_t(b) * a.H + hh) * a.T + tt) * dw + c, sacc[r]);
        }
    } else {
        const float bias = a.bias ? load_elem<BF16>(a.bias, n) : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t mr = m0 + 4 * lg + r;
            if (mr >= a.M) continue;
            float o = sacc[r] + bias;
            if (a.res) o += load_elem<BF16>(a.res, mr * a.N + n);
            store_elem<BF16>(a.out, mr * a.N + n, o);
        }
    }
    }
}

template <int MODE>
static hipError_t launch_linear(const LinArgs& a0, bool bf16, hipStream_t stream) {
    if (a0.M == 0 || a0.N == 0) return hipSuccess;
    // 32 x 32 tiles where they still give the GPU enough workgroups (the projections of a
    // decode step: 392 at 256 x 1544), else 16 x 32 (the output map: 256 at 256 x 512).  Both
    // were measured against the 16 x 16 tiles of before (17 and 8.7 us: now 11.3 and 8.7 us);
    // 32 x 64 took 12.7 us on the projection.
    const int64_t m32 = (int64_t(a0.M) + 31) / 32, n32 = (int64_t(a0.N) + 31) / 32;
    const bool tall = m32 * n32 >= 384;
    const int rows = tall ? 32 : 16;
    const int mblocks = static_cast<int>((int64_t(a0.M) + rows - 1) / rows);
    for (int b0 = 0; b0 < mblocks; b0 += 65535) {
        LinArgs a = a0;
        a.mblk0 = b0;
        const int nb = mblocks - b0 < 65535 ? mblocks - b0 : 65535;
        const dim3 grid(static_cast<unsigned>(n32), static_cast<unsigned>(nb));
        auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, a); };
        if (bf16) {
            if (tall) go(linear_kernel<true, MODE, 2, 2>);
            else go(linear_kernel<true, MODE, 1, 2>);
        } else {
            if (tall) go(linear_kernel<false, MODE, 2, 2>);
            else go(linear_kernel<false, MODE, 1, 2>);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_layer_project(const void* x, const void* Wqkvb, void* q, void* k, void* v,
                                void* bl, int B, int T, int d_model, int H, int d_k, int d_v,
                                bool bf16, hipStream_t stream) {
    LinArgs a = {};
    a.A = x;
    a.Bw = Wqkvb;
    a.q = q;
    a.k = k;
    a.v = v;
    a.bl = bl;
    a.M = B * T;
    a.N = 2 * H * d_k + H * d_v + H;
    a.K = d_model;
    a.T = T;
    a.H = H;
    a.d_k = d_k;
    a.d_v = d_v;
    return launch_linear<kLinProject>(a, bf16, stream);
}

hipError_t launch_layer_output(const void* y, const void* Wo, const void* bo, const void* res,
                               void* out, int B, int T, int H, int d_v, int d_model, bool bf16,
                               hipStream_t stream) {
    LinArgs a = {};
    a.A = y;
    a.Bw = Wo;
    a.bias = bo;
    a.res = res;
    a.out = out;
    a.M = B * T;
    a.N = d_model;
    a.K = H * d_v;
    a.T = T;
    a.H = H;
    a.d_v = d_v;
    return launch_linear<kLinOutput>(a, bf16, stream);
}

}  // namespace fwa
