// The linear maps around the layer ("Fast Weights Transformer" guide, xdnf.cn/news/308600,
// section "FastWeightsAttention / module structure and source walkthrough"): the bias-free
// query, key, value and interpolation-weight projections of x, written straight into the
// head-split [B, H, T, d] layout the layer reads, and the output map (with bias) of the heads'
// concatenated outputs, read straight from [B, H, T, d_v] and added to a residual.
//
// Both are C[M x N] = A[M x K] B^T with B an [N x K] weight (out = x W^T).  A workgroup of 4
// waves computes one 16 x 16 tile of C with the k range split over its waves (stages of four
// 16-byte loads per operand and lane, stage s to wave s % 4), so a token-wise decode (M = the
// number of sequences, a few hundred) spreads over a thousand or more workgroups and each wave
// waits for about one memory round trip: its stages' loads go out two at a time, ahead of their
// products.  The four partial tiles are summed through LDS.  bf16 operands use
// v_mfma_f32_16x16x32_bf16; fp32 operands v_mfma_f32_16x16x4f32 (four per 16-deep k block).  In
// both, lane l supplies row l % 16 of A and of B^T over a run of consecutive k (8 bf16 or 4
// fp32: one 16-byte load each, contiguous in x, y and the weights).
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
    int mblk0;           // first 16-row block of this launch (grids are at most 65535 tall)
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

template <bool BF16, int MODE>
__global__ __launch_bounds__(256) void linear_kernel(LinArgs a) {
    constexpr int KL = BF16 ? 32 : 16;          // k covered by one 16-byte load per lane
    constexpr int U = 4;                         // loads per operand per stage
    constexpr int ES = BF16 ? 2 : 4;
    __shared__ f32x4 part[4][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t m0 = (int64_t(a.mblk0) + blockIdx.y) * 16;
    const int n0 = blockIdx.x * 16;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t m = m0 + li;
    const int n = n0 + li;
    const bool mok = m < a.M, nok = n < a.N;
    const unsigned mu = mok ? static_cast<unsigned>(m) : 0u;
    const int mb = static_cast<int>(mu / static_cast<unsigned>(a.T)), mt = static_cast<int>(mu) - mb * a.T;
    const char* Ab = static_cast<const char*>(a.A);
    const char* Bb = static_cast<const char*>(a.Bw) + (nok ? int64_t(n) * a.K * ES : 0);
    uint4 ra0[U], rb0[U], ra1[U], rb1[U];
    // stage st: k runs kk = st U KL + u KL + (KL / 4) lg; a run past K (or a row past M / N)
    // loads nothing and reads as zero
    auto load = [&](int st, uint4 (&xa)[U], uint4 (&xb)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = (st * U + u) * KL + (KL / 4) * lg;
            const bool kok = kk < a.K;
            xa[u] = make_uint4(0u, 0u, 0u, 0u);
            xb[u] = make_uint4(0u, 0u, 0u, 0u);
            if (mok && kok) xa[u] = *reinterpret_cast<const uint4*>(Ab + a_offset<MODE>(a, m, mb, mt, kk) * ES);
            if (nok && kok) xb[u] = *reinterpret_cast<const uint4*>(Bb + int64_t(kk) * ES);
        }
    };
    f32x4 acc = zero4(), acc2 = zero4();
    auto products = [&](const uint4 (&xa)[U], const uint4 (&xb)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            f32x4& ac = (u & 1) ? acc2 : acc;
            if constexpr (BF16) {
                ac = mfma_bf16_k32(__builtin_bit_cast(bf16x8, xa[u]), __builtin_bit_cast(bf16x8, xb[u]), ac);
            } else {
                // sub-step s takes k = kk + s from lane group lg: the same k for A and B
                const f32x4 fa = __builtin_bit_cast(f32x4, xa[u]), fb = __builtin_bit_cast(f32x4, xb[u]);
                ac = mfma_f32_k4(fa[0], fb[0], ac);
                ac = mfma_f32_k4(fa[1], fb[1], ac);
                ac = mfma_f32_k4(fa[2], fb[2], ac);
                ac = mfma_f32_k4(fa[3], fb[3], ac);
            }
        }
    };
    // this wave's stages wave, wave + 4, ...: two register sets, the next pair's loads issued
    // before the current pair's products
    const int stages = (a.K + U * KL - 1) / (U * KL);
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
    part[wave][lane] = acc + acc2;
    __syncthreads();
    if (wave != 0) return;
    acc = part[0][lane] + part[1][lane];
    acc2 = part[2][lane] + part[3][lane];
    acc += acc2;
    // result slot r: row m0 + 4 lg + r, column n0 + li
    if (!nok) return;
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
            store_elem<BF16>(dst, ((int64_t(b) * a.H + hh) * a.T + tt) * dw + c, acc[r]);
        }
    } else {
        const float bias = a.bias ? load_elem<BF16>(a.bias, n) : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t mr = m0 + 4 * lg + r;
            if (mr >= a.M) continue;
            float o = acc[r] + bias;
            if (a.res) o += load_elem<BF16>(a.res, mr * a.N + n);
            store_elem<BF16>(a.out, mr * a.N + n, o);
        }
    }
}

template <int MODE>
static hipError_t launch_linear(const LinArgs& a0, bool bf16, hipStream_t stream) {
    if (a0.M == 0 || a0.N == 0) return hipSuccess;
    const int mblocks = static_cast<int>((int64_t(a0.M) + 15) / 16);
    for (int b0 = 0; b0 < mblocks; b0 += 65535) {
        LinArgs a = a0;
        a.mblk0 = b0;
        const int nb = mblocks - b0 < 65535 ? mblocks - b0 : 65535;
        const dim3 grid(static_cast<unsigned>((a.N + 15) / 16), static_cast<unsigned>(nb));
        if (bf16) hipLaunchKernelGGL((linear_kernel<true, MODE>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((linear_kernel<false, MODE>), grid, dim3(256), 0, stream, a);
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
