// The linear maps around the layer ("Fast Weights Transformer" guide, xdnf.cn/news/308600,
// section "FastWeightsAttention / module structure and source walkthrough"): the bias-free
// query, key, value and interpolation-weight projections of x, written straight into the
// head-split [B, H, T, d] layout the layer reads, and the output map (with bias) of the heads'
// concatenated outputs, read straight from [B, H, T, d_v] and added to a residual.
//
// Both are C[M x N] = A[M x K] B^T with B an [N x K] weight (out = x W^T).  Each wave computes
// one 16 x 16 tile of C; a workgroup of 4 waves covers 32 x 32, so a token-wise decode (M = the
// number of sequences, a few hundred) still spreads over hundreds of workgroups.  bf16 operands
// use v_mfma_f32_16x16x32_bf16; fp32 operands v_mfma_f32_16x16x4f32 (four per 16-deep k block).
// In both, lane l supplies row l % 16 of A and of B^T over a run of consecutive k (8 bf16 or 4
// fp32: one 16-byte load each, contiguous in x, y and the weights).  The k loop runs in stages of
// four such loads per operand, the next stage's loads issued before the current stage's products,
// so one memory round trip is in flight behind the MFMAs instead of one per k-step.
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
};

enum { kLinProject = 0, kLinOutput = 1 };

// Element offset of A[m][kk] (the first of a run of consecutive kk within one head).
template <int MODE>
__device__ __forceinline__ int64_t a_offset(const LinArgs& a, int64_t m, int kk) {
    if constexpr (MODE == kLinProject) return m * a.K + kk;
    const int64_t b = m / a.T, t = m % a.T;
    return ((b * a.H + kk / a.d_v) * a.T + t) * a.d_v + kk % a.d_v;
}

template <bool BF16, int MODE>
__global__ __launch_bounds__(256) void linear_kernel(LinArgs a) {
    constexpr int KL = BF16 ? 32 : 16;          // k covered by one 16-byte load per lane
    constexpr int U = 4;                         // loads per operand per stage
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t m0 = int64_t(blockIdx.y) * 32 + (wave >> 1) * 16;
    const int n0 = blockIdx.x * 32 + (wave & 1) * 16;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t m = m0 + li;
    const int n = n0 + li;
    const bool mok = m < a.M, nok = n < a.N;
    const char* Ab = static_cast<const char*>(a.A);
    const char* Bb = static_cast<const char*>(a.Bw) + (nok ? int64_t(n) * a.K * (BF16 ? 2 : 4) : 0);
    constexpr int ES = BF16 ? 2 : 4;
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
            if (mok && kok) xa[u] = *reinterpret_cast<const uint4*>(Ab + a_offset<MODE>(a, m, kk) * ES);
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
    // two register sets, alternating: the next stage's loads go out before this stage's MFMAs
    const int stages = (a.K + U * KL - 1) / (U * KL);
    load(0, ra0, rb0);
    for (int st = 0; st < stages; st += 2) {
        if (st + 1 < stages) load(st + 1, ra1, rb1);
        products(ra0, rb0);
        if (st + 1 >= stages) break;
        if (st + 2 < stages) load(st + 2, ra0, rb0);
        products(ra1, rb1);
    }
    acc += acc2;
    // result slot r: row m0 + 4 lg + r, column n0 + li
    if (!nok) return;
    const int nq = a.H * a.d_k, nv = a.H * a.d_v;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t mr = m0 + 4 * lg + r;
        if (mr >= a.M) continue;
        const float val = acc[r];
        if constexpr (MODE == kLinProject) {
            const int64_t b = mr / a.T, t = mr % a.T;
            if (n < nq) {
                store_elem<BF16>(a.q, ((b * a.H + n / a.d_k) * a.T + t) * a.d_k + n % a.d_k, val);
            } else if (n < 2 * nq) {
                const int c = n - nq;
                store_elem<BF16>(a.k, ((b * a.H + c / a.d_k) * a.T + t) * a.d_k + c % a.d_k, val);
            } else if (n < 2 * nq + nv) {
                const int c = n - 2 * nq;
                store_elem<BF16>(a.v, ((b * a.H + c / a.d_v) * a.T + t) * a.d_v + c % a.d_v, val);
            } else {
                store_elem<BF16>(a.bl, (b * a.H + (n - 2 * nq - nv)) * a.T + t, val);
            }
        } else {
            float o = val;
            if (a.bias) o += load_elem<BF16>(a.bias, n);
            if (a.res) o += load_elem<BF16>(a.res, mr * a.N + n);
            store_elem<BF16>(a.out, mr * a.N + n, o);
        }
    }
}

template <int MODE>
static hipError_t launch_linear(const LinArgs& a, bool bf16, hipStream_t stream) {
    if (a.M == 0 || a.N == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((a.N + 31) / 32), static_cast<unsigned>((int64_t(a.M) + 31) / 32));
    if (bf16) hipLaunchKernelGGL((linear_kernel<true, MODE>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((linear_kernel<false, MODE>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
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
