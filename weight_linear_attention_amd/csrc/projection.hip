// The linear maps around the layer ("Fast Weights Transformer" guide, xdnf.cn/news/308600,
// section "FastWeightsAttention / module structure and source walkthrough"): the bias-free
// query, key, value and interpolation-weight projections of x, written straight into the
// head-split [B, H, T, d] layout the layer reads, and the output map (with bias) of the heads'
// concatenated outputs, read straight from [B, H, T, d_v] and added to a residual.
//
// Both are C[M x N] = A[M x K] B^T with B an [N x K] weight (out = x W^T).  One workgroup of 4
// waves computes a 64 x 64 tile of C; each wave a 32 x 32 block as 2 x 2 MFMA tiles of 16 x 16.
// bf16 operands use v_mfma_f32_16x16x32_bf16; fp32 operands v_mfma_f32_16x16x4f32 (four per
// 16-deep k block).  In both, lane l of a tile supplies row l % 16 of A and of B^T over a run of
// consecutive k (8 bf16 or 4 fp32: one 16-byte load each, contiguous in x, y and the weights).
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
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t m0 = int64_t(blockIdx.y) * 64 + (wave >> 1) * 32;
    const int n0 = blockIdx.x * 64 + (wave & 1) * 32;
    const int li = lane & 15, lg = lane >> 4;
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = zero4();
    if constexpr (BF16) {
        const u16* Ab = static_cast<const u16*>(a.A);
        const u16* Bb = static_cast<const u16*>(a.Bw);
        for (int k0 = 0; k0 < a.K; k0 += 32) {
            const int kk = k0 + 8 * lg;
            bf16x8 af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int64_t m = m0 + 16 * i + li;
                af[i] = bf16x8{};
                if (m < a.M && kk < a.K)
                    af[i] = *reinterpret_cast<const bf16x8*>(Ab + a_offset<MODE>(a, m, kk));
                const int n = n0 + 16 * i + li;
                bf[i] = bf16x8{};
                if (n < a.N && kk < a.K)
                    bf[i] = *reinterpret_cast<const bf16x8*>(Bb + int64_t(n) * a.K + kk);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16_k32(af[i], bf[j], acc[i][j]);
        }
    } else {
        const float* Af = static_cast<const float*>(a.A);
        const float* Bf = static_cast<const float*>(a.Bw);
        for (int k0 = 0; k0 < a.K; k0 += 16) {
            const int kk = k0 + 4 * lg;
            float4 af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int64_t m = m0 + 16 * i + li;
                af[i] = float4{0.0f, 0.0f, 0.0f, 0.0f};
                if (m < a.M && kk < a.K)
                    af[i] = *reinterpret_cast<const float4*>(Af + a_offset<MODE>(a, m, kk));
                const int n = n0 + 16 * i + li;
                bf[i] = float4{0.0f, 0.0f, 0.0f, 0.0f};
                if (n < a.N && kk < a.K)
                    bf[i] = *reinterpret_cast<const float4*>(Bf + int64_t(n) * a.K + kk);
            }
            // sub-step s takes k = k0 + 4 g + s from lane group g: the same k for A and B
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[i][j] = mfma_f32_k4(af[i].x, bf[j].x, acc[i][j]);
                    acc[i][j] = mfma_f32_k4(af[i].y, bf[j].y, acc[i][j]);
                    acc[i][j] = mfma_f32_k4(af[i].z, bf[j].z, acc[i][j]);
                    acc[i][j] = mfma_f32_k4(af[i].w, bf[j].w, acc[i][j]);
                }
        }
    }
    // result element r of tile (i, j): row m0 + 16 i + 4 lg + r, column n0 + 16 j + li
    const int nq = a.H * a.d_k, nv = a.H * a.d_v;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 16 * j + li;
            if (n >= a.N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + 16 * i + 4 * lg + r;
                if (m >= a.M) continue;
                const float val = acc[i][j][r];
                if constexpr (MODE == kLinProject) {
                    const int64_t b = m / a.T, t = m % a.T;
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
                    if (a.res) o += load_elem<BF16>(a.res, m * a.N + n);
                    store_elem<BF16>(a.out, m * a.N + n, o);
                }
            }
        }
}

template <int MODE>
static hipError_t launch_linear(const LinArgs& a, bool bf16, hipStream_t stream) {
    if (a.M == 0 || a.N == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((a.N + 63) / 64), static_cast<unsigned>((int64_t(a.M) + 63) / 64));
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
