// fp32 chunk helpers shared by the backward (backward.hip) and the sum-update forward
// (sum_forward.hip): chunks of kBC = 32 rows and normalised DPFP tiles built in LDS.
#pragma once

#include "fwa_common.h"

namespace fwa {

constexpr int kBC = 32;              // rows per chunk

// x rows for DPFP: xs[c][j] = relu(r_c[j]), xs[c][d_k + j] = relu(-r_c[j]) for the `rows` valid
// rows c of the chunk starting at t0 of the slice at element row `base` (zeros beyond), from
// [.., T, d_k] input of the caller's dtype.
template <bool BF16>
__device__ __forceinline__ void load_relu_rows(const void* src, float* xs, int64_t base, int rows,
                                               int t0, int d_k, int tid, int nthr) {
    // d_k is a power of two up to 64 and nthr >= 256: at most 8 elements per thread, all loads
    // issued before the first store
    const int two = 2 * d_k, lg = __builtin_ctz(d_k);
    constexpr int kMax = kBC * 64 / 256;
    float xv[kMax];
#pragma unroll
    for (int m = 0; m < kMax; ++m) {
        const int i = tid + nthr * m, c = i >> lg, j = i & (d_k - 1);
        xv[m] = (i < kBC * d_k && c < rows) ? load_elem<BF16>(src, (base + t0 + c) * d_k + j) : 0.0f;
    }
#pragma unroll
    for (int m = 0; m < kMax; ++m) {
        const int i = tid + nthr * m, c = i >> lg, j = i & (d_k - 1);
        if (i < kBC * d_k) {
            xs[c * two + j] = relu(xv[m]);
            xs[c * two + d_k + j] = relu(-xv[m]);
        }
    }
}

// Row stride (floats) of the [C][D] feature tiles that the chunk-parallel kernels keep in LDS:
// D + 8 puts rows c and c + 1 eight banks apart, so reads where the lanes of a wave span 8 rows
// (and 8 consecutive columns) hit 64 distinct banks.
__host__ __device__ inline int tile_stride(int D) { return D + 8; }

// Normalised DPFP features of the kBC rows of two x tiles (xa, xb: [C][2 d_k]) into Fa, Fb
// ([C][SD], SD = tile_stride(D)): block i - 1 holds x[j] x[(j - i) mod 2 d_k] ("Fast Weights
// Transformer" guide, section "DPFP"), divided by the row's sum + 1e-6 (section "DPFP /
// normalisation").  Thread t owns row t / 8 of both tiles and every 8th column from t % 8, so
// each row sum reduces over 8 adjacent lanes.  Needs 256 threads; starts with a barrier (the x
// tiles must be written before the call) and ends with one.
__device__ __forceinline__ void dpfp_tiles(const float* xa, const float* xb, float* Fa, float* Fb,
                                           int D, int d_k, int tid) {
    const int two = 2 * d_k, SD = tile_stride(D);
    const int c = tid >> 3, s0 = tid & 7;
    __syncthreads();
    const float* xra = xa + c * two;
    const float* xrb = xb + c * two;
    float sa = 0.0f, sb = 0.0f;
    // position j and shift i of column p = (i - 1) 2 d_k + j, advanced without divisions
    int i = 1, j = s0;
    for (int p = s0; p < D; p += 8) {
        int src = j - i;
        src += (src < 0) ? two : 0;
        const float ra = xra[j] * xra[src], rb = xrb[j] * xrb[src];
        Fa[c * SD + p] = ra;
        Fb[c * SD + p] = rb;
        sa += ra;
        sb += rb;
        j += 8;
        if (j >= two) {
            j -= two;
            ++i;
        }
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        sa += __shfl_xor(sa, m);
        sb += __shfl_xor(sb, m);
    }
    const float da = sa + kDpfpEps, db = sb + kDpfpEps;
    for (int p = s0; p < D; p += 8) {                 // this thread's own entries
        Fa[c * SD + p] = Fa[c * SD + p] / da;
        Fb[c * SD + p] = Fb[c * SD + p] / db;
    }
    __syncthreads();
}

}  // namespace fwa
