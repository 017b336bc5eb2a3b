// fp32 chunk helpers shared by the backward (backward.hip) and the sum-update forward
// (sum_forward.hip): chunks of kBC = 32 rows, normalised DPFP tiles built in LDS, and the wave
// reductions of the one-wave-per-memory-row serial passes.
#pragma once

#include "fwa_common.h"

namespace fwa {

constexpr int kBC = 32;              // rows per chunk
constexpr int kRowWaves = 8;         // memory rows per serial workgroup (one wave each)

// x rows for DPFP: xs[c][j] = relu(r_c[j]), xs[c][d_k + j] = relu(-r_c[j]) for the `rows` valid
// rows c of the chunk starting at t0 of the slice at element row `base` (zeros beyond), from
// [.., T, d_k] input of the caller's dtype.
template <bool BF16>
__device__ __forceinline__ void load_relu_rows(const void* src, float* xs, int64_t base, int rows,
                                               int t0, int d_k, int tid, int nthr) {
    const int two = 2 * d_k;
    for (int i = tid; i < kBC * d_k; i += nthr) {
        const int c = i / d_k, j = i % d_k;
        const float x = c < rows ? load_elem<BF16>(src, (base + t0 + c) * d_k + j) : 0.0f;
        xs[c * two + j] = relu(x);
        xs[c * two + d_k + j] = relu(-x);
    }
}

// Normalised DPFP features of the kBC rows of two x tiles (xa, xb: [C][2 d_k]) into Fa, Fb
// ([C][D]): block i - 1 holds x[j] x[(j - i) mod 2 d_k] ("Fast Weights Transformer" guide,
// section "DPFP"), divided by the row's sum + 1e-6 (section "DPFP / normalisation").  `rs`
// holds 2 C floats of scratch (the row sums + eps on return).  Starts and ends with a barrier
// (all threads of the workgroup must call it); expects the x tiles written before the call.
__device__ __forceinline__ void dpfp_tiles(const float* xa, const float* xb, float* Fa, float* Fb,
                                           float* rs, int D, int d_k, int tid, int nthr) {
    const int two = 2 * d_k;
    __syncthreads();
    for (int e = tid; e < kBC * D; e += nthr) {
        const int c = e / D, p = e % D;
        const int i = p / two + 1, j = p % two;
        int src = j - i;
        src += (src < 0) ? two : 0;
        Fa[e] = xa[c * two + j] * xa[c * two + src];
        Fb[e] = xb[c * two + j] * xb[c * two + src];
    }
    __syncthreads();
    if (tid < 2 * kBC) {
        const float* row = (tid < kBC ? Fa : Fb) + (tid % kBC) * D;
        float s = 0.0f;
        for (int p = 0; p < D; ++p) s += row[p];
        rs[tid] = s + kDpfpEps;
    }
    __syncthreads();
    for (int e = tid; e < kBC * D; e += nthr) {
        const int c = e / D;
        Fa[e] = Fa[e] / rs[c];
        Fb[e] = Fb[e] / rs[kBC + c];
    }
    __syncthreads();
}

// Reduce-scatter of 32 per-lane partial sums over the wave: on return, lane l holds the sum
// over all 64 lanes of entry l >> 1.
__device__ __forceinline__ float wave_reduce_scatter32(float (&v)[kBC]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int half = 16, mask = 32; half >= 1; half >>= 1, mask >>= 1) {
        const bool up = (lane & mask) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float send = up ? v[i] : v[i + half];
            const float keep = up ? v[i + half] : v[i];
            v[i] = keep + __shfl_xor(send, mask);
        }
    }
    return v[0] + __shfl_xor(v[0], 1);
}

// Value of `x` held by lane `l` (a wave-uniform index), in every lane.
__device__ __forceinline__ float lane_value(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Stages `n` floats (a multiple of 4, both pointers 16-byte aligned) from global to LDS with
// all threads of the workgroup.
__device__ __forceinline__ void stage(float* dst, const float* src, int n, int tid, int nthr) {
    for (int i = 4 * tid; i < n; i += 4 * nthr)
        *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(src + i);
}

}  // namespace fwa
