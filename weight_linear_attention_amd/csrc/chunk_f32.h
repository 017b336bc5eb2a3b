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

// Register staging of a [C][D] fp32 tile from global memory (row stride D) into LDS with the
// padded row stride 64 * NPL by the 512 threads of a serial workgroup.  The pad columns are
// zeroed once (zero_tile_pads) and never written again, so the one-wave-per-row passes read
// every lane's NPL columns unconditionally (with zero memory entries in the pad).
// prefetch_tile() issues the loads of up to NPL float4 per thread (NPL >= C * D / 2048) and
// commit_tile() writes them at offsets tile_slots() computed once per kernel.  Issued before a
// chunk's compute phase for the next chunk, the loads overlap that phase.
template <int NPL>
__device__ __forceinline__ void tile_slots(int (&slot)[NPL], int D, int tid) {
    const int n = kBC * D;
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
        const int i = 4 * (tid + 512 * m);
        slot[m] = i < n ? (i / D) * (64 * NPL) + i % D : -1;
    }
}

template <int NPL>
__device__ __forceinline__ void zero_tile_pads(float* dst, int D, int tid) {
    const int SDP = 64 * NPL;
    for (int e = tid; e < kBC * (SDP - D); e += 512) {
        const int c = e / (SDP - D), p = D + e % (SDP - D);
        dst[c * SDP + p] = 0.0f;
    }
}

template <int NPL>
__device__ __forceinline__ void prefetch_tile(f32x4 (&r)[NPL], const float* src, int n, int tid) {
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
        // an index past the tile loads its last 16 bytes again (unconditional loads keep r in
        // registers); commit_tile skips those
        const int i = min(4 * (tid + 512 * m), n - 4);
        r[m] = *reinterpret_cast<const f32x4*>(src + i);
    }
}

template <int NPL>
__device__ __forceinline__ void commit_tile(float* dst, const f32x4 (&r)[NPL], const int (&slot)[NPL]) {
#pragma unroll
    for (int m = 0; m < NPL; ++m)
        if (slot[m] >= 0) *reinterpret_cast<f32x4*>(dst + slot[m]) = r[m];
}

// One halving step of the reduce-scatter below: lanes whose bit 2*HALF is set keep entries
// HALF .. 2*HALF - 1 (moved to 0 .. HALF - 1), the others keep 0 .. HALF - 1, each adding the
// partner's copy of what it keeps.  HALF is a template argument so every index is static.
template <int HALF>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[kBC], int lane) {
    const bool up = (lane & (2 * HALF)) != 0;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
        const float send = up ? v[i] : v[i + HALF];
        const float keep = up ? v[i + HALF] : v[i];
        v[i] = keep + __shfl_xor(send, 2 * HALF);
    }
}

// Reduce-scatter of 32 per-lane partial sums over the wave: on return, lane l holds the sum
// over all 64 lanes of entry l >> 1.
__device__ __forceinline__ float wave_reduce_scatter32(float (&v)[kBC]) {
    const int lane = threadIdx.x & 63;
    reduce_scatter_step<16>(v, lane);
    reduce_scatter_step<8>(v, lane);
    reduce_scatter_step<4>(v, lane);
    reduce_scatter_step<2>(v, lane);
    reduce_scatter_step<1>(v, lane);
    return v[0] + __shfl_xor(v[0], 1);
}

// Value of `x` held by lane `l` (a wave-uniform index), in every lane.
__device__ __forceinline__ float lane_value(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

}  // namespace fwa
