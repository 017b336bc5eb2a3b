// fp32 chunk helpers shared by the backward (backward.hip) and the sum-update forward
// (sum_forward.hip): chunks of kBC = 32 rows and normalised DPFP tiles built in LDS.
#pragma once

#include "fwa_common.h"

#include <type_traits>

namespace fwa {

constexpr int kBC = 32;              // rows per chunk

// One chunk's inputs into LDS, every load issued before the first store (one memory round trip):
// the x rows for DPFP, xk[c][j] = relu(k_c[j]), xk[c][d_k + j] = relu(-k_c[j]) (the same for q),
// and the v rows Vs[c][r], for the `rows` valid rows c of the chunk starting at t0 of the slice
// at element row `base` (zeros beyond), from [.., T, d_k] / [.., T, d_v] input of the caller's
// dtype.  Loads use clamped indices and are selected when stored, so none sits in a branch.
// d_k is a power of two up to 64 and d_v <= MAXDV (a multiple of 64); NTHR threads.
template <bool BF16, int NTHR, int MAXDV>
__device__ __forceinline__ void load_chunk_inputs(const void* k, const void* q, const void* v,
                                                  float* xk, float* xq, float* Vs, int64_t base,
                                                  int rows, int t0, int d_k, int d_v, int tid) {
    using ET = std::conditional_t<BF16, u16, float>;
    const ET* kp = static_cast<const ET*>(k);
    const ET* qp = static_cast<const ET*>(q);
    const ET* vp = static_cast<const ET*>(v);
    const int two = 2 * d_k, lg = __builtin_ctz(d_k);
    constexpr int kMax = kBC * 64 / NTHR;            // k / q elements per thread
    constexpr int kRowsPerPass = NTHR / 64;          // v rows per pass (one per wave)
    constexpr int kVr = kBC / kRowsPerPass, kVh = MAXDV / 64;
    const int wv = tid >> 6, lane = tid & 63;
    ET kr[kMax], qr[kMax], vr[kVr][kVh];
#pragma unroll
    for (int m = 0; m < kMax; ++m) {
        const int i = min(tid + NTHR * m, kBC * d_k - 1), c = min(i >> lg, rows - 1), j = i & (d_k - 1);
        kr[m] = kp[(base + t0 + c) * d_k + j];
        qr[m] = qp[(base + t0 + c) * d_k + j];
    }
#pragma unroll
    for (int m = 0; m < kVr; ++m)
#pragma unroll
        for (int h = 0; h < kVh; ++h) {
            const int c = min(wv + kRowsPerPass * m, rows - 1), r = min(lane + 64 * h, d_v - 1);
            vr[m][h] = vp[(base + t0 + c) * d_v + r];
        }
#pragma unroll
    for (int m = 0; m < kMax; ++m) {
        const int i = tid + NTHR * m, c = i >> lg, j = i & (d_k - 1);
        if (i < kBC * d_k) {
            const float kv = c < rows ? to_f32(kr[m]) : 0.0f, qv = c < rows ? to_f32(qr[m]) : 0.0f;
            xk[c * two + j] = relu(kv);
            xk[c * two + d_k + j] = relu(-kv);
            xq[c * two + j] = relu(qv);
            xq[c * two + d_k + j] = relu(-qv);
        }
    }
#pragma unroll
    for (int m = 0; m < kVr; ++m)
#pragma unroll
        for (int h = 0; h < kVh; ++h) {
            const int c = wv + kRowsPerPass * m, r = lane + 64 * h;
            if (r < d_v) Vs[c * d_v + r] = c < rows ? to_f32(vr[m][h]) : 0.0f;
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
    sa = sum8_dpp(sa);
    sb = sum8_dpp(sb);
    const float ia = 1.0f / (sa + kDpfpEps), ib = 1.0f / (sb + kDpfpEps);
    for (int p = s0; p < D; p += 8) {                 // this thread's own entries
        Fa[c * SD + p] *= ia;
        Fb[c * SD + p] *= ib;
    }
    __syncthreads();
}

}  // namespace fwa
