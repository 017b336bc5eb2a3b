// Single-token decode step of the fast-weight delta rule, W updated in place.
//
// Per (b, h), with f = phi(k), g = phi(q), beta = sigmoid(beta_logit) ("Fast Weights
// Transformer" guide, xdnf.cn/news/308600, sections "FastWeightsAttention / update formula"
// and "token_wise variant"):
//     v_bar = W f;  W <- W + beta (v - v_bar) f^T;  y = W g  (read after the write).
// Row r of W evolves independently: with u_r = beta (v_r - W_r.f),
//     y_r = (W_r + u_r f).g = W_r.g + u_r (f.g),
// so one pass over the rows reads W once (two dot products per row against the old row) and
// writes it once (W_r + u_r f).  The step is bound by HBM traffic on W (8 * d_v * D bytes per
// (b, h)), the decode regime the "Transformer" page (wineandchord.com), section "Complexity",
// describes.
//
// Mapping: one workgroup (4 waves) per (b, h), or, when there are few (b, h) slices, a power
// of two of workgroups per (b, h) that split its rows (each recomputes f and g).  A row of D
// floats is spread over LR lanes of one wave, CPL float4 columns per lane (D = 4 * LR * CPL,
// both compile-time), so every row dot product is a
// lane-shuffle reduction inside a wave and each lane issues 16-byte loads and stores.  Each
// lane computes the f and g entries of its own columns from 4-wide loads of k and q and a
// per-wave LDS copy of relu([k,-k]) and relu([q,-q]), and the group reduces the DPFP sums, so
// the kernel needs no barrier; every load (W rows, v, beta, k, q) is in flight before the
// first arithmetic.
#include "fwa_common.h"
#include "fwa_internal.h"

namespace fwa {

// Sum of x over each aligned group of LR lanes (LR in {8, 16, 32, 64}), in every lane of the
// group: DPP inside 16-lane rows (quad permutes, then row rotations), one cross-row permute per
// doubling beyond 16.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int LR>
__device__ __forceinline__ float lane_group_sum(float x) {
    x = dpp_add<0xB1>(x);                    // quad_perm [1,0,3,2]: lane ^ 1
    x = dpp_add<0x4E>(x);                    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (LR == 8) return x + __shfl_xor(x, 4, 8);
    x = dpp_add<0x124>(x);                   // row_ror:4
    x = dpp_add<0x128>(x);                   // row_ror:8
    if constexpr (LR >= 32) x += __shfl_xor(x, 16);
    if constexpr (LR == 64) x += __shfl_xor(x, 32);
    return x;
}

// Elements i .. i+3 of an fp32 or bf16 vector (i a multiple of 4, the base 16-byte aligned).
template <bool BF16>
__device__ __forceinline__ void load4(const void* p, int64_t i, float (&x)[4]) {
    if constexpr (BF16) {
        const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const u16*>(p) + i);
        x[0] = __uint_as_float(r.x << 16);
        x[1] = __uint_as_float(r.x & 0xffff0000u);
        x[2] = __uint_as_float(r.y << 16);
        x[3] = __uint_as_float(r.y & 0xffff0000u);
    } else {
        const float4 r = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
        x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w;
    }
}

template <bool BF16, int CPL, int LR>
__global__ __launch_bounds__(256) void delta_step_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ bl, float* __restrict__ W, void* __restrict__ y, int d_k, int d_v,
    int nu, int rsplit) {
    constexpr int RB = (CPL == 1) ? 8 : (CPL == 2 ? 4 : 2);  // row rounds per batch
    const int64_t s = blockIdx.x / rsplit;                    // (b, h)
    const int part = blockIdx.x % rsplit;                     // its share of the row rounds
    const int two_dk = 2 * d_k;                // a power of two (d_k in {16, 32, 64, 128})
    const int sh = __builtin_ctz(two_dk);
    const int D = two_dk * nu;
    float* Ws = W + s * static_cast<int64_t>(d_v) * D;
    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
    constexpr int rpw = 64 / LR;       // rows per wave per round
    constexpr int RPR = 4 * rpw;       // rows per workgroup round
    const int rr = wv * rpw + l / LR;  // this lane's row inside a round
    const int c = l % LR;
    const int all_rounds = (d_v + RPR - 1) / RPR;
    const int rpp = (all_rounds + rsplit - 1) / rsplit;       // rounds per workgroup
    const int rbase = part * rpp;                             // first round of this workgroup
    const int rounds = max(0, min(all_rounds - rbase, rpp));
    const int64_t vb = s * d_v;

    // Every load is issued up front: the first batch of W rows, then this lane's v entries,
    // beta's logit and the k and q entries its columns need.
    float4 wrow[RB][CPL];
    float vrow[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        const int row = rr + RPR * (rbase + b);
        const int rs = b < rounds && row < d_v ? row : 0;   // a row that exists; not stored
#pragma unroll
        for (int m = 0; m < CPL; ++m)
            wrow[b][m] = *reinterpret_cast<const float4*>(Ws + static_cast<int64_t>(rs) * D + 4 * (c + LR * m));
        vrow[b] = load_elem<BF16>(v, vb + rs);
    }
    const float blog = load_elem<BF16>(bl, s);

    // f and g on this lane's 4*CPL columns.  Position d lies in the block of shift
    // i = d / (2 d_k) + 1 at j = d mod 2 d_k; its factors are x[j] and x[(j - i) mod 2 d_k] with
    // x = relu([k, -k]).  A lane's four columns d0 .. d0+3 share i and one half of x, so their
    // first factors come from one 4-wide load of k.  The rolled factors come from a copy of x
    // in LDS, one per wave: the first 2 d_k / 4 lanes of the wave hold x's blocks in their
    // first column group (2 d_k / 4 <= LR always, since CPL <= nu), and write them there.
    // Two vector loads per column group for k and q instead of sixteen scalar ones.
    __shared__ __attribute__((aligned(16))) float xs_all[4][2][256];   // 2 d_k <= 256
    float* xk = xs_all[wv][0];
    float* xq = xs_all[wv][1];
    const int64_t kb = s * d_k;
    float xa_k[CPL][4], xa_q[CPL][4];
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int j0 = (4 * (c + LR * m)) & (two_dk - 1);
        const float sa = j0 < d_k ? 1.0f : -1.0f;
        float kv[4], qv[4];
        load4<BF16>(k, kb + (j0 & (d_k - 1)), kv);
        load4<BF16>(q, kb + (j0 & (d_k - 1)), qv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xa_k[m][e] = relu(sa * kv[e]);
            xa_q[m][e] = relu(sa * qv[e]);
        }
    }
    if (l < two_dk / 4) {
        *reinterpret_cast<float4*>(xk + 4 * l) = make_float4(xa_k[0][0], xa_k[0][1], xa_k[0][2], xa_k[0][3]);
        *reinterpret_cast<float4*>(xq + 4 * l) = make_float4(xa_q[0][0], xa_q[0][1], xa_q[0][2], xa_q[0][3]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own LDS writes are done
    float f[CPL * 4], g[CPL * 4];
    float Sf = 0.0f, Sg = 0.0f;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int d0 = 4 * (c + LR * m);
        const int i = (d0 >> sh) + 1;
        const int ws = ((d0 & (two_dk - 1)) - i) & (two_dk - 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int jr = (ws + e) & (two_dk - 1);
            const float fk = xa_k[m][e] * xk[jr];
            const float fq = xa_q[m][e] * xq[jr];
            f[m * 4 + e] = fk;
            g[m * 4 + e] = fq;
            Sf += fk;
            Sg += fq;
        }
    }
    Sf = lane_group_sum<LR>(Sf);
    Sg = lane_group_sum<LR>(Sg);
    const float rf = 1.0f / (Sf + kDpfpEps), rg = 1.0f / (Sg + kDpfpEps);
    float fg = 0.0f;
#pragma unroll
    for (int e = 0; e < CPL * 4; ++e) {
        f[e] *= rf;
        g[e] *= rg;
        fg += f[e] * g[e];
    }
    fg = lane_group_sum<LR>(fg);
    const float beta = sigmoid_stable(blog);

    for (int r0 = 0; r0 < rounds; r0 += RB) {
        if (r0 > 0) {
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const int row = rr + RPR * (rbase + r0 + b);
                const int rs = r0 + b < rounds && row < d_v ? row : 0;
#pragma unroll
                for (int m = 0; m < CPL; ++m)
                    wrow[b][m] = *reinterpret_cast<const float4*>(Ws + static_cast<int64_t>(rs) * D + 4 * (c + LR * m));
                vrow[b] = load_elem<BF16>(v, vb + rs);
            }
        }
        float dk[RB], dq[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            dk[b] = dq[b] = 0.0f;
#pragma unroll
            for (int m = 0; m < CPL; ++m) {
                const float4 w4 = wrow[b][m];
                dk[b] += w4.x * f[m * 4 + 0] + w4.y * f[m * 4 + 1] + w4.z * f[m * 4 + 2] +
                         w4.w * f[m * 4 + 3];
                dq[b] += w4.x * g[m * 4 + 0] + w4.y * g[m * 4 + 1] + w4.z * g[m * 4 + 2] +
                         w4.w * g[m * 4 + 3];
            }
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            dk[b] = lane_group_sum<LR>(dk[b]);
            dq[b] = lane_group_sum<LR>(dq[b]);
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const int row = rr + RPR * (rbase + r0 + b);
            if (r0 + b < rounds && row < d_v) {
                const float u = beta * (vrow[b] - dk[b]);
                if (c == 0) store_elem<BF16>(y, vb + row, dq[b] + u * fg);
#pragma unroll
                for (int m = 0; m < CPL; ++m) {
                    float4 w4 = wrow[b][m];
                    w4.x += u * f[m * 4 + 0];
                    w4.y += u * f[m * 4 + 1];
                    w4.z += u * f[m * 4 + 2];
                    w4.w += u * f[m * 4 + 3];
                    *reinterpret_cast<float4*>(Ws + static_cast<int64_t>(row) * D +
                                               4 * (c + LR * m)) = w4;
                }
            }
        }
    }
}

// Columns per lane for a row of D floats: the smallest CPL in 1..4 with D / (4 CPL) a power of
// two in [8, 64].  Returns 0 when none exists (shape not implemented).
int step_cpl_for(int D, int* LR_out) {
    for (int cpl = 1; cpl <= 4; ++cpl) {
        if (D % (4 * cpl)) continue;
        const int lr = D / (4 * cpl);
        if (lr == 8 || lr == 16 || lr == 32 || lr == 64) {
            *LR_out = lr;
            return cpl;
        }
    }
    return 0;
}

hipError_t launch_delta_step(const void* q, const void* k, const void* v, const void* bl,
                             float* W, void* y, int64_t BH, int d_k, int d_v, int nu, bool bf16,
                             hipStream_t stream) {
    const int D = 2 * d_k * nu;
    int LR = 0;
    const int cpl = step_cpl_for(D, &LR);
    if (cpl == 0) return hipErrorInvalidValue;
    // Few (b, h) slices: split each slice's rows over several workgroups (up to one row round
    // each) so that at least ~256 workgroups share the latency-bound step.
    const int RPR = 4 * (64 / LR), all_rounds = (d_v + RPR - 1) / RPR;
    int rsplit = 1;
    while (rsplit < all_rounds && BH * rsplit < 256) rsplit *= 2;
    if (rsplit > all_rounds) rsplit = all_rounds;
    const dim3 grid(static_cast<unsigned>(BH * rsplit)), block(256);
#define FWA_STEP_CASE(BF, C, L)                                                              \
    if (bf16 == BF && cpl == C && LR == L) {                                                 \
        hipLaunchKernelGGL((delta_step_kernel<BF, C, L>), grid, block, 0, stream, q, k, v, bl, \
                           W, y, d_k, d_v, nu, rsplit);                                      \
        return hipGetLastError();                                                            \
    }
#define FWA_STEP_LR(BF, C) \
    FWA_STEP_CASE(BF, C, 8) FWA_STEP_CASE(BF, C, 16) FWA_STEP_CASE(BF, C, 32) FWA_STEP_CASE(BF, C, 64)
    FWA_STEP_LR(false, 1) FWA_STEP_LR(false, 2) FWA_STEP_LR(false, 3) FWA_STEP_LR(false, 4)
    FWA_STEP_LR(true, 1) FWA_STEP_LR(true, 2) FWA_STEP_LR(true, 3) FWA_STEP_LR(true, 4)
#undef FWA_STEP_LR
#undef FWA_STEP_CASE
    return hipErrorInvalidValue;
}

}  // namespace fwa
