// Host-side planning of the chunked forward: the d_v split across workgroups, the waves'
// share of the memory, and the LDS layout; then dispatch to the (dtype, chunk) instantiation.
#include "forward_kernel.h"

namespace fwa {

static int align16(int x) { return (x + 15) & ~15; }


constexpr int kMaxLds = 160 * 1024;

// Chooses the d_v split and the LDS layout; returns false when the shape does not fit.
bool plan_forward(int BH, int d_k, int d_v, int nu, int C, bool bf16, FwdPlan* plan) {
    const int D = 2 * d_k * nu;
    if (D % 32 != 0 || d_v % 16 != 0 || D > 512) return false;
    const int ND = D / 16, NVT_total = d_v / 16;
    const int pair = bf16 ? 2 : 1;
    const int es = bf16 ? 2 : 4;
    // Candidate splits: fewest workgroups per (b, h) that still give >= 256 workgroups.
    int R0 = NVT_total > 4 ? NVT_total / 4 : 1;
    if (NVT_total % R0) return false;
    for (int R = R0; R <= NVT_total; R *= 2) {
        if (NVT_total % R) continue;
        const int NVT = NVT_total / R;
        if (NVT > 4) continue;
        const bool enough = static_cast<int64_t>(BH) * R >= 256 || R == NVT_total;
        if (!enough) continue;
        for (int DP = 4 / NVT; DP >= 1; DP /= 2) {
            if (ND % (DP * pair)) continue;
            const int NDP = ND / DP;
            if (NDP > 32) continue;
            FwdArgs fa = {};
            fa.krs = bf16 ? D + 8 : D + 4;
            fa.lss = C + 4;
            fa.pss = C + 4;
            int off = 0;
            fa.off_kr = off;                      // K lives through the memory update
            off = align16(off + C * fa.krs * es);
            const int ustart = off;               // Q, then (after it dies) the phase-C/D buffers
            fa.off_qr = ustart;
            const int uend1 = align16(fa.off_qr + C * fa.krs * es);
            fa.off_ls = ustart;
            fa.off_ps = align16(fa.off_ls + C * fa.lss * 4);
            fa.off_li = align16(fa.off_ps + C * fa.pss * es);
            fa.off_red = align16(fa.off_li + C * kLiStride * 4);
            const int uend2 = align16(fa.off_red + (DP > 1 ? 4 * 2 * 16 * (C + 4) * 4 : 0));
            off = uend1 > uend2 ? uend1 : uend2;
            fa.off_xs = off;                      // raw k and q rows of the chunk
            off = align16(off + (2 * C * d_k + C * 16 * NVT) * es);
            fa.off_small = off;
            off = align16(off + 3 * C * 4);
            if (off > kMaxLds) continue;
            fa.R = R;
            fa.NVT = NVT;
            fa.DP = DP;
            fa.NDP = NDP;
            plan->R = R;
            plan->NVT = NVT;
            plan->DP = DP;
            plan->NDP = NDP;
            plan->NDPM = fwd_ndpm_bucket(NDP, C);
            if (plan->NDPM == 0) continue;
            plan->args = fa;
            plan->lds_bytes = off;
            return true;
        }
    }
    return false;
}


hipError_t launch_delta_forward(const FwdPlan& plan_in, const void* q, const void* k,
                                const void* v, const void* bl, const float* W0, void* y,
                                float* Wf, int BH, int H, int T, int d_k, int d_v, int nu, int C,
                                bool bf16, hipStream_t stream) {
    FwdPlan p = plan_in;
    FwdArgs& a = p.args;
    a.q = q; a.k = k; a.v = v; a.bl = bl; a.W0 = W0; a.y = y; a.Wf = Wf;
    a.BH = BH; a.H = H; a.T = T; a.d_k = d_k; a.d_v = d_v; a.nu = nu;
    switch (C) {
        case 16: return bf16 ? launch_fwd_bf16_c16(p, BH, stream) : launch_fwd_f32_c16(p, BH, stream);
        case 32: return bf16 ? launch_fwd_bf16_c32(p, BH, stream) : launch_fwd_f32_c32(p, BH, stream);
        case 64: return bf16 ? launch_fwd_bf16_c64(p, BH, stream) : launch_fwd_f32_c64(p, BH, stream);
        case 128: return bf16 ? launch_fwd_bf16_c128(p, BH, stream) : launch_fwd_f32_c128(p, BH, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fwa
