// Host-side planning of the chunked forward: the chain kernel's split of D over
// waves, the prep kernel's LDS layout and the workspace layout; then dispatch to the
// (dtype, chunk) instantiation.
#include "chunked_kernels.h"

#include <map>
#include <mutex>
#include <utility>

namespace fwa {

static int align16(int x) { return (x + 15) & ~15; }

hipError_t ensure_lds_attr(const void* kernel, int bytes) {
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, int> done;   // (kernel, device) -> bytes set
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    int& cur = done[{kernel, dev}];
    if (cur >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) cur = bytes;
    return e;
}

// Workgroups of `kernel` (threads, lds bytes) that fit on the device at once, times its CUs,
// rounded down to a multiple of 8 (so a workgroup that strides through its chunks by the grid
// size stays on one XCD); at most `want` and at least 1.  Cached per (kernel, device, lds).
hipError_t resident_grid(const void* kernel, int threads, int lds, int64_t want, unsigned* grid) {
    static std::mutex mu;
    static std::map<std::pair<std::pair<const void*, int>, int>, int64_t> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int64_t cap;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find({{kernel, dev}, lds});
        if (it != cache.end()) {
            cap = it->second;
        } else {
            int per_cu = 0, cus = 0;
            if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds)) != hipSuccess) return e;
            if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
            cap = static_cast<int64_t>(per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
            if (cap >= 8) cap &= ~static_cast<int64_t>(7);
            cache[{{kernel, dev}, lds}] = cap;
        }
    }
    const int64_t g = want < cap ? want : cap;
    *grid = static_cast<unsigned>(g > 0 ? g : 1);
    return hipSuccess;
}

constexpr int kMaxLdsPrep = 160 * 1024;

bool plan_chunked(int BH, int T, int d_k, int d_v, int nu, int C, bool bf16, ChunkPlan* plan) {
    if (C != 32 && C != 64) return false;
    const int D = 2 * d_k * nu;
    if (D % 32 != 0 || d_v % 16 != 0 || D > 512) return false;
    const int es = bf16 ? 2 : 4, pair = bf16 ? 2 : 1;
    const int ND = D / 16;
    // Waves of the chain kernel (up to 8) split the d-tiles of W^T evenly, in whole bf16
    // pairs, 1-2 fp32 or 2-4 bf16 tiles per wave: the fewest such waves, but at least 4 where
    // the tiles allow, since more waves shorten the serial chain.
    const int min_dp = ND / pair < 4 ? ND / pair : 4;
    int DP = 0;
    for (int dp : {1, 2, 3, 4, 6, 8})
        if (dp >= min_dp && ND % (dp * pair) == 0 && chain_config_ok(bf16, ND / dp, dp)) {
            DP = dp;
            break;
        }
    if (DP == 0) return false;
    const int NDP = ND / DP;

    ChunkArgs a = {};
    a.krs = bf16 ? D + 8 : D + 4;
    a.lss = C + 4;
    a.pss = C + 4;
    int off = 0;
    a.l_kr = off;
    off = align16(off + C * a.krs * es);
    a.l_qr = off;                                  // Q, then A' and A'' (fp32 or bf16 hi + lo)
    a.aps = bf16 ? C + 8 : C + 4;
    const int qbytes = C * a.krs * es, abytes = 8 * C * a.aps;   // two fp32-sized copies
    off = align16(off + (qbytes > abytes ? qbytes : abytes));
    a.l_x = off;                                   // raw k, q rows; then L, P~ and Li
    const int xend = align16(off + 2 * C * d_k * es);
    a.l_ls = off;
    a.l_ps = align16(a.l_ls + C * a.lss * 4);
    a.l_li = align16(a.l_ps + C * a.pss * es);
    const int lend = align16(a.l_li + C * kLiStride * 4);
    off = xend > lend ? xend : lend;
    a.l_xv = off;
    off = align16(off + C * d_v * es);
    a.l_small = off;
    off = align16(off + 3 * C * 4);
    if (off > kMaxLdsPrep) return false;

    const int NC = (T + C - 1) / C;
    const int64_t NU = static_cast<int64_t>(BH) * NC;
    const int64_t szCD = static_cast<int64_t>(C) * D * es, szCC = static_cast<int64_t>(C) * C * es;
    const int64_t szUy = static_cast<int64_t>(C) * d_v * 4, szR = C * 4;
    const int64_t szWn = static_cast<int64_t>(D) * d_v * es, szUn = static_cast<int64_t>(C) * d_v * es;
    a.o_wy = 0;
    a.o_kt = a.o_wy + NU * szCD;
    a.o_qa = a.o_kt + NU * szCD;
    a.o_pa = a.o_qa + NU * szCD;
    a.o_uy = a.o_pa + NU * szCC;
    a.o_rk = a.o_uy + NU * szUy;
    a.o_rq = a.o_rk + NU * szR;
    a.o_wn = a.o_rq + NU * szR;
    a.o_un = a.o_wn + NU * szWn;

    a.BH = BH;
    a.T = T;
    a.NC = NC;
    a.d_k = d_k;
    a.d_v = d_v;
    a.nu = nu;
    a.D = D;
    a.DP = DP;
    a.NDP = NDP;
    plan->args = a;
    plan->C = C;
    plan->lds_prep = off;
    plan->ws_bytes = a.o_un + NU * szUn;
    // The staged chain kernel (loader waves, LDS operand ring) where its LDS fits: 4 compute
    // waves, ND / 4 d-tiles each.
    plan->staged_ndp = 0;
    plan->lds_chain = 0;
    // (fp32: the staged chain stores y through a buffer whose byte offsets must fit 31 bits)
    const bool y_fits = (static_cast<int64_t>(T) + C) * d_v * 4 < (int64_t(1) << 31);
    if (ND % kChainWaves == 0 && (bf16 || y_fits)) {
        const int sndp = ND / kChainWaves;
        const int lds = staged_chain_lds(bf16, C, sndp);
        if (lds > 0 && lds <= kMaxLdsPrep) {
            plan->staged_ndp = sndp;
            plan->lds_chain = lds;
        }
    }
    // the staged chain kernel takes fp32 operands in the split bf16 hi + lo format
    plan->args.split = !bf16 && plan->staged_ndp > 0;
    // bf16 at chunk 64 runs the direct variant (y through a buffer whose byte offsets must fit
    // 31 bits); it and the fp32 staged kernel form y in the chain, so the workspace ends
    // before the chunk-start memories and U that the output kernel would read
    const bool ybf_fits = (static_cast<int64_t>(T) + C) * d_v * 2 < (int64_t(1) << 31);
    plan->direct = bf16 && C == 64 && plan->staged_ndp > 0 && ybf_fits;
    plan->chain_outputs = plan->direct || (!bf16 && plan->staged_ndp > 0);
    if (plan->chain_outputs) plan->ws_bytes = a.o_wn;
    return true;
}

hipError_t launch_chunked(const ChunkPlan& plan_in, const void* q, const void* k, const void* v,
                          const void* bl, const float* W0, void* y, float* Wf, char* ws,
                          bool bf16, hipStream_t stream) {
    ChunkPlan p = plan_in;
    ChunkArgs& a = p.args;
    a.q = q;
    a.k = k;
    a.v = v;
    a.bl = bl;
    a.W0 = W0;
    a.y = y;
    a.Wf = Wf;
    a.ws = ws;
    switch (p.C) {
        case 32: return bf16 ? launch_chunked_bf16_c32(p, stream) : launch_chunked_f32_c32(p, stream);
        case 64: return bf16 ? launch_chunked_bf16_c64(p, stream) : launch_chunked_f32_c64(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fwa
