// Shift-sliced streaming forward (bf16, d_k = 64): host planning of the LDS and workspace
// layouts, and the launches of the sliced prep kernel and the chunk-128 serial kernel.
#include "stream_sliced.h"

namespace fwa {

static int align16v(int x) { return (x + 15) & ~15; }

constexpr int kMaxLdsSliced = 160 * 1024;

// LDS layout of the sliced prep kernel for chunk C; returns its bytes (0 if it does not fit).
int plan_prep_sliced(int C, ChunkArgs* a) {
    a->ss = kSliceCols + 8;                           // 272-byte rows: 16-byte aligned, no bank clash
    a->lss = C + 4;
    a->pss = C + 4;
    a->aps = C + 8;
    // phase 1: raw k, q rows, then one K and one Q slice
    a->l_x = 0;
    a->l_kr = align16v(2 * C * (C == 64 ? kRawRow : kSliceDk) * 2);   // raw rows (padded at 64)
    a->l_qr = align16v(a->l_kr + C * a->ss * 2);
    const int p1 = align16v(a->l_qr + C * a->ss * 2);
    // phase 2 (over phase 1): L, the diagonal-block inverses, P~ and then A'' hi / lo
    a->l_ls = 0;
    a->l_li = align16v(C * a->lss * 4);
    a->l_ps = align16v(a->l_li + C * kLiStride * 4);
    const int pb = C * a->pss * 2, ab = 2 * C * a->aps * 2;
    const int p2 = align16v(a->l_ps + (pb > ab ? pb : ab));
    a->l_small = p1 > p2 ? p1 : p2;
    const int total = a->l_small + 3 * C * 4;
    return total <= kMaxLdsSliced ? total : 0;
}

bool plan_stream_sliced(int BH, int T, int d_k, int d_v, int nu, int C, StreamPlan* plan) {
    const int D = 2 * d_k * nu;
    if (d_k != kSliceDk || nu < 1 || nu > 4 || (C != 64 && C != 128)) return false;
    const int NCT = C / 64, CW = 16 * NCT;          // column tiles and columns per workgroup
    if (d_v % CW != 0) return false;
    // the y buffer's byte offsets (up to the last chunk's padded rows) fit 32 bits
    if ((static_cast<int64_t>(T) + C) * d_v * 2 >= (int64_t(1) << 32)) return false;
    ChunkArgs a = {};
    const int lds_prep = plan_prep_sliced(C, &a);
    if (lds_prep == 0) return false;
    const int NC = (T + C - 1) / C;
    const int64_t NU = static_cast<int64_t>(BH) * NC;
    // A'' hi, lo and P~: the blocks on and below the diagonal (the sliced prep's order)
    const int64_t szCC = static_cast<int64_t>(tri_nblocks(C)) * 1024, szR = C * 4;
    a.o_pa = 0;
    a.o_ah = a.o_pa + NU * szCC;
    a.o_al = a.o_ah + NU * szCC;
    a.o_rk = a.o_al + NU * szCC;
    a.o_rq = a.o_rk + NU * szR;
    // serial kernel LDS: raw slot (k rows, q rows, v columns), W^T copy, K slice, Q slice (Z and
    // U over it), y rows
    int off = 0;
    a.s_raw = off;
    a.s_qoff = C * kSliceDk * 2;
    a.s_voff = 2 * C * kSliceDk * 2;
    off = align16v(a.s_voff + C * CW * 2);
    a.s_wt = off;
    off += (D / 32) * NCT * 1024;
    a.s_k = off;
    off = align16v(off + C * a.ss * 2);
    a.s_q = off;
    a.s_z = off;
    a.s_u = off + C * CW * 4;
    const int qb = C * a.ss * 2, zu = 2 * C * CW * 4;
    off = align16v(off + (qb > zu ? qb : zu));
    a.s_y = off;
    off += C * CW * 2;
    if (off > kMaxLdsSliced) return false;
    a.BH = BH;
    a.T = T;
    a.NC = NC;
    a.d_k = d_k;
    a.d_v = d_v;
    a.nu = nu;
    a.D = D;
    plan->args = a;
    plan->C = C;
    plan->lds_prep = lds_prep;
    plan->lds_stream = off;
    plan->ndw = nu;
    plan->sliced_prep = true;
    plan->sliced_stream = true;
    plan->pipe = false;
    plan->ws_bytes = a.o_rq + NU * szR;
    return true;
}

// Chunk 64 runs the prep as 4-wave workgroups: at 52 KB of LDS three share a CU, and the
// 8x16x16384 prep takes 606 us against 697 us with 8-wave workgroups (two per CU).  Chunk 128
// needs one wave per block column of A, so 8 waves.
template <int C, int NU>
static hipError_t launch_prep_sliced_nu(const StreamPlan& p, hipStream_t stream) {
    constexpr int NTH = C == 64 ? 256 : kSliceThreads;
    // the persistent form where more chunks than fit at once and it keeps as many workgroups
    // resident as the one-chunk form (chunk 128: one per CU either way, 3% faster; at chunk 64
    // its registers cost the third workgroup per CU, 800 against 578 us), else one per chunk
    auto prep1 = delta_prep_sliced_kernel<C, NU, NTH, false>;
    auto prepp = delta_prep_sliced_kernel<C, NU, NTH, true>;
    hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(prepp), p.lds_prep);
    if (e != hipSuccess) return e;
    if ((e = ensure_lds_attr(reinterpret_cast<const void*>(prep1), p.lds_prep)) != hipSuccess) return e;
    const int64_t units = static_cast<int64_t>(p.args.BH) * p.args.NC;
    unsigned grid = 0, cap1 = 0;
    if ((e = resident_grid(reinterpret_cast<const void*>(prepp), NTH, p.lds_prep, units, &grid)) != hipSuccess) return e;
    if ((e = resident_grid(reinterpret_cast<const void*>(prep1), NTH, p.lds_prep, INT64_MAX, &cap1)) != hipSuccess) return e;
    if (static_cast<int64_t>(grid) < units && grid >= cap1) {
        hipLaunchKernelGGL(prepp, dim3(grid), dim3(NTH), p.lds_prep, stream, p.args);
    } else {
        hipLaunchKernelGGL(prep1, dim3(static_cast<unsigned>(units)), dim3(NTH), p.lds_prep, stream, p.args);
    }
    return hipGetLastError();
}

hipError_t launch_prep_sliced(const StreamPlan& p, hipStream_t stream) {
    if (static_cast<int64_t>(p.args.BH) * p.args.NC == 0) return hipSuccess;
    if (p.C == 64) {
        switch (p.args.nu) {
            case 1: return launch_prep_sliced_nu<64, 1>(p, stream);
            case 2: return launch_prep_sliced_nu<64, 2>(p, stream);
            case 3: return launch_prep_sliced_nu<64, 3>(p, stream);
            case 4: return launch_prep_sliced_nu<64, 4>(p, stream);
            default: return hipErrorInvalidValue;
        }
    }
    if (p.C == 128) {
        switch (p.args.nu) {
            case 1: return launch_prep_sliced_nu<128, 1>(p, stream);
            case 2: return launch_prep_sliced_nu<128, 2>(p, stream);
            case 3: return launch_prep_sliced_nu<128, 3>(p, stream);
            case 4: return launch_prep_sliced_nu<128, 4>(p, stream);
            default: return hipErrorInvalidValue;
        }
    }
    return hipErrorInvalidValue;
}

template <int C, int NU>
static hipError_t launch_stream_sliced_nu(const StreamPlan& p, hipStream_t stream) {
    constexpr int NCT = C / 64;
    auto kern = delta_stream_sliced_kernel<C, NU, NCT>;
    hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kern), p.lds_stream);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.args.BH) * (p.args.d_v / (16 * NCT))));
    hipLaunchKernelGGL(kern, grid, dim3(4 * C), p.lds_stream, stream, p.args);
    return hipGetLastError();
}

template <int C>
static hipError_t launch_stream_sliced_c(const StreamPlan& p, hipStream_t stream) {
    switch (p.args.nu) {
        case 1: return launch_stream_sliced_nu<C, 1>(p, stream);
        case 2: return launch_stream_sliced_nu<C, 2>(p, stream);
        case 3: return launch_stream_sliced_nu<C, 3>(p, stream);
        case 4: return launch_stream_sliced_nu<C, 4>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_stream_sliced(const StreamPlan& p, hipStream_t stream) {
    hipError_t e = launch_prep_sliced(p, stream);
    if (e != hipSuccess) return e;
    if (p.C == 64) return launch_stream_sliced_c<64>(p, stream);
    if (p.C == 128) return launch_stream_sliced_c<128>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace fwa
