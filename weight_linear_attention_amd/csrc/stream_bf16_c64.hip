// Streaming forward (bf16, chunk 64): host planning, the LDS and workspace layouts, and the two
// launches (prep kernel in compact mode, then the stream kernel).
#include "stream_kernel.h"


namespace fwa {

static int align16s(int x) { return (x + 15) & ~15; }

constexpr int kMaxLdsStream = 160 * 1024;

// Which kernels the streaming path runs.  Chunk 128 takes the shift-sliced kernels (d_k = 64,
// nu <= 4).  Chunk 64 takes a 32-column serial kernel: the pipelined one for d_k = 64 and
// nu <= 3, the full-tile one for d_k 16 and 32, with the sliced prep for d_k = 64 and nu <= 4
// and the full-tile compact prep otherwise; shapes neither serial kernel takes (d_v 16, D 512)
// fall back to the sliced serial kernel with 16-column workgroups, which builds the DPFP tiles
// three times per chunk and column group and is bound by that VALU work.
static bool plan_stream_full(int BH, int T, int d_k, int d_v, int nu, int C, StreamPlan* plan);

bool plan_stream(int BH, int T, int d_k, int d_v, int nu, int C, bool bf16, StreamPlan* plan) {
    if (!bf16) return false;
    if (C == 128) return plan_stream_sliced(BH, T, d_k, d_v, nu, C, plan);
    if (!plan_stream_full(BH, T, d_k, d_v, nu, C, plan))
        return C == 64 && plan_stream_sliced(BH, T, d_k, d_v, nu, C, plan);
    return true;
}

static bool plan_stream_full(int BH, int T, int d_k, int d_v, int nu, int C, StreamPlan* plan) {
    const int D = 2 * d_k * nu;
    // chunk 64, 32-column pairs of d_v, D in whole 8-wave shares of 16-row tiles, and rolls of
    // at most 8 positions (the extended q rows hold 8 positions before 0)
    if (C != 64 || d_v % 32 != 0 || D % 128 != 0 || nu > 8) return false;
    if (d_k != 16 && d_k != 32 && d_k != 64) return false;
    ChunkPlan cp;
    if (!plan_chunked(BH, T, d_k, d_v, nu, C, true, &cp)) return false;   // prep LDS layout
    ChunkArgs a = cp.args;
    const int64_t NU = static_cast<int64_t>(BH) * a.NC;
    a.o_wy = a.o_kt = a.o_qa = a.o_uy = a.o_wn = a.o_un = 0;
    // the y buffer's byte offsets (up to the last chunk's padded rows) fit 32 bits
    if ((static_cast<int64_t>(T) + C) * d_v * 2 >= (int64_t(1) << 32)) return false;
    // stream kernel LDS: K and Q tiles, the raw slot, W^T copy, Z (then y) and U tiles
    int off = 0;
    a.s_k = off;
    off = align16s(off + C * a.krs * 2);
    a.s_q = off;
    off = align16s(off + C * a.krs * 2);
    const int kbytes = C * d_k * 2;
    a.s_raw = off;
    a.s_qoff = kbytes;
    a.s_voff = align16s(a.s_qoff + kbytes);
    off = align16s(off + a.s_voff + C * 32 * 2);
    a.s_wt = off;
    off += (D / 32) * 2 * 1024;
    a.s_z = off;
    off += 8 * 1024;
    a.s_u = off;
    off += 8 * 1024;
    if (off > kMaxLdsStream) return false;
    plan->C = C;
    plan->lds_prep = cp.lds_prep;
    plan->sliced_prep = false;
    plan->sliced_stream = false;
    if (d_k == 64 && nu <= 4) {
        const int lds = plan_prep_sliced(C, &a);
        if (lds > 0) {
            plan->lds_prep = lds;
            plan->sliced_prep = true;
        }
    }
    plan->pipe = false;
    if (d_k == 64 && nu <= 3 && plan->sliced_prep) {
        // pipelined kernel: two K tiles, W^T copy, Z tiles, the bf16 U and rho_k o U blocks, Q W^T
        // exchange tiles, y and v rows.  Its K rows are 800 bytes at D = 384 (row stride = 32
        // mod 256 bytes), where both the 16-byte operand reads of 16 rows x 4 lanes and the
        // transposed reads hit distinct banks; the sliced prep does not use this stride.
        a.krs = D + 16;
        int o = 0;
        a.s_k = o;
        o = align16s(o + C * a.krs * 2);
        a.s_q = o;
        o = align16s(o + C * a.krs * 2);
        a.s_wt = o;
        o += (D / 32) * 2 * 1024;
        a.s_z = o;
        o += 8 * 1024;
        a.s_u = o;
        o += 8 * 1024;
        a.s_raw = o;
        o += 8 * 1024;
        a.s_y = o;
        o += C * 32 * 2;
        a.s_voff = o;
        o += C * 32 * 2;
        if (o > kMaxLdsStream) return false;
        off = o;
        plan->pipe = true;
    } else if (plan->sliced_prep) {
        // the 32-column full-tile serial kernel reads every block: it takes the compact prep
        plan->sliced_prep = false;
        plan->lds_prep = cp.lds_prep;
    }
    // workspace: A'' hi, lo and P~ blocks (the sliced prep stores those on and below the
    // diagonal only, the compact prep all of them), then rho_k and rho_q
    const int64_t szCC = plan->sliced_prep ? static_cast<int64_t>(tri_nblocks(C)) * 1024
                                           : static_cast<int64_t>(C) * C * 2;
    const int64_t szR = C * 4;
    a.o_pa = 0;
    a.o_ah = a.o_pa + NU * szCC;
    a.o_al = a.o_ah + NU * szCC;
    a.o_rk = a.o_al + NU * szCC;
    a.o_rq = a.o_rk + NU * szR;
    plan->args = a;
    plan->lds_stream = off;
    plan->ndw = D / 128;
    plan->ws_bytes = a.o_rq + NU * szR;
    return true;
}

template <int NU>
static hipError_t launch_stream_pipe(const StreamPlan& p, hipStream_t stream) {
    if (p.args.krs != 2 * 64 * NU + 16) return hipErrorInvalidValue;   // the kernel's fixed K stride
    auto kern = delta_stream_pipe_kernel<NU>;
    hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kern), p.lds_stream);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.args.BH) * (p.args.d_v / 32)));
    hipLaunchKernelGGL(kern, grid, dim3(64 * kStreamWaves), p.lds_stream, stream, p.args);
    return hipGetLastError();
}

template <int NDW>
static hipError_t launch_stream_ndw(const StreamPlan& p, hipStream_t stream) {
    auto kern = delta_stream_kernel<64, NDW>;
    hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kern), p.lds_stream);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.args.BH) * (p.args.d_v / 32)));
    hipLaunchKernelGGL(kern, grid, dim3(64 * kStreamWaves), p.lds_stream, stream, p.args);
    return hipGetLastError();
}

hipError_t launch_stream_c64(const StreamPlan& p, hipStream_t stream) {
    const ChunkArgs& a = p.args;
    const int64_t NU = static_cast<int64_t>(a.BH) * a.NC;
    if (p.sliced_prep) {
        hipError_t e = launch_prep_sliced(p, stream);
        if (e != hipSuccess) return e;
    } else if (NU > 0) {
        auto prep = delta_prep_kernel<true, 64, true>;
        hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(prep), p.lds_prep);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(prep, dim3(static_cast<unsigned>(NU)), dim3(kPrepThreads), p.lds_prep, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (p.pipe) {
        switch (a.nu) {
            case 1: return launch_stream_pipe<1>(p, stream);
            case 2: return launch_stream_pipe<2>(p, stream);
            case 3: return launch_stream_pipe<3>(p, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.ndw) {
        case 1: return launch_stream_ndw<1>(p, stream);
        case 2: return launch_stream_ndw<2>(p, stream);
        case 3: return launch_stream_ndw<3>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_stream(const StreamPlan& plan_in, const void* q, const void* k, const void* v,
                         const void* bl, const float* W0, void* y, float* Wf, char* ws,
                         hipStream_t stream) {
    StreamPlan p = plan_in;
    ChunkArgs& a = p.args;
    a.q = q;
    a.k = k;
    a.v = v;
    a.bl = bl;
    a.W0 = W0;
    a.y = y;
    a.Wf = Wf;
    a.ws = ws;
    if (p.sliced_stream) return launch_stream_sliced(p, stream);
    if (p.C != 64) return hipErrorInvalidValue;
    return launch_stream_c64(p, stream);
}

}  // namespace fwa
