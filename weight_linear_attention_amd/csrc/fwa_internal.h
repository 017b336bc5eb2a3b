// Host-side interface between the C ABI (fwa_api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fwa {

// Kernel arguments of the chunked forward, including its LDS layout (byte offsets and row
// strides in elements of each region's type).
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* bl;
    const float* W0;
    void* y;
    float* Wf;
    int BH, H, T, d_k, d_v, nu;
    int R, NVT, DP, NDP;
    int off_kr, off_qr, off_ls, off_ps, off_li, off_red, off_xs, off_small;
    int krs, lss, pss;
};

struct FwdPlan {
    int R, NVT, DP, NDP, NDPM;
    FwdArgs args;
    int lds_bytes;
};

hipError_t launch_dpfp(const void* x, void* phi, int64_t n_vec, int d_k, int nu, bool bf16,
                       hipStream_t stream);

int step_cpl_for(int D, int* LR_out);
hipError_t launch_delta_step(const void* q, const void* k, const void* v, const void* bl,
                             float* W, void* y, int64_t BH, int d_k, int d_v, int nu, bool bf16,
                             hipStream_t stream);

bool plan_forward(int BH, int d_k, int d_v, int nu, int C, bool bf16, FwdPlan* plan);
hipError_t launch_delta_forward(const FwdPlan& plan, const void* q, const void* k,
                                const void* v, const void* bl, const float* W0, void* y,
                                float* Wf, int BH, int H, int T, int d_k, int d_v, int nu, int C,
                                bool bf16, hipStream_t stream);

// Arguments of the chunked forward (prep, chain and, where it runs, output kernels): inputs and
// outputs, the workspace and the byte offsets of its regions, the chain split, and the prep
// kernel's LDS layout (byte offsets; row strides in elements).
struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* bl;
    const float* W0;
    void* y;
    float* Wf;
    char* ws;
    int64_t o_wy, o_kt, o_qa, o_pa, o_uy, o_rk, o_rq, o_wn, o_un;
    int64_t o_ah, o_al;          // streaming forward: (I + L)^-1 diag(beta) as bf16 hi, lo blocks
    int BH, T, NC, d_k, d_v, nu, D;
    int DP, NDP;
    int split;                   // fp32: W_y and K^T blocks in the split bf16 hi + lo format
    int krs, lss, pss, aps;
    int ss;                      // row stride (elements) of the shift-sliced K and Q tiles
    int l_kr, l_qr, l_x, l_ls, l_ps, l_li, l_xv, l_small;
    // streaming kernel LDS layout (byte offsets): K and Q tiles, the raw-input slot (k rows,
    // then q rows at s_qoff and v columns at s_voff inside it), W^T copy, Z (then y) and U tiles
    int s_k, s_q, s_raw, s_qoff, s_voff, s_wt, s_z, s_u;
    int s_y;                     // sliced streaming kernel: the chunk's y rows (bf16 [C][32])
};

struct ChunkPlan {
    ChunkArgs args;
    int C;
    int lds_prep;
    int64_t ws_bytes;
    int staged_ndp;      // > 0: the staged chain kernel with this many d-tiles per compute wave
    int lds_chain;       // its LDS bytes
    bool direct;         // bf16, chunk 64: the direct chain variant of the staged decomposition
    bool chain_outputs;  // the chain forms y itself (no chunk-start memories, no output launch)
};

// hipFuncSetAttribute(kernel, MaxDynamicSharedMemorySize, bytes) once per (kernel, device,
// size): the attribute persists, so later launches skip the runtime call.
hipError_t ensure_lds_attr(const void* kernel, int bytes);

// Workgroups of `kernel` that fit on the current device at once (a multiple of 8 from 8 on),
// capped at `want`.
hipError_t resident_grid(const void* kernel, int threads, int lds, int64_t want, unsigned* grid);

bool plan_chunked(int BH, int T, int d_k, int d_v, int nu, int C, bool bf16, ChunkPlan* plan);
hipError_t launch_chunked(const ChunkPlan& plan, const void* q, const void* k, const void* v,
                          const void* bl, const float* W0, void* y, float* Wf, char* ws,
                          bool bf16, hipStream_t stream);

// Streaming forward (bf16): the prep kernel in its compact mode, then one serial kernel per
// (b, h, 32 columns of d_v).  plan_stream returns false for shapes it does not implement.
struct StreamPlan {
    ChunkArgs args;
    int C;
    int lds_prep;
    int lds_stream;
    int ndw;             // d-tiles of W^T per wave (of 8)
    bool sliced_prep;    // prep with shift-sliced K and Q tiles (d_k = 64, nu <= 4)
    bool sliced_stream;  // serial kernel with shift-sliced K and Q tiles (chunk 64 or 128)
    bool pipe;           // pipelined serial kernel (d_k = 64, nu <= 3, chunk 64)
    int64_t ws_bytes;
};
bool plan_stream(int BH, int T, int d_k, int d_v, int nu, int C, bool bf16, StreamPlan* plan);
// Shift-sliced pieces (bf16, d_k = 64, nu <= 4): the prep kernel's LDS layout for chunk C (its
// bytes, 0 if it does not fit), the sliced plan (chunk 64 or 128), and the launches.
int plan_prep_sliced(int C, ChunkArgs* a);
bool plan_stream_sliced(int BH, int T, int d_k, int d_v, int nu, int C, StreamPlan* plan);
hipError_t launch_prep_sliced(const StreamPlan& plan, hipStream_t stream);
hipError_t launch_stream_sliced(const StreamPlan& plan, hipStream_t stream);
hipError_t launch_stream(const StreamPlan& plan, const void* q, const void* k, const void* v,
                         const void* bl, const float* W0, void* y, float* Wf, char* ws,
                         hipStream_t stream);

// Gradient of the forward (backward.hip): plan_backward gives the workspace bytes and returns
// false for shapes it does not implement.
bool plan_backward(int BH, int T, int d_k, int d_v, int nu, int64_t* ws_bytes);
hipError_t launch_backward(const void* q, const void* k, const void* v, const void* bl,
                           const float* W0, const void* dy, const float* dWf, void* dq, void* dk,
                           void* dv, void* dbl, float* dW0, int BH, int T, int d_k, int d_v,
                           int nu, bool bf16, void* workspace, hipStream_t stream);

// Sum-update linear attention with the z normaliser (sum_forward.hip).
bool plan_sum_forward(int BH, int T, int d_k, int d_v, int nu, int64_t* ws_bytes);
hipError_t launch_sum_forward(const void* q, const void* k, const void* v, const float* W0,
                              const float* z0, void* y, float* Wf, float* zf, int BH, int T,
                              int d_k, int d_v, int nu, bool bf16, void* workspace,
                              hipStream_t stream);

// Linear maps around the layer (projection.hip).
hipError_t launch_layer_project(const void* x, const void* Wqkvb, void* q, void* k, void* v,
                                void* bl, int B, int T, int d_model, int H, int d_k, int d_v,
                                bool bf16, hipStream_t stream);
hipError_t launch_layer_output(const void* y, const void* Wo, const void* bo, const void* res,
                               void* out, int B, int T, int H, int d_v, int d_model, bool bf16,
                               hipStream_t stream);

}  // namespace fwa
