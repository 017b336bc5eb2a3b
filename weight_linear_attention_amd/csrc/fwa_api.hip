// C ABI of the fast-weight delta-rule library: argument checks on the host, then one launch
// on the caller's stream.  Every check runs before any HIP call, so an invalid call touches
// neither the device nor the outputs.
#include "fwa.h"
#include "fwa_internal.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstring>
#include <mutex>
#include <cstdint>
#include <cstdio>
#include <string>


namespace {

thread_local std::string g_last_error;

fwa_status fail(fwa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
fwa_status fail(fwa_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

fwa_status ok() {
    g_last_error.clear();
    return FWA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [lo, lo + bytes) as an address range.
struct Span {
    uintptr_t lo, hi;
};
Span span(const void* p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, lo + static_cast<uintptr_t>(bytes)};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

bool valid_dtype(int d) { return d == FWA_F32 || d == FWA_BF16; }
int elem_bytes(int d) { return d == FWA_BF16 ? 2 : 4; }

// a * b * c ... <= limit without overflow (all factors >= 0)
bool mul_le(int64_t limit, std::initializer_list<int64_t> fs) {
    int64_t acc = 1;
    for (int64_t f : fs) {
        if (f == 0) return true;
        if (acc > limit / f) return false;
        acc *= f;
    }
    return acc <= limit;
}
constexpr int64_t kIndexLimit = int64_t(1) << 61;

fwa_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(FWA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The planner takes the chunked implementation where it applies and its workspace stays within
// kAutoWorkspaceLimit: beyond that the workspace traffic (about 7 D-wide rows per token)
// outweighs the parallelism it buys.  Larger bf16 problems take the streaming implementation
// where it applies, else the fused kernel.  Where both apply, the streaming one is taken once
// its serial workgroups (one per head and 32 columns of d_v) number kStreamFill, or half that
// at D >= 384, where the chunked workspace traffic is largest: on MI355X the streaming forward
// of 128 heads x 4096 at D 256 takes 387 us against 672, of 32 heads x 4096 at D 384 256 us
// against 379, while 32 heads x 4096 at D 256 (227 against 264 us) and 16 heads x 16384 stay
// chunked.
constexpr int64_t kAutoWorkspaceLimit = int64_t(2) << 30;
constexpr int64_t kStreamFill = 128;
}  // namespace

extern "C" {

const char* fwa_status_string(fwa_status s) {
    switch (s) {
        case FWA_OK: return "FWA_OK";
        case FWA_ERR_INVALID_ARG: return "FWA_ERR_INVALID_ARG";
        case FWA_ERR_UNSUPPORTED: return "FWA_ERR_UNSUPPORTED";
        case FWA_ERR_HIP: return "FWA_ERR_HIP";
    }
    return "FWA_UNKNOWN_STATUS";
}

const char* fwa_last_error(void) { return g_last_error.c_str(); }

int fwa_version(void) { return 1 * 10000 + 2 * 100 + 0; }

fwa_status fwa_dpfp(const void* x, void* phi, int64_t n_vec, int d_k, int nu, int dtype,
                    hipStream_t stream) {
    if (!valid_dtype(dtype)) return fail(FWA_ERR_INVALID_ARG, "fwa_dpfp: unknown dtype %d", dtype);
    if (n_vec < 0) return fail(FWA_ERR_INVALID_ARG, "fwa_dpfp: n_vec < 0");
    if (d_k < 1) return fail(FWA_ERR_INVALID_ARG, "fwa_dpfp: d_k < 1");
    if (nu < 1 || nu > 2 * d_k - 1)
        return fail(FWA_ERR_INVALID_ARG, "fwa_dpfp: nu=%d outside [1, 2*d_k-1]", nu);
    if (n_vec == 0) return ok();
    if (!x || !phi) return fail(FWA_ERR_INVALID_ARG, "fwa_dpfp: NULL pointer");
    if (!aligned16(x) || !aligned16(phi))
        return fail(FWA_ERR_INVALID_ARG, "fwa_dpfp: pointers must be 16-byte aligned");
    if (d_k != 16 && d_k != 32 && d_k != 64 && d_k != 128)
        return fail(FWA_ERR_UNSUPPORTED, "fwa_dpfp: d_k=%d not in {16,32,64,128}", d_k);
    const int64_t D = 2 * static_cast<int64_t>(d_k) * nu;
    if (!mul_le(kIndexLimit, {n_vec, D}))
        return fail(FWA_ERR_UNSUPPORTED, "fwa_dpfp: n_vec * D overflows the index range");
    const int es = elem_bytes(dtype);
    if (overlap(span(x, n_vec * d_k * es), span(phi, n_vec * D * es)))
        return fail(FWA_ERR_INVALID_ARG, "fwa_dpfp: x and phi overlap");
    return hip_status(fwa::launch_dpfp(x, phi, n_vec, d_k, nu, dtype == FWA_BF16, stream),
                      "fwa_dpfp launch");
}

}  // extern "C"

namespace {

// Checks of the sizes shared by fwa_delta_forward and fwa_delta_forward_info.
fwa_status check_forward_sizes(const char* fn, int B, int H, int T, int d_k, int d_v, int nu,
                               int chunk, int dtype) {
    if (!valid_dtype(dtype)) return fail(FWA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (B < 0 || H < 0 || T < 0) return fail(FWA_ERR_INVALID_ARG, "%s: negative B/H/T", fn);
    if (d_k < 1 || d_v < 1) return fail(FWA_ERR_INVALID_ARG, "%s: d_k and d_v must be >= 1", fn);
    if (nu < 1 || nu > 2 * d_k - 1)
        return fail(FWA_ERR_INVALID_ARG, "%s: nu=%d outside [1, 2*d_k-1]", fn, nu);
    if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128)
        return fail(FWA_ERR_INVALID_ARG, "%s: chunk=%d not in {16,32,64,128}", fn, chunk);
    return ok();
}

fwa_status check_forward_shape(const char* fn, int64_t BH, int T, int d_k, int d_v, int nu) {
    if (d_k != 16 && d_k != 32 && d_k != 64)
        return fail(FWA_ERR_UNSUPPORTED, "%s: d_k=%d not in {16,32,64}", fn, d_k);
    if (d_v != 16 && d_v != 32 && d_v != 64)
        return fail(FWA_ERR_UNSUPPORTED, "%s: d_v=%d not in {16,32,64}", fn, d_v);
    const int64_t D = 2 * static_cast<int64_t>(d_k) * nu;
    if (D > 512) return fail(FWA_ERR_UNSUPPORTED, "%s: D=2*d_k*nu=%lld > 512", fn, (long long)D);
    if (!mul_le(kIndexLimit, {BH, T, d_k > d_v ? d_k : d_v}) || !mul_le(kIndexLimit, {BH, d_v, D}))
        return fail(FWA_ERR_UNSUPPORTED, "%s: sizes overflow the index range", fn);
    if (BH > (int64_t(1) << 26) || static_cast<int64_t>(T) * d_v >= (int64_t(1) << 31) ||
        static_cast<int64_t>(T) * d_k >= (int64_t(1) << 31))
        return fail(FWA_ERR_UNSUPPORTED, "%s: too many (b, h) slices for one launch", fn);
    return ok();
}

// The implementation a forward call takes (the request and the shape), with its plan.
struct ForwardChoice {
    int path;                       // FWA_PATH_CHUNKED, FWA_PATH_STREAM or FWA_PATH_FUSED
    fwa::ChunkPlan cplan;
    fwa::StreamPlan splan;
    fwa::FwdPlan fplan;
    int64_t ws_bytes;
};

fwa_status choose_forward(const char* fn, int request, int BH, int T, int d_k, int d_v, int nu,
                          int chunk, bool bf16, ForwardChoice* c) {
    if (request != FWA_PATH_AUTO && request != FWA_PATH_CHUNKED && request != FWA_PATH_STREAM &&
        request != FWA_PATH_FUSED)
        return fail(FWA_ERR_INVALID_ARG, "%s: unknown forward path %d", fn, request);
    const bool auto_ = request == FWA_PATH_AUTO;
    const bool can_chunk = (auto_ || request == FWA_PATH_CHUNKED) &&
                           fwa::plan_chunked(BH, T, d_k, d_v, nu, chunk, bf16, &c->cplan);
    const bool can_stream = (auto_ || request == FWA_PATH_STREAM) &&
                            fwa::plan_stream(BH, T, d_k, d_v, nu, chunk, bf16, &c->splan);
    const bool can_fuse = (auto_ || request == FWA_PATH_FUSED) &&
                          fwa::plan_forward(BH, d_k, d_v, nu, chunk, bf16, &c->fplan);
    c->ws_bytes = 0;
    const int64_t serial_wgs = static_cast<int64_t>(BH) * (d_v / 32);
    const bool stream_fills = can_stream && (serial_wgs >= kStreamFill ||
                                             (2 * d_k * nu >= 384 && 2 * serial_wgs >= kStreamFill));
    if (can_chunk && (!auto_ || (c->cplan.ws_bytes <= kAutoWorkspaceLimit && !stream_fills) ||
                      (!can_stream && !can_fuse))) {
        c->path = FWA_PATH_CHUNKED;
        c->ws_bytes = c->cplan.ws_bytes;
        return ok();
    }
    if (can_stream) {
        c->path = FWA_PATH_STREAM;
        c->ws_bytes = c->splan.ws_bytes;
        return ok();
    }
    if (can_fuse) {
        c->path = FWA_PATH_FUSED;
        return ok();
    }
    if (request == FWA_PATH_CHUNKED || request == FWA_PATH_STREAM)
        return fail(FWA_ERR_UNSUPPORTED,
                    "%s: the %s path does not support d_k=%d d_v=%d nu=%d chunk=%d%s", fn,
                    request == FWA_PATH_CHUNKED ? "chunked" : "stream", d_k, d_v, nu, chunk,
                    request == FWA_PATH_STREAM && !bf16 ? " (it takes bf16 inputs)" : "");
    return fail(FWA_ERR_UNSUPPORTED,
                "%s: d_k=%d d_v=%d nu=%d chunk=%d does not fit the on-chip working set", fn, d_k,
                d_v, nu, chunk);
}

// Checks every argument of a forward call (sizes, pointers, overlaps, the workspace) and picks
// the implementation; nothing is launched.
fwa_status check_forward_call(const char* fn, int request, const void* q, const void* k,
                              const void* v, const void* beta_logit, const float* W0,
                              const void* y, const float* W_final, int B, int H, int T, int d_k,
                              int d_v, int nu, int chunk, int dtype, const void* workspace,
                              int64_t workspace_bytes, ForwardChoice* c,
                              bool check_workspace = true) {
    fwa_status st = check_forward_sizes(fn, B, H, T, d_k, d_v, nu, chunk, dtype);
    if (st != FWA_OK) return st;
    const int64_t BH = static_cast<int64_t>(B) * H;
    c->path = FWA_PATH_NONE;
    c->ws_bytes = 0;
    if (BH == 0) return ok();
    if (T > 0 && (!q || !k || !v || !beta_logit || !y))
        return fail(FWA_ERR_INVALID_ARG, "%s: NULL input or output pointer", fn);
    if (workspace_bytes < 0) return fail(FWA_ERR_INVALID_ARG, "%s: workspace_bytes < 0", fn);
    const void* ptrs[] = {q, k, v, beta_logit, W0, y, W_final, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p))
            return fail(FWA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    if ((st = check_forward_shape(fn, BH, T, d_k, d_v, nu)) != FWA_OK) return st;
    const int64_t D = 2 * static_cast<int64_t>(d_k) * nu;
    const int es = elem_bytes(dtype);
    const int64_t nqk = BH * T * d_k * es, nv = BH * T * d_v * es, nb = BH * T * es;
    const int64_t nW = BH * d_v * D * 4;
    const Span in[] = {span(q, T ? nqk : 0), span(k, T ? nqk : 0), span(v, T ? nv : 0),
                       span(beta_logit, T ? nb : 0), span(W0, W0 ? nW : 0)};
    const Span sy = span(y, T && y ? nv : 0), sw = span(W_final, W_final ? nW : 0);
    for (const Span& s : in)
        if (overlap(s, sy)) return fail(FWA_ERR_INVALID_ARG, "%s: y overlaps an input", fn);
    for (int i = 0; i < 4; ++i)
        if (overlap(in[i], sw)) return fail(FWA_ERR_INVALID_ARG, "%s: W_final overlaps an input", fn);
    if (W0 && W_final && W0 != W_final && overlap(in[4], sw))
        return fail(FWA_ERR_INVALID_ARG, "%s: W0 and W_final partially overlap", fn);
    if (overlap(sy, sw)) return fail(FWA_ERR_INVALID_ARG, "%s: y overlaps W_final", fn);

    if ((st = choose_forward(fn, request, static_cast<int>(BH), T, d_k, d_v, nu, chunk,
                             dtype == FWA_BF16, c)) != FWA_OK)
        return st;
    if (c->ws_bytes > 0 && check_workspace) {
        if (!workspace || workspace_bytes < c->ws_bytes)
            return fail(FWA_ERR_INVALID_ARG,
                        "%s: the %s path needs a workspace of %lld bytes (got %lld%s)", fn,
                        c->path == FWA_PATH_CHUNKED ? "chunked" : "stream",
                        (long long)c->ws_bytes, (long long)workspace_bytes,
                        workspace ? "" : ", NULL");
        const Span sws = span(workspace, c->ws_bytes);
        for (const Span& s : in)
            if (overlap(s, sws)) return fail(FWA_ERR_INVALID_ARG, "%s: workspace overlaps an input", fn);
        if (overlap(sws, sy) || overlap(sws, sw))
            return fail(FWA_ERR_INVALID_ARG, "%s: workspace overlaps an output", fn);
    }
    return ok();
}

// Enqueues the chosen implementation (arguments already checked).
fwa_status launch_forward(const ForwardChoice& c, const void* q, const void* k, const void* v,
                          const void* beta_logit, const float* W0, void* y, float* W_final,
                          int BH, int H, int T, int d_k, int d_v, int nu, int chunk, bool bf16,
                          void* workspace, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    switch (c.path) {
        case FWA_PATH_NONE:
            return ok();
        case FWA_PATH_STREAM:
            return hip_status(fwa::launch_stream(c.splan, q, k, v, beta_logit, W0, y, W_final, ws,
                                                 stream),
                              "fwa_delta_forward launch");
        case FWA_PATH_CHUNKED:
            return hip_status(fwa::launch_chunked(c.cplan, q, k, v, beta_logit, W0, y, W_final,
                                                  ws, bf16, stream),
                              "fwa_delta_forward launch");
        default:
            return hip_status(fwa::launch_delta_forward(c.fplan, q, k, v, beta_logit, W0, y,
                                                        W_final, BH, H, T, d_k, d_v, nu, chunk,
                                                        bf16, stream),
                              "fwa_delta_forward launch");
    }
}

}  // namespace

extern "C" {

fwa_status fwa_delta_forward_info(int B, int H, int T, int d_k, int d_v, int nu, int chunk,
                                  int dtype, int request, int* path,
                                  int64_t* workspace_bytes) {
    const char* fn = "fwa_delta_forward_info";
    fwa_status st = check_forward_sizes(fn, B, H, T, d_k, d_v, nu, chunk, dtype);
    if (st != FWA_OK) return st;
    const int64_t BH = static_cast<int64_t>(B) * H;
    int p = FWA_PATH_NONE;
    int64_t ws = 0;
    if (BH > 0) {
        if ((st = check_forward_shape(fn, BH, T, d_k, d_v, nu)) != FWA_OK) return st;
        ForwardChoice c;
        if ((st = choose_forward(fn, request, static_cast<int>(BH), T, d_k, d_v, nu, chunk,
                                 dtype == FWA_BF16, &c)) != FWA_OK)
            return st;
        p = c.path;
        ws = c.ws_bytes;
    } else if (request != FWA_PATH_AUTO && request != FWA_PATH_CHUNKED &&
               request != FWA_PATH_STREAM && request != FWA_PATH_FUSED) {
        return fail(FWA_ERR_INVALID_ARG, "%s: unknown forward path %d", fn, request);
    }
    if (path) *path = p;
    if (workspace_bytes) *workspace_bytes = ws;
    return ok();
}

fwa_status fwa_delta_forward_path(int request, const void* q, const void* k, const void* v,
                                  const void* beta_logit, const float* W0, void* y,
                                  float* W_final, int B, int H, int T, int d_k, int d_v, int nu,
                                  int chunk, int dtype, void* workspace,
                                  int64_t workspace_bytes, hipStream_t stream) {
    const char* fn = "fwa_delta_forward";
    ForwardChoice c;
    fwa_status st = check_forward_call(fn, request, q, k, v, beta_logit, W0, y, W_final, B, H, T,
                                       d_k, d_v, nu, chunk, dtype, workspace, workspace_bytes, &c);
    if (st != FWA_OK) return st;
    return launch_forward(c, q, k, v, beta_logit, W0, y, W_final, B * H, H, T, d_k, d_v, nu,
                          chunk, dtype == FWA_BF16, workspace, stream);
}

fwa_status fwa_delta_forward(const void* q, const void* k, const void* v, const void* beta_logit,
                             const float* W0, void* y, float* W_final, int B, int H, int T,
                             int d_k, int d_v, int nu, int chunk, int dtype,
                             void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    return fwa_delta_forward_path(FWA_PATH_AUTO, q, k, v, beta_logit, W0, y, W_final, B, H, T,
                                  d_k, d_v, nu, chunk, dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of fwa_delta_forward_noalloc: a file-scope device array that every GPU the library
// runs on holds until the process ends.  Host code never uses its name as an address: each
// device's copy lives at its own address, taken once per device with hipGetSymbolAddress
// (with that device current) and kept in g_scratch_ptr.
constexpr int64_t kNoAllocScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call on that device).
hipError_t scratch_for_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

fwa_status fwa_delta_forward_noalloc(const void* q, const void* k, const void* v,
                                     const void* beta_logit, const float* W0, void* y,
                                     float* W_final, int B, int H, int T, int d_k, int d_v, int nu,
                                     int chunk, int dtype, hipStream_t stream) {
    const char* fn = "fwa_delta_forward_noalloc";
    ForwardChoice c;
    fwa_status st = check_forward_call(fn, FWA_PATH_AUTO, q, k, v, beta_logit, W0, y, W_final, B,
                                       H, T, d_k, d_v, nu, chunk, dtype, nullptr, 0, &c, false);
    if (st != FWA_OK) return st;
    if (c.path == FWA_PATH_NONE) return ok();
    if (c.ws_bytes > kNoAllocScratchBytes) {
        // the planner's choice needs more scratch than the static array holds: the fused
        // implementation needs none, where it takes these sizes
        const int64_t need = c.ws_bytes;
        ForwardChoice f;
        st = check_forward_call(fn, FWA_PATH_FUSED, q, k, v, beta_logit, W0, y, W_final, B, H, T,
                                d_k, d_v, nu, chunk, dtype, nullptr, 0, &f, false);
        if (st != FWA_OK)
            return fail(FWA_ERR_UNSUPPORTED,
                        "%s: the planned forward needs %lld bytes of scratch, more than the %lld "
                        "the static scratch holds, and the fused implementation (no scratch) does "
                        "not take these sizes",
                        fn, (long long)need, (long long)kNoAllocScratchBytes);
        c = f;
    }
    void* ws = nullptr;
    const hipError_t e = scratch_for_current_device(&ws);
    if (e != hipSuccess) return hip_status(e, "fwa_delta_forward_noalloc scratch address");
    return launch_forward(c, q, k, v, beta_logit, W0, y, W_final, B * H, H, T, d_k, d_v, nu,
                          chunk, dtype == FWA_BF16, ws, stream);
}

}  // extern "C"

namespace {

fwa_status check_backward_shape(const char* fn, int B, int H, int T, int d_k, int d_v, int nu,
                                int dtype, int64_t* ws_bytes) {
    if (!valid_dtype(dtype)) return fail(FWA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (B < 0 || H < 0 || T < 0) return fail(FWA_ERR_INVALID_ARG, "%s: negative B/H/T", fn);
    if (d_k < 1 || d_v < 1) return fail(FWA_ERR_INVALID_ARG, "%s: d_k and d_v must be >= 1", fn);
    if (nu < 1 || nu > 2 * d_k - 1)
        return fail(FWA_ERR_INVALID_ARG, "%s: nu=%d outside [1, 2*d_k-1]", fn, nu);
    const int64_t BH = static_cast<int64_t>(B) * H;
    *ws_bytes = 0;
    if (BH == 0) return ok();
    const int64_t D = 2 * static_cast<int64_t>(d_k) * nu;
    if (d_k != 16 && d_k != 32 && d_k != 64)
        return fail(FWA_ERR_UNSUPPORTED, "%s: d_k=%d not in {16,32,64}", fn, d_k);
    if (d_v > 64) return fail(FWA_ERR_UNSUPPORTED, "%s: d_v=%d > 64", fn, d_v);
    if (D > 384) return fail(FWA_ERR_UNSUPPORTED, "%s: D=2*d_k*nu=%lld > 384", fn, (long long)D);
    if (!mul_le(kIndexLimit / 64, {BH, static_cast<int64_t>(T) + 64, D}) ||
        !mul_le(kIndexLimit / 64, {BH, static_cast<int64_t>(T) + 64, d_v}) ||
        BH > (int64_t(1) << 26) || static_cast<int64_t>(T) * d_v >= (int64_t(1) << 31))
        return fail(FWA_ERR_UNSUPPORTED, "%s: sizes overflow the index range", fn);
    if (!fwa::plan_backward(static_cast<int>(BH), T, d_k, d_v, nu, ws_bytes))
        return fail(FWA_ERR_UNSUPPORTED, "%s: no backward plan for these sizes", fn);
    return ok();
}

}  // namespace

extern "C" {

fwa_status fwa_delta_backward_info(int B, int H, int T, int d_k, int d_v, int nu,
                                   int dtype, int64_t* workspace_bytes) {
    int64_t ws = 0;
    const fwa_status st = check_backward_shape("fwa_delta_backward_info", B, H, T, d_k, d_v, nu,
                                               dtype, &ws);
    if (st != FWA_OK) return st;
    if (workspace_bytes) *workspace_bytes = ws;
    return ok();
}

fwa_status fwa_delta_backward(const void* q, const void* k, const void* v,
                              const void* beta_logit, const float* W0, const void* dy,
                              const float* dW_final, void* dq, void* dk, void* dv,
                              void* dbeta_logit, float* dW0, int B, int H, int T, int d_k,
                              int d_v, int nu, int dtype, void* workspace,
                              int64_t workspace_bytes, hipStream_t stream) {
    const char* fn = "fwa_delta_backward";
    int64_t need = 0;
    fwa_status st = check_backward_shape(fn, B, H, T, d_k, d_v, nu, dtype, &need);
    if (st != FWA_OK) return st;
    const int64_t BH = static_cast<int64_t>(B) * H;
    if (BH == 0) return ok();
    if (T > 0 && (!q || !k || !v || !beta_logit || !dy || !dq || !dk || !dv || !dbeta_logit))
        return fail(FWA_ERR_INVALID_ARG, "%s: NULL input or gradient pointer", fn);
    if (workspace_bytes < 0) return fail(FWA_ERR_INVALID_ARG, "%s: workspace_bytes < 0", fn);
    const void* ptrs[] = {q, k, v, beta_logit, W0, dy, dW_final, dq, dk, dv, dbeta_logit, dW0,
                          workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p))
            return fail(FWA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(FWA_ERR_INVALID_ARG, "%s: needs a workspace of %lld bytes (got %lld%s)", fn,
                    (long long)need, (long long)workspace_bytes, workspace ? "" : ", NULL");
    const int64_t D = 2 * static_cast<int64_t>(d_k) * nu;
    const int es = elem_bytes(dtype);
    const int64_t nqk = T ? BH * T * d_k * es : 0, nv = T ? BH * T * d_v * es : 0;
    const int64_t nb = T ? BH * T * es : 0, nW = BH * d_v * D * 4;
    const Span in[] = {span(q, nqk), span(k, nqk), span(v, nv), span(beta_logit, nb),
                       span(W0, W0 ? nW : 0), span(dy, nv), span(dW_final, dW_final ? nW : 0)};
    const Span out[] = {span(dq, nqk), span(dk, nqk), span(dv, nv), span(dbeta_logit, nb),
                        span(dW0, dW0 ? nW : 0), span(workspace, need)};
    for (int i = 0; i < 6; ++i) {
        for (const Span& s : in)
            if (overlap(out[i], s)) return fail(FWA_ERR_INVALID_ARG, "%s: an output overlaps an input", fn);
        for (int j = 0; j < i; ++j)
            if (overlap(out[i], out[j])) return fail(FWA_ERR_INVALID_ARG, "%s: two outputs overlap", fn);
    }
    return hip_status(fwa::launch_backward(q, k, v, beta_logit, W0, dy, dW_final, dq, dk, dv,
                                           dbeta_logit, dW0, static_cast<int>(BH), T, d_k, d_v,
                                           nu, dtype == FWA_BF16, workspace, stream),
                      "fwa_delta_backward launch");
}

}  // extern "C"

namespace {

fwa_status check_sum_shape(const char* fn, int B, int H, int T, int d_k, int d_v, int nu,
                           int dtype, int64_t* ws_bytes) {
    if (!valid_dtype(dtype)) return fail(FWA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (B < 0 || H < 0 || T < 0) return fail(FWA_ERR_INVALID_ARG, "%s: negative B/H/T", fn);
    if (d_k < 1 || d_v < 1) return fail(FWA_ERR_INVALID_ARG, "%s: d_k and d_v must be >= 1", fn);
    if (nu < 1 || nu > 2 * d_k - 1)
        return fail(FWA_ERR_INVALID_ARG, "%s: nu=%d outside [1, 2*d_k-1]", fn, nu);
    const int64_t BH = static_cast<int64_t>(B) * H;
    *ws_bytes = 0;
    if (BH == 0) return ok();
    const int64_t D = 2 * static_cast<int64_t>(d_k) * nu;
    if (d_k != 16 && d_k != 32 && d_k != 64)
        return fail(FWA_ERR_UNSUPPORTED, "%s: d_k=%d not in {16,32,64}", fn, d_k);
    if (d_v > 128) return fail(FWA_ERR_UNSUPPORTED, "%s: d_v=%d > 128", fn, d_v);
    if (D > 384) return fail(FWA_ERR_UNSUPPORTED, "%s: D=2*d_k*nu=%lld > 384", fn, (long long)D);
    if (!mul_le(kIndexLimit / 64, {BH, static_cast<int64_t>(T) + 64, D}) ||
        !mul_le(kIndexLimit / 64, {BH, static_cast<int64_t>(T) + 64, d_v}) ||
        BH > (int64_t(1) << 26) || static_cast<int64_t>(T) * d_v >= (int64_t(1) << 31))
        return fail(FWA_ERR_UNSUPPORTED, "%s: sizes overflow the index range", fn);
    if (!fwa::plan_sum_forward(static_cast<int>(BH), T, d_k, d_v, nu, ws_bytes))
        return fail(FWA_ERR_UNSUPPORTED, "%s: no plan for these sizes", fn);
    return ok();
}

}  // namespace

extern "C" {

fwa_status fwa_sum_forward_info(int B, int H, int T, int d_k, int d_v, int nu, int dtype,
                                int64_t* workspace_bytes) {
    int64_t ws = 0;
    const fwa_status st = check_sum_shape("fwa_sum_forward_info", B, H, T, d_k, d_v, nu, dtype, &ws);
    if (st != FWA_OK) return st;
    if (workspace_bytes) *workspace_bytes = ws;
    return ok();
}

fwa_status fwa_sum_forward(const void* q, const void* k, const void* v, const float* W0,
                           const float* z0, void* y, float* W_final, float* z_final, int B, int H,
                           int T, int d_k, int d_v, int nu, int dtype, void* workspace,
                           int64_t workspace_bytes, hipStream_t stream) {
    const char* fn = "fwa_sum_forward";
    int64_t need = 0;
    fwa_status st = check_sum_shape(fn, B, H, T, d_k, d_v, nu, dtype, &need);
    if (st != FWA_OK) return st;
    const int64_t BH = static_cast<int64_t>(B) * H;
    if (BH == 0) return ok();
    if (T > 0 && (!q || !k || !v || !y))
        return fail(FWA_ERR_INVALID_ARG, "%s: NULL input or output pointer", fn);
    if (workspace_bytes < 0) return fail(FWA_ERR_INVALID_ARG, "%s: workspace_bytes < 0", fn);
    const void* ptrs[] = {q, k, v, W0, z0, y, W_final, z_final, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p))
            return fail(FWA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(FWA_ERR_INVALID_ARG, "%s: needs a workspace of %lld bytes (got %lld%s)", fn,
                    (long long)need, (long long)workspace_bytes, workspace ? "" : ", NULL");
    const int64_t D = 2 * static_cast<int64_t>(d_k) * nu;
    const int es = elem_bytes(dtype);
    const int64_t nqk = T ? BH * T * d_k * es : 0, nv = T ? BH * T * d_v * es : 0;
    const int64_t nW = BH * d_v * D * 4, nz = BH * D * 4;
    const Span in[] = {span(q, nqk), span(k, nqk), span(v, nv), span(W0, W0 ? nW : 0),
                       span(z0, z0 ? nz : 0)};
    const Span out[] = {span(y, nv), span(W_final, W_final ? nW : 0),
                        span(z_final, z_final ? nz : 0), span(workspace, need)};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 5; ++j) {
            // in-place carry: W_final may be W0 and z_final z0 (exactly)
            if ((i == 1 && j == 3 && W_final == W0) || (i == 2 && j == 4 && z_final == z0)) continue;
            if (overlap(out[i], in[j])) return fail(FWA_ERR_INVALID_ARG, "%s: an output overlaps an input", fn);
        }
        for (int j = 0; j < i; ++j)
            if (overlap(out[i], out[j])) return fail(FWA_ERR_INVALID_ARG, "%s: two outputs overlap", fn);
    }
    return hip_status(fwa::launch_sum_forward(q, k, v, W0, z0, y, W_final, z_final,
                                              static_cast<int>(BH), T, d_k, d_v, nu,
                                              dtype == FWA_BF16, workspace, stream),
                      "fwa_sum_forward launch");
}

}  // extern "C"

namespace {

fwa_status check_linear_dims(const char* fn, int B, int T, int d_model, int H, int d_k, int d_v,
                             int dtype) {
    if (!valid_dtype(dtype)) return fail(FWA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (B < 0 || T < 0 || H < 0) return fail(FWA_ERR_INVALID_ARG, "%s: negative B/T/H", fn);
    if (d_model < 1 || d_k < 1 || d_v < 1)
        return fail(FWA_ERR_INVALID_ARG, "%s: d_model, d_k and d_v must be >= 1", fn);
    if (d_model % 8 || d_k % 8 || d_v % 8)
        return fail(FWA_ERR_UNSUPPORTED, "%s: d_model, d_k and d_v must be multiples of 8", fn);
    const int64_t N = 2 * int64_t(H) * d_k + int64_t(H) * d_v + H;
    if (!mul_le(kIndexLimit, {int64_t(B), int64_t(T), N + d_model}) ||
        static_cast<int64_t>(B) * T >= (int64_t(1) << 31) || N * d_model >= (int64_t(1) << 31) ||
        int64_t(H) * d_v * d_model >= (int64_t(1) << 31))
        return fail(FWA_ERR_UNSUPPORTED, "%s: sizes overflow the index range", fn);
    return ok();
}

}  // namespace

extern "C" {

fwa_status fwa_layer_project(const void* x, const void* W_qkvb, void* q, void* k, void* v,
                             void* beta_logit, int B, int T, int d_model, int H, int d_k, int d_v,
                             int dtype, hipStream_t stream) {
    const char* fn = "fwa_layer_project";
    fwa_status st = check_linear_dims(fn, B, T, d_model, H, d_k, d_v, dtype);
    if (st != FWA_OK) return st;
    const int64_t M = int64_t(B) * T;
    if (M == 0 || H == 0) return ok();
    if (!x || !W_qkvb || !q || !k || !v || !beta_logit)
        return fail(FWA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    const void* ptrs[] = {x, W_qkvb, q, k, v, beta_logit};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(FWA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    const int es = elem_bytes(dtype);
    const int64_t N = 2 * int64_t(H) * d_k + int64_t(H) * d_v + H;
    const Span in[] = {span(x, M * d_model * es), span(W_qkvb, N * d_model * es)};
    const Span out[] = {span(q, M * H * d_k * es), span(k, M * H * d_k * es),
                        span(v, M * H * d_v * es), span(beta_logit, M * H * es)};
    for (int i = 0; i < 4; ++i) {
        for (const Span& s : in)
            if (overlap(out[i], s)) return fail(FWA_ERR_INVALID_ARG, "%s: an output overlaps an input", fn);
        for (int j = 0; j < i; ++j)
            if (overlap(out[i], out[j])) return fail(FWA_ERR_INVALID_ARG, "%s: two outputs overlap", fn);
    }
    return hip_status(fwa::launch_layer_project(x, W_qkvb, q, k, v, beta_logit, B, T, d_model, H,
                                                d_k, d_v, dtype == FWA_BF16, stream),
                      "fwa_layer_project launch");
}

fwa_status fwa_layer_output(const void* y, const void* W_o, const void* b_o,
                            const void* residual, void* out, int B, int T, int H, int d_v,
                            int d_model, int dtype, hipStream_t stream) {
    const char* fn = "fwa_layer_output";
    fwa_status st = check_linear_dims(fn, B, T, d_model, H, 8, d_v, dtype);
    if (st != FWA_OK) return st;
    const int64_t M = int64_t(B) * T;
    if (M == 0) return ok();
    if (!out || !W_o || (H > 0 && !y)) return fail(FWA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    const void* ptrs[] = {y, W_o, b_o, residual, out};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(FWA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    const int es = elem_bytes(dtype);
    const Span so = span(out, M * d_model * es);
    const Span in[] = {span(y, y ? M * H * d_v * es : 0), span(W_o, int64_t(d_model) * H * d_v * es),
                       span(b_o, b_o ? d_model * es : 0)};
    for (const Span& s : in)
        if (overlap(so, s)) return fail(FWA_ERR_INVALID_ARG, "%s: out overlaps an input", fn);
    if (residual && residual != out && overlap(so, span(residual, M * d_model * es)))
        return fail(FWA_ERR_INVALID_ARG, "%s: out partially overlaps residual", fn);
    return hip_status(fwa::launch_layer_output(y, W_o, b_o, residual, out, B, T, H, d_v, d_model,
                                               dtype == FWA_BF16, stream),
                      "fwa_layer_output launch");
}

fwa_status fwa_decode_layers_info(int B, int d_model, int H, int d_k, int d_v, int nu,
                                  int dtype, int64_t* workspace_bytes) {
    const char* fn = "fwa_decode_layers_info";
    fwa_status st = check_linear_dims(fn, B, 1, d_model, H, d_k, d_v, dtype);
    if (st != FWA_OK) return st;
    if (nu < 1 || nu > 2 * d_k - 1)
        return fail(FWA_ERR_INVALID_ARG, "%s: nu=%d outside [1, 2*d_k-1]", fn, nu);
    const int64_t BH = int64_t(B) * H;
    const int es = elem_bytes(dtype);
    auto up16 = [](int64_t n) { return (n + 15) & ~int64_t(15); };
    if (workspace_bytes)
        *workspace_bytes = 2 * up16(BH * d_k * es) + 2 * up16(BH * d_v * es) + up16(BH * es);
    return ok();
}

fwa_status fwa_decode_layers(void* x, int L, const void* const* W_qkvb, const void* const* W_o,
                             const void* const* b_o, float* const* W, int B, int d_model, int H,
                             int d_k, int d_v, int nu, int dtype, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream) {
    const char* fn = "fwa_decode_layers";
    int64_t need = 0;
    fwa_status st = fwa_decode_layers_info(B, d_model, H, d_k, d_v, nu, dtype, &need);
    if (st != FWA_OK) return st;
    if (L < 0) return fail(FWA_ERR_INVALID_ARG, "%s: L < 0", fn);
    const int64_t BH = int64_t(B) * H;
    if (L == 0 || BH == 0) return ok();
    if (!x || !W_qkvb || !W_o || !W) return fail(FWA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!workspace || workspace_bytes < need)
        return fail(FWA_ERR_INVALID_ARG, "%s: needs a workspace of %lld bytes (got %lld%s)", fn,
                    (long long)need, (long long)workspace_bytes, workspace ? "" : ", NULL");
    if (d_k != 16 && d_k != 32 && d_k != 64 && d_k != 128)
        return fail(FWA_ERR_UNSUPPORTED, "%s: d_k=%d not in {16,32,64,128}", fn, d_k);
    const int64_t D = 2 * static_cast<int64_t>(d_k) * nu;
    int LR = 0;
    if (D > 1024 || fwa::step_cpl_for(static_cast<int>(D), &LR) == 0)
        return fail(FWA_ERR_UNSUPPORTED, "%s: D=%lld has no decode-step row layout", fn, (long long)D);
    const int es = elem_bytes(dtype);
    const int64_t N = 2 * int64_t(H) * d_k + int64_t(H) * d_v + H;
    const Span sx = span(x, int64_t(B) * d_model * es), sws = span(workspace, need);
    if (!aligned16(x) || !aligned16(workspace))
        return fail(FWA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    if (overlap(sx, sws)) return fail(FWA_ERR_INVALID_ARG, "%s: x overlaps the workspace", fn);
    for (int l = 0; l < L; ++l) {
        if (!W_qkvb[l] || !W_o[l] || !W[l])
            return fail(FWA_ERR_INVALID_ARG, "%s: NULL pointer for layer %d", fn, l);
        const void* lp[] = {W_qkvb[l], W_o[l], b_o ? b_o[l] : nullptr, W[l]};
        for (const void* p : lp)
            if (p && !aligned16(p))
                return fail(FWA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned (layer %d)", fn, l);
        const Span ls[] = {span(W_qkvb[l], N * d_model * es),
                           span(W_o[l], int64_t(d_model) * H * d_v * es),
                           span(b_o ? b_o[l] : nullptr, b_o && b_o[l] ? d_model * es : 0),
                           span(W[l], BH * d_v * D * 4)};
        for (const Span& s : ls)
            if (overlap(s, sx) || overlap(s, sws))
                return fail(FWA_ERR_INVALID_ARG, "%s: layer %d's parameters overlap x or the workspace", fn, l);
        for (int m = 0; m < l; ++m)
            if (overlap(ls[3], span(W[m], BH * d_v * D * 4)))
                return fail(FWA_ERR_INVALID_ARG, "%s: the memories of layers %d and %d overlap", fn, m, l);
    }
    auto up16 = [](int64_t n) { return (n + 15) & ~int64_t(15); };
    char* ws = static_cast<char*>(workspace);
    void* q = ws;
    void* k = ws + up16(BH * d_k * es);
    void* v = ws + 2 * up16(BH * d_k * es);
    void* y = ws + 2 * up16(BH * d_k * es) + up16(BH * d_v * es);
    void* bl = ws + 2 * up16(BH * d_k * es) + 2 * up16(BH * d_v * es);
    const bool bf16 = dtype == FWA_BF16;
    for (int l = 0; l < L; ++l) {
        hipError_t e = fwa::launch_layer_project(x, W_qkvb[l], q, k, v, bl, B, 1, d_model, H, d_k,
                                                 d_v, bf16, stream);
        if (e == hipSuccess)
            e = fwa::launch_delta_step(q, k, v, bl, W[l], y, BH, d_k, d_v, nu, bf16, stream);
        if (e == hipSuccess)
            e = fwa::launch_layer_output(y, W_o[l], b_o ? b_o[l] : nullptr, x, x, B, 1, H, d_v,
                                         d_model, bf16, stream);
        if (e != hipSuccess) return hip_status(e, "fwa_decode_layers launch");
    }
    return ok();
}

fwa_status fwa_delta_step(const void* q, const void* k, const void* v, const void* beta_logit,
                          float* W, void* y, int B, int H, int d_k, int d_v, int nu,
                          int dtype, hipStream_t stream) {
    const char* fn = "fwa_delta_step";
    if (!valid_dtype(dtype)) return fail(FWA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (B < 0 || H < 0) return fail(FWA_ERR_INVALID_ARG, "%s: negative B/H", fn);
    if (d_k < 1 || d_v < 1) return fail(FWA_ERR_INVALID_ARG, "%s: d_k and d_v must be >= 1", fn);
    if (nu < 1 || nu > 2 * d_k - 1)
        return fail(FWA_ERR_INVALID_ARG, "%s: nu=%d outside [1, 2*d_k-1]", fn, nu);
    const int64_t BH = static_cast<int64_t>(B) * H;
    if (BH == 0) return ok();
    if (!q || !k || !v || !beta_logit || !W || !y)
        return fail(FWA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    const void* ptrs[] = {q, k, v, beta_logit, W, y};
    for (const void* p : ptrs)
        if (!aligned16(p))
            return fail(FWA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    if (d_k != 16 && d_k != 32 && d_k != 64 && d_k != 128)
        return fail(FWA_ERR_UNSUPPORTED, "%s: d_k=%d not in {16,32,64,128}", fn, d_k);
    const int64_t D = 2 * static_cast<int64_t>(d_k) * nu;
    int LR = 0;
    if (D > 1024 || fwa::step_cpl_for(static_cast<int>(D), &LR) == 0)
        return fail(FWA_ERR_UNSUPPORTED, "%s: D=%lld has no row layout (D <= 1024, D/4 = 8..64 x 1..4)",
                    fn, (long long)D);
    if (!mul_le(kIndexLimit, {BH, d_v, D}) || BH > (int64_t(1) << 31) - 1)
        return fail(FWA_ERR_UNSUPPORTED, "%s: sizes overflow the index range", fn);
    const int es = elem_bytes(dtype);
    const Span sW = span(W, BH * d_v * D * 4), sy = span(y, BH * d_v * es);
    const Span in[] = {span(q, BH * d_k * es), span(k, BH * d_k * es), span(v, BH * d_v * es),
                       span(beta_logit, BH * es)};
    for (const Span& s : in)
        if (overlap(s, sW) || overlap(s, sy))
            return fail(FWA_ERR_INVALID_ARG, "%s: an output overlaps an input", fn);
    if (overlap(sW, sy)) return fail(FWA_ERR_INVALID_ARG, "%s: y overlaps W", fn);
    return hip_status(fwa::launch_delta_step(q, k, v, beta_logit, W, y, BH, d_k, d_v, nu,
                                             dtype == FWA_BF16, stream),
                      "fwa_delta_step launch");
}

}  // extern "C"
