// C ABI of the fast-weight delta-rule library: argument checks on the host, then one launch
// on the caller's stream.  Every check runs before any HIP call, so an invalid call touches
// neither the device nor the outputs.
#include "fwa.h"
#include "fwa_internal.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
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

bool valid_dtype(fwa_dtype d) { return d == FWA_F32 || d == FWA_BF16; }
int elem_bytes(fwa_dtype d) { return d == FWA_BF16 ? 2 : 4; }

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

// Forward implementation: FWA_FORWARD_PATH = "chunked" (two or three launches with a D-wide
// workspace), "stream" (bf16: compact prep plus one serial kernel, a 24.5 KB-per-chunk
// workspace), "fused" (one launch, no workspace), or unset / "auto".  Auto takes the chunked
// path where it applies and its workspace stays within kAutoWorkspaceLimit: beyond that the
// workspace traffic (about 7 D-wide rows per token) outweighs the parallelism it buys.  Larger
// bf16 problems take the streaming path where it applies, else the fused kernel.
enum class ForwardPath { kAuto, kChunked, kStream, kFused, kInvalid };
constexpr int64_t kAutoWorkspaceLimit = int64_t(2) << 30;
ForwardPath forward_path() {
    const char* s = std::getenv("FWA_FORWARD_PATH");
    if (!s || !*s || std::strcmp(s, "auto") == 0) return ForwardPath::kAuto;
    if (std::strcmp(s, "chunked") == 0) return ForwardPath::kChunked;
    if (std::strcmp(s, "stream") == 0) return ForwardPath::kStream;
    if (std::strcmp(s, "fused") == 0) return ForwardPath::kFused;
    return ForwardPath::kInvalid;
}

// Workspace of the chunked forward: one buffer per (device, stream), reused by every call on
// that stream (calls on one stream run in order, so reuse needs no synchronisation) and grown
// when a call needs more: the stream is synchronised, the old buffer freed and a larger one
// allocated.  Buffers are held until the process ends.
hipError_t workspace_get(char** ptr, int64_t bytes, hipStream_t stream) {
    static std::mutex mu;
    static std::map<std::pair<int, uintptr_t>, std::pair<char*, int64_t>> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    auto& ent = cache[{dev, reinterpret_cast<uintptr_t>(stream)}];
    if (ent.second < bytes) {
        if (ent.first) {
            if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
            if ((e = hipFree(ent.first)) != hipSuccess) return e;
            ent = {nullptr, 0};
        }
        void* p = nullptr;
        if ((e = hipMalloc(&p, static_cast<size_t>(bytes))) != hipSuccess) return e;
        ent = {static_cast<char*>(p), bytes};
    }
    *ptr = ent.first;
    return hipSuccess;
}
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

int fwa_version(void) { return 1 * 10000 + 1 * 100 + 0; }

fwa_status fwa_dpfp(const void* x, void* phi, int64_t n_vec, int d_k, int nu, fwa_dtype dtype,
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
                               int chunk, fwa_dtype dtype) {
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

// The implementation a forward call takes (FWA_FORWARD_PATH and the shape), with its plan.
struct ForwardChoice {
    int path;                       // FWA_PATH_CHUNKED, FWA_PATH_STREAM or FWA_PATH_FUSED
    fwa::ChunkPlan cplan;
    fwa::StreamPlan splan;
    fwa::FwdPlan fplan;
    int64_t ws_bytes;
};

fwa_status choose_forward(const char* fn, int BH, int T, int d_k, int d_v, int nu, int chunk,
                          bool bf16, ForwardChoice* c) {
    const ForwardPath want = forward_path();
    if (want == ForwardPath::kInvalid)
        return fail(FWA_ERR_INVALID_ARG,
                    "%s: FWA_FORWARD_PATH must be auto, chunked, stream or fused", fn);
    const bool auto_ = want == ForwardPath::kAuto;
    const bool can_chunk = (auto_ || want == ForwardPath::kChunked) &&
                           fwa::plan_chunked(BH, T, d_k, d_v, nu, chunk, bf16, &c->cplan);
    const bool can_stream = (auto_ || want == ForwardPath::kStream) &&
                            fwa::plan_stream(BH, T, d_k, d_v, nu, chunk, bf16, &c->splan);
    const bool can_fuse = (auto_ || want == ForwardPath::kFused) &&
                          fwa::plan_forward(BH, d_k, d_v, nu, chunk, bf16, &c->fplan);
    c->ws_bytes = 0;
    if (can_chunk && (!auto_ || c->cplan.ws_bytes <= kAutoWorkspaceLimit || (!can_stream && !can_fuse))) {
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
    if (want == ForwardPath::kChunked || want == ForwardPath::kStream)
        return fail(FWA_ERR_UNSUPPORTED,
                    "%s: the %s path does not support d_k=%d d_v=%d nu=%d chunk=%d%s", fn,
                    want == ForwardPath::kChunked ? "chunked" : "stream", d_k, d_v, nu, chunk,
                    want == ForwardPath::kStream && !bf16 ? " (it takes bf16 inputs)" : "");
    return fail(FWA_ERR_UNSUPPORTED,
                "%s: d_k=%d d_v=%d nu=%d chunk=%d does not fit the on-chip working set", fn, d_k,
                d_v, nu, chunk);
}

}  // namespace

extern "C" {

fwa_status fwa_delta_forward_info(int B, int H, int T, int d_k, int d_v, int nu, int chunk,
                                  fwa_dtype dtype, int* path, int64_t* workspace_bytes) {
    const char* fn = "fwa_delta_forward_info";
    fwa_status st = check_forward_sizes(fn, B, H, T, d_k, d_v, nu, chunk, dtype);
    if (st != FWA_OK) return st;
    const int64_t BH = static_cast<int64_t>(B) * H;
    int p = FWA_PATH_NONE;
    int64_t ws = 0;
    if (BH > 0) {
        if ((st = check_forward_shape(fn, BH, T, d_k, d_v, nu)) != FWA_OK) return st;
        ForwardChoice c;
        if ((st = choose_forward(fn, static_cast<int>(BH), T, d_k, d_v, nu, chunk,
                                 dtype == FWA_BF16, &c)) != FWA_OK)
            return st;
        p = c.path;
        ws = c.ws_bytes;
    }
    if (path) *path = p;
    if (workspace_bytes) *workspace_bytes = ws;
    return ok();
}

fwa_status fwa_delta_forward(const void* q, const void* k, const void* v, const void* beta_logit,
                             const float* W0, void* y, float* W_final, int B, int H, int T,
                             int d_k, int d_v, int nu, int chunk, fwa_dtype dtype,
                             hipStream_t stream) {
    const char* fn = "fwa_delta_forward";
    fwa_status st = check_forward_sizes(fn, B, H, T, d_k, d_v, nu, chunk, dtype);
    if (st != FWA_OK) return st;
    const int64_t BH = static_cast<int64_t>(B) * H;
    if (BH == 0) return ok();
    if (T > 0 && (!q || !k || !v || !beta_logit || !y))
        return fail(FWA_ERR_INVALID_ARG, "%s: NULL input or output pointer", fn);
    const void* ptrs[] = {q, k, v, beta_logit, W0, y, W_final};
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

    const bool bf16 = dtype == FWA_BF16;
    ForwardChoice c;
    if ((st = choose_forward(fn, static_cast<int>(BH), T, d_k, d_v, nu, chunk, bf16, &c)) != FWA_OK)
        return st;
    if (c.path != FWA_PATH_FUSED) {
        char* ws = nullptr;
        if (c.ws_bytes > 0) {
            const hipError_t e = workspace_get(&ws, c.ws_bytes, stream);
            if (e != hipSuccess)
                return fail(FWA_ERR_HIP, "%s: workspace of %lld bytes: %s", fn,
                            (long long)c.ws_bytes, hipGetErrorString(e));
        }
        if (c.path == FWA_PATH_STREAM)
            return hip_status(fwa::launch_stream(c.splan, q, k, v, beta_logit, W0, y, W_final, ws,
                                                 stream),
                              "fwa_delta_forward launch");
        return hip_status(fwa::launch_chunked(c.cplan, q, k, v, beta_logit, W0, y, W_final, ws,
                                              bf16, stream),
                          "fwa_delta_forward launch");
    }
    return hip_status(fwa::launch_delta_forward(c.fplan, q, k, v, beta_logit, W0, y, W_final,
                                                static_cast<int>(BH), H, T, d_k, d_v, nu, chunk,
                                                bf16, stream),
                      "fwa_delta_forward launch");
}

fwa_status fwa_delta_step(const void* q, const void* k, const void* v, const void* beta_logit,
                          float* W, void* y, int B, int H, int d_k, int d_v, int nu,
                          fwa_dtype dtype, hipStream_t stream) {
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
