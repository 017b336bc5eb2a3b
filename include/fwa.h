/*
 * fwa.h -- C ABI of the MI355X (gfx950) fast-weight delta-rule layer with DPFP projection.
 *
 * The method (sources are web pages, cited by title and section):
 *   [FWT] "Fast Weights Transformer" technical guide for the labml annotated implementation,
 *         xdnf.cn/news/308600;
 *   [FWA] "Deep dive into Fast Weight Attention (lucidrains)", gitcode.csdn.net;
 *   [TRF] "Transformer", wineandchord.com/llm/architecture/transformer/.
 *
 *   DPFP    phi(k): x = relu([k, -k]) (length 2*d_k); for shift i = 1..nu the block at
 *           offset (i-1)*2*d_k holds x[j] * x[(j - i) mod 2*d_k] (x times x rolled by +i);
 *           then phi = raw / (sum(raw) + 1e-6).  D = d_dot = 2*d_k*nu.
 *           [FWT] sections "DPFP / projection formula and hyper-parameters", "DPFP /
 *           normalisation".
 *   step    per (batch, head), with beta = sigmoid(beta_logit):
 *             v_bar = W phi(k);  W <- W + beta (v - v_bar) phi(k)^T;  y = W phi(q)
 *           (the read uses the W just written).  [FWT] sections "FastWeightsAttention /
 *           update formula" and "FastWeightsAttention / module structure and source
 *           walkthrough".  No 1/sqrt(d) scale and no z normaliser.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  Every launch goes on
 *     `stream` (0 = the legacy default stream) and FWA_OK means "enqueued".  No entry point
 *     allocates device memory, frees it or synchronises a stream; scratch memory comes from
 *     the caller (fwa_delta_forward's workspace).  The only state the library keeps between
 *     calls is which kernels already carry their LDS-size attribute and how many workgroups
 *     of a kernel fit on a device (both fixed per device), so a call after a first one on
 *     the same device can be captured into a HIP graph.
 *   - Layouts are row-major and contiguous (the [B, H, T, d] convention of [TRF], section
 *     "Scaled dot-product attention").  The fast-weight memory W is [B, H, d_v, D] fp32
 *     (d_value x d_key orientation of [FWT], module walkthrough).
 *   - `dtype` is the element type of q, k, v, beta_logit, y and phi (FWA_F32 or FWA_BF16);
 *     W is always fp32.  Arithmetic is fp32 with fp32 state; bf16 results are rounded to
 *     nearest-even.
 *   - Arguments are checked on the host before anything is launched.  On any error nothing
 *     is launched and no output is written:
 *       FWA_ERR_INVALID_ARG   a required pointer is NULL, a size is negative, d_k < 1,
 *                             d_v < 1, nu outside [1, 2*d_k - 1] (the range [FWT] gives for
 *                             nu), chunk not in {16, 32, 64, 128}, an unknown dtype, or a
 *                             pointer not aligned to 16 bytes;
 *       FWA_ERR_UNSUPPORTED   valid arguments outside the shapes the kernels implement
 *                             (listed per entry point), or sizes whose index arithmetic would
 *                             overflow 64 bits;
 *       FWA_ERR_HIP           the HIP runtime rejected a launch (the message is available
 *                             from fwa_last_error()).
 *   - Inputs holding NaN or Inf give unspecified values but never a fault.
 */
#ifndef FWA_H
#define FWA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FWA_OK = 0,
    FWA_ERR_INVALID_ARG = 1,
    FWA_ERR_UNSUPPORTED = 2,
    FWA_ERR_HIP = 3
} fwa_status;

/* Element types.  Entry points take the value as a plain int `dtype` (any other value is
 * rejected with FWA_ERR_INVALID_ARG), so a caller may pass what it likes without undefined
 * behaviour in the library. */
typedef enum {
    FWA_F32 = 0,
    FWA_BF16 = 1
} fwa_dtype;

/* Implementation of fwa_delta_forward (see there). */
typedef enum {
    FWA_PATH_AUTO = 0,      /* request only: the planner's choice (what fwa_delta_forward does) */
    FWA_PATH_CHUNKED = 1,
    FWA_PATH_FUSED = 2,
    FWA_PATH_STREAM = 3,
    FWA_PATH_NONE = 4       /* report only: nothing to launch (B*H == 0) */
} fwa_forward_path;

/*
 * fwa_dpfp -- phi[n, :] = DPFP(x[n, :]) for n in [0, n_vec).
 *   [FWT] sections "DPFP / projection formula and hyper-parameters" and "DPFP /
 *   normalisation" (eps = 1e-6, added to the sum).
 *   x    [n_vec, d_k]        input, `dtype`
 *   phi  [n_vec, 2*d_k*nu]   output, `dtype`; entry (i-1)*2*d_k + j is the shift-i product
 *                            at position j.  Exact zeros are written as +0.0.
 *   n_vec == 0 is a no-op.
 *   Implemented shapes: d_k in {16, 32, 64, 128}, any valid nu.
 */
fwa_status fwa_dpfp(const void* x, void* phi, int64_t n_vec, int d_k, int nu,
                    int dtype, hipStream_t stream);

/*
 * fwa_delta_forward -- causal forward of the delta rule over T steps for every (b, h),
 * starting from W0 and returning the final memory.
 *   [FWT] section "FastWeightsAttention / module structure and source walkthrough" (the
 *   per-step loop this reproduces), [FWA] section 4.2 (chunked processing that passes the
 *   memory between chunks and returns it).
 *   q, k        [B, H, T, d_k]  `dtype`
 *   v           [B, H, T, d_v]  `dtype`
 *   beta_logit  [B, H, T]       `dtype`  (pre-sigmoid; beta = sigmoid(beta_logit))
 *   W0          [B, H, d_v, D]  fp32, or NULL for a zero initial memory ([FWT]'s default)
 *   y           [B, H, T, d_v]  `dtype`, output: y_t = W_t phi(q_t) after the step-t write
 *   W_final     [B, H, d_v, D]  fp32 output, or NULL to skip it; may equal W0 (in-place
 *                               carry), must not overlap any other argument
 *   chunk       rows per chunk of the chunk-parallel evaluation, one of {16, 32, 64, 128}.
 *               It changes only the rounding order: results agree for every chunk within
 *               the stated tolerances.
 *   T == 0 leaves y untouched and writes W_final = W0 (or zeros).  B*H == 0 is a no-op.
 *   T need not be a multiple of chunk.
 *   workspace   device scratch owned by the caller, at least the bytes fwa_delta_forward_info
 *               reports for the same sizes (NULL / 0 where that is 0), 16-byte aligned, not
 *               overlapping any other argument.  The call's kernels use it in stream order on
 *               `stream`; the caller keeps it alive and unused by other work until they have
 *               run (memory from a stream-ordered allocator on `stream` satisfies this).  Its
 *               contents on entry do not matter and are undefined on return.  Too small a
 *               workspace gives FWA_ERR_INVALID_ARG before anything is launched.
 *   Three implementations compute the same result (within the tolerances above); the planner
 *   picks one from the sizes alone:
 *     chunked  every chunk's memory-independent part in parallel, then the memory carried
 *              through the chunks.  The chain forms the outputs itself for fp32 with D in
 *              {64, 128} and for bf16 at chunk 64 with D in {128, 256} (two launches; y of
 *              one (b, h) under 2 GiB); otherwise a third launch forms them from the
 *              chunk-start memories and U that the chain leaves in the workspace.  The
 *              workspace holds B*H*ceil(T/chunk) * (3*chunk*D + chunk*chunk) elements of
 *              `dtype`, plus B*H*ceil(T/chunk) * (D*d_v + chunk*d_v) more where the third
 *              launch runs, plus B*H*ceil(T/chunk)*chunk*(d_v + 2) fp32 values.  Chunks of
 *              32 or 64 rows; D in {32, 64, 96, 128, 192, 256}, and for bf16 also 384, 512;
 *              the prep kernel's working set (2*chunk*(D + 8) elements plus chunk-sized
 *              scratch) must fit the 160 KiB of LDS, which leaves out chunk 64 for fp32 D = 256
 *              and bf16 D = 512.
 *     stream   bf16 only, two launches: every chunk's (I + L)^-1 diag(beta), P~ and DPFP
 *              normalisers in parallel, then one serial pass per (b, h, 32 columns of d_v)
 *              that rebuilds the DPFP features from the raw rows and keeps the memory on chip.
 *              Workspace of B*H*ceil(T/chunk) * (3*S + 2*chunk*4) bytes, S the bytes of one
 *              chunk's block-lower-triangular operand matrix: for d_k = 64 only its 16 x 32
 *              blocks on and below the diagonal, S = 1024*(chunk/32)*(chunk/32 + 1) (18.5 KiB
 *              per chunk of 64, 61 KiB per chunk of 128); for d_k = 16 and 32 the full
 *              S = chunk*chunk*2 (24.5 KiB per chunk of 64).
 *              Chunk 64: d_v in {32, 64}, D in {128, 256, 384}, nu <= 8; and, for d_k = 64
 *              with nu <= 4, also d_v = 16 and D = 512.  Chunk 128: d_k = 64, nu <= 4,
 *              d_v in {32, 64} (the DPFP features are built one shift block of 128 columns
 *              at a time, so D up to 512 fits on chip).
 *     fused    one launch that keeps the chunk and the memory on chip; no workspace.
 *              Needs the chunk's working set (3*chunk*D elements plus chunk-sized scratch)
 *              within the 160 KiB of LDS of one compute unit.
 *   The planner takes the chunked path where it applies, its workspace is at most 2 GiB and
 *   the streaming path does not fill the GPU (B*H*(d_v/32) serial workgroups of at least 128,
 *   or 64 at D >= 384); else the streaming one where it applies, else the fused one.
 *   Implemented shapes: d_k in {16, 32, 64}, d_v in {16, 32, 64}, D = 2*d_k*nu <= 512, and
 *   the conditions of at least one implementation above; other valid shapes give
 *   FWA_ERR_UNSUPPORTED.
 */
fwa_status fwa_delta_forward(const void* q, const void* k, const void* v,
                             const void* beta_logit, const float* W0, void* y, float* W_final,
                             int B, int H, int T, int d_k, int d_v, int nu, int chunk,
                             int dtype, void* workspace, int64_t workspace_bytes,
                             hipStream_t stream);

/*
 * fwa_delta_forward_path -- fwa_delta_forward with the implementation named by `request`
 * (an fwa_forward_path: FWA_PATH_AUTO is exactly fwa_delta_forward).  For callers that must
 * pin the implementation, such as tests that check each one against the others.  A named
 * implementation that does not take the sizes gives FWA_ERR_UNSUPPORTED; an unknown request
 * FWA_ERR_INVALID_ARG.  Same sources, arguments, workspace rule and errors otherwise.
 */
fwa_status fwa_delta_forward_path(int request, const void* q, const void* k, const void* v,
                                  const void* beta_logit, const float* W0, void* y,
                                  float* W_final, int B, int H, int T, int d_k, int d_v, int nu,
                                  int chunk, int dtype, void* workspace,
                                  int64_t workspace_bytes, hipStream_t stream);

/*
 * fwa_delta_forward_noalloc -- fwa_delta_forward for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments as fwa_delta_forward without the workspace, same
 * results and errors.  Its scratch is a static device array of 64 MiB (FWA_NOALLOC_SCRATCH_BYTES)
 * that each GPU the library runs on holds until the process ends; the call allocates nothing.
 * Where the planner's implementation needs more scratch than that, the fused implementation
 * (which needs none) runs instead; where that does not take the sizes either, the call returns
 * FWA_ERR_UNSUPPORTED before launching anything.  Every call on one GPU shares that GPU's
 * scratch: calls that may overlap in time on one GPU (different streams, or host threads
 * without ordering) race and must not be issued; calls in order on one stream are safe.  The
 * scratch needs no initial contents.
 */
#define FWA_NOALLOC_SCRATCH_BYTES (64ll << 20)
fwa_status fwa_delta_forward_noalloc(const void* q, const void* k, const void* v,
                                     const void* beta_logit, const float* W0, void* y,
                                     float* W_final, int B, int H, int T, int d_k, int d_v, int nu,
                                     int chunk, int dtype, hipStream_t stream);

/*
 * fwa_delta_forward_info -- which implementation a forward call with `request` (an
 * fwa_forward_path; FWA_PATH_AUTO for fwa_delta_forward) takes for these sizes and the
 * workspace bytes it needs, without touching the device.
 *   path             out (may be NULL): FWA_PATH_CHUNKED, _STREAM, _FUSED or _NONE
 *   workspace_bytes  out (may be NULL): bytes of workspace the call needs (chunked and stream
 *                    paths), 0 for fused
 *   Size errors are those the forward gives for the same sizes; outputs are untouched on error.
 */
fwa_status fwa_delta_forward_info(int B, int H, int T, int d_k, int d_v, int nu, int chunk,
                                  int dtype, int request, int* path,
                                  int64_t* workspace_bytes);

/*
 * fwa_delta_backward -- gradient of fwa_delta_forward: given dy = dL/dy and dW_final =
 * dL/dW_final, returns dL/dq, dL/dk, dL/dv, dL/dbeta_logit and dL/dW0 for the same inputs.
 *   The pages train this layer with a cross-entropy loss and gradient clipping ([FWT] section
 *   "Training experiment"), which takes the derivative of the forward of [FWT] sections
 *   "FastWeightsAttention / update formula" and "DPFP"; this is that derivative (ReLU's
 *   derivative at 0 taken as 0).
 *   q, k, v, beta_logit, W0   the forward's inputs, as fwa_delta_forward takes them (W0 NULL
 *                             for zeros)
 *   dy          [B, H, T, d_v]  `dtype`
 *   dW_final    [B, H, d_v, D]  fp32, or NULL when the loss does not depend on W_final
 *   dq, dk      [B, H, T, d_k]  `dtype`, output
 *   dv          [B, H, T, d_v]  `dtype`, output
 *   dbeta_logit [B, H, T]       `dtype`, output
 *   dW0         [B, H, d_v, D]  fp32 output, or NULL to skip it
 *   workspace   caller-owned device scratch of at least the bytes fwa_delta_backward_info
 *               reports, under the same rule as fwa_delta_forward's
 *   The memory is recomputed (no forward state is taken from the caller).  Outputs must not
 *   overlap the inputs, each other or the workspace.  T == 0 writes dW0 = dW_final (or zeros).
 *   Arithmetic is fp32 throughout (fp32 state and gradients), chunks of 32 rows.
 *   Implemented shapes: d_k in {16, 32, 64}, d_v <= 64, D = 2*d_k*nu <= 384.
 */
fwa_status fwa_delta_backward(const void* q, const void* k, const void* v,
                              const void* beta_logit, const float* W0, const void* dy,
                              const float* dW_final, void* dq, void* dk, void* dv,
                              void* dbeta_logit, float* dW0, int B, int H, int T, int d_k,
                              int d_v, int nu, int dtype, void* workspace,
                              int64_t workspace_bytes, hipStream_t stream);

/*
 * fwa_delta_backward_info -- the workspace bytes fwa_delta_backward needs for these sizes
 * (0 when B*H == 0), without touching the device.  Size errors are those of the backward.
 */
fwa_status fwa_delta_backward_info(int B, int H, int T, int d_k, int d_v, int nu,
                                   int dtype, int64_t* workspace_bytes);

/*
 * fwa_sum_forward -- causal sum-update linear attention with the z normaliser over DPFP
 * features, for every (b, h):
 *     W_t = W_{t-1} + v_t phi(k_t)^T,  z_t = z_{t-1} + phi(k_t),  y_t = W_t phi(q_t) / (z_t . phi(q_t))
 *   [FWT] section "Background / fast computation form of linear self-attention" (the form the
 *   delta rule replaces: attention with the kernel phi(k)^T phi(q), computed recurrently).
 *   Where the denominator z_t . phi(q_t) is exactly 0, y_t is 0.
 *   q, k        [B, H, T, d_k]  `dtype`
 *   v, y        [B, H, T, d_v]  `dtype` (y output)
 *   W0          [B, H, d_v, D]  fp32 or NULL (zeros);  z0 [B, H, D] fp32 or NULL (zeros)
 *   W_final     [B, H, d_v, D]  fp32 output or NULL;   z_final [B, H, D] fp32 output or NULL;
 *                               W_final may equal W0 and z_final z0 (in-place carry)
 *   workspace   caller-owned device scratch of at least the bytes fwa_sum_forward_info reports,
 *               under fwa_delta_forward's rule
 *   Arithmetic is fp32 (fp32 state), chunks of 32 rows.  T == 0 copies the initial state.
 *   Implemented shapes: d_k in {16, 32, 64}, d_v <= 128, D = 2*d_k*nu <= 384.
 */
fwa_status fwa_sum_forward(const void* q, const void* k, const void* v, const float* W0,
                           const float* z0, void* y, float* W_final, float* z_final, int B, int H,
                           int T, int d_k, int d_v, int nu, int dtype, void* workspace,
                           int64_t workspace_bytes, hipStream_t stream);

/* fwa_sum_forward_info -- workspace bytes fwa_sum_forward needs (0 when B*H == 0). */
fwa_status fwa_sum_forward_info(int B, int H, int T, int d_k, int d_v, int nu, int dtype,
                                int64_t* workspace_bytes);

/*
 * fwa_layer_project -- the projections in front of the layer, written straight into its
 * head-split inputs: for x [B, T, d_model] and the stacked bias-free weights
 * W_qkvb [2*H*d_k + H*d_v + H, d_model] (rows: H*d_k query, H*d_k key, H*d_v value, then H
 * interpolation-weight rows; out = x W^T), writes q, k [B, H, T, d_k], v [B, H, T, d_v] and
 * beta_logit [B, H, T] (the layer applies the sigmoid).
 *   [FWT] section "FastWeightsAttention / module structure and source walkthrough" (query,
 *   key and value maps without bias, one interpolation-weight scalar per head).
 *   All tensors `dtype`; fp32 accumulation.  d_model, d_k and d_v must be multiples of 8.
 */
fwa_status fwa_layer_project(const void* x, const void* W_qkvb, void* q, void* k, void* v,
                             void* beta_logit, int B, int T, int d_model, int H, int d_k, int d_v,
                             int dtype, hipStream_t stream);

/*
 * fwa_layer_output -- the output map behind the layer, reading its head-split output:
 *   out[b, t, :] = residual[b, t, :] + b_o + W_o concat_h(y[b, h, t, :])
 * with y [B, H, T, d_v], W_o [d_model, H*d_v], b_o [d_model] (or NULL), residual and out
 * [B, T, d_model] (residual may be NULL, or equal out for the in-place residual add the
 * Transformer layer does).  [FWT] same section ("output" linear map) and section "Assembling
 * the Transformer / layer" (the attention residual).  All `dtype`; fp32 accumulation;
 * d_model and d_v multiples of 8.
 */
fwa_status fwa_layer_output(const void* y, const void* W_o, const void* b_o,
                            const void* residual, void* out, int B, int T, int H, int d_v,
                            int d_model, int dtype, hipStream_t stream);

/*
 * fwa_decode_layers -- one new token through L fast-weight attention layers, each with its
 * own memory: for l = 0 .. L-1,
 *   (q, k, v, beta_logit) = fwa_layer_project(x, W_qkvb[l]);
 *   y = fwa_delta_step(q, k, v, beta_logit, W[l]);
 *   x = fwa_layer_output(y, W_o[l], b_o[l], residual = x)
 * with x [B, d_model] (`dtype`) updated in place and every W[l] [B, H, d_v, D] (fp32) updated
 * in place.  [FWT] sections "token_wise variant" (one memory per layer, carried from token to
 * token) and "Inference and sampling".  W_qkvb, W_o, b_o and W are HOST arrays of L device
 * pointers (b_o may be NULL, or hold NULL entries); they are read during the call, so the
 * 3*L launches can be captured into a HIP graph and replayed for later tokens.  workspace: at
 * least fwa_decode_layers_info's bytes (the per-layer q, k, v, beta_logit and y).
 * Implemented shapes: those of fwa_layer_project and fwa_delta_step together.
 */
fwa_status fwa_decode_layers(void* x, int L, const void* const* W_qkvb, const void* const* W_o,
                             const void* const* b_o, float* const* W, int B, int d_model, int H,
                             int d_k, int d_v, int nu, int dtype, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream);

/* fwa_decode_layers_info -- workspace bytes fwa_decode_layers needs. */
fwa_status fwa_decode_layers_info(int B, int d_model, int H, int d_k, int d_v, int nu,
                                  int dtype, int64_t* workspace_bytes);

/*
 * fwa_delta_step -- one decode step (a single new token) for every (b, h), with the memory
 * carried in and out through W, updated in place.
 *   [FWT] sections "token_wise variant" and "Inference and sampling" (each new token updates
 *   the carried fast weights with no recomputation over the history); [TRF] section
 *   "Complexity" (decode streams its state, so it is bandwidth-bound).
 *   q, k        [B, H, d_k]     `dtype`
 *   v           [B, H, d_v]     `dtype`
 *   beta_logit  [B, H]          `dtype`
 *   W           [B, H, d_v, D]  fp32, read and written in place (read once, written once)
 *   y           [B, H, d_v]     `dtype`, output
 *   B*H == 0 is a no-op.  y must not overlap W or the inputs.
 *   Implemented shapes: d_k in {16, 32, 64, 128}, d_v >= 1, D = 2*d_k*nu <= 1024.
 */
fwa_status fwa_delta_step(const void* q, const void* k, const void* v, const void* beta_logit,
                          float* W, void* y, int B, int H, int d_k, int d_v, int nu,
                          int dtype, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* fwa_status_string(fwa_status s);

/* Detail of the most recent non-OK status returned on the calling thread ("" if none). */
const char* fwa_last_error(void);

/* Version of this ABI, as major * 10000 + minor * 100 + patch. */
int fwa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FWA_H */
