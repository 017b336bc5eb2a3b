"""Benchmark of the fast-weight delta-rule layer (DPFP + chunked forward + decode step) on one
MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step of a forward workload is one pass of the whole hot path over one batch: the chunked
causal forward over B x T tokens (DPFP, beta, intra-chunk work, state work, y and the final
memory) followed by one decode step per sequence that continues from that memory.  Tokens per
step = B * (T + 1).  The default workload is the largest, b8_h16_t16384_d64_nu3_bf16 (8 x 16
heads x 16384 tokens, D 384, bf16, chunk 64; --chunk 128 for the sweep's other point).  Inputs
are seeded synthetic tensors (weight_linear_attention_amd/synthetic.py) already resident in HBM
when timing starts.  Other workloads (--workload):
    h8_t1024_d64_nu1_f32, b4_h8_t4096_d64_nu2_bf16_carried, tiny_t64_d16_nu1_f32
                                                                    forward + decode step
    decode_b256_h8_d64_nu1_f32                                      one fwa_delta_step per step
    backward_<forward workload>                                     one fwa_delta_backward
    sum_<forward workload>                                          one fwa_sum_forward (the
                                                                    sum-update form with z)
    layers6_decode_b256_h8_d64_nu1_f32                              one token through 6 layers
                                                                    (fwa_decode_layers, d_model
                                                                    512, random-init weights)
    dpfp_b8_h16_t16384_d64_nu3_bf16                                 fwa_dpfp on q and k
    copy_calibration                                                a 1 GiB device copy (the
                                                                    reference for HBM counters)

--flush (decode and DPFP workloads) reads a 1 GiB scratch buffer before every timed step,
outside the timed events, so that no step finds its data in the 256 MB Infinity Cache; the
rate then comes from per-step event pairs and `roofline.flushed` says so.

Prints ONE JSON line.  `roofline` describes the dominant call: the forward (one launch on the
fused path, two on the streaming path, three on the chunked path) or, for the decode and DPFP
workloads, that kernel.
`achieved` is its algorithmic bytes or flops divided by its mean duration, measured with HIP
events on the launch stream: one event pair around the back-to-back calls, divided by their
number (forward workloads: a second region of back-to-back forwards after the timed steps);
`traffic` is the HBM bytes per call that
rocprofv3 counted on the same sources (profiles/traffic.json), or null.  `cpu_baseline` times
the fp64 oracle on the host (rank 0 only).
"""
import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBPS = 8000.0
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}
PEAK_VALU_F32_TFLOPS = 157.3   # 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2 issue x 2.4 GHz
DEFAULT_WORKLOAD = "b8_h16_t16384_d64_nu3_bf16"
WARMUP_SECONDS = 0.3       # default warm-up length
DECODE_WARM_SLICES = 64    # decode: input slices the warm-up cycles through
FLUSH_BYTES = 1 << 30      # --flush: scratch read before every timed step


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--chunk", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--flush", action="store_true",
                   help="decode and DPFP workloads: read a 1 GiB scratch buffer before every timed "
                        "step (outside the timed events), so no step finds its data in the 256 MB "
                        "Infinity Cache; the rate is summed from per-step event pairs")
    return p.parse_args()


# Kernel sources behind each measured unit (their hash keys the committed counter data).
SOURCES = {
    "chunked": ("chunked_kernels.h", "chunk_tile.h"),
    "stream": ("stream_kernel.h", "stream_bf16_c64.hip", "stream_sliced.h", "stream_sliced_bf16.hip",
               "chunked_kernels.h", "chunk_tile.h"),
    "fused": ("forward_kernel.h", "chunk_tile.h"),
    "decode": ("step_kernel.hip",),
    "dpfp": ("dpfp_kernel.hip",),
    "backward": ("backward.hip", "chunk_f32.h"),
    "sum": ("sum_forward.hip", "chunk_f32.h"),
    "layers": ("projection.hip", "step_kernel.hip"),
}


def kernel_source_hash(unit):
    h = hashlib.sha256()
    for name in SOURCES[unit]:
        with open(os.path.join(HERE, "weight_linear_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stream_kernels(w):
    """Kernel names of the streaming path for this shape, by the planner's rule (chunk 128: the
    shift-sliced prep and serial kernels; chunk 64: the sliced prep for d_k 64 and nu <= 4, then
    the pipelined serial kernel for d_k 64 and nu <= 3, the full-tile one where it applies, else
    the sliced one)."""
    sliced_prep = w.d_k == 64 and w.nu <= 4
    full_ok = w.chunk == 64 and w.d_v % 32 == 0 and w.D % 128 == 0 and w.nu <= 8 and w.D <= 384
    if w.chunk == 128 or not full_ok:
        return "delta_prep_sliced_kernel + delta_stream_sliced_kernel"
    serial = "delta_stream_pipe_kernel" if w.d_k == 64 and w.nu <= 3 else "delta_stream_kernel"
    return ("delta_prep_sliced_kernel" if sliced_prep else "delta_prep_kernel (compact)") + \
        " + " + serial


def chunked_kernels(w):
    """Kernel names of the chunked path for this shape, by the planner's rule: the prep as two
    workgroups per chunk (K side, Q side) at chunk 64 with D a multiple of 128 where twice the
    chunks fit the GPU at once (one prep workgroup per CU at these sizes); the staged chain for
    fp32 D 64 / 128 and bf16 D 128 / 256, as its direct variant for bf16 at chunk 64, both
    forming the outputs themselves."""
    chunks = w.B * w.H * -(-w.T // w.chunk)
    split = w.chunk == 64 and w.D % 128 == 0 and 2 * chunks <= 256
    prep = "delta_prep_split_kernel" if split else "delta_prep_kernel"
    if w.dtype == "f32" and w.D in (64, 128):
        return prep + " + delta_chain_staged_kernel (outputs in the chain)"
    if w.dtype == "bf16" and w.D in (128, 256) and w.chunk == 64:
        return prep + " + delta_chain_direct_kernel (outputs in the chain)"
    if w.dtype == "bf16" and w.D in (128, 256):
        return prep + " + delta_chain_staged_kernel + delta_output_kernel"
    return prep + " + delta_chain_kernel + delta_output_kernel"


def measured_traffic(unit, workload):
    """HBM bytes per call from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources for this workload; otherwise None."""
    path = os.path.join(HERE, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    ent = table.get(f"{unit}:{workload}")
    if not ent or ent.get("source_sha256_16") != kernel_source_hash(unit):
        return None
    return ent.get("bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from weight_linear_attention_amd import fwa
    from weight_linear_attention_amd.synthetic import (WORKLOADS, make_decode_inputs,
                                                       make_inputs, workload)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = args.workload
    if name == "copy_calibration":
        # A plain device-to-device copy of a known size (1 GiB read + 1 GiB written): the
        # reference that HBM byte counters (FETCH_SIZE, WRITE_SIZE) are scaled against.
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dst.copy_(src)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        print(json.dumps({"workload": "copy_calibration", "bytes_read": 4 * n,
                          "bytes_written": 4 * n, "seconds": dt}), flush=True)
        return
    kind = "prefill+decode"
    n_layers = 0
    if name.startswith("dpfp_"):
        kind, w = "dpfp", workload(name[len("dpfp_"):])
    elif name.startswith("decode_"):
        kind, w = "decode", workload(name)
    elif name.startswith("backward_"):
        kind, w = "backward", workload(name[len("backward_"):])
    elif name.startswith("sum_"):
        kind, w = "sum", workload(name[len("sum_"):])
    elif name.startswith("layers"):
        n_layers = int(name[len("layers"):name.index("_")])
        kind, w = "layers", workload(name[name.index("_") + 1:])
    else:
        w = workload(name)
    if args.chunk is not None:
        w = workload(w.name, chunk=args.chunk)
    steps = args.steps if args.steps is not None else {
        "prefill+decode": 100 if w.B * w.H * w.T >= (1 << 20) else 1000,
        "decode": 1024, "dpfp": 50, "backward": 20, "sum": 50, "layers": 256}[kind]
    # Warm-up: --warmup steps, else as many as fill WARMUP_SECONDS (at least 3): the GPU's
    # clocks reach their steady state only after some tens of milliseconds of work.
    warmup = args.warmup
    es = 2 if w.dtype == "bf16" else 4
    D, BH = w.D, w.B * w.H

    # ------------------------------------------------------------------ inputs in HBM
    nxt = None
    if kind == "layers":
        # random-init weights of the projections and output maps (N(0, 1/fan_in)), one token
        # embedding per step, a zero memory per layer
        d_model = w.H * w.d_k
        gl = torch.Generator().manual_seed(w.seed + 11)
        Nq = 2 * w.H * w.d_k + w.H * w.d_v + w.H
        layer_w = [(torch.randn(Nq, d_model, generator=gl).div(d_model ** 0.5).to(w.torch_dtype).to(dev),
                    torch.randn(d_model, w.H * w.d_v, generator=gl).div((w.H * w.d_v) ** 0.5).to(w.torch_dtype).to(dev),
                    (0.1 * torch.randn(d_model, generator=gl)).to(w.torch_dtype).to(dev))
                   for _ in range(n_layers)]
        mems = [torch.zeros(w.B, w.H, w.d_v, w.D, device=dev) for _ in range(n_layers)]
        toks = torch.randn(64, w.B, d_model, generator=gl).to(w.torch_dtype).to(dev)
        xl = torch.empty(w.B, d_model, dtype=w.torch_dtype, device=dev)
        inp = None
    elif kind == "decode":
        # DECODE_WARM_SLICES slices for the warm-up (cycled), then one fresh slice per timed step
        inp = make_decode_inputs(w, steps=DECODE_WARM_SLICES + steps)
        d = {k: v.to(dev) for k, v in inp.items()}
        W = d["W0"].clone()
    else:
        inp = make_inputs(w)
        d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    if kind == "backward":
        from weight_linear_attention_amd.synthetic import make_cotangents
        cot = {k: (None if v is None else v.to(dev)) for k, v in make_cotangents(w).items()}
    if kind == "prefill+decode":
        g = torch.Generator().manual_seed(w.seed + 7)
        nxt = {n: torch.randn(w.B, w.H, dd, generator=g).to(w.torch_dtype).to(dev)
               for n, dd in (("q", w.d_k), ("k", w.d_k), ("v", w.d_v))}
        nxt["beta_logit"] = torch.randn(w.B, w.H, generator=g).to(w.torch_dtype).to(dev)
    y = Wf = phi_q = phi_k = ws = None
    if kind == "prefill+decode":
        y = torch.empty(w.B, w.H, w.T, w.d_v, dtype=w.torch_dtype, device=dev)
        Wf = torch.empty(w.B, w.H, w.d_v, D, dtype=torch.float32, device=dev)
        unit, ws_bytes = fwa.delta_forward_info(w.B, w.H, w.T, w.d_k, w.d_v, w.nu, w.chunk,
                                                w.torch_dtype)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    if kind == "dpfp":
        phi_q = torch.empty(w.B, w.H, w.T, D, dtype=w.torch_dtype, device=dev)
        phi_k = torch.empty_like(phi_q)
    ystep = torch.empty(w.B, w.H, w.d_v, dtype=w.torch_dtype, device=dev)

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def forward():
        fwa.delta_forward(d["q"], d["k"], d["v"], d["beta_logit"], d["W0"], chunk=w.chunk,
                          nu=w.nu, out=y, W_final=Wf, workspace=ws)

    def decode_next():
        fwa.delta_step(nxt["q"], nxt["k"], nxt["v"], nxt["beta_logit"], Wf, nu=w.nu, out=ystep)

    def one_step(i):
        if kind == "prefill+decode":
            forward()
            decode_next()
        elif kind == "decode":
            fwa.delta_step(d["q"][i], d["k"][i], d["v"][i], d["beta_logit"][i], W, nu=w.nu,
                           out=ystep)
        elif kind == "backward":
            fwa.delta_backward(d["q"], d["k"], d["v"], d["beta_logit"], cot["dy"], W0=d["W0"],
                               dW_final=cot["dW_final"], nu=w.nu)
        elif kind == "sum":
            fwa.sum_forward(d["q"], d["k"], d["v"], d["W0"], nu=w.nu)
        elif kind == "layers":
            xl.copy_(toks[i % toks.shape[0]])
            fwa.decode_layers(xl, layer_w, mems, w.H, w.d_k, w.d_v, w.nu)
        else:
            fwa.dpfp(d["q"], w.nu, out=phi_q)
            fwa.dpfp(d["k"], w.nu, out=phi_k)

    def region(fn, n):
        """Milliseconds per call of fn over n back-to-back calls inside one event pair."""
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    # Every step runs back to back, as a serving loop would, inside one event pair around the
    # timed region (an event recorded between two launches stalls the queue for a few
    # microseconds, so no call inside the region is bracketed).  For the forward workloads a
    # second region of back-to-back forwards alone (and a third of decode steps alone) then
    # gives the forward's mean duration for the roofline.
    warm_idx = lambda i: i % DECODE_WARM_SLICES if kind == "decode" else i
    if warmup is None:
        warmup, t_w = 0, time.perf_counter()
        while warmup < 3 or time.perf_counter() - t_w < WARMUP_SECONDS:
            one_step(warm_idx(warmup))
            warmup += 1
            if warmup % 64 == 0:
                torch.cuda.synchronize()
    else:
        for i in range(warmup):
            one_step(warm_idx(i))
    torch.cuda.synchronize()
    flush = args.flush and kind in ("decode", "dpfp")
    step_ms = None
    if flush:
        # Every timed step starts with the caches cold: a 1 GiB read (4x the Infinity Cache)
        # goes before it, outside its event pair; value and duration come from the step events.
        # A read, not a write, so that the step does not also pay for writing back dirty lines.
        scratch = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        pairs = [(ev(), ev()) for _ in range(steps)]
        for i in range(steps):
            torch.sum(scratch, dim=0, out=sink)
            pairs[i][0].record()
            one_step(DECODE_WARM_SLICES + i if kind == "decode" else i)
            pairs[i][1].record()
        torch.cuda.synchronize()
        main_ms = sum(a.elapsed_time(b) for a, b in pairs) / steps
        elapsed = main_ms * 1e-3 * steps
        del scratch
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step_region_ms = region(lambda i: one_step(DECODE_WARM_SLICES + i if kind == "decode" else i),
                                steps)
        elapsed = time.perf_counter() - t0
        if kind == "prefill+decode":
            main_ms = region(lambda i: forward(), steps)
            step_ms = region(lambda i: decode_next(), steps)
        else:
            main_ms = step_region_ms

    # ------------------------------------------------------------------ metric + roofline
    if kind == "prefill+decode":
        tokens = w.B * (w.T + 1)
    elif kind in ("backward", "sum"):
        tokens = w.B * w.T
    elif kind in ("decode", "layers"):
        tokens = w.B
    else:
        tokens = 2 * BH * w.T          # DPFP vectors (q and k) per step
    value = tokens * steps / elapsed

    if kind == "prefill+decode":
        flops = BH * w.T * (6 * D * w.d_v + 6 * D)
        nbytes = (BH * w.T * ((3 * w.d_k + 1) * es + w.d_v * es)
                  + BH * w.d_v * D * 4 * (1 + (d["W0"] is not None)))
        t_mfma = flops / (PEAK_TFLOPS[w.dtype] * 1e12)
        t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9)
        if t_mfma >= t_hbm:
            ach = flops / (main_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": ach, "peak": PEAK_TFLOPS[w.dtype],
                    "unit": "TFLOP/s", "frac": ach / PEAK_TFLOPS[w.dtype]}
        else:
            ach = nbytes / (main_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": ach / PEAK_HBM_GBPS}
        kname = {"chunked": "fwa_delta_forward, chunked: " + chunked_kernels(w),
                 "stream": "fwa_delta_forward, stream: " + stream_kernels(w),
                 "fused": "fwa_delta_forward, fused: delta_forward_kernel"}[unit]
        roof.update(kernel=kname, algorithmic_flops=flops, algorithmic_bytes=nbytes,
                    mean_launch_ms=main_ms,
                    timing="one event pair around %d back-to-back forwards" % steps,
                    algorithmic_mfma_frac=flops / (main_ms * 1e-3) / (PEAK_TFLOPS[w.dtype] * 1e12))
        if w.dtype == "f32" and unit == "chunked":
            split_peak = PEAK_TFLOPS["bf16"] / 3.0
            roof["note"] = ("fp32 inputs and state; the prep's and the chain's contractions run on the "
                            "bf16 MFMA with fp32 operands split into bf16 hi + lo pairs (three "
                            "products, about 2^-16 relative); the peak quoted is the fp32 MFMA one")
            roof["split_bf16_ceiling"] = {"peak": split_peak, "unit": "TFLOP/s",
                                          "frac": flops / (main_ms * 1e-3) / 1e12 / split_peak}
    elif kind in ("backward", "sum"):
        unit = kind
        if kind == "backward":
            # the gradient of the literal recurrence: six rank-1 / mat-vec passes over the
            # memory per token-head (12 D d_v) plus DPFP's derivative; no forward recompute
            flops = BH * w.T * (12 * D * w.d_v + 12 * D)
            nbytes = (BH * w.T * ((4 * w.d_k + 2 * w.d_v + 2 + w.d_v) * es)
                      + BH * w.d_v * D * 4 * (2 + (d["W0"] is not None)))
            kname = "fwa_delta_backward: bwd_prep + bwd_states + bwd_chunk_grads + bwd_dpfp"
        else:
            flops = BH * w.T * (4 * D * w.d_v + 9 * D)
            nbytes = (BH * w.T * (2 * w.d_k + 2 * w.d_v) * es
                      + BH * (w.d_v * D + D) * 4 * (1 + (d["W0"] is not None)))
            kname = "fwa_sum_forward: sum_prep + sum_scan + sum_zfinal"
        t_alu = flops / (PEAK_VALU_F32_TFLOPS * 1e12)
        t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9)
        if t_alu >= t_hbm:
            ach = flops / (main_ms * 1e-3) / 1e12
            roof = {"bound": "alu", "achieved": ach, "peak": PEAK_VALU_F32_TFLOPS,
                    "unit": "TFLOP/s", "frac": ach / PEAK_VALU_F32_TFLOPS}
        else:
            ach = nbytes / (main_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": ach / PEAK_HBM_GBPS}
        roof.update(kernel=kname, algorithmic_flops=flops, algorithmic_bytes=nbytes,
                    mean_launch_ms=main_ms,
                    timing="one event pair around %d back-to-back calls" % steps)
    elif kind == "layers":
        unit = "layers"
        d_model = w.H * w.d_k
        Nq = 2 * w.H * w.d_k + w.H * w.d_v + w.H
        per_layer = (BH * (2 * w.d_v * D * 4 + (2 * w.d_k + 1 + 2 * w.d_v) * es * 2)
                     + (Nq * d_model + d_model * w.H * w.d_v + d_model) * es + 2 * w.B * d_model * es)
        nbytes = n_layers * per_layer
        ach = nbytes / (main_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBPS,
                "kernel": f"fwa_decode_layers ({n_layers} x linear_kernel<project> + "
                          "delta_step_kernel + linear_kernel<output>)",
                "algorithmic_bytes": nbytes, "mean_launch_ms": main_ms,
                "timing": "one event pair around %d back-to-back tokens" % steps}
    else:
        if kind == "decode":
            unit = "decode"
            nbytes = BH * (2 * w.d_v * D * 4 + (2 * w.d_k + 1 + 2 * w.d_v) * es)
            kname = "delta_step_kernel"
        else:
            unit = "dpfp"
            nbytes = 2 * BH * w.T * (w.d_k + D) * es
            kname = "dpfp_kernel (q and k launches)"
        ach = nbytes / (main_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBPS, "kernel": kname, "algorithmic_bytes": nbytes,
                "mean_launch_ms": main_ms}
    roof["traffic"] = measured_traffic(
        unit, name if kind in ("dpfp", "decode", "backward", "sum", "layers")
        else f"{w.name}:c{w.chunk}")
    if flush:
        roof["flushed"] = "a 1 GiB scratch read before every timed step; per-step events"

    out = {
        "metric": "tokens/sec through fast-weight layer (fwd + decode step) & % of MFMA/HBM roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": elapsed * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name if kind != "prefill+decode" else
                   f"{w.name}: forward over B*T tokens (chunk {w.chunk}) + 1 decode step per sequence",
                   "B": w.B, "H": w.H, "T": w.T, "d_k": w.d_k, "d_v": w.d_v, "nu": w.nu,
                   "D": D, "chunk": w.chunk, "tokens_per_step": tokens,
                   "initial_memory": "zeros" if w.w0_std is None else f"N(0,{w.w0_std}^2)"},
        "roofline": roof,
        "kernels_ms": {"main": main_ms, "decode_step": step_ms},
    }

    # ------------------------------------------------------------------ CPU baseline
    if not args.no_cpu_baseline:
        extra = (cot if kind == "backward" else
                 (layer_w, n_layers) if kind == "layers" else nxt)
        out["cpu_baseline"] = cpu_baseline(w, kind, inp, extra)
    print(json.dumps(out), flush=True)


def host_cpu():
    """The host's logical CPU count, the CPUs this process may run on, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_count": os.cpu_count(), "usable_cpus": usable, "model": model}


def cpu_baseline(w, kind, inp, nxt):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload, timed on the
    host; the sample is scaled to tokens/s exactly like the GPU value."""
    import numpy as np
    import oracle
    from weight_linear_attention_amd.synthetic import to_f64

    threads = oracle.num_threads()
    host = host_cpu()
    BH = w.B * w.H
    sl = lambda t, n: None if t is None else to_f64(t).reshape(1, BH, *t.shape[2:])[:, :n]
    if kind in ("backward", "sum"):
        # whole (b, h) slices, a bounded sample (at most ~1e10 flops of oracle work per rep)
        per_slice = w.T * w.D * w.d_v * (18 if kind == "backward" else 4)
        nsl = max(1, min(BH, threads, int(1e10 // per_slice)))
        args = [sl(inp[n], nsl) for n in ("q", "k", "v", "beta_logit", "W0")]
        reps, dt, t0 = 0, 0.0, time.perf_counter()
        while dt < 10.0 or reps == 0:
            if kind == "backward":
                oracle.delta_backward(*args, sl(nxt["dy"], nsl), sl(nxt["dW_final"], nsl), nu=w.nu)
            else:
                oracle.sum_forward(args[0], args[1], args[2], args[4], None, nu=w.nu)
            reps += 1
            dt = time.perf_counter() - t0
        tok = w.T * nsl / w.H * reps
        return {"value": tok / dt, "unit": "tokens/s", "cores": min(threads, nsl),
                "kind": "oracle", "sample": f"{nsl} of {BH} (b,h) slices x T={w.T}, {reps} rep(s)",
                "threads": threads, "host": host}
    if kind == "layers":
        layer_w, n_layers = nxt
        d_model = w.H * w.d_k
        lw = [tuple(to_f64(t) for t in p) for p in layer_w]
        Ws = [np.zeros((w.B, w.H, w.d_v, w.D)) for _ in range(n_layers)]
        rng = np.random.default_rng(0)
        reps, dt, t0 = 0, 0.0, time.perf_counter()
        while dt < 10.0 or reps == 0:
            x = rng.normal(size=(w.B, d_model))
            for l, (Wp, Wo, bo) in enumerate(lw):
                q, k, v, bl = oracle.layer_project(x[:, None], Wp, w.H, w.d_k, w.d_v)
                y, Ws[l] = oracle.delta_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], bl[:, :, 0], Ws[l],
                                             nu=w.nu)
                x = oracle.layer_output(y[:, :, None], Wo, bo, x[:, None])[:, 0]
            reps += 1
            dt = time.perf_counter() - t0
        return {"value": w.B * reps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"{reps} token(s) x {w.B} sequences through {n_layers} layers",
                "threads": threads, "host": host}
    if kind == "decode":
        # 16 successive steps over all 2048 (b, h) slices (the oracle's step function)
        S = 16
        Wd = to_f64(inp["W0"])
        t0 = time.perf_counter()
        for s in range(S):
            _, Wd = oracle.delta_step(to_f64(inp["q"][s]), to_f64(inp["k"][s]), to_f64(inp["v"][s]),
                                      to_f64(inp["beta_logit"][s]), Wd, nu=w.nu)
        dt = time.perf_counter() - t0
        return {"value": w.B * S / dt, "unit": "tokens/s", "cores": min(threads, w.B * w.H),
                "kind": "oracle", "sample": f"{S} decode steps x {w.B}x{w.H} slices (full state)",
                "threads": threads, "host": host}
    if kind == "dpfp":
        n = 65536
        x = to_f64(inp["q"].reshape(-1, w.d_k)[:n])
        t0 = time.perf_counter()
        oracle.dpfp(x, w.nu)
        dt = time.perf_counter() - t0
        return {"value": n / dt, "unit": "vectors/s", "cores": threads, "kind": "oracle",
                "sample": f"{n} q vectors", "threads": threads, "host": host}
    # forward (+ decode): whole (b, h) slices, as many as needed for a bounded sample (a
    # multiple of the thread count where the flop cap allows, so every thread has work)
    BH = w.B * w.H
    nsl = min(BH, max(1, threads))
    if w.T * w.D * w.d_v * 6 * nsl > 4e10:      # cap the sample at roughly 1e10..4e10 flops
        nsl = max(1, int(4e10 // (w.T * w.D * w.d_v * 6)))
    q = to_f64(inp["q"]).reshape(1, BH, w.T, w.d_k)[:, :nsl]
    k = to_f64(inp["k"]).reshape(1, BH, w.T, w.d_k)[:, :nsl]
    v = to_f64(inp["v"]).reshape(1, BH, w.T, w.d_v)[:, :nsl]
    l = to_f64(inp["beta_logit"]).reshape(1, BH, w.T)[:, :nsl]
    W0 = None if inp["W0"] is None else to_f64(inp["W0"]).reshape(1, BH, w.d_v, w.D)[:, :nsl]
    reps, dt = 0, 0.0
    t0 = time.perf_counter()
    while dt < 10.0 or reps == 0:
        _, Wf = oracle.delta_forward(q, k, v, l, W0, nu=w.nu)
        if nxt is not None:
            sel = lambda t: to_f64(t).reshape(1, BH, -1)[:, :nsl]
            oracle.delta_step(sel(nxt["q"]), sel(nxt["k"]), sel(nxt["v"]),
                              to_f64(nxt["beta_logit"]).reshape(1, BH)[:, :nsl], Wf, nu=w.nu)
        reps += 1
        dt = time.perf_counter() - t0
    # tokens of the sample, scaled like the GPU metric: a (b, h) slice is 1/H of a sequence
    tok = (w.T + (1 if nxt is not None else 0)) * nsl / w.H * reps
    return {"value": tok / dt, "unit": "tokens/s", "cores": min(threads, nsl), "kind": "oracle",
            "sample": f"{nsl} of {BH} (b,h) slices x T={w.T}"
                      + (" + 1 decode step" if nxt is not None else "") + f", {reps} rep(s)",
            "threads": threads, "host": host,
            "cores_note": "OpenMP threads over independent (b, h) slices: min(threads, slices)"}


if __name__ == "__main__":
    main()
