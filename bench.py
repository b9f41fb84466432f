"""Benchmark: batched routed-MoE FFN prefill on one MI355X.

One step = one full pass of the layer (router logits, routing + int8
quantiser, CSR bucketing, grouped gate/up + SwiGLU GEMM, grouped down GEMM,
ordered combine) over one batch of synthetic tokens, inputs resident in HBM.

Prints ONE JSON line with tokens/s, the roofline fraction of the dominant
kernel (timed live with HIP events on the launch stream) and the CPU oracle's
rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE FFN prefill tokens/sec (OLMoE-shape N=2048) + % int8 MFMA peak"
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
# The gate/up kernel's own roof: per 32-block and 32x32 output tile it issues
# three MFMAs of equal cost on the matrix pipe (the int8 product, the exact
# int32-to-float conversion and the scale outer product), so the pipe caps it
# at a third of the int8 peak.
PIPE_ROOF_TOPS = INT8_PEAK_TOPS / 3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime (recorded by the library on
    the stream it launches on)."""

    def __init__(self):
        self.h = C.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.h.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = C.c_void_p()
            if self.h.hipEventCreate(C.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = C.c_float()
        if self.h.hipEventElapsedTime(C.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.h.hipEventDestroy(e)


def gemm_ops(shape, n_tokens):
    """Useful int8 ops (2 per multiply-add, no padding) of the two grouped GEMMs."""
    P = n_tokens * shape.top_k
    gu = 2 * P * (2 * shape.ffn) * shape.d
    dn = 2 * P * shape.d * shape.ffn
    if shape.shared_ffn:
        gu += 2 * n_tokens * (2 * shape.shared_ffn) * shape.d
        dn += 2 * n_tokens * shape.d * shape.shared_ffn
    return gu, dn


def stage_bytes(shape, n_tokens, counts, fmt="q8_0"):
    """Algorithmic HBM bytes per stage: what the method must read or write
    once (weights of the experts the batch touches, activations, partials).
    Weight bytes per value: Q8_0 34/32, Q4_K 144/256, Q3_K 110/256 (the
    format's bytes; the library reads Q3_K experts from int8 planes)."""
    d, F, k, E = shape.d, shape.ffn, shape.top_k, shape.n_experts
    kk = k + (1 if shape.shared_ffn else 0)
    touched = sum(1 for c in counts[:E] if c > 0)
    q8 = {"q4_k": 144.0 / 256.0, "q3_k": 110.0 / 256.0}.get(fmt, 34.0 / 32.0)
    gu_w = touched * 2 * F * d * q8 + (2 * shape.shared_ffn * d * q8 if shape.shared_ffn else 0)
    dn_w = touched * d * F * q8 + (d * shape.shared_ffn * q8 if shape.shared_ffn else 0)
    P = n_tokens * k + (n_tokens if shape.shared_ffn else 0)
    x_q = n_tokens * d * (1 + 2 / 32)
    h_q = n_tokens * k * F * (1 + 2 / 32) + (n_tokens * shape.shared_ffn * (1 + 2 / 32) if shape.shared_ffn else 0)
    part = n_tokens * kk * d * 4
    return {
        "router_logits": n_tokens * d * 4 + E * d * 4 + n_tokens * E * 4,
        "gateup_swiglu": gu_w + x_q + h_q,
        "down": dn_w + h_q + part,
        "combine": part + n_tokens * k * 4 + n_tokens * d * 4,
        "P": P,
    }


# The sources each measured kernel is compiled from: a traffic summary is
# valid only while their digest matches the one it records.
KERNEL_SOURCES = {
    "grouped_gemm": ("gemm.hip", "gemm_common.h", "internal.h", "device_util.h"),
    "grouped_gemm_q4k": ("gemm_q4k.hip", "gemm_common.h", "internal.h", "device_util.h"),
    "decode_gemv": ("decode.hip", "internal.h", "device_util.h", "route_util.h"),
}


def kernel_source_sha256(family="grouped_gemm"):
    """Digest of the sources a kernel family is compiled from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "mixture_experts_ffn_gemm_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(kernel_tag, family="grouped_gemm"):
    """HBM bytes per launch of a kernel from the committed rocprofv3 PMC
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy kernel's
    reading), valid only while the kernel's sources are unchanged."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            rec[key.strip()] = val.strip()
    if rec.get("sources_sha256") != kernel_source_sha256(family):
        return None
    try:
        return int(float(rec["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_calibration(mib, reps):
    """Launch a plain streaming kernel (read N bytes, write N bytes) so that
    rocprofv3's FETCH_SIZE / WRITE_SIZE readings can be scaled to bytes."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "torch neg (float32, contiguous)",
                                           "bytes_read": n * 4, "bytes_written": n * 4,
                                           "launches": reps}}), flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_pass(layers, x, toks, eps):
    """The sampled tokens through the oracle's layers: one layer is the
    per-token loop on x; a stack is h <- h + layer(RMSNorm(h)) per layer."""
    import numpy as np
    from oracle import oracle as O
    if len(layers) == 1:
        O.moe_tokens(layers[0], x, tokens=toks)
        return
    h = x[toks].astype(np.float32)
    for lw in layers:
        xn = O.rmsnorm(h, eps).astype(np.float32)
        y = O.moe_tokens(lw, xn)["out"]
        h = (h + y.astype(np.float32)).astype(np.float32)


def cpu_baseline(layers, x, target_s, eps=1e-5):
    """The oracle as it stands on a bounded sample of the same workload: m
    tokens (the batch's first m, cycled when m exceeds a small batch) through
    the layer or the whole stack, timed three times with every host thread and
    three times with one; the median of each is reported."""
    import statistics
    from oracle import oracle as O
    n = x.shape[0]
    threads = O.num_threads()

    def timed(m):
        toks = [i % n for i in range(m)]
        t0 = time.perf_counter()
        _oracle_pass(layers, x, toks, eps)
        return time.perf_counter() - t0

    res = {}
    for label, nthr, share, probe in (("all", threads, 0.6, 2 * threads), ("single", 1, 0.4, 2)):
        O.set_num_threads(nthr)
        per = timed(probe) / probe   # seconds per token at this thread count
        m = int(max(probe, min(max(n, probe), share * target_s / 3 / max(per, 1e-9))))
        rates = [m / timed(m) for _ in range(3)]
        res[label] = (statistics.median(rates), rates, m, nthr)
    O.set_num_threads(threads)
    v, rates, m, nthr = res["all"]
    v1, rates1, m1, _ = res["single"]
    what = "one layer (per-token loop: router + top-k + quantiser + k experts + combine)" if len(layers) == 1 \
        else f"the whole {len(layers)}-layer stack (per layer: RMSNorm, per-token layer loop, residual add)"
    return {"value": v, "unit": "tokens/s", "cores": nthr, "kind": "oracle",
            "sample": f"{m} of the batch's {n} tokens through {what}; median of 3 runs "
                      f"({', '.join('%.1f' % r for r in rates)} tokens/s)",
            "cpu_model": cpu_model(),
            "single_thread": {"value": v1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{m1} tokens, median of 3 runs "
                                        f"({', '.join('%.2f' % r for r in rates1)} tokens/s)"}}


def measured_peaks(stream, settle_s=0.3):
    """The int8 matrix-core rate and HBM streaming rate of this GPU, measured
    with the calibration kernels of libmoe_probe.so (timed with HIP events on
    the launch stream, each after settle_s seconds of the same launches, so at
    the clock the GPU holds under that load): the ceilings next to the
    datasheet peaks."""
    import torch
    from mixture_experts_ffn_gemm_amd import build as hb
    P = C.CDLL(hb.PROBE_LIB)
    P.moe_probe_int8_mfma.argtypes = [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    P.moe_probe_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    dev = torch.cuda.current_device()
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    st = stream.cuda_stream

    def time_launches(fn, reps=5):
        t0 = time.perf_counter()
        while True:
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= settle_s:
                break
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    wgs, iters = 2 * n_cu, 4096  # two workgroups of 4 wavefronts per CU: 2 wavefronts per SIMD
    sink = torch.empty(wgs * 256, dtype=torch.int32, device="cuda")

    def mfma():
        if P.moe_probe_int8_mfma(iters, wgs, sink.data_ptr(), st) != 0:
            raise RuntimeError("moe_probe_int8_mfma failed")
    ms = time_launches(mfma)
    tops = wgs * 4 * iters * 4 * 65536 / (ms * 1e-3) / 1e12
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)

    def copy():
        if P.moe_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, st) != 0:
            raise RuntimeError("moe_probe_copy failed")
    ms_c = time_launches(copy)
    gbs = 2 * nbytes / (ms_c * 1e-3) / 1e9
    del src, dst
    return {"int8_mfma_TOPs": round(tops, 1), "copy_GBps": round(gbs, 1),
            "how": f"int8: {wgs} workgroups x 4 wavefronts x {iters} x 4 independent v_mfma_i32_32x32x32_i8, "
                   f"{ms:.3f} ms; copy: 1 GiB read + 1 GiB written with 16-byte loads/stores, {ms_c:.3f} ms"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="olmoe_n2048")
    ap.add_argument("--stack-form", choices=("fused", "fused-graph", "unfused"), default="fused",
                    help="stack workloads: each layer as moe_ffn_prefill_residual (combine + residual + "
                         "RMSNorm in one kernel), the same replayed from one HIP graph of the whole pass, "
                         "or moe_ffn_prefill + moe_ffn_residual_rmsnorm")
    ap.add_argument("--decode-launch", choices=("eager", "graph"), default="eager",
                    help="decode workloads: call moe_ffn_decode directly, or replay one HIP graph of a call "
                         "per timed step")
    ap.add_argument("--chunk", type=int, default=0, metavar="TOKENS",
                    help="prefill workloads: time moe_ffn_prefill_chunked with chunks of TOKENS tokens "
                         "(stages and roofline then describe one chunk-sized call)")
    ap.add_argument("--chunk-order", choices=("forward", "serpentine"), default="serpentine")
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="untimed: run the step back to back for this long before the warmup steps, so that "
                         "the GPU clock has reached its steady state under this load (0 disables it)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="wall-time budget of the CPU oracle sample (0 disables it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain MIB-MiB streaming kernel (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, args.steps))
        return

    import numpy as np
    import torch

    import moe_workloads as mw
    from mixture_experts_ffn_gemm_amd import binding as B
    from mixture_experts_ffn_gemm_amd.layer import MoeLayer

    B.lib()
    wl = mw.WORKLOADS[args.workload]
    s = wl.shape
    n_layers = wl.n_layers
    # decode workloads (1 <= N <= 8) run through moe_ffn_decode
    decode = wl.n_tokens <= 8
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    t0 = time.perf_counter()
    lw = mw.workload_layer(args.workload)
    x_np = mw.workload_tokens(args.workload)
    layer = MoeLayer.from_workload(lw, device=dev)
    n = x_np.shape[0]
    stack = [layer]
    for li in range(1, n_layers):  # a stack: every layer resident in HBM
        stack.append(MoeLayer.from_workload(mw.workload_layer(args.workload, layer=li), device=dev))
        log(f"[bench] {args.workload}: layer {li} created")
    log(f"[bench] {args.workload}: inputs generated in {time.perf_counter() - t0:.1f} s")
    x = torch.from_numpy(x_np).to(dev)
    eps = 1e-5
    if n_layers > 1:
        # the stack's input is h0; each layer sees RMSNorm(h) (unit gain) and
        # adds its output to the residual stream
        h0 = x
        h = torch.empty_like(h0)
        x = torch.empty_like(h0)
        B.moe_ffn_residual_rmsnorm(h0, None, x, n, s.d, eps, stream)
    out = torch.empty((n, s.d), dtype=torch.float32, device=dev)
    ws = layer.workspace(n)
    chunk = args.chunk if (args.chunk and not decode and n_layers == 1) else 0

    def stack_pass(st=stream):
        h.copy_(h0)
        B.moe_ffn_residual_rmsnorm(h, None, x, n, s.d, eps, st)
        for lay in stack:
            if args.stack_form == "unfused":
                B.moe_ffn_prefill(lay.handle, x, n, out, ws, ws.numel(), None, st)
                B.moe_ffn_residual_rmsnorm(h, out, x, n, s.d, eps, st)
            else:  # the next layer's input is written over this one's
                B.moe_ffn_prefill_residual(lay.handle, x, n, h, x, eps, ws, ws.numel(), None, st)
    exp_start = torch.empty(s.n_experts + 1 + (1 if s.shared_ffn else 0), dtype=torch.int32, device=dev)
    step_fn = B.moe_ffn_decode if decode else B.moe_ffn_prefill
    if chunk:
        flags = B.CHUNK_SERPENTINE if args.chunk_order == "serpentine" else 0

        def step_fn(h, xx, nn, oo, w_, wb, r, st):  # the whole batch, chunk by chunk
            B.moe_ffn_prefill_chunked(h, xx, nn, chunk, flags, oo, w_, wb, st)
    step_fn(layer.handle, x, n, out, ws, ws.numel(), B.make_routing(exp_start=exp_start), stream)
    # Clock settling (untimed): from idle the GPU ramps its clock up over tens
    # of milliseconds, so a few warmup steps would time a partly ramped clock.
    settle_t0 = time.perf_counter()
    settle_calls = 0
    while time.perf_counter() - settle_t0 < args.settle_seconds:
        for _ in range(20):
            if n_layers > 1:
                stack_pass()
            else:
                step_fn(layer.handle, x, n, out, ws, ws.numel(), None, stream)
        settle_calls += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step_fn(layer.handle, x, n, out, ws, ws.numel(), None, stream)
    torch.cuda.synchronize()
    counts = np.diff(exp_start.cpu().numpy())

    # Timed region: K plain prefill passes (the product entry point; no events
    # between its kernels), K passes through the whole stack, or K decode
    # calls.
    graph = None
    if decode and args.decode_launch == "graph":
        # one HIP graph of a decode call (kernels only), captured on a side
        # stream and replayed on the timed stream
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                step_fn(layer.handle, x, n, out, ws, ws.numel(), None, torch.cuda.current_stream(dev))
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
    if n_layers > 1:
        for _ in range(args.warmup):
            stack_pass()
        if args.stack_form == "fused-graph":
            # one HIP graph of the whole pass (kernels only, no memset nodes),
            # captured on a side stream and replayed on the timed stream
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream(dev)
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                with torch.cuda.graph(graph, stream=side):
                    stack_pass(torch.cuda.current_stream(dev))
            torch.cuda.synchronize()
            for _ in range(args.warmup):
                graph.replay()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        elif n_layers > 1:
            stack_pass()
        else:
            step_fn(layer.handle, x, n, out, ws, ws.numel(), None, stream)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    if n_layers > 1:
        # the per-stage passes below run the first layer on its normalised input
        B.moe_ffn_residual_rmsnorm(h0, None, x, n, s.d, eps, stream)

    # Then K passes of the profiled entry point: the library records HIP events
    # between its stages on its launch stream (each event adds a dispatch gap,
    # so these passes are slower and are not the timed region).
    hip = HipEvents()
    if decode:
        n_ev, stage_names, prof_fn = B.N_DECODE_STAGE_EVENTS, B.DECODE_STAGES, B.moe_ffn_decode_profiled
    else:
        n_ev, stage_names, prof_fn = B.N_STAGE_EVENTS, B.STAGES, B.moe_ffn_prefill_profiled
    evs = [hip.create(n_ev) for _ in range(args.steps)]
    n_prof = min(n, chunk) if chunk else n   # a chunked run profiles one chunk-sized call
    for i in range(args.steps):
        prof_fn(layer.handle, x, n_prof, out, ws, ws.numel(), evs[i], None, stream)
    torch.cuda.synchronize()
    stage_ms = {name: 0.0 for name in stage_names}
    for i in range(args.steps):
        for j, name in enumerate(stage_names):
            stage_ms[name] += hip.elapsed_ms(evs[i][j], evs[i][j + 1]) / args.steps
    for e in evs:
        hip.destroy(e)

    if chunk:  # the routing of the profiled chunk
        B.moe_ffn_prefill(layer.handle, x, n_prof, out, ws, ws.numel(), B.make_routing(exp_start=exp_start), stream)
        torch.cuda.synchronize()
        counts = np.diff(exp_start.cpu().numpy())
    gu_ops, dn_ops = gemm_ops(s, n_prof)
    sb = stage_bytes(s, n_prof, counts, wl.fmt)
    if decode:
        # decode stages: the router launch also quantises; the gate/up launch
        # also routes
        sb["router_quantise"] = sb.pop("router_logits") + n * s.d * (1 + 2 / 32)
        sb["route_gateup_swiglu"] = sb.pop("gateup_swiglu")
        gu_us = stage_ms["route_gateup_swiglu"] * 1e3
    else:
        gu_us = stage_ms["gateup_swiglu"] * 1e3
    dn_us = stage_ms["down"] * 1e3
    gu_tops = gu_ops / (gu_us * 1e-6) / 1e12
    if decode:
        # a handful of tokens: the matvecs stream each touched expert's weights
        # once, so HBM bandwidth is the roof
        gu_gbs = sb["route_gateup_swiglu"] / (gu_us * 1e-6) / 1e9
        roofline = {"bound": "hbm",
                    "kernel": "decode_gemv_kernel<true> (routing + gathered gate/up int8 matvec + SwiGLU + requantise)",
                    "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                    "traffic": read_traffic(f"decode_gateup_{args.workload}", "decode_gemv"),
                    "algorithmic_bytes_per_launch": int(sb["route_gateup_swiglu"]), "avg_launch_us": round(gu_us, 2),
                    "layer_hbm_frac": round(sum(sb[k] for k in ("router_quantise", "route_gateup_swiglu", "down",
                                                                "combine"))
                                            / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    else:
        q4k = wl.fmt == "q4_k"
        # Q4_K adds one min-term MFMA (about 34 cycles) per tile and k-step of 4 blocks
        pipe_roof = INT8_PEAK_TOPS * 32 / (3 * 32 + 34 / 4) if q4k else PIPE_ROOF_TOPS
        roofline = {"bound": "mfma",
                    "kernel": ("grouped_gemm_q4k_kernel<true> (grouped Q4_K gate/up + SwiGLU + requantise)" if q4k
                               else "grouped_gemm_kernel<true> (grouped gate/up + SwiGLU + requantise)"),
                    "achieved": round(gu_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                    "frac": round(gu_tops / INT8_PEAK_TOPS, 4),
                    "traffic": (read_traffic(f"gateup_{args.workload}", "grouped_gemm_q4k" if q4k else "grouped_gemm")
                                if not chunk else None),
                    "algorithmic_ops_per_launch": gu_ops, "avg_launch_us": round(gu_us, 2),
                    "pipe_roof": {"peak": round(pipe_roof, 1), "unit": "TOP/s",
                                  "frac": round(gu_tops / pipe_roof, 4),
                                  "why": ("3 MFMAs per 32-block per 32x32 tile (int8, conversion, scale) plus one "
                                          "min-term MFMA per tile and k-step" if q4k else
                                          "3 MFMAs per 32-block per 32x32 tile (int8, conversion, scale)")}}
    stages = {}
    for name in stage_names:
        us = stage_ms[name] * 1e3
        ent = {"avg_us": round(us, 2)}
        if name in sb:
            ent["hbm_GBps_algorithmic"] = round(sb[name] / (us * 1e-6) / 1e9, 1)
            ent["hbm_frac"] = round(sb[name] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        stages[name] = ent
    stages["route_gateup_swiglu" if decode else "gateup_swiglu"]["int8_TOPs"] = round(gu_tops, 1)
    stages["down"]["int8_TOPs"] = round(dn_ops / (dn_us * 1e-6) / 1e12, 1)
    gemm_frac = (gu_ops + dn_ops) / ((gu_us + dn_us) * 1e-6) / 1e12 / INT8_PEAK_TOPS

    log("[bench] measuring the int8 MFMA and copy ceilings")
    peaks = measured_peaks(stream, settle_s=min(args.settle_seconds, 0.3))
    peak_key = "copy_GBps" if roofline["unit"] == "GB/s" else "int8_mfma_TOPs"
    roofline["measured_peak"] = peaks[peak_key]
    roofline["frac_of_measured_peak"] = round(roofline["achieved"] / peaks[peak_key], 4)

    cpu = None
    if args.cpu_seconds > 0:
        log("[bench] timing the CPU oracle sample")
        layers_cpu = [lw] + [mw.workload_layer(args.workload, layer=li) for li in range(1, n_layers)]
        cpu = cpu_baseline(layers_cpu, h0.cpu().numpy() if n_layers > 1 else x_np, args.cpu_seconds, eps)

    res = {
        "metric": METRIC, "value": round(n / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "clock_settle": {"seconds": args.settle_seconds, "steps": settle_calls,
                         "why": "untimed steps before the warmup, so that the timed steps run at the clock "
                                "the GPU holds under this load rather than one still ramping up from idle"},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights packed as %s)"
                % {"q4_k": "Q4_K", "q3_k": "Q3_K"}.get(wl.fmt, "Q8_0"),
        "config": {"workload": args.workload, **{k: v for k, v in mw.describe(args.workload).items()
                                                 if k != "workload"}},
        "grouped_gemm_int8_frac": round(gemm_frac, 4),
        "launch": ("graph replay" if graph is not None else "eager calls"),
        "experts_touched": int((counts[:s.n_experts] > 0).sum()),
        "stages": stages, "roofline": roofline, "measured_peaks": peaks, "cpu_baseline": cpu,
    }
    if chunk:
        res["chunked"] = {"chunk_tokens": chunk, "order": args.chunk_order, "chunks": (n + chunk - 1) // chunk,
                          "entry_point": "moe_ffn_prefill_chunked",
                          "stages_and_roofline": f"one {n_prof}-token call (the first chunk)"}
    if n_layers > 1:
        res["stack"] = {"layers": n_layers, "ms_per_layer": round(ms_step / n_layers, 5),
                        "step": "h = h0; xn = RMSNorm(h); per layer: y = MoE(xn), h += y, xn = RMSNorm(h)",
                        "form": args.stack_form,
                        "stages_and_roofline": "first layer, profiled passes on its normalised input"}
    for lay in stack:
        lay.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
