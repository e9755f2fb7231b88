"""Benchmark of the NVFP4 W4A4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|NAME] [--no-cpu-baseline]

The metric is the NVFP4 W4A4 GEMV/GEMM's HBM GB/s and fraction of peak at M=1 and M=16, and its
TFLOP/s and fraction of the matrix-core peak at M=512.  By default one run measures all of it
and prints ONE JSON line: the headline is single-stream decode of an FFN up-projection (M=1,
K=5120, N=25600: nvfp4_quantize_gemm, activation quantization inside the FP4 GEMV), the
bandwidth-bound product behind the decode speedup of the page "TensorRT Edge-LLM Completes the
MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor" (section "Using NVFP4 quantization to
accelerate Qwen3.6-27B inference"); the line's "workloads" object carries the M=16 records (the
tree-verification down-projection, the LM head over the 16-node tree, the LM head with the fused
greedy acceptance) and the M=512 suffix-prefill record (two GEMMs, the first emitting its output's
NVFP4 form for the second).  --workload NAME measures one workload alone (one record as the line);
--workload kv_fp8 measures the FP8 E4M3 KV-cache codec (its own metric, not part of the default line).

A step is one pass of the workload's hot path over one batch of synthetic, seeded input already
resident in HBM: activation quantization then the product(s).  Steps rotate over enough copies of
the quantized weights (> 512 MB in total) that the 256 MB Infinity Cache cannot serve them.  The
timed region is exactly K steps captured as ONE HIP graph (uploaded before timing) and replayed
once, bracketed by synchronizations; HIP events on the replay stream time it.  Just before the
start event, outside the region, a spin kernel and a 512 MiB read keep the GPU busy while the host
submits the graph, so neither the host's launch latency nor an idle GPU's first moments are
counted.  Per record:

  value        algorithmic weight bytes (packed codes + block scales) per step / step time, GB/s
               (prefill: 2*M*N*K flops of both GEMMs / step time, TFLOP/s);
  roofline     the dominant kernel's algorithmic bytes (flops) per launch / its average duration,
               from K launches of that kernel alone in one graph timed the same way, against
               MI355X's published peak (8 TB/s HBM3E; 2.5 PFLOP/s dense f16), with the HBM
               traffic per launch from the committed rocprofv3 counter record (null when the
               kernel's sources changed since the counters were taken) and, for the weight
               streams, the read-only ceiling: nvfp4_stream_read over the same bytes, timed the
               same way;
  cpu_baseline the CPU oracle (oracle/) on a bounded sample of the same step, with all BLAS
               threads and with one, and the host CPU model (rank 0, N=1 only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

from nvfp4_w4a4_block_amd import binding as B
from nvfp4_w4a4_block_amd import workloads as WL

METRIC = "NVFP4 W4A4 GEMM: HBM GB/s & % peak at M=1/16; TFLOP/s & % MFMA at M=512"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense f16/bf16 matrix cores
ROTATE_BYTES = 600 * 2 ** 20   # weight bytes cycled through per pass (> 2x the Infinity Cache)
PRIMER_US = 200.0              # GPU busy time enqueued before each timed region's start event
DEV = "cuda:0"
ROOT = os.path.dirname(os.path.abspath(__file__))

# the arithmetic each product runs in
DTYPE_FP4 = "e2m1 x e2m1 MFMA (exact), fp32 scale and accumulation"
DTYPE_F16 = "f16 MFMA on exactly dequantized NVFP4, fp32 accumulation"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def calibrated_scale(x: np.ndarray) -> np.float32:
    """Static activation decode scale from calibration data: amax / (6 * 448)."""
    return np.float32(np.float32(np.max(np.abs(x))) / np.float32(2688.0))


def to_dev_acts(inp: WL.Inputs) -> torch.Tensor:
    if inp.wl.act_dtype == "bf16":
        return torch.from_numpy(inp.A.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(inp.A).to(DEV)


# ---------------------------------------------------------------------------------------------
# Timing
# ---------------------------------------------------------------------------------------------

class Primer:
    """GPU work enqueued just before a timed region's start event, outside it: a short spin
    kernel (covers the host's submission of the graph) and two reads of a 256 MiB buffer
    (nvfp4_stream_read, about 80 us: the memory system is busy and the Infinity Cache holds
    none of the workload's data when the region starts)."""

    def __init__(self):
        self.buf = torch.zeros((256 << 20,), dtype=torch.uint8, device=DEV)
        self.sink = torch.zeros((1,), dtype=torch.int32, device=DEV)
        self.half = self.buf.numel() // 2

    def __call__(self):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(1 << 16)
        for _ in range(2):
            B.nvfp4_stream_read(self.buf[:self.half], self.buf[self.half:], sink=self.sink)


_PRIMER = None
_HIP = None


def upload(g: torch.cuda.CUDAGraph) -> None:
    """hipGraphUpload of an instantiated graph, so that its first replay does not pay for it."""
    global _HIP
    import ctypes
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _HIP.hipGraphUpload.restype = ctypes.c_int
    st = _HIP.hipGraphUpload(g.raw_cuda_graph_exec(), torch.cuda.current_stream().cuda_stream)
    if st != 0:
        raise RuntimeError(f"hipGraphUpload failed ({st})")


def capture(fn, count: int) -> torch.cuda.CUDAGraph:
    """One graph of fn(0) .. fn(count - 1)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)  # warm the allocator and any lazily set kernel attributes on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        for i in range(count):
            fn(i)
    return g


def timed(fn, steps: int, warmup: int) -> float:
    """Milliseconds per call of fn over exactly `steps` calls in one replayed graph (after
    `warmup` untimed calls in a graph of their own)."""
    global _PRIMER
    if _PRIMER is None:
        _PRIMER = Primer()
    g = capture(fn, steps)
    upload(g)
    if warmup:
        capture(fn, warmup).replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _PRIMER()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


# ---------------------------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------------------------

class Layer:
    """One NVFP4 weight matrix, quantized on the GPU, replicated `copies` times."""

    def __init__(self, W: np.ndarray, copies: int):
        wd = torch.from_numpy(W).to(DEV)
        wc, ws, gw = B.nvfp4_quantize_weights(wd)
        del wd
        self.N, self.K = W.shape
        self.copies = [(wc, ws, gw)] + [(wc.clone(), ws.clone(), gw.clone()) for _ in range(copies - 1)]
        self.bytes = self.N * self.K // 2 + self.N * self.K // 16

    def __getitem__(self, i):
        return self.copies[i % len(self.copies)]


def tree16() -> list:
    """16 nodes over 8 depths: a main chain plus one alternative per depth (8 draft steps, top-2
    candidates per depth)."""
    parent, chain = [-1], [0]
    for _ in range(7):
        parent += [chain[-1], chain[-1]]
        chain.append(len(parent) - 2)
    parent.append(chain[-1])
    return parent


def read_ceiling(layer: Layer, steps: int, warmup: int) -> dict:
    """nvfp4_stream_read over the layer's codes and scales (the same rotating copies): the
    measured read-only ceiling for these bytes."""
    sink = torch.zeros((1,), dtype=torch.int32, device=DEV)
    ms = timed(lambda i: B.nvfp4_stream_read(layer[i][0], layer[i][1], sink=sink), steps, warmup)
    gbs = layer.bytes / (ms * 1e-3) / 1e9
    return {"kernel": "read_stream_kernel (nvfp4_stream_read)", "us": ms * 1e3, "achieved": gbs,
            "frac_of_peak": gbs / HBM_PEAK_GBS}


def hbm_roofline(kname: str, nbytes: int, kern_ms: float, traffic) -> dict:
    gbs = nbytes / (kern_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": traffic, "kernel": kname, "us_per_launch": kern_ms * 1e3, "algorithmic_bytes": nbytes}


def mfma_roofline(kname: str, flops: float, kern_ms: float, traffic) -> dict:
    tf = flops / (kern_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": tf, "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": tf / F16_MFMA_PEAK_TFLOPS, "traffic": traffic, "kernel": kname, "us_per_launch": kern_ms * 1e3,
            "algorithmic_flops": flops}


def measured_traffic(name: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter record
    (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter on a copy of known size), or None
    when there is no record or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as g:
            h.update(g.read())
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def base_record(wl: WL.Workload, steps: int, warmup: int, step_ms: float, value: float, unit: str, dtype: str,
                copies: int, extra_config=None) -> dict:
    cfg = {"workload": f"{wl.name}: M={wl.M} K={wl.K} N={wl.N} ({wl.note})", "M": wl.M, "K": wl.K, "N": wl.N,
           "act_dtype": wl.act_dtype, "out_dtype": wl.out_dtype, "weight_copies": copies,
           "parallelism": "none (1 GPU)"}
    cfg.update(extra_config or {})
    return {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": dtype, "data": "synthetic", "config": cfg}


def copies_for(nbytes: int) -> int:
    return max(1, math.ceil(ROTATE_BYTES / nbytes))


def bench_decode(args, wl: WL.Workload) -> dict:
    """M <= 2 decode step: nvfp4_quantize_gemm (one kernel where the FP4 GEMV takes the shape), or
    with --dynamic-act-scale nvfp4_quantize_gemm_dynamic (the tensor scale computed inside it)."""
    inp = WL.generate(wl)
    layer = Layer(inp.W, copies_for(wl.weight_bytes))
    a = to_dev_acts(inp)
    g_a = torch.tensor([float(calibrated_scale(inp.a_f32()))], device=DEV)
    ac = torch.empty((wl.M, wl.K // 2), dtype=torch.uint8, device=DEV)
    asc = torch.empty((wl.M, wl.K // 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((wl.M, wl.N), dtype=torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32, device=DEV)
    one_kernel = B.gemm_dispatch(wl.M, wl.K, wl.N) == B.KERNEL_GEMV_FP4

    def step(i):
        wc, ws, gw = layer[i]
        if args.dynamic_act_scale:
            B.nvfp4_quantize_gemm_dynamic(a, wc, ws, gw, out_dtype=out.dtype, out=out, a_codes=ac, a_scales=asc,
                                          g_a=g_a)
        else:
            B.nvfp4_quantize_gemm(a, g_a, wc, ws, gw, out_dtype=out.dtype, out=out, a_codes=ac, a_scales=asc)

    step_ms = timed(step, args.steps, args.warmup)
    if one_kernel:  # the step is one launch of the kernel
        kern_ms = step_ms
        kname = "gemv_fp4_kernel (fused " + ("scale, " if args.dynamic_act_scale else "") + "quantization + FP4 GEMV)"
    else:
        kern_ms = timed(lambda i: B.nvfp4_gemm(ac, asc, g_a, *layer[i], out_dtype=out.dtype, out=out),
                        args.steps, args.warmup)
        kname = B.KERNEL_NAMES[B.gemm_dispatch(wl.M, wl.K, wl.N)]
    log(f"[bench] {wl.name}: step {step_ms * 1e3:.2f} us, {kname} {kern_ms * 1e3:.2f} us per launch")
    rec = base_record(wl, args.steps, args.warmup, step_ms, wl.weight_bytes / (step_ms * 1e-3) / 1e9, "GB/s",
                      DTYPE_FP4 if one_kernel else DTYPE_F16, len(layer.copies),
                      {"act_scale": "dynamic (device amax per step)" if args.dynamic_act_scale else
                       "static (calibrated)", "step": "nvfp4_quantize_gemm" +
                       ("_dynamic" if args.dynamic_act_scale else "") + (" (one kernel)" if one_kernel else "")})
    rec["roofline"] = hbm_roofline(kname, wl.weight_bytes, kern_ms, measured_traffic(wl.name))
    rec["roofline"]["ceiling"] = read_ceiling(layer, args.steps, args.warmup)
    rec["roofline"]["frac_of_ceiling"] = rec["roofline"]["achieved"] / rec["roofline"]["ceiling"]["achieved"]
    return rec


def bench_m16(args, wl: WL.Workload, layer=None, inp=None) -> dict:
    """3..16-row products: quantize the node rows (nvfp4_quantize_act), then the GEMM (with the
    cached split-K workspace where the product splits: verify_down), or the LM head with the
    fused argmax and greedy acceptance (tree_verify, no logits written)."""
    inp = inp or WL.generate(wl)
    layer = layer or Layer(inp.W, copies_for(wl.weight_bytes))
    a = to_dev_acts(inp)
    g_a = torch.tensor([float(calibrated_scale(inp.a_f32()))], device=DEV)
    ac = torch.empty((wl.M, wl.K // 2), dtype=torch.uint8, device=DEV)
    asc = torch.empty((wl.M, wl.K // 16), dtype=torch.uint8, device=DEV)
    out_dtype = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
    out = torch.empty((wl.M, wl.N), dtype=out_dtype, device=DEV)
    tree = wl.name == "tree_verify"
    ws = None if tree else B.gemm_workspace(wl.M, wl.K, wl.N, torch.device(DEV))
    kernel = B.gemm_dispatch(wl.M, wl.K, wl.N, ws.numel() if ws is not None else 0)
    parent = torch.tensor(tree16(), dtype=torch.int32, device=DEV)
    draft = torch.zeros(wl.M, dtype=torch.int32, device=DEV)

    def product(i):
        wc, wsc, gw = layer[i]
        if tree:
            B.nvfp4_tree_verify(ac, asc, g_a, wc, wsc, gw, parent, draft)
        else:
            B.nvfp4_gemm(ac, asc, g_a, wc, wsc, gw, out_dtype=out_dtype, out=out, workspace=ws)

    def step(i):
        B.nvfp4_quantize_act(a, g_a, ac, asc)
        product(i)

    step_ms = timed(step, args.steps, args.warmup)
    kern_ms = timed(product, args.steps, args.warmup)
    if tree:
        kname = B.KERNEL_NAMES[kernel] + (" with fused argmax and acceptance (one launch)"
                                          if kernel == B.KERNEL_M16_STREAM else
                                          " + fused argmax, then tree_accept_kernel")
    else:
        kname = B.KERNEL_NAMES[kernel] + (", K split over workgroups" if ws is not None else "")
    log(f"[bench] {wl.name}: step {step_ms * 1e3:.2f} us, {kname} {kern_ms * 1e3:.2f} us per launch")
    step_desc = ("nvfp4_quantize_act + nvfp4_tree_verify (LM head with fused argmax, acceptance)" if tree else
                 "nvfp4_quantize_act + nvfp4_gemm" + ("_ws (split-K workspace)" if ws is not None else ""))
    rec = base_record(wl, args.steps, args.warmup, step_ms, wl.weight_bytes / (step_ms * 1e-3) / 1e9, "GB/s",
                      DTYPE_F16, len(layer.copies), {"step": step_desc})
    rec["roofline"] = hbm_roofline(kname, wl.weight_bytes, kern_ms, measured_traffic(wl.name))
    return rec, layer


def bench_prefill(args, wl: WL.Workload) -> dict:
    """Suffix prefill: quantize A1, the up-projection emitting Y1 and its NVFP4 form under the
    static scale g2 (nvfp4_gemm_quantize_output), the down-projection on those codes."""
    inp = WL.generate(wl)
    R = copies_for(2 * wl.weight_bytes)
    l1, l2 = Layer(inp.W, R), Layer(inp.W2, R)
    M, K, N = wl.M, wl.K, wl.N
    a = to_dev_acts(inp)
    g1 = torch.tensor([float(calibrated_scale(inp.a_f32()))], device=DEV)
    ac1 = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    as1 = torch.empty((M, K // 16), dtype=torch.uint8, device=DEV)
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ac2 = torch.empty((M, N // 2), dtype=torch.uint8, device=DEV)
    as2 = torch.empty((M, N // 16), dtype=torch.uint8, device=DEV)
    y2 = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    # static scale of the second GEMM's input, calibrated once on this batch's Y1 (outside timing)
    B.nvfp4_quantize_act(a, g1, ac1, as1)
    B.nvfp4_gemm(ac1, as1, g1, *l1[0], out_dtype=torch.bfloat16, out=y1)
    torch.cuda.synchronize()
    g2 = torch.tensor([float(np.float32(np.float32(y1.float().abs().max().item()) / np.float32(2688.0)))],
                      device=DEV)

    def gemm1(i):
        B.nvfp4_gemm_quantize_output(ac1, as1, g1, *l1[i], g2, out_dtype=torch.bfloat16, out=y1, y_codes=ac2,
                                     y_scales=as2)

    def gemm2(i):
        B.nvfp4_gemm(ac2, as2, g2, *l2[i], out_dtype=torch.bfloat16, out=y2)

    def step(i):
        B.nvfp4_quantize_act(a, g1, ac1, as1)
        gemm1(i)
        gemm2(i)

    step_ms = timed(step, args.steps, args.warmup)
    k1_ms = timed(gemm1, args.steps, args.warmup)
    k2_ms = timed(gemm2, args.steps, args.warmup)
    flops = 2.0 * M * N * K
    log(f"[bench] prefill: step {step_ms * 1e3:.2f} us, GEMM1 {k1_ms * 1e3:.2f} us, GEMM2 {k2_ms * 1e3:.2f} us")
    rec = base_record(wl, args.steps, args.warmup, step_ms, 2 * flops / (step_ms * 1e-3) / 1e12, "TFLOP/s",
                      DTYPE_F16, R, {"step": "nvfp4_quantize_act + nvfp4_gemm_quantize_output (up, output NVFP4 "
                                             "form in the epilogue) + nvfp4_gemm (down)"})
    rec["roofline"] = mfma_roofline(B.KERNEL_NAMES[B.KERNEL_TILED_PERSISTENT] + " (up-projection, output quantized "
                                    "in the epilogue)", flops, k1_ms, measured_traffic("prefill"))
    rec["roofline_down"] = mfma_roofline(B.KERNEL_NAMES[B.KERNEL_TILED_PERSISTENT] + " (down-projection)", flops,
                                         k2_ms, measured_traffic("prefill_down"))
    return rec


# ---------------------------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------------------------

KV_METRIC = "FP8 E4M3 KV-cache codec: HBM GB/s (bf16 in + E4M3 out, then back) & % peak"


def bench_kv(args) -> dict:
    """FP8 KV-cache codec (page section "Reusing KV cache across agent turns": the KV cache is kept
    in FP8): a step encodes one layer's bf16 K and V (23,552 tokens x 8 heads x 128) to E4M3 with
    a static calibrated scale and decodes them back to bf16, 6 bytes of HBM traffic per element
    (2 + 1, then 1 + 2).  Input, code and output sets rotate so that the Infinity Cache cannot
    serve them.  roofline: the encode kernel (3 bytes per element); roofline_decode: the decode."""
    bits = WL.make_kv()
    n = bits.size
    x = torch.from_numpy(bits.view(np.int16).reshape(-1)).view(torch.bfloat16).to(DEV)
    amax = float(torch.max(torch.abs(x.float())))
    scale = torch.tensor([float(np.float32(np.float32(amax) / np.float32(448.0)))], device=DEV)  # calibration
    R = max(2, math.ceil(ROTATE_BYTES / (6 * n)))
    xs = [x] + [x.clone() for _ in range(R - 1)]
    qs = [torch.empty(n, dtype=torch.uint8, device=DEV) for _ in range(R)]
    ys = [torch.empty(n, dtype=torch.bfloat16, device=DEV) for _ in range(R)]
    for i in range(R):  # codes to decode in the decode-only timing
        B.nvfp4_kv_fp8_encode(xs[i], scale, qs[i])

    def enc(i):
        B.nvfp4_kv_fp8_encode(xs[i % R], scale, qs[i % R])

    def dec(i):
        B.nvfp4_kv_fp8_decode(qs[i % R], scale, torch.bfloat16, ys[i % R])

    def step(i):
        enc(i)
        dec(i)

    step_ms = timed(step, args.steps, args.warmup)
    enc_ms = timed(enc, args.steps, args.warmup)
    dec_ms = timed(dec, args.steps, args.warmup)
    log(f"[bench] kv_fp8: n={n}, step {step_ms * 1e3:.2f} us, kv_encode_kernel {enc_ms * 1e3:.2f} us, "
        f"kv_decode_kernel {dec_ms * 1e3:.2f} us per launch")
    rec = {"metric": KV_METRIC, "value": 6.0 * n / (step_ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"kv_fp8: one layer's K and V, {WL.KV_TOKENS} tokens x {WL.KV_HEADS} heads x "
                                  f"{WL.KV_DIM}, bf16 <-> E4M3", "elements": n, "copies": R,
                      "step": "nvfp4_kv_fp8_encode + nvfp4_kv_fp8_decode", "parallelism": "none (1 GPU)"}}
    rec["roofline"] = hbm_roofline("kv_encode_kernel (bf16 -> E4M3)", 3 * n, enc_ms, measured_traffic("kv_fp8"))
    rec["roofline_decode"] = hbm_roofline("kv_decode_kernel (E4M3 -> bf16)", 3 * n, dec_ms, None)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = kv_cpu_baseline(bits, args.cpu_seconds)
    return rec


def kv_cpu_baseline(bits: np.ndarray, budget_s: float) -> dict:
    """The oracle's encode + decode (NumPy) on the first 2^22 elements of the same layer."""
    from oracle import kvfp8 as KVO
    xs = WL.bf16_bits_to_f32(bits.reshape(-1)[: 1 << 22])
    s = KVO.calibrated_scale(xs)
    reps, t0 = 0, time.perf_counter()
    while True:
        KVO.decode_bf16_bits(KVO.encode(xs, s), s)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": 6.0 * xs.size * reps / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} x encode + decode of the first {xs.size} elements, {el:.1f} s (NumPy, one thread)",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl: WL.Workload, budget_s: float) -> dict:
    """The CPU oracle on a bounded sample of the same step: activation quantization plus the fp64
    product against the first rows of the pre-quantized weights, timed for budget_s with all
    BLAS threads, then for budget_s with one."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import gemm as G
    from oracle import quant as Q
    rows = min(2048 if wl.M <= 16 else 256, wl.N)
    inp = WL.generate(wl)
    a = inp.a_f32()
    g_a = calibrated_scale(a)
    g_w = Q.global_scale(inp.W)
    wp, ws = Q.quantize_packed(inp.W[:rows], g_w)

    def run(budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            ap, asc = Q.quantize_packed(a, g_a)
            G.gemm_ref(ap, asc, g_a, wp, ws, g_w, want_tol=False)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    def rate(reps, el):
        if wl.chain:
            return 2.0 * wl.M * rows * wl.K * reps / el / 1e12
        return (rows * wl.K // 2 + rows * wl.K // 16) * reps / el / 1e9

    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    reps, el = run(budget_s)
    with threadpool_limits(limits=1):
        reps1, el1 = run(budget_s)
    sample = (f"quantize A[{wl.M}x{wl.K}] + fp64 GEMM against the first {rows} of {wl.N} weight rows "
              f"(weights pre-quantized)")
    return {"value": rate(reps, el), "unit": "TFLOP/s" if wl.chain else "GB/s", "cores": int(threads),
            "kind": "oracle", "sample": f"{reps} x {sample}, {el:.1f} s, BLAS threads={threads}",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "single_thread": {"value": rate(reps1, el1), "cores": 1, "sample": f"{reps1} x the same, {el1:.1f} s"}}


# ---------------------------------------------------------------------------------------------

def run_workload(args, name: str, cache: dict) -> dict:
    wl = WL.get(name)
    if name in ("tiny", "decode_up"):
        rec = bench_decode(args, wl)
    elif name == "prefill":
        rec = bench_prefill(args, wl)
    else:
        # lm_head and tree_verify draw the same weights: quantize and copy them once
        key = (wl.K, wl.N, wl.w_sigma, wl.seed)
        layer, inp = cache.get(key, (None, None))
        inp = inp or WL.generate(wl)
        rec, layer = bench_m16(args, wl, layer, inp)
        cache[key] = (layer, inp)
        if name in ("verify_down", "lm_head"):
            rec["roofline"]["ceiling"] = read_ceiling(layer, args.steps, args.warmup)
            rec["roofline"]["frac_of_ceiling"] = rec["roofline"]["achieved"] / rec["roofline"]["ceiling"]["achieved"]
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds if name == args.headline else args.cpu_seconds_other)
    return rec


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(WL.WORKLOADS) + ["kv_fp8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dynamic-act-scale", action="store_true",
                    help="decode: compute the activation scale on the device in every step (inside the fused "
                         "GEMV) instead of the static calibrated one")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="oracle seconds per thread setting for the headline workload")
    ap.add_argument("--cpu-seconds-other", type=float, default=2.0,
                    help="oracle seconds per thread setting for every other workload")
    ap.add_argument("--copy-reference-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (a known-size "
                         "reference for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the NVFP4 path is built and measured on a single MI355X)", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    B.load()
    cache: dict = {}
    if args.workload == "all":
        args.headline = "decode_up"
        line = run_workload(args, "decode_up", cache)
        line["workloads"] = {}
        for name in ("verify_down", "lm_head", "tree_verify", "prefill"):
            line["workloads"][name] = run_workload(args, name, cache)
            if name == "tree_verify":  # the LM-head weights are no longer needed
                cache.clear()
            torch.cuda.empty_cache()
    elif args.workload == "kv_fp8":
        line = bench_kv(args)
    else:
        args.headline = args.workload
        line = run_workload(args, args.workload, cache)
    if args.copy_reference_mib:
        x = torch.ones(args.copy_reference_mib * 2 ** 18, dtype=torch.float32, device=DEV)
        for _ in range(3):
            x.clone()
        torch.cuda.synchronize()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
