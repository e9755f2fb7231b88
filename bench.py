"""Benchmark of the NVFP4 W4A4 decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one pass of the hot path over one batch of synthetic input:
on-the-fly activation quantization followed by the NVFP4 GEMV/GEMM against
weights quantized offline, through nvfp4_quantize_gemm (one kernel for one or
two activation rows, otherwise nvfp4_quantize_act's kernel then the GEMM's);
the prefill workload runs its two GEMMs, the first one emitting its output's NVFP4 form
(nvfp4_gemm_quantize_output) for the second.  The default
workload is single-stream decode of an FFN up-projection (M=1, K=5120,
N=25600), the bandwidth-bound product behind the decode speedup of the page
"TensorRT Edge-LLM Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on
Jetson AGX Thor" (section "Using NVFP4 quantization to accelerate Qwen3.6-27B
inference").

Inputs are seeded synthetic tensors already resident in HBM.  Steps rotate
over enough copies of the quantized weights (> 512 MB in total) that the
256 MB Infinity Cache cannot serve them, and run as a replayed HIP graph so
that host launch overhead does not hide the kernels' time.  Prints one JSON
line on stdout:
  value      algorithmic weight bytes (packed codes + block scales) per step / step time, GB/s
             (prefill: 2*M*N*K flops per GEMM pair / step time, TFLOP/s);
  roofline   the dominant kernel's algorithmic bytes (or flops) per launch / its average
             duration from HIP events around graph-replayed launches, against MI355X's peak;
  cpu_baseline  the CPU oracle on a bounded sample of the same step (rank 0, N=1).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

from nvfp4_w4a4_block_amd import binding as B
from nvfp4_w4a4_block_amd import workloads as WL

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense f16/bf16 matrix cores
ROTATE_BYTES = 600 * 2 ** 20   # weight bytes cycled through per pass (> 2x the Infinity Cache)
DEV = "cuda:0"
ROOT = os.path.dirname(os.path.abspath(__file__))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def calibrated_scale(x: np.ndarray) -> np.float32:
    """Static activation decode scale from calibration data: amax / (6 * 448)."""
    return np.float32(np.float32(np.max(np.abs(x))) / np.float32(2688.0))


def to_dev_acts(inp: WL.Inputs) -> torch.Tensor:
    if inp.wl.act_dtype == "bf16":
        return torch.from_numpy(inp.A.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(inp.A).to(DEV)


class Layer:
    """One NVFP4 weight matrix, quantized on the GPU, replicated `copies` times."""

    def __init__(self, W: np.ndarray, copies: int):
        wd = torch.from_numpy(W).to(DEV)
        wc, ws, gw = B.nvfp4_quantize_weights(wd)
        del wd
        self.N, self.K = W.shape
        self.copies = [(wc, ws, gw)] + [(wc.clone(), ws.clone(), gw.clone()) for _ in range(copies - 1)]
        self.bytes = self.N * self.K // 2 + self.N * self.K // 16


class Pipeline:
    """Preallocated buffers and the step of one workload."""

    def __init__(self, wl: WL.Workload):
        self.wl = wl
        inp = WL.generate(wl)
        wbytes = wl.weight_bytes * (2 if wl.chain else 1)
        self.R = max(1, math.ceil(ROTATE_BYTES / wbytes))
        log(f"[bench] {wl.name}: M={wl.M} K={wl.K} N={wl.N}, {self.R} weight copies "
            f"({self.R * wbytes / 2**20:.0f} MiB)")
        self.l1 = Layer(inp.W, self.R)
        self.l2 = Layer(inp.W2, self.R) if wl.chain else None
        self.a = to_dev_acts(inp)
        self.g1 = torch.tensor([float(calibrated_scale(inp.a_f32()))], device=DEV)
        M, K, N = wl.M, wl.K, wl.N
        self.ac1 = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
        self.as1 = torch.empty((M, K // 16), dtype=torch.uint8, device=DEV)
        self.out_dtype = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
        self.y1 = torch.empty((M, N), dtype=self.out_dtype, device=DEV)
        # 3..16 rows: the workspace with which the GEMM splits a long K over workgroups (None
        # when it needs none); zeroed once, left zeroed by every call
        self.split_ws = B.gemm_workspace(M, K, N, torch.device(DEV)) if 3 <= M <= 16 else None
        self.tree = wl.name == "tree_verify"
        if self.tree:  # 16 nodes over 8 depths: a main chain plus one alternative per depth
            parent, chain = [-1], [0]
            for _ in range(7):
                parent += [chain[-1], chain[-1]]
                chain.append(len(parent) - 2)
            parent.append(chain[-1])
            self.parent = torch.tensor(parent, dtype=torch.int32, device=DEV)
            self.draft = torch.zeros(M, dtype=torch.int32, device=DEV)
            B.nvfp4_quantize_act(self.a, self.g1, self.ac1, self.as1)
        if wl.chain:
            self.ac2 = torch.empty((M, N // 2), dtype=torch.uint8, device=DEV)
            self.as2 = torch.empty((M, N // 16), dtype=torch.uint8, device=DEV)
            self.y2 = torch.empty((M, K), dtype=self.out_dtype, device=DEV)
            # static scale of the second GEMM's input, calibrated once on this batch's Y1
            self._gemm1(0)
            torch.cuda.synchronize()
            amax = self.y1.float().abs().max().item()
            self.g2 = torch.tensor([float(np.float32(np.float32(amax) / np.float32(2688.0)))], device=DEV)

    dynamic_scale = False  # set by --dynamic-act-scale: g_a computed on the device every step

    def _gemm1(self, i):
        wc, ws, gw = self.l1.copies[i % self.R]
        if self.dynamic_scale and self.split_ws is None:  # scale, quantization and GEMM in one call
            B.nvfp4_quantize_gemm_dynamic(self.a, wc, ws, gw, out_dtype=self.out_dtype, out=self.y1,
                                          a_codes=self.ac1, a_scales=self.as1, g_a=self.g1)
            return
        if self.dynamic_scale:
            B.nvfp4_act_global_scale(self.a, out=self.g1)
        if self.split_ws is not None:  # quantization, then the GEMM with its K split over workgroups
            B.nvfp4_quantize_act(self.a, self.g1, self.ac1, self.as1)
            B.nvfp4_gemm(self.ac1, self.as1, self.g1, wc, ws, gw, out_dtype=self.out_dtype, out=self.y1,
                         workspace=self.split_ws)
            return
        B.nvfp4_quantize_gemm(self.a, self.g1, wc, ws, gw, out_dtype=self.out_dtype, out=self.y1,
                              a_codes=self.ac1, a_scales=self.as1)

    def _verify(self, i):
        """Tree verification: quantize the 16 node rows, then LM head + fused argmax + greedy
        acceptance (nvfp4_tree_verify, three launches, no logits written)."""
        wc, ws, gw = self.l1.copies[i % self.R]
        B.nvfp4_tree_verify(self.ac1, self.as1, self.g1, wc, ws, gw, self.parent, self.draft)

    def step(self, i):
        if self.tree:
            B.nvfp4_quantize_act(self.a, self.g1, self.ac1, self.as1)
            self._verify(i)
            return
        if self.l2 is not None and not self.dynamic_scale:
            # prefill chain: the first GEMM emits Y1 and its NVFP4 form (static scale g2) in
            # one kernel, the second GEMM consumes those codes
            wc, ws, gw = self.l1.copies[i % self.R]
            B.nvfp4_quantize_act(self.a, self.g1, self.ac1, self.as1)
            B.nvfp4_gemm_quantize_output(self.ac1, self.as1, self.g1, wc, ws, gw, self.g2, out_dtype=self.out_dtype,
                                         out=self.y1, y_codes=self.ac2, y_scales=self.as2)
            wc, ws, gw = self.l2.copies[i % self.R]
            B.nvfp4_gemm(self.ac2, self.as2, self.g2, wc, ws, gw, out_dtype=self.out_dtype, out=self.y2)
            return
        self._gemm1(i)
        if self.l2 is not None:
            wc, ws, gw = self.l2.copies[i % self.R]
            if self.dynamic_scale:
                B.nvfp4_act_global_scale(self.y1, out=self.g2)
            B.nvfp4_quantize_gemm(self.y1, self.g2, wc, ws, gw, out_dtype=self.out_dtype, out=self.y2,
                                  a_codes=self.ac2, a_scales=self.as2)

    @property
    def fused_single_kernel(self) -> bool:
        """nvfp4_quantize_gemm runs as one kernel for M <= 2 and K a multiple of 1024 in
        [1024, 8192] (include/nvfp4.h)."""
        wl = self.wl
        return not wl.chain and wl.M <= 2 and wl.K % 1024 == 0 and 1024 <= wl.K <= 8192

    def gemm_only(self, i):
        """The dominant kernel alone, for its per-launch duration: the fused kernel where the
        step is one kernel, else the first GEMM on already quantized activations."""
        if self.tree:
            self._verify(i)
            return
        if self.fused_single_kernel:
            self._gemm1(i)
            return
        wc, ws, gw = self.l1.copies[i % self.R]
        if self.l2 is not None and not self.dynamic_scale:  # the step's first GEMM, output quantization fused
            B.nvfp4_gemm_quantize_output(self.ac1, self.as1, self.g1, wc, ws, gw, self.g2, out_dtype=self.out_dtype,
                                         out=self.y1, y_codes=self.ac2, y_scales=self.as2)
            return
        B.nvfp4_gemm(self.ac1, self.as1, self.g1, wc, ws, gw, out_dtype=self.out_dtype, out=self.y1,
                     workspace=self.split_ws)


def capture(fn, count: int) -> torch.cuda.CUDAGraph:
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)  # warm the allocator/caches on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        for i in range(count):
            fn(i)
    return g


def timed_replays(graphs, total: int, per_graph: int) -> float:
    """Runs exactly `total` units (full graphs, then a remainder graph); returns elapsed ms."""
    full, rem = divmod(total, per_graph)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(full):
        graphs[0].replay()
    if rem:
        graphs[1].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def build_graphs(fn, R: int, total: int):
    rem = total % R
    return [capture(fn, R), capture(fn, rem) if rem else None]


def measured_traffic(wl: WL.Workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter on a copy of known size), or
    None when there is no summary or the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as g:
            h.update(g.read())
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def cpu_baseline(wl: WL.Workload, budget_s: float) -> dict:
    """The CPU oracle timed on a bounded sample of the same step: activation quantization plus
    the fp64 product against a sample of pre-quantized weight rows."""
    from oracle import gemm as G
    from oracle import quant as Q
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    rng_rows = 2048 if wl.M <= 16 else 256
    inp = WL.generate(wl)
    a = inp.a_f32()
    g_a = calibrated_scale(a)
    W = inp.W[:rng_rows]
    g_w = Q.global_scale(inp.W)
    wp, ws = Q.quantize_packed(W, g_w)
    reps, t0 = 0, time.perf_counter()
    while True:
        ap, asc = Q.quantize_packed(a, g_a)
        G.gemm_ref(ap, asc, g_a, wp, ws, g_w, want_tol=False)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    sample_bytes = rng_rows * wl.K // 2 + rng_rows * wl.K // 16
    if wl.chain:
        value, unit = 2.0 * wl.M * rng_rows * wl.K * reps / el / 1e12, "TFLOP/s"
    else:
        value, unit = sample_bytes * reps / el / 1e9, "GB/s"
    return {"value": value, "unit": unit, "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} x (quantize A[{wl.M}x{wl.K}] + fp64 GEMM against the first {rng_rows} of "
                      f"{wl.N} weight rows, weights pre-quantized), {el:.1f} s; BLAS threads={threads}, "
                      f"host cpus={len(os.sched_getaffinity(0))}"}


def kv_bench(args) -> dict:
    """FP8 KV-cache codec: one step encodes one layer's bf16 K and V (23,552 tokens x 8 heads x 128)
    to E4M3 and decodes it back to bf16; 6 bytes of HBM traffic per element (2 + 1, then 1 + 2).
    Three input/code/output sets rotate so the 256 MB Infinity Cache cannot serve them."""
    bits = WL.make_kv()
    n = bits.size
    x = torch.from_numpy(bits.view(np.int16).reshape(-1)).view(torch.bfloat16).to(DEV)
    amax = float(torch.max(torch.abs(x.float())))
    scale = torch.tensor([float(np.float32(np.float32(amax) / np.float32(448.0)))], device=DEV)  # calibration
    R = 3
    xs = [x] + [x.clone() for _ in range(R - 1)]
    qs = [torch.empty(n, dtype=torch.uint8, device=DEV) for _ in range(R)]
    ys = [torch.empty(n, dtype=torch.bfloat16, device=DEV) for _ in range(R)]

    def step(i):
        B.nvfp4_kv_fp8_encode(xs[i % R], scale, qs[i % R])
        B.nvfp4_kv_fp8_decode(qs[i % R], scale, torch.bfloat16, ys[i % R])

    def enc(i):
        B.nvfp4_kv_fp8_encode(xs[i % R], scale, qs[i % R])

    K, W = args.steps, args.warmup
    if W:
        timed_replays(build_graphs(step, R, W), W, R)
    step_ms = timed_replays(build_graphs(step, R, K), K, R) / K
    enc_ms = timed_replays(build_graphs(enc, R, K), K, R) / K
    log(f"[bench] kv_fp8: n={n}, step {step_ms * 1e3:.2f} us, encode {enc_ms * 1e3:.2f} us")
    roof = {"bound": "hbm", "achieved": 3.0 * n / (enc_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "kernel": "kv_encode_kernel (bf16 -> E4M3)", "traffic": None, "algorithmic_bytes": 3 * n}
    roof["frac"] = roof["achieved"] / roof["peak"]
    line = {
        "metric": "FP8 E4M3 KV-cache codec HBM GB/s (bf16 in + E4M3 out, then back)", "value": 6.0 * n / (step_ms * 1e-3) / 1e9,
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": step_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"kv_fp8: one layer's K and V, {WL.KV_TOKENS} tokens x {WL.KV_HEADS} heads x "
                               f"{WL.KV_DIM} dims, bf16 <-> E4M3", "elements": n, "copies": R,
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import kvfp8 as KVO
        xs_host = WL.bf16_bits_to_f32(bits.reshape(-1)[: 1 << 22])
        s = KVO.calibrated_scale(xs_host)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            KVO.decode_bf16_bits(KVO.encode(xs_host, s), s)
            reps += 1
        el = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": 6.0 * xs_host.size * reps / el / 1e9, "unit": "GB/s", "cores": 1,
                                "kind": "oracle", "sample": f"{reps} x encode + decode of the first {xs_host.size} "
                                                            f"elements, {el:.1f} s (NumPy, one thread)"}
    return line


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode_up", choices=sorted(WL.WORKLOADS) + ["kv_fp8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dynamic-act-scale", action="store_true",
                    help="compute the activation scale on the device in every step (inside the fused GEMV "
                         "where the step is one kernel, else nvfp4_act_global_scale) instead of the static "
                         "calibrated one")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
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
    if args.workload == "kv_fp8":
        print(json.dumps(kv_bench(args)), flush=True)
        return 0
    wl = WL.get(args.workload)
    Pipeline.dynamic_scale = args.dynamic_act_scale
    P = Pipeline(wl)
    K, W = args.steps, args.warmup

    step_graphs = build_graphs(P.step, P.R, K)
    gemm_graphs = build_graphs(P.gemm_only, P.R, K)
    if W:
        timed_replays(build_graphs(P.step, P.R, W), W, P.R)
    torch.cuda.synchronize()
    step_ms = timed_replays(step_graphs, K, P.R) / K
    kern_ms = timed_replays(gemm_graphs, K, P.R) / K
    kname = ("LM head + fused argmax + tree acceptance" if P.tree else
             "fused scale + quantize + FP4 GEMV" if P.fused_single_kernel and args.dynamic_act_scale else
             "fused quantize + FP4 GEMV" if P.fused_single_kernel else
             "M<=16 weight-streaming GEMM (gemm_m16_kernel)" if 3 <= wl.M <= 16 else
             "first GEMM (its output's NVFP4 form emitted in the epilogue)" if wl.chain and not args.dynamic_act_scale else
             "first GEMM")
    log(f"[bench] step {step_ms * 1e3:.2f} us, {kname} {kern_ms * 1e3:.2f} us per launch")

    if wl.chain:
        flops = 2.0 * wl.M * wl.N * wl.K
        value, unit = 2 * flops / (step_ms * 1e-3) / 1e12, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": flops / (kern_ms * 1e-3) / 1e12, "peak": F16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
        metric = "NVFP4 W4A4 GEMM TFLOP/s at M=512 (suffix prefill, up+down projection)"
    else:
        value, unit = wl.weight_bytes / (step_ms * 1e-3) / 1e9, "GB/s"
        roof = {"bound": "hbm", "achieved": wl.weight_bytes / (kern_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
        metric = "NVFP4 W4A4 GEMV/GEMM HBM GB/s (packed weight codes + block scales per step)"
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = kname
    roof["traffic"] = measured_traffic(wl)
    roof["algorithmic_bytes"] = wl.weight_bytes if not wl.chain else None
    line = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: M={wl.M} K={wl.K} N={wl.N} ({wl.note})", "M": wl.M, "K": wl.K,
                   "N": wl.N, "act_dtype": wl.act_dtype, "out_dtype": wl.out_dtype,
                   "weight_copies": P.R, "parallelism": "none (1 GPU)",
                   "act_scale": "dynamic (device amax per step)" if args.dynamic_act_scale else "static (calibrated)"},
        "roofline": roof,
    }
    if args.copy_reference_mib:
        x = torch.ones(args.copy_reference_mib * 2 ** 18, dtype=torch.float32, device=DEV)
        for _ in range(3):
            x.clone()
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
