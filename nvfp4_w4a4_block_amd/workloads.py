"""Seeded synthetic inputs for the NVFP4 W4A4 GEMV/GEMM workloads.

This module only draws random arrays and rounds them to the storage dtype the
workload names (fp32 or bf16).  It holds none of the quantization or GEMM
arithmetic, so both the HIP path and the CPU oracle can take their inputs from
it without sharing any of the method.

The shapes stand in for the linear layers of the decode, tree-verification and
suffix-prefill passes described in "TensorRT Edge-LLM Completes the MLPerf Edge
Agentic Benchmark 6.4x Faster on Jetson AGX Thor" (sections "Using NVFP4
quantization to accelerate Qwen3.6-27B inference", "Reusing KV cache across
agent turns" and "Using tree-based multi-token prediction to accelerate LLM
inference"): M=1 single-stream decode, M=16 for one pass over a 16-node
candidate tree, M=512 for a suffix prefill.

Recipe (the same for every workload):
  * ``numpy.random.default_rng(seed)`` (PCG64), weights drawn before activations;
  * weights: float32 standard normals times sigma, row-major [N, K];
  * activations: float32 standard normals, then the workload's structure
    (outlier channels, abs + zeroed entries), then a round-to-nearest-even cast
    to bf16 (torch's CPU cast) when the workload stores activations in bf16.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_weights", "make_acts", "bf16_bits_to_f32",
           "f32_to_bf16_bits"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    w_sigma: float
    act: str              # "normal" | "normal_outliers" | "abs_zeros"
    act_dtype: str        # "f32" | "bf16"
    out_dtype: str        # "f32" | "bf16"
    outlier_frac: float = 0.0
    outlier_gain: float = 1.0
    zero_frac: float = 0.0
    # second GEMM of a chained up/down projection pair (prefill): K2 = N, N2 = K
    chain: bool = False
    seed: int = 0
    note: str = ""

    @property
    def weight_bytes(self) -> int:
        """Packed E2M1 codes plus E4M3 block scales of one weight matrix."""
        return self.N * self.K // 2 + self.N * self.K // 16


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, 256, 256, 0.02, "normal", "f32", "f32",
                 note="tiny GEMV, oracle runs in well under a second"),
        Workload("decode_up", 1, 5120, 25600, 0.02, "normal_outliers", "bf16", "bf16",
                 outlier_frac=0.005, outlier_gain=20.0,
                 note="single-stream decode, FFN up-projection"),
        Workload("verify_down", 16, 25600, 5120, 0.01, "abs_zeros", "bf16", "bf16",
                 zero_frac=0.01,
                 note="16-node tree verification pass, FFN down-projection"),
        Workload("lm_head", 16, 5120, 151936, 0.02, "normal", "bf16", "f32",
                 note="LM head over the 16-node verification tree, fp32 logits"),
        Workload("tree_verify", 16, 5120, 151936, 0.02, "normal", "bf16", "f32",
                 note="LM head over the 16-node verification tree with fused greedy acceptance "
                      "(argmax inside the GEMM, no logits written)"),
        Workload("prefill", 512, 5120, 25600, 0.02, "normal_outliers", "bf16", "bf16",
                 outlier_frac=0.005, outlier_gain=20.0, chain=True,
                 note="suffix prefill: up-proj 5120->25600 then down-proj 25600->5120"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even, torch's CPU cast); return the uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_weights(rng: np.random.Generator, N: int, K: int, sigma: float) -> np.ndarray:
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def make_acts(rng: np.random.Generator, M: int, K: int, kind: str, dtype: str, *,
              outlier_frac: float = 0.0, outlier_gain: float = 1.0,
              zero_frac: float = 0.0) -> np.ndarray:
    """Activations [M, K]: float32 array, or uint16 bf16 bit patterns when dtype == "bf16"."""
    a = rng.standard_normal((M, K), dtype=np.float32)
    if kind == "normal_outliers":
        n_out = int(round(outlier_frac * K))
        cols = rng.choice(K, size=n_out, replace=False)
        a[:, cols] *= np.float32(outlier_gain)
    elif kind == "abs_zeros":
        np.abs(a, out=a)
        n_zero = int(round(zero_frac * M * K))
        flat = rng.choice(M * K, size=n_zero, replace=False)
        a.reshape(-1)[flat] = 0.0
    elif kind != "normal":
        raise ValueError(f"unknown activation kind {kind!r}")
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    if dtype != "f32":
        raise ValueError(f"unknown activation dtype {dtype!r}")
    return a


@dataclasses.dataclass
class Inputs:
    wl: Workload
    W: np.ndarray                  # float32 [N, K]
    A: np.ndarray                  # float32 [M, K] or uint16 bf16 bits
    W2: Optional[np.ndarray] = None  # float32 [K, N] (chained down-projection), prefill only

    def a_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.A) if self.wl.act_dtype == "bf16" else self.A


def generate(wl: Workload, *, M: Optional[int] = None, K: Optional[int] = None,
             N: Optional[int] = None, seed: Optional[int] = None) -> Inputs:
    """Draw one workload's inputs.  M/K/N/seed override the workload's sizes (for small parity cases)."""
    M = wl.M if M is None else M
    K = wl.K if K is None else K
    N = wl.N if N is None else N
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    W = make_weights(rng, N, K, wl.w_sigma)
    W2 = make_weights(rng, K, N, wl.w_sigma) if wl.chain else None
    A = make_acts(rng, M, K, wl.act, wl.act_dtype, outlier_frac=wl.outlier_frac,
                  outlier_gain=wl.outlier_gain, zero_frac=wl.zero_frac)
    return Inputs(wl, W, A, W2)


# KV cache of one attention layer for the FP8 codec: K and V of a context as long as the
# benchmark's longest agent turns (about 23.5K prompt tokens on the page "TensorRT Edge-LLM
# Completes the MLPerf Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor"), 8 KV heads of
# dimension 128 (grouped-query attention of a model of this size; the pages give no layer
# shapes).  Values N(0, 1) with 1% of the channels of each head scaled by 8 (keys carry a few
# large channels); stored as bf16.
KV_TOKENS, KV_HEADS, KV_DIM = 23552, 8, 128


def make_kv(seed: int = 0, tokens: int = KV_TOKENS, heads: int = KV_HEADS, dim: int = KV_DIM) -> np.ndarray:
    """uint16 bf16 bit patterns of [2, tokens, heads, dim] (K then V)."""
    rng = np.random.default_rng(seed)
    kv = rng.standard_normal((2, tokens, heads, dim), dtype=np.float32)
    n_out = max(1, int(round(0.01 * dim)))
    for h in range(heads):
        cols = rng.choice(dim, size=n_out, replace=False)
        kv[0, :, h, cols] *= np.float32(8.0)
    return f32_to_bf16_bits(kv)
