"""CPU oracle for NVFP4 W4A4 block-scaled quantization and GEMM -- TEST INFRASTRUCTURE.

A plain, slow NumPy implementation written from the NVFP4 format definition
(E2M1 4-bit codes, one FP8 E4M3 scale per 16 contiguous K-elements, one fp32
per-tensor scale) and from the page "TensorRT Edge-LLM Completes the MLPerf
Edge Agentic Benchmark 6.4x Faster on Jetson AGX Thor", section "Using NVFP4
quantization to accelerate Qwen3.6-27B inference" (weights and activations in
NVFP4, LM head included; post-training quantization done once offline).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library and its Python binding never do, and the
two share no code: the oracle decodes with lookup tables in fp64, encodes by
nearest-value search, and multiplies dense dequantized matrices in fp64.

Pinned by tests/test_oracle_*.py against closed forms, torch's float8_e4m3fn
casts, hand-worked blocks (tests/golden/) and exact rational brute force.
`tree` adds the greedy verification of a candidate tree over the LM head
(section "Using tree-based multi-token prediction to accelerate LLM
inference"), pinned by hand-worked trees and an exhaustive path search.
`kvfp8` adds the FP8 E4M3 KV-cache codec (same section as NVFP4: the KV cache
is FP8), pinned by hand-worked elements, exact round trips and torch's casts.
Parity unpinned by the pages themselves: the per-tensor scale formula
amax/(6*448) and the static activation scale are readings, not page facts.
"""
from . import formats, quant, gemm, tree, kvfp8  # noqa: F401
