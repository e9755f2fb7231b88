"""Helpers shared by the GPU parity tests: device copies, oracle quantization, tolerances.

The HIP path is reached only through nvfp4_w4a4_block_amd.binding (the C ABI);
expected values come only from oracle/ applied to the seeded inputs.
"""
from __future__ import annotations

import numpy as np
import torch

from nvfp4_w4a4_block_amd import binding as B
from nvfp4_w4a4_block_amd import workloads as WL
from oracle import quant as Q

DEV = "cuda:0"


def require_gpu_lib() -> None:
    """On a GPU run the library must be present and load: no silent fallback."""
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    B.load()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def dev_bf16_bits(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> a bfloat16 device tensor (bit-identical)."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def dev_acts(inp: WL.Inputs) -> torch.Tensor:
    return dev_bf16_bits(inp.A) if inp.wl.act_dtype == "bf16" else dev_f32(inp.A)


def scalar(v: np.float32) -> torch.Tensor:
    return torch.tensor([float(v)], dtype=torch.float32, device=DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return WL.bf16_bits_to_f32(bits)
    return t.cpu().numpy()


def f32_bits(v) -> int:
    return int(np.float32(v).view(np.uint32))


def oracle_quant(x_f32: np.ndarray, g) -> tuple[np.ndarray, np.ndarray]:
    return Q.quantize_packed(x_f32, np.float32(g))


def out_rounding_slack(ref: np.ndarray, out_dtype: torch.dtype) -> np.ndarray:
    """Worst-case rounding of the stored result: bf16 keeps 8 significant bits (RNE)."""
    return np.abs(ref) * 2.0 ** -8 if out_dtype == torch.bfloat16 else np.zeros_like(ref)


def assert_within(gpu: np.ndarray, ref: np.ndarray, tol: np.ndarray, what: str) -> None:
    err = np.abs(gpu.astype(np.float64) - ref)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:8]
        rows = [(tuple(i), float(gpu[tuple(i)]), float(ref[tuple(i)]), float(tol[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs outside tolerance; first {rows}")
    assert np.all(np.isfinite(gpu)), what
