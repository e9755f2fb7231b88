"""Thin Python binding of the C ABI in include/nvfp4.h (ctypes; marshalling only).

Every function here checks tensor placement, dtype, shape and contiguity,
allocates outputs with torch (device memory is torch's job), passes raw
device pointers and the current HIP stream to libnvfp4.so, and raises
NVFP4Error on a non-zero status.  All arithmetic runs in the library's HIP
kernels; there is no fallback: without the built library (or without a GPU)
these functions raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")

NVFP4_OK, NVFP4_ERR_NULL, NVFP4_ERR_SHAPE, NVFP4_ERR_ALIGN, NVFP4_ERR_DTYPE, NVFP4_ERR_HIP, NVFP4_ERR_SCRATCH = range(7)
SCRATCH_BYTES = 4 << 20  # NVFP4_SCRATCH_BYTES
NVFP4_F32, NVFP4_BF16 = 0, 1
PATH_AUTO, PATH_SKINNY, PATH_TILED = 0, 1, 2
# kernel selectors of nvfp4_gemm_ex (and values of nvfp4_gemm_dispatch)
(KERNEL_GEMV_FP4, KERNEL_GEMV_FLAT, KERNEL_M16, KERNEL_SKINNY256, KERNEL_SKINNY16,
 KERNEL_TILED_PERSISTENT, KERNEL_TILED, KERNEL_M16_STREAM) = range(3, 11)
KERNEL_NAMES = {KERNEL_GEMV_FP4: "gemv_fp4_kernel", KERNEL_GEMV_FLAT: "gemv_flat_kernel", KERNEL_M16: "gemm_m16_kernel",
                KERNEL_SKINNY256: "gemm_skinny256_kernel", KERNEL_SKINNY16: "gemm_skinny_kernel",
                KERNEL_TILED_PERSISTENT: "gemm_wg_tiled_kernel", KERNEL_TILED: "gemm_tiled_kernel",
                KERNEL_M16_STREAM: "gemm_m16_stream_kernel"}

EXPORTS = ("nvfp4_abi_version", "nvfp4_act_global_scale", "nvfp4_gemm", "nvfp4_gemm_dispatch", "nvfp4_gemm_ex",
           "nvfp4_gemm_quantize_output", "nvfp4_gemm_scratch", "nvfp4_gemm_workspace_bytes", "nvfp4_gemm_ws", "nvfp4_kv_fp8_decode", "nvfp4_kv_fp8_encode",
           "nvfp4_quantize_act",
           "nvfp4_quantize_gemm", "nvfp4_quantize_gemm_dynamic", "nvfp4_quantize_weights", "nvfp4_status_string",
           "nvfp4_stream_read",
           "nvfp4_tree_accept",
           "nvfp4_tree_verify")

_lib: Optional[ctypes.CDLL] = None


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def load() -> ctypes.CDLL:
    """Loads libnvfp4.so and declares the signatures (no GPU needed)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m nvfp4_w4a4_block_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.nvfp4_quantize_weights.argtypes = [p, i32, i64, i64, p, p, p, p]
    lib.nvfp4_quantize_act.argtypes = [p, i32, i64, i64, p, p, p, p]
    lib.nvfp4_gemm.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, i32, p]
    lib.nvfp4_gemm_ex.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, i32, i32, p]
    lib.nvfp4_gemm_ws.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, i32, p, i64, p]
    lib.nvfp4_gemm_scratch.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, i32, p]
    lib.nvfp4_gemm_quantize_output.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, i32, p, p, p, p]
    lib.nvfp4_gemm_workspace_bytes.argtypes = [i64, i64, i64]
    lib.nvfp4_gemm_workspace_bytes.restype = i64
    lib.nvfp4_gemm_dispatch.argtypes = [i64, i64, i64, i64]
    lib.nvfp4_stream_read.argtypes = [p, i64, p, i64, p, ctypes.c_uint32, p]
    lib.nvfp4_gemm_dispatch.restype = i32
    lib.nvfp4_quantize_gemm.argtypes = [i64, i64, i64, p, i32, p, p, p, p, p, i32, p, p, p]
    lib.nvfp4_quantize_gemm_dynamic.argtypes = [i64, i64, i64, p, i32, p, p, p, p, p, i32, p, p, p]
    lib.nvfp4_tree_accept.argtypes = [i64, p, p, p, p, p]
    lib.nvfp4_kv_fp8_encode.argtypes = [p, i32, i64, p, p, p]
    lib.nvfp4_act_global_scale.argtypes = [p, i32, i64, i64, p, p]
    lib.nvfp4_kv_fp8_decode.argtypes = [p, i64, p, p, i32, p]
    lib.nvfp4_tree_verify.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, p, p, p, p, p, p]
    for f in ("nvfp4_quantize_weights", "nvfp4_quantize_act", "nvfp4_gemm", "nvfp4_gemm_ex", "nvfp4_gemm_ws",
              "nvfp4_gemm_scratch",
              "nvfp4_gemm_quantize_output",
              "nvfp4_quantize_gemm", "nvfp4_tree_accept", "nvfp4_tree_verify", "nvfp4_kv_fp8_encode",
              "nvfp4_kv_fp8_decode", "nvfp4_act_global_scale", "nvfp4_stream_read"):
        getattr(lib, f).restype = i32
    lib.nvfp4_status_string.argtypes = [i32]
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    lib.nvfp4_abi_version.argtypes = []
    lib.nvfp4_abi_version.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().nvfp4_status_string(status).decode()


def _dt(t: torch.dtype) -> int:
    if t == torch.float32:
        return NVFP4_F32
    if t == torch.bfloat16:
        return NVFP4_BF16
    raise TypeError(f"unsupported dtype {t} (float32 or bfloat16)")


def _dev(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _check(status: int, where: str) -> None:
    if status != NVFP4_OK:
        raise NVFP4Error(status, where)


def nvfp4_quantize_weights(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """w [N, K] float32/bfloat16 -> (codes uint8 [N, K/2], scales uint8 [N, K/16], g_w float32 [1])."""
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    dev = _dev(w)
    N, K = w.shape
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
    g = torch.empty((1,), dtype=torch.float32, device=dev)
    _check(load().nvfp4_quantize_weights(w.data_ptr(), _dt(w.dtype), N, K, codes.data_ptr(),
                                         scales.data_ptr(), g.data_ptr(), _stream(dev)),
           "nvfp4_quantize_weights")
    return codes, scales, g


def nvfp4_quantize_act(a: torch.Tensor, g_a: torch.Tensor, codes: Optional[torch.Tensor] = None,
                       scales: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """a [M, K] float32/bfloat16 with device decode scale g_a [1] -> (codes [M, K/2], scales [M, K/16])."""
    if a.dim() != 2:
        raise ValueError("a must be [M, K]")
    if g_a.dtype != torch.float32 or g_a.numel() != 1:
        raise ValueError("g_a must be a float32 tensor of one element")
    dev = _dev(a, g_a)
    M, K = a.shape
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    _dev(a, codes, scales)
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8 or \
            codes.numel() != M * (K // 2) or scales.numel() != M * (K // 16):
        raise ValueError("codes/scales must be uint8 of [M, K/2] / [M, K/16] elements")
    _check(load().nvfp4_quantize_act(a.data_ptr(), _dt(a.dtype), M, K, g_a.data_ptr(),
                                     codes.data_ptr(), scales.data_ptr(), _stream(dev)),
           "nvfp4_quantize_act")
    return codes, scales


_gemm_workspaces: dict = {}


def gemm_workspace(M: int, K: int, N: int, dev: torch.device) -> Optional[torch.Tensor]:
    """A zeroed workspace of at least nvfp4_gemm_workspace_bytes(M, K, N) bytes on `dev`, or None
    when the product needs none.  Cached per device and grown when too small; every call leaves
    its counters zero, so it is zeroed only when allocated.  Shared by the calls of this module:
    keep them on one stream, or pass a workspace of your own."""
    need = int(load().nvfp4_gemm_workspace_bytes(M, K, N))
    if need <= 0:
        return None
    ws = _gemm_workspaces.get(dev)
    if ws is None or ws.numel() < need:
        ws = _gemm_workspaces[dev] = torch.zeros((need,), dtype=torch.uint8, device=dev)
    return ws


def gemm_dispatch(M: int, K: int, N: int, workspace_bytes: int = 0) -> int:
    """The kernel selector (KERNEL_*) the automatic path runs for an (M, K, N) product with a
    workspace of that size (nvfp4_gemm_dispatch); 0 for an empty or invalid product."""
    return int(load().nvfp4_gemm_dispatch(M, K, N, workspace_bytes))


def nvfp4_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, g_a: torch.Tensor,
               w_codes: torch.Tensor, w_scales: torch.Tensor, g_w: torch.Tensor,
               out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
               path: int = PATH_AUTO, workspace=None) -> torch.Tensor:
    """NVFP4 W4A4 product: out [M, N] = dequant(A) @ dequant(W)^T, fp32 accumulation.
    workspace: None (nvfp4_gemm_ex with `path`), "auto" (gemm_workspace(), nvfp4_gemm_ws) or a
    uint8 device tensor (nvfp4_gemm_ws; zero before its first use)."""
    if a_codes.dim() != 2 or w_codes.dim() != 2:
        raise ValueError("codes must be 2-D")
    M, K2 = a_codes.shape
    N = w_codes.shape[0]
    K = 2 * K2
    if w_codes.shape[1] != K2 or a_scales.shape != (M, K // 16) or w_scales.shape != (N, K // 16):
        raise ValueError("inconsistent operand shapes")
    for t in (a_codes, a_scales, w_codes, w_scales):
        if t.dtype != torch.uint8:
            raise ValueError("codes and scales must be uint8")
    for g in (g_a, g_w):
        if g.dtype != torch.float32 or g.numel() != 1:
            raise ValueError("tensor scales must be float32 tensors of one element")
    dev = _dev(a_codes, a_scales, g_a, w_codes, w_scales, g_w)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    elif out.shape != (M, N) or out.dtype != out_dtype:
        raise ValueError("out must be [M, N] of out_dtype")
    _dev(a_codes, out)
    if workspace is None:
        _check(load().nvfp4_gemm_ex(M, K, N, a_codes.data_ptr(), a_scales.data_ptr(), g_a.data_ptr(),
                                    w_codes.data_ptr(), w_scales.data_ptr(), g_w.data_ptr(),
                                    out.data_ptr(), _dt(out_dtype), path, _stream(dev)),
               "nvfp4_gemm")
        return out
    if path != PATH_AUTO:
        raise ValueError("a workspace is used by the automatic path only")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be None, "auto" or a uint8 tensor')
        workspace = gemm_workspace(M, K, N, dev)
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.device != dev or
                                  not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor on the operands' device")
    _check(load().nvfp4_gemm_ws(M, K, N, a_codes.data_ptr(), a_scales.data_ptr(), g_a.data_ptr(),
                                w_codes.data_ptr(), w_scales.data_ptr(), g_w.data_ptr(),
                                out.data_ptr(), _dt(out_dtype),
                                workspace.data_ptr() if workspace is not None else None,
                                workspace.numel() if workspace is not None else 0, _stream(dev)),
           "nvfp4_gemm_ws")
    return out


def nvfp4_gemm_quantize_output(a_codes: torch.Tensor, a_scales: torch.Tensor, g_a: torch.Tensor,
                               w_codes: torch.Tensor, w_scales: torch.Tensor, g_w: torch.Tensor,
                               g_y: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                               out: Optional[torch.Tensor] = None, y_codes: Optional[torch.Tensor] = None,
                               y_scales: Optional[torch.Tensor] = None
                               ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """NVFP4 product whose output is also quantized with the device scale g_y [1]: returns
    (out [M, N], y_codes [M, N/2], y_scales [M, N/16])."""
    if a_codes.dim() != 2 or w_codes.dim() != 2:
        raise ValueError("codes must be 2-D")
    M, K2 = a_codes.shape
    N = w_codes.shape[0]
    K = 2 * K2
    if w_codes.shape[1] != K2 or a_scales.shape != (M, K // 16) or w_scales.shape != (N, K // 16):
        raise ValueError("inconsistent operand shapes")
    for t in (a_codes, a_scales, w_codes, w_scales):
        if t.dtype != torch.uint8:
            raise ValueError("codes and scales must be uint8")
    for g in (g_a, g_w, g_y):
        if g.dtype != torch.float32 or g.numel() != 1:
            raise ValueError("tensor scales must be float32 tensors of one element")
    dev = _dev(a_codes, a_scales, g_a, w_codes, w_scales, g_w, g_y)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    elif out.shape != (M, N) or out.dtype != out_dtype:
        raise ValueError("out must be [M, N] of out_dtype")
    if y_codes is None:
        y_codes = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
    if y_scales is None:
        y_scales = torch.empty((M, N // 16), dtype=torch.uint8, device=dev)
    if y_codes.dtype != torch.uint8 or y_scales.dtype != torch.uint8 or \
            y_codes.numel() != M * (N // 2) or y_scales.numel() != M * (N // 16):
        raise ValueError("y_codes/y_scales must be uint8 of [M, N/2] / [M, N/16] elements")
    _dev(a_codes, out, y_codes, y_scales)
    _check(load().nvfp4_gemm_quantize_output(M, K, N, a_codes.data_ptr(), a_scales.data_ptr(), g_a.data_ptr(),
                                             w_codes.data_ptr(), w_scales.data_ptr(), g_w.data_ptr(),
                                             out.data_ptr(), _dt(out_dtype), g_y.data_ptr(), y_codes.data_ptr(),
                                             y_scales.data_ptr(), _stream(dev)),
           "nvfp4_gemm_quantize_output")
    return out, y_codes, y_scales


def nvfp4_quantize_gemm(a: torch.Tensor, g_a: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor,
                        g_w: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                        out: Optional[torch.Tensor] = None, a_codes: Optional[torch.Tensor] = None,
                        a_scales: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Raw activations a [M, K] (float32/bfloat16) with device scale g_a [1] times the NVFP4
    weights: returns (out [M, N], a_codes [M, K/2], a_scales [M, K/16])."""
    if a.dim() != 2 or w_codes.dim() != 2:
        raise ValueError("a and w_codes must be 2-D")
    M, K = a.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] != K // 2 or w_scales.shape != (N, K // 16):
        raise ValueError("inconsistent operand shapes")
    if w_codes.dtype != torch.uint8 or w_scales.dtype != torch.uint8:
        raise ValueError("codes and scales must be uint8")
    for g in (g_a, g_w):
        if g.dtype != torch.float32 or g.numel() != 1:
            raise ValueError("tensor scales must be float32 tensors of one element")
    dev = _dev(a, g_a, w_codes, w_scales, g_w)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    elif out.shape != (M, N) or out.dtype != out_dtype:
        raise ValueError("out must be [M, N] of out_dtype")
    if a_codes is None:
        a_codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if a_scales is None:
        a_scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    if a_codes.dtype != torch.uint8 or a_scales.dtype != torch.uint8 or \
            a_codes.numel() != M * (K // 2) or a_scales.numel() != M * (K // 16):
        raise ValueError("a_codes/a_scales must be uint8 of [M, K/2] / [M, K/16] elements")
    _dev(a, out, a_codes, a_scales)
    _check(load().nvfp4_quantize_gemm(M, K, N, a.data_ptr(), _dt(a.dtype), g_a.data_ptr(),
                                      w_codes.data_ptr(), w_scales.data_ptr(), g_w.data_ptr(),
                                      out.data_ptr(), _dt(out_dtype), a_codes.data_ptr(),
                                      a_scales.data_ptr(), _stream(dev)),
           "nvfp4_quantize_gemm")
    return out, a_codes, a_scales


def nvfp4_quantize_gemm_dynamic(a: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, g_w: torch.Tensor,
                                out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                                a_codes: Optional[torch.Tensor] = None, a_scales: Optional[torch.Tensor] = None,
                                g_a: Optional[torch.Tensor] = None
                                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """Raw activations a [M, K] times the NVFP4 weights with the activations' tensor scale
    computed on the device: returns (out [M, N], a_codes, a_scales, g_a [1])."""
    if a.dim() != 2 or w_codes.dim() != 2:
        raise ValueError("a and w_codes must be 2-D")
    M, K = a.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] != K // 2 or w_scales.shape != (N, K // 16):
        raise ValueError("inconsistent operand shapes")
    if w_codes.dtype != torch.uint8 or w_scales.dtype != torch.uint8:
        raise ValueError("codes and scales must be uint8")
    if g_w.dtype != torch.float32 or g_w.numel() != 1:
        raise ValueError("tensor scales must be float32 tensors of one element")
    dev = _dev(a, w_codes, w_scales, g_w)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    elif out.shape != (M, N) or out.dtype != out_dtype:
        raise ValueError("out must be [M, N] of out_dtype")
    if a_codes is None:
        a_codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if a_scales is None:
        a_scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    if g_a is None:
        g_a = torch.empty((1,), dtype=torch.float32, device=dev)
    if g_a.dtype != torch.float32 or g_a.numel() != 1:
        raise ValueError("g_a must be a float32 tensor of one element")
    if a_codes.dtype != torch.uint8 or a_scales.dtype != torch.uint8 or \
            a_codes.numel() != M * (K // 2) or a_scales.numel() != M * (K // 16):
        raise ValueError("a_codes/a_scales must be uint8 of [M, K/2] / [M, K/16] elements")
    _dev(a, out, a_codes, a_scales, g_a)
    _check(load().nvfp4_quantize_gemm_dynamic(M, K, N, a.data_ptr(), _dt(a.dtype), g_a.data_ptr(),
                                              w_codes.data_ptr(), w_scales.data_ptr(), g_w.data_ptr(),
                                              out.data_ptr(), _dt(out_dtype), a_codes.data_ptr(),
                                              a_scales.data_ptr(), _stream(dev)),
           "nvfp4_quantize_gemm_dynamic")
    return out, a_codes, a_scales, g_a


def _int32_vec(t: torch.Tensor, n: int, name: str) -> None:
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() != n:
        raise ValueError(f"{name} must be an int32 vector of {n} elements")


def nvfp4_tree_accept(parent: torch.Tensor, draft: torch.Tensor, greedy: torch.Tensor) -> torch.Tensor:
    """Greedy acceptance of a candidate tree: returns result int32 [3 + n] = (end node, accepted
    count L, bonus token, L path nodes, -1 padding)."""
    n = parent.numel()
    for t, name in ((parent, "parent"), (draft, "draft"), (greedy, "greedy")):
        _int32_vec(t, n, name)
    dev = _dev(parent, draft, greedy)
    result = torch.empty((3 + n,), dtype=torch.int32, device=dev)
    _check(load().nvfp4_tree_accept(n, parent.data_ptr(), draft.data_ptr(), greedy.data_ptr(),
                                    result.data_ptr(), _stream(dev)), "nvfp4_tree_accept")
    return result


_key_workspaces: dict = {}


def tree_key_workspace(dev: torch.device) -> torch.Tensor:
    """The argmax-key workspace of nvfp4_tree_verify for `dev` (1024 int64, zeroed once; every
    call leaves it zeroed).  Shared by the calls of this module: keep them on one stream, or
    pass a workspace of your own."""
    ws = _key_workspaces.get(dev)
    if ws is None:
        ws = _key_workspaces[dev] = torch.zeros((1024,), dtype=torch.int64, device=dev)
    return ws


def nvfp4_tree_verify(a_codes: torch.Tensor, a_scales: torch.Tensor, g_a: torch.Tensor,
                      w_codes: torch.Tensor, w_scales: torch.Tensor, g_w: torch.Tensor,
                      parent: torch.Tensor, draft: torch.Tensor, want_logits: bool = False,
                      keys: Optional[torch.Tensor] = None):
    """LM head over the M tree nodes plus greedy acceptance: returns (greedy int32 [M],
    result int32 [3 + M], logits fp32 [M, N] or None)."""
    M, K2 = a_codes.shape
    N = w_codes.shape[0]
    K = 2 * K2
    if w_codes.shape[1] != K2 or a_scales.shape != (M, K // 16) or w_scales.shape != (N, K // 16):
        raise ValueError("inconsistent operand shapes")
    _int32_vec(parent, M, "parent")
    _int32_vec(draft, M, "draft")
    dev = _dev(a_codes, a_scales, g_a, w_codes, w_scales, g_w, parent, draft)
    greedy = torch.empty((M,), dtype=torch.int32, device=dev)
    result = torch.empty((3 + M,), dtype=torch.int32, device=dev)
    if keys is None:
        keys = tree_key_workspace(dev)
    elif keys.dtype != torch.int64 or keys.numel() != 1024 or keys.device != dev:
        raise ValueError("keys must be 1024 int64 on the operands' device, zero on entry")
    logits = torch.empty((M, N), dtype=torch.float32, device=dev) if want_logits else None
    _check(load().nvfp4_tree_verify(M, K, N, a_codes.data_ptr(), a_scales.data_ptr(), g_a.data_ptr(),
                                    w_codes.data_ptr(), w_scales.data_ptr(), g_w.data_ptr(),
                                    parent.data_ptr(), draft.data_ptr(),
                                    logits.data_ptr() if logits is not None else None,
                                    greedy.data_ptr(), result.data_ptr(), keys.data_ptr(), _stream(dev)),
           "nvfp4_tree_verify")
    return greedy, result, logits


def nvfp4_kv_fp8_encode(x: torch.Tensor, scale: torch.Tensor, q: Optional[torch.Tensor] = None) -> torch.Tensor:
    """KV values x (float32/bfloat16, any shape, contiguous) with device decode scale [1] -> E4M3
    bytes (uint8, same shape)."""
    if scale.dtype != torch.float32 or scale.numel() != 1:
        raise ValueError("scale must be a float32 tensor of one element")
    dev = _dev(x, scale)
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    elif q.dtype != torch.uint8 or q.numel() != x.numel():
        raise ValueError("q must be uint8 with x's element count")
    _dev(x, q)
    _check(load().nvfp4_kv_fp8_encode(x.data_ptr(), _dt(x.dtype), x.numel(), scale.data_ptr(), q.data_ptr(),
                                      _stream(dev)), "nvfp4_kv_fp8_encode")
    return q


def nvfp4_kv_fp8_decode(q: torch.Tensor, scale: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """E4M3 bytes q (uint8) with device decode scale [1] -> values (out_dtype, same shape)."""
    if q.dtype != torch.uint8:
        raise ValueError("q must be uint8")
    if scale.dtype != torch.float32 or scale.numel() != 1:
        raise ValueError("scale must be a float32 tensor of one element")
    dev = _dev(q, scale)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=dev)
    elif out.dtype != out_dtype or out.numel() != q.numel():
        raise ValueError("out must have q's element count and out_dtype")
    _dev(q, out)
    _check(load().nvfp4_kv_fp8_decode(q.data_ptr(), q.numel(), scale.data_ptr(), out.data_ptr(), _dt(out_dtype),
                                      _stream(dev)), "nvfp4_kv_fp8_decode")
    return out


def nvfp4_act_global_scale(a: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dynamic activation decode scale g_a = amax|a| / 2688 of a [M, K] float32/bfloat16 tensor,
    computed on the device -> float32 [1] (device)."""
    if a.dim() != 2:
        raise ValueError("a must be [M, K]")
    dev = _dev(a)
    if out is None:
        out = torch.empty((1,), dtype=torch.float32, device=dev)
    elif out.dtype != torch.float32 or out.numel() != 1:
        raise ValueError("out must be a float32 tensor of one element")
    M, K = a.shape
    _check(load().nvfp4_act_global_scale(a.data_ptr(), _dt(a.dtype), M, K, out.data_ptr(), _stream(dev)),
           "nvfp4_act_global_scale")
    return out


def nvfp4_stream_read(a: torch.Tensor, b: torch.Tensor, sink: Optional[torch.Tensor] = None,
                      magic: int = 0x9E3779B9) -> torch.Tensor:
    """Reads every byte of a and b once (the read-only streaming ceiling of nvfp4_stream_read);
    returns the sink (int32 [1] on the device, written only by a lane whose XOR fold of the words
    it read equals `magic`)."""
    dev = _dev(a, b)
    if sink is None:
        sink = torch.zeros((1,), dtype=torch.int32, device=dev)
    _dev(a, sink)
    _check(load().nvfp4_stream_read(a.data_ptr(), a.numel() * a.element_size(), b.data_ptr(),
                                    b.numel() * b.element_size(), sink.data_ptr(), magic, _stream(dev)),
           "nvfp4_stream_read")
    return sink
