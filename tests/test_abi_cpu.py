"""The C-ABI library loads, exports what include/nvfp4.h declares, and validates arguments
on the host (CPU only: every call here is rejected, or empty, before any HIP call)."""
import ctypes
import os
import re

import pytest

from nvfp4_w4a4_block_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "nvfp4.h")
A16 = 0x10000  # a fake, 16-byte aligned address: never dereferenced by a rejected call


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 6
    for n in names:
        assert hasattr(lib, n), f"{n} declared in nvfp4.h but not exported"
    assert sorted(B.EXPORTS) == names


def test_exported_symbols_are_c_linkage():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    syms = set(re.findall(r"\b(nvfp4_\w+)\b", out))
    assert set(declared_functions()) <= syms


def test_status_strings_and_version(lib):
    for s in range(7):
        assert B.status_string(s) and B.status_string(s) != "unknown status"
    assert B.status_string(99) == "unknown status"
    assert lib.nvfp4_abi_version() == 11


def gemm(lib, M, K, N, ptrs=(A16,) * 7, out_dt=B.NVFP4_BF16, path=B.PATH_AUTO):
    ac, asc, ga, wc, wsc, gw, out = ptrs
    return lib.nvfp4_gemm_ex(M, K, N, ac, asc, ga, wc, wsc, gw, out, out_dt, path, None)


@pytest.mark.parametrize("K", [0, 8, 15, 17, 24, -16])
def test_gemm_rejects_bad_k(lib, K):
    assert gemm(lib, 1, K, 16) == B.NVFP4_ERR_SHAPE


def test_gemm_rejects_bad_sizes(lib):
    assert gemm(lib, -1, 32, 16) == B.NVFP4_ERR_SHAPE
    assert gemm(lib, 1, 32, -3) == B.NVFP4_ERR_SHAPE
    assert gemm(lib, 1, 1 << 27, 16) == B.NVFP4_ERR_SHAPE          # N * K = 2^31
    assert gemm(lib, 1 << 20, 16, 1 << 11) == B.NVFP4_ERR_SHAPE    # M * N = 2^31
    assert gemm(lib, 1 << 21, 16, 16, path=B.PATH_SKINNY) == B.NVFP4_ERR_SHAPE  # grid rows > 65535


def test_gemm_rejects_null_align_dtype_path(lib):
    assert gemm(lib, 1, 32, 16, ptrs=(A16,) * 6 + (0,)) == B.NVFP4_ERR_NULL
    assert gemm(lib, 1, 32, 16, ptrs=(0,) + (A16,) * 6) == B.NVFP4_ERR_NULL
    assert gemm(lib, 1, 32, 16, ptrs=(A16 + 8,) + (A16,) * 6) == B.NVFP4_ERR_ALIGN
    assert gemm(lib, 1, 32, 16, ptrs=(A16,) * 2 + (A16 + 2,) + (A16,) * 4) == B.NVFP4_ERR_ALIGN
    # scalar scale pointers only need 4-byte alignment: this one passes validation up to the
    # dtype check, which fails first here
    assert gemm(lib, 1, 32, 16, ptrs=(A16,) * 2 + (A16 + 4,) + (A16,) * 4, out_dt=7) == B.NVFP4_ERR_DTYPE
    assert gemm(lib, 1, 32, 16, path=11) == B.NVFP4_ERR_DTYPE
    assert gemm(lib, 1, 32, 16, path=-1) == B.NVFP4_ERR_DTYPE


def test_gemm_kernel_selectors_refuse_shapes_they_do_not_take(lib):
    """An explicitly selected kernel that does not take the product is refused (the checks below
    decide on the shape alone, before any HIP call)."""
    assert gemm(lib, 1, 32, 16, path=B.KERNEL_GEMV_FP4) == B.NVFP4_ERR_SHAPE      # K % 1024 != 0
    assert gemm(lib, 3, 1024, 16, path=B.KERNEL_GEMV_FP4) == B.NVFP4_ERR_SHAPE    # M > 2
    assert gemm(lib, 1, 32, 16, path=B.KERNEL_GEMV_FLAT) == B.NVFP4_ERR_SHAPE     # K < 2048
    assert gemm(lib, 17, 128, 16, path=B.KERNEL_M16) == B.NVFP4_ERR_SHAPE         # M > 16
    assert gemm(lib, 4, 144, 16, path=B.KERNEL_M16) == B.NVFP4_ERR_SHAPE          # K % 128 != 0
    assert gemm(lib, 17, 1024, 16, path=B.KERNEL_M16_STREAM) == B.NVFP4_ERR_SHAPE  # M > 16
    assert gemm(lib, 4, 1152, 16, path=B.KERNEL_M16_STREAM) == B.NVFP4_ERR_SHAPE   # 9 lines: no chunk length
    assert gemm(lib, 4, 144, 16, path=B.KERNEL_SKINNY256) == B.NVFP4_ERR_SHAPE    # K % 256 != 0
    assert gemm(lib, 40, 1280, 16, path=B.KERNEL_TILED_PERSISTENT) == B.NVFP4_ERR_SHAPE  # K % 1024 != 0
    assert gemm(lib, 0, 32, 16, ptrs=(0,) * 7, path=B.KERNEL_GEMV_FP4) == B.NVFP4_OK  # empty: nothing to run
    assert gemm(lib, 1 << 21, 16, 16, path=B.KERNEL_SKINNY16) == B.NVFP4_ERR_SHAPE   # grid rows > 65535


def test_gemm_dispatch_host_cases(lib):
    """nvfp4_gemm_dispatch on shapes decided without a device query: invalid or empty products
    (0), one or two rows with K a multiple of 1024 up to 8192 (the FP4 GEMV), more than 16 rows
    (the persistent tiled kernel for K % 1024 == 0, else the simple one)."""
    f = lib.nvfp4_gemm_dispatch
    assert f(0, 5120, 100, 0) == 0
    assert f(1, 5120, 0, 0) == 0
    assert f(1, 24, 100, 0) == 0
    assert f(1, 5120, 100, -1) == 0
    assert f(1, 5120, 25600, 0) == B.KERNEL_GEMV_FP4
    assert f(2, 1024, 7, 0) == B.KERNEL_GEMV_FP4
    assert f(512, 5120, 25600, 0) == B.KERNEL_TILED_PERSISTENT
    assert f(512, 25600, 5120, 0) == B.KERNEL_TILED_PERSISTENT
    assert f(17, 768, 100, 0) == B.KERNEL_TILED
    assert lib.nvfp4_gemm(1, 32, 16, A16, A16, A16, A16, A16, A16, A16, 2, None) == B.NVFP4_ERR_DTYPE


def test_gemm_ws_validation(lib):
    """nvfp4_gemm_ws validates like nvfp4_gemm, plus its workspace (size, NULL, alignment)."""
    def ws(M, K, N, work=A16, nbytes=4096, out_dt=B.NVFP4_BF16, ptrs=(A16,) * 7):
        ac, asc, ga, wc, wsc, gw, out = ptrs
        return lib.nvfp4_gemm_ws(M, K, N, ac, asc, ga, wc, wsc, gw, out, out_dt, work, nbytes, None)
    assert ws(16, 256, 64, out_dt=3) == B.NVFP4_ERR_DTYPE
    assert ws(16, 24, 64) == B.NVFP4_ERR_SHAPE
    assert ws(16, 256, 64, nbytes=-1) == B.NVFP4_ERR_SHAPE
    assert ws(16, 256, 64, work=0) == B.NVFP4_ERR_NULL
    assert ws(16, 256, 64, work=A16 + 8) == B.NVFP4_ERR_ALIGN
    assert ws(16, 256, 64, ptrs=(A16,) * 6 + (0,)) == B.NVFP4_ERR_NULL
    assert ws(0, 256, 64, work=0, nbytes=0, ptrs=(0,) * 7) == B.NVFP4_OK


def test_gemm_quantize_output_validation(lib):
    """nvfp4_gemm_quantize_output: nvfp4_gemm's rules plus N % 16 == 0 and the output-quantization
    pointers (scale 4-byte aligned, codes and scales 16-byte aligned)."""
    def qo(M, K, N, out_dt=B.NVFP4_BF16, ptrs=(A16,) * 10):
        ac, asc, ga, wc, wsc, gw, out, gy, yc, ys = ptrs
        return lib.nvfp4_gemm_quantize_output(M, K, N, ac, asc, ga, wc, wsc, gw, out, out_dt, gy, yc, ys, None)
    assert qo(64, 256, 64, out_dt=5) == B.NVFP4_ERR_DTYPE
    assert qo(64, 256, 40) == B.NVFP4_ERR_SHAPE      # output blocks run along N
    assert qo(64, 24, 64) == B.NVFP4_ERR_SHAPE
    assert qo(0, 256, 64, ptrs=(0,) * 10) == B.NVFP4_OK
    for k in range(10):
        ptrs = [A16] * 10
        ptrs[k] = 0
        assert qo(64, 256, 64, ptrs=tuple(ptrs)) == B.NVFP4_ERR_NULL, k
    for k, off in ((7, 2), (8, 8), (9, 4), (6, 8)):
        ptrs = [A16] * 10
        ptrs[k] = A16 + off
        assert qo(64, 256, 64, ptrs=tuple(ptrs)) == B.NVFP4_ERR_ALIGN, k


def test_gemm_workspace_bytes_host_cases(lib):
    """Shapes the split path never takes need no workspace (decided from the shape alone, before
    any device query): one or two rows (the GEMV), more than 16 rows (the tiled path), K not a
    multiple of 128, short-K products with N <= 16384 (the skinny kernel), invalid shapes.  The
    shapes that do split depend on the device's compute-unit count and are checked on the GPU."""
    f = lib.nvfp4_gemm_workspace_bytes
    assert f(1, 25600, 5120) == 0
    assert f(2, 25600, 5120) == 0
    assert f(17, 25600, 5120) == 0
    assert f(512, 5120, 25600) == 0
    assert f(16, 25616, 5120) == 0
    assert f(16, 25600, 0) == 0
    assert f(16, 24, 5120) == 0
    assert f(-1, 256, 64) == 0
    assert f(16, 5120, 5120) == 0  # short K, N <= 16384: the skinny kernel, unsplit
    assert f(16, 8192, 16384) == 0


def test_empty_gemm_is_ok_without_pointers(lib):
    assert gemm(lib, 0, 32, 16, ptrs=(0,) * 7) == B.NVFP4_OK
    assert gemm(lib, 4, 32, 0, ptrs=(0,) * 7) == B.NVFP4_OK


def test_quantize_validation(lib):
    q = lib.nvfp4_quantize_act
    assert q(A16, B.NVFP4_BF16, 1, 20, A16, A16, A16, None) == B.NVFP4_ERR_SHAPE
    assert q(A16, 5, 1, 32, A16, A16, A16, None) == B.NVFP4_ERR_DTYPE
    assert q(0, B.NVFP4_F32, 1, 32, A16, A16, A16, None) == B.NVFP4_ERR_NULL
    assert q(A16, B.NVFP4_F32, 1, 32, 0, A16, A16, None) == B.NVFP4_ERR_NULL
    assert q(A16 + 4, B.NVFP4_F32, 1, 32, A16, A16, A16, None) == B.NVFP4_ERR_ALIGN
    assert q(A16, B.NVFP4_F32, 1, 32, A16 + 1, A16, A16, None) == B.NVFP4_ERR_ALIGN
    assert q(0, B.NVFP4_F32, 0, 32, 0, 0, 0, None) == B.NVFP4_OK           # empty
    w = lib.nvfp4_quantize_weights
    assert w(A16, B.NVFP4_F32, 4, 40, A16, A16, A16, None) == B.NVFP4_ERR_SHAPE
    assert w(A16, 9, 4, 32, A16, A16, A16, None) == B.NVFP4_ERR_DTYPE
    assert w(A16, B.NVFP4_F32, 4, 32, A16, A16, 0, None) == B.NVFP4_ERR_NULL
    assert w(0, B.NVFP4_F32, 4, 32, A16, A16, A16, None) == B.NVFP4_ERR_NULL
    assert w(A16, B.NVFP4_F32, 4, 32, A16 + 8, A16, A16, None) == B.NVFP4_ERR_ALIGN
    assert w(A16, B.NVFP4_F32, 4, 32, A16, A16, A16 + 2, None) == B.NVFP4_ERR_ALIGN
    assert w(A16, B.NVFP4_F32, 1 << 16, 1 << 15, A16, A16, A16, None) == B.NVFP4_ERR_SHAPE


def test_binding_has_no_cpu_fallback():
    """The tensor-level functions refuse CPU tensors instead of computing anything."""
    import torch
    with pytest.raises(ValueError):
        B.nvfp4_quantize_weights(torch.zeros(4, 32))


def qgemm(lib, M, K, N, ptrs=(A16,) * 8, a_dt=B.NVFP4_BF16, out_dt=B.NVFP4_BF16):
    a, ga, wc, wsc, gw, out, ac, asc = ptrs
    return lib.nvfp4_quantize_gemm(M, K, N, a, a_dt, ga, wc, wsc, gw, out, out_dt, ac, asc, None)


def test_quantize_gemm_validation(lib):
    assert qgemm(lib, 1, 5120, 64, a_dt=7) == B.NVFP4_ERR_DTYPE
    assert qgemm(lib, 1, 5120, 64, out_dt=2) == B.NVFP4_ERR_DTYPE
    assert qgemm(lib, 1, 24, 64) == B.NVFP4_ERR_SHAPE
    assert qgemm(lib, -1, 32, 64) == B.NVFP4_ERR_SHAPE
    assert qgemm(lib, 1, 32, -1) == B.NVFP4_ERR_SHAPE
    assert qgemm(lib, 0, 32, 64, ptrs=(None,) * 8) == B.NVFP4_OK  # empty: nothing to do
    for k in range(8):
        ptrs = [A16] * 8
        ptrs[k] = None
        assert qgemm(lib, 1, 5120, 64, ptrs=tuple(ptrs)) == B.NVFP4_ERR_NULL, k
        ptrs[k] = A16 + (2 if k in (1, 4) else 8)  # scalars need 4 bytes, arrays 16
        assert qgemm(lib, 1, 5120, 64, ptrs=tuple(ptrs)) == B.NVFP4_ERR_ALIGN, k


def test_quantize_gemm_dynamic_validation(lib):
    """Same rules as nvfp4_quantize_gemm, with the tensor scale an output that is always
    required (checked before anything else that could launch)."""
    def dq(M, K, N, ptrs=(A16,) * 8, a_dt=B.NVFP4_BF16, out_dt=B.NVFP4_BF16):
        a, ga, wc, wsc, gw, out, ac, asc = ptrs
        return lib.nvfp4_quantize_gemm_dynamic(M, K, N, a, a_dt, ga, wc, wsc, gw, out, out_dt, ac, asc, None)
    assert dq(1, 5120, 64, a_dt=7) == B.NVFP4_ERR_DTYPE
    assert dq(1, 5120, 64, out_dt=2) == B.NVFP4_ERR_DTYPE
    assert dq(1, 24, 64) == B.NVFP4_ERR_SHAPE
    assert dq(-1, 32, 64) == B.NVFP4_ERR_SHAPE
    assert dq(1, 32, -1) == B.NVFP4_ERR_SHAPE
    assert dq(0, 32, 64, ptrs=(A16, None) + (A16,) * 6) == B.NVFP4_ERR_NULL  # g_a is written even for M == 0
    for k in range(8):
        ptrs = [A16] * 8
        ptrs[k] = None
        assert dq(1, 5120, 64, ptrs=tuple(ptrs)) == B.NVFP4_ERR_NULL, k
        ptrs[k] = A16 + (2 if k in (1, 4) else 8)  # scalars need 4 bytes, arrays 16
        assert dq(1, 5120, 64, ptrs=tuple(ptrs)) == B.NVFP4_ERR_ALIGN, k


def test_tree_entry_points_validate(lib):
    A = A16
    assert lib.nvfp4_tree_accept(0, A, A, A, A, None) == B.NVFP4_ERR_SHAPE
    assert lib.nvfp4_tree_accept(65, A, A, A, A, None) == B.NVFP4_ERR_SHAPE
    assert lib.nvfp4_tree_accept(16, None, A, A, A, None) == B.NVFP4_ERR_NULL
    assert lib.nvfp4_tree_accept(16, A + 2, A, A, A, None) == B.NVFP4_ERR_ALIGN

    def verify(M, K, N, ptrs=None, logits=A):
        ptrs = ptrs or (A,) * 6 + (A, A, A, A, A)
        ac, asc, ga, wc, wsc, gw, par, dr, gr, res, keys = ptrs
        return lib.nvfp4_tree_verify(M, K, N, ac, asc, ga, wc, wsc, gw, par, dr, logits, gr, res, keys, None)
    assert verify(0, 5120, 100) == B.NVFP4_ERR_SHAPE
    assert verify(17, 5120, 100) == B.NVFP4_ERR_SHAPE
    assert verify(16, 5120, 0) == B.NVFP4_ERR_SHAPE
    assert verify(16, 24, 100) == B.NVFP4_ERR_SHAPE
    ptrs = [A] * 11
    ptrs[10] = A + 4  # keys need 8-byte alignment
    assert verify(16, 5120, 100, tuple(ptrs)) == B.NVFP4_ERR_ALIGN
    ptrs[10] = None
    assert verify(16, 5120, 100, tuple(ptrs)) == B.NVFP4_ERR_NULL
    # logits may be omitted only where the argmax is fused (K % 128 == 0)
    assert verify(16, 1040, 100, logits=None) == B.NVFP4_ERR_NULL


def test_kv_fp8_validation(lib):
    A = A16
    for f in (lambda *a: lib.nvfp4_kv_fp8_encode(a[0], a[4], a[1], a[2], a[3], None),
              lambda *a: lib.nvfp4_kv_fp8_decode(a[3], a[1], a[2], a[0], a[4], None)):
        assert f(A, 100, A, A, 9) == B.NVFP4_ERR_DTYPE
        assert f(A, -1, A, A, B.NVFP4_BF16) == B.NVFP4_ERR_SHAPE
        assert f(None, 0, None, None, B.NVFP4_BF16) == B.NVFP4_OK
        assert f(None, 100, A, A, B.NVFP4_BF16) == B.NVFP4_ERR_NULL
        assert f(A, 100, A + 2, A, B.NVFP4_BF16) == B.NVFP4_ERR_ALIGN
        assert f(A + 8, 100, A, A, B.NVFP4_BF16) == B.NVFP4_ERR_ALIGN


def test_act_global_scale_validation(lib):
    A = A16
    assert lib.nvfp4_act_global_scale(A, 9, 1, 16, A, None) == B.NVFP4_ERR_DTYPE
    assert lib.nvfp4_act_global_scale(A, B.NVFP4_BF16, 1, 24, A, None) == B.NVFP4_ERR_SHAPE
    assert lib.nvfp4_act_global_scale(A, B.NVFP4_BF16, 1, 16, None, None) == B.NVFP4_ERR_NULL
    assert lib.nvfp4_act_global_scale(None, B.NVFP4_BF16, 1, 16, A, None) == B.NVFP4_ERR_NULL
    assert lib.nvfp4_act_global_scale(A, B.NVFP4_BF16, 1, 16, A + 2, None) == B.NVFP4_ERR_ALIGN
    assert lib.nvfp4_act_global_scale(A + 8, B.NVFP4_BF16, 1, 16, A, None) == B.NVFP4_ERR_ALIGN
