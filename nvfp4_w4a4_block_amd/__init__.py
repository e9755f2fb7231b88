"""NVFP4 W4A4 block-scaled quantization and GEMV/GEMM for AMD Instinct MI355X (gfx950).

The compute path is libnvfp4.so (HIP kernels behind the C ABI of include/nvfp4.h);
`binding` marshals torch tensors into it.  `workloads` draws the seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    NVFP4Error, nvfp4_gemm, nvfp4_quantize_act, nvfp4_quantize_weights, PATH_AUTO, PATH_SKINNY,
    PATH_TILED,
)
