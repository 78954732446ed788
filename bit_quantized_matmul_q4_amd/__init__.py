"""MI355X (gfx950) 4-bit group-256 weight-quantized matmul: dequant-fused GEMV
for decode and an int8-MFMA MMQ GEMM on Q8_1 activations for prefill.

The compute lives in libq4mi.so (HIP kernels behind the C ABI of
include/q4mi.h); this package is the Python binding of that ABI.
"""
from ._lib import (  # noqa: F401
    GEMV_MAX_M,
    Q4Error,
    lib,
    q4_abi_version,
    q4_gemv,
    q4_gemv_g32,
    q4_gemv_g32_workspace_bytes,
    q4_gemv_workspace_bytes,
    q4_mmq_block_dots,
    q4_mmq_gemm,
    q4_mmq_gemm_g32,
    q4_mmq_gemm_q8_1,
    q4_mmq_workspace_bytes,
    q4_pack,
    q4_pack_g32,
    q8_1_quantize,
    strerror,
)
