"""C-ABI checks that need no GPU: the library loads, exports every function
include/q4mi.h declares, and rejects invalid arguments with the documented
error codes before any HIP call (so nothing here touches a device)."""
import ctypes
import os
import re

import pytest

import bit_quantized_matmul_q4_amd as q4
from bit_quantized_matmul_q4_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4mi.h")

ARG, ALIGN, WORKSPACE = -1, -2, -3
FAKE = ctypes.c_void_p(0x10000)       # 64 KiB-aligned non-null host-side token (never dereferenced)
ODD = ctypes.c_void_p(0x10002)        # misaligned token
NULL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q[48]\w*)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(names) == set(_lib.SYMBOLS), names


def test_library_exports_every_declared_symbol():
    L = q4.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_strerror():
    assert q4.q4_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6, -99):
        assert isinstance(q4.strerror(code), str) and q4.strerror(code)


@pytest.mark.parametrize("K", [0, -256, 100, 255, 2 ** 21])
def test_bad_k_rejected(K):
    L = q4.lib()
    assert L.q4_pack(FAKE, 4, K, FAKE, FAKE, NULL) == ARG
    assert L.q4_gemv(FAKE, 1, FAKE, FAKE, 4, K, FAKE, NULL, 0, NULL) == ARG
    assert L.q4_mmq_gemm(FAKE, FAKE, 4, FAKE, FAKE, 4, K, FAKE, NULL, 0, NULL) == ARG
    assert L.q4_mmq_block_dots(FAKE, 4, FAKE, 4, K, FAKE, NULL) == ARG
    assert L.q4_gemv_workspace_bytes(1, 4, K) == 0


def test_q8_1_k_multiple_of_32():
    L = q4.lib()
    assert L.q8_1_quantize(FAKE, 2, 48, FAKE, FAKE, NULL) == ARG
    assert L.q8_1_quantize(FAKE, -1, 64, FAKE, FAKE, NULL) == ARG


@pytest.mark.parametrize("M", [-1, 17, 100])
def test_gemv_m_range(M):
    assert q4.lib().q4_gemv(FAKE, M, FAKE, FAKE, 8, 256, FAKE, NULL, 0, NULL) == ARG


def test_negative_n_rejected():
    L = q4.lib()
    assert L.q4_pack(FAKE, -1, 256, FAKE, FAKE, NULL) == ARG
    assert L.q4_gemv(FAKE, 1, FAKE, FAKE, -5, 256, FAKE, NULL, 0, NULL) == ARG
    assert L.q4_mmq_gemm(FAKE, FAKE, 1, FAKE, FAKE, -5, 256, FAKE, NULL, 0, NULL) == ARG


def test_null_pointers_rejected():
    L = q4.lib()
    assert L.q4_pack(NULL, 4, 256, FAKE, FAKE, NULL) == ARG
    assert L.q4_pack(FAKE, 4, 256, NULL, FAKE, NULL) == ARG
    assert L.q8_1_quantize(FAKE, 4, 256, FAKE, NULL, NULL) == ARG
    assert L.q4_gemv(FAKE, 1, FAKE, FAKE, 4, 256, NULL, NULL, 0, NULL) == ARG
    assert L.q4_mmq_gemm(FAKE, NULL, 4, FAKE, FAKE, 4, 256, FAKE, NULL, 0, NULL) == ARG
    assert L.q4_mmq_block_dots(FAKE, 4, FAKE, 4, 256, NULL, NULL) == ARG


def test_misaligned_pointers_rejected():
    L = q4.lib()
    assert L.q4_pack(ODD, 4, 256, FAKE, FAKE, NULL) == ALIGN
    assert L.q4_pack(FAKE, 4, 256, ODD, FAKE, NULL) == ALIGN
    assert L.q8_1_quantize(FAKE, 4, 256, ODD, FAKE, NULL) == ALIGN
    assert L.q4_gemv(ODD, 1, FAKE, FAKE, 4, 256, FAKE, NULL, 0, NULL) == ALIGN
    assert L.q4_gemv(FAKE, 1, FAKE, ctypes.c_void_p(0x10001), 4, 256, FAKE, NULL, 0, NULL) == ALIGN
    assert L.q4_mmq_gemm(ODD, FAKE, 4, FAKE, FAKE, 4, 256, FAKE, NULL, 0, NULL) == ALIGN
    assert L.q4_mmq_block_dots(FAKE, 4, ODD, 4, 256, FAKE, NULL) == ALIGN


def test_empty_products_are_no_ops():
    L = q4.lib()
    # nothing to do: valid, no device needed, null data pointers allowed
    assert L.q4_pack(NULL, 0, 256, NULL, NULL, NULL) == 0
    assert L.q8_1_quantize(NULL, 0, 64, NULL, NULL, NULL) == 0
    assert L.q4_gemv(NULL, 0, NULL, NULL, 16, 256, NULL, NULL, 0, NULL) == 0
    assert L.q4_gemv(NULL, 3, NULL, NULL, 0, 256, NULL, NULL, 0, NULL) == 0
    assert L.q4_mmq_gemm(NULL, NULL, 0, NULL, NULL, 9, 512, NULL, NULL, 0, NULL) == 0
    assert L.q4_mmq_block_dots(NULL, 5, NULL, 0, 512, NULL, NULL) == 0


def test_block_dots_size_limit():
    # M * N * K/32 beyond 2^31 int32 entries is refused
    assert q4.lib().q4_mmq_block_dots(FAKE, 1 << 16, FAKE, 1 << 16, 256, FAKE, NULL) == ARG


def test_workspace_queries_are_host_only():
    for M in (1, 2, 4, 8, 16):
        assert q4.q4_gemv_workspace_bytes(M, 151936, 4096) >= 0
    assert q4.q4_mmq_workspace_bytes(2048, 12288, 4096) >= 0


def test_binding_rejects_host_tensors():
    import torch
    W = torch.zeros((4, 256), dtype=torch.float32)
    with pytest.raises(ValueError):
        q4.q4_pack(W)


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libq4mi.so")
    with pytest.raises(ImportError):
        _lib.lib()


def test_mmq_q8_1_output_argument_checks():
    L = q4.lib()
    fn = L.q4_mmq_gemm_q8_1
    # N must be a multiple of 32 (Q8_1 blocks along n)
    assert fn(FAKE, FAKE, 4, FAKE, FAKE, 48, 256, FAKE, FAKE, NULL, 0, NULL) == ARG
    assert fn(FAKE, FAKE, 4, FAKE, FAKE, 64, 100, FAKE, FAKE, NULL, 0, NULL) == ARG
    # empty problems are no-ops; missing outputs are argument errors
    assert fn(NULL, NULL, 0, NULL, NULL, 64, 256, NULL, NULL, NULL, 0, NULL) == 0
    assert fn(FAKE, FAKE, 4, FAKE, FAKE, 64, 256, NULL, FAKE, NULL, 0, NULL) == ARG
    assert fn(FAKE, FAKE, 4, FAKE, FAKE, 64, 256, FAKE, NULL, NULL, 0, NULL) == ARG


def test_gemv_plan_is_made_for_the_whole_shape():
    # 1048576 x 4096 weights run as two row ranges (1048512 rows and 64); the
    # plan, and with it the workspace, comes from the whole shape: no K split
    # at M = 8 (a 64-row matrix on its own would split K)
    assert q4.q4_gemv_workspace_bytes(8, 1048576, 4096) == 0
    assert q4.q4_gemv_workspace_bytes(8, 64, 4096) > 0
    # the K-split partials of the largest row range: nsplit x M x rows
    ws = q4.q4_gemv_workspace_bytes(8, 300, 2560)
    assert ws > 0 and ws % (8 * 300 * 4) == 0


def test_gemv_output_beyond_one_descriptor_rejected():
    # the matrix-core arm without a K split addresses y through one 2 GiB
    # descriptor: M * N <= 2^29
    L = q4.lib()
    assert L.q4_gemv(FAKE, 16, FAKE, FAKE, 40000000, 256, FAKE, NULL, 0, NULL) == ARG
    assert q4.q4_gemv_workspace_bytes(16, 40000000, 256) == 0
    # one activation row on the VALU arm writes y with 64-bit indexing: allowed
    assert q4.q4_gemv_workspace_bytes(1, 40000000, 256) == 0


def test_gemv_noalloc_validates_before_any_device_call():
    L = q4.lib()
    # more K-split partials than the library's fixed scratch array holds
    assert q4.q4_gemv_workspace_bytes(16, 151936, 65536) > q4.NOALLOC_SCRATCH_BYTES
    assert L.q4_gemv_noalloc(FAKE, 16, FAKE, FAKE, 151936, 65536, FAKE, NULL) == WORKSPACE
    assert L.q4_gemv_noalloc(FAKE, 17, FAKE, FAKE, 8, 256, FAKE, NULL) == ARG
    assert L.q4_gemv_noalloc(ODD, 1, FAKE, FAKE, 8, 256, FAKE, NULL) == ALIGN
    assert L.q4_gemv_noalloc(NULL, 0, NULL, NULL, 8, 256, NULL, NULL) == 0
