"""ctypes binding of libq4mi.so (the C ABI in include/q4mi.h).

Argument marshalling only: every function checks devices, dtypes and shapes of
its torch tensors, allocates missing outputs with torch on the input's device,
and calls the C entry point of the same name on the current torch stream.
All arithmetic happens in the library's HIP kernels.  There is no fallback:
if libq4mi.so is missing or the call fails, an exception is raised.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4mi.so")

Q4_OK = 0
ERRORS = {
    -1: "Q4_ERR_ARG",
    -2: "Q4_ERR_ALIGN",
    -3: "Q4_ERR_WORKSPACE",
    -4: "Q4_ERR_ARCH",
    -5: "Q4_ERR_LAUNCH",
    -6: "Q4_ERR_DEVICE",
}
GEMV_MAX_M = 16
SYMBOLS = [
    "q4_abi_version", "q4_strerror", "q4_pack", "q8_1_quantize", "q4_gemv_workspace_bytes",
    "q4_gemv", "q4_mmq_workspace_bytes", "q4_mmq_gemm", "q4_mmq_gemm_q8_1", "q4_mmq_block_dots",
    "q4_pack_g32", "q4_gemv_g32_workspace_bytes", "q4_gemv_g32", "q4_mmq_gemm_g32",
    "q4_gemv_noalloc", "q4_mmq_int8_workspace_bytes", "q4_mmq_gemm_int8",
]
NOALLOC_SCRATCH_BYTES = 32 << 20

_lib = None


class Q4Error(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__("%s: %s (%s)" % (where, ERRORS.get(code, code), strerror(code)))


def lib():
    """Load libq4mi.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libq4mi.so not found at %s; build it with "
                          "`python -m bit_quantized_matmul_q4_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sig = {
        "q4_abi_version": ([], I),
        "q4_strerror": ([I], ctypes.c_char_p),
        "q4_pack": ([P, I64, I64, P, P, P], I),
        "q8_1_quantize": ([P, I64, I64, P, P, P], I),
        "q4_gemv_workspace_bytes": ([I64, I64, I64], SZ),
        "q4_gemv": ([P, I64, P, P, I64, I64, P, P, SZ, P], I),
        "q4_mmq_workspace_bytes": ([I64, I64, I64], SZ),
        "q4_mmq_gemm": ([P, P, I64, P, P, I64, I64, P, P, SZ, P], I),
        "q4_mmq_gemm_q8_1": ([P, P, I64, P, P, I64, I64, P, P, P, SZ, P], I),
        "q4_mmq_block_dots": ([P, I64, P, I64, I64, P, P], I),
        "q4_pack_g32": ([P, I64, I64, P, P, P], I),
        "q4_gemv_g32_workspace_bytes": ([I64, I64, I64], SZ),
        "q4_gemv_g32": ([P, I64, P, P, I64, I64, P, P, SZ, P], I),
        "q4_mmq_gemm_g32": ([P, P, I64, P, P, I64, I64, P, P, SZ, P], I),
        "q4_gemv_noalloc": ([P, I64, P, P, I64, I64, P, P], I),
        "q4_mmq_int8_workspace_bytes": ([I64, I64, I64], SZ),
        "q4_mmq_gemm_int8": ([P, P, I64, P, P, I64, I64, P, P, SZ, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def strerror(code):
    return lib().q4_strerror(int(code)).decode()


def q4_abi_version():
    return lib().q4_abi_version()


def _stream(stream, t):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, shape, name):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check(rc, where):
    if rc != Q4_OK:
        raise Q4Error(rc, where)


def q4_pack(W, qs=None, sm=None, stream=None):
    """W fp32 [N][K] -> (qs uint8 [N][K/2], sm float16 [N][K/256][2])."""
    N, K = W.shape
    _need(W, torch.float32, (N, K), "W")
    if qs is None:
        qs = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    if sm is None:
        sm = torch.empty((N, K // 256, 2), dtype=torch.float16, device=W.device)
    _need(qs, torch.uint8, (N, K // 2), "qs")
    _need(sm, torch.float16, (N, K // 256, 2), "sm")
    _check(lib().q4_pack(_ptr(W), N, K, _ptr(qs), _ptr(sm), _stream(stream, W)), "q4_pack")
    return qs, sm


def q8_1_quantize(x, qa=None, ds=None, stream=None):
    """x fp32 [M][K] -> (qa int8 [M][K], ds float16 [M][K/32][2] = (d, s))."""
    M, K = x.shape
    _need(x, torch.float32, (M, K), "x")
    if qa is None:
        qa = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if ds is None:
        ds = torch.empty((M, K // 32, 2), dtype=torch.float16, device=x.device)
    _need(qa, torch.int8, (M, K), "qa")
    _need(ds, torch.float16, (M, K // 32, 2), "ds")
    _check(lib().q8_1_quantize(_ptr(x), M, K, _ptr(qa), _ptr(ds), _stream(stream, x)), "q8_1_quantize")
    return qa, ds


def q4_gemv_workspace_bytes(M, N, K):
    return lib().q4_gemv_workspace_bytes(int(M), int(N), int(K))


def q4_mmq_workspace_bytes(M, N, K):
    return lib().q4_mmq_workspace_bytes(int(M), int(N), int(K))


def _workspace(nbytes, ws, device):
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.empty((nbytes,), dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace too small: need %d bytes" % nbytes)
    return ws, ws.numel() * ws.element_size()


def q4_gemv(x, qs, sm, y=None, workspace=None, stream=None):
    """y fp32 [M][N] = x fp32 [M][K] . dequant(qs, sm)^T, 1 <= M <= 16."""
    M, K = x.shape
    N = qs.shape[0]
    _need(x, torch.float32, (M, K), "x")
    _need(qs, torch.uint8, (N, K // 2), "qs")
    _need(sm, torch.float16, (N, K // 256, 2), "sm")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need(y, torch.float32, (M, N), "y")
    ws, wsb = _workspace(q4_gemv_workspace_bytes(M, N, K), workspace, x.device)
    _check(lib().q4_gemv(_ptr(x), M, _ptr(qs), _ptr(sm), N, K, _ptr(y), _ptr(ws), wsb,
                         _stream(stream, x)), "q4_gemv")
    return y


def q4_gemv_noalloc(x, qs, sm, y, stream=None):
    """q4_gemv with the K-split partials in the library's fixed device array
    (no workspace); y fp32 [M][N] must be given."""
    M, K = x.shape
    N = qs.shape[0]
    _need(x, torch.float32, (M, K), "x")
    _need(qs, torch.uint8, (N, K // 2), "qs")
    _need(sm, torch.float16, (N, K // 256, 2), "sm")
    _need(y, torch.float32, (M, N), "y")
    _check(lib().q4_gemv_noalloc(_ptr(x), M, _ptr(qs), _ptr(sm), N, K, _ptr(y), _stream(stream, x)),
           "q4_gemv_noalloc")
    return y


def q4_pack_g32(W, qs=None, sm=None, stream=None):
    """W fp32 [N][K] -> (qs uint8 [N][K/2], sm float16 [N][K/32][2]): group-32 pairs."""
    N, K = W.shape
    _need(W, torch.float32, (N, K), "W")
    if qs is None:
        qs = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    if sm is None:
        sm = torch.empty((N, K // 32, 2), dtype=torch.float16, device=W.device)
    _need(qs, torch.uint8, (N, K // 2), "qs")
    _need(sm, torch.float16, (N, K // 32, 2), "sm")
    _check(lib().q4_pack_g32(_ptr(W), N, K, _ptr(qs), _ptr(sm), _stream(stream, W)), "q4_pack_g32")
    return qs, sm


def q4_gemv_g32_workspace_bytes(M, N, K):
    return lib().q4_gemv_g32_workspace_bytes(int(M), int(N), int(K))


def q4_gemv_g32(x, qs, sm, y=None, workspace=None, stream=None):
    """q4_gemv on group-32 weights (sm float16 [N][K/32][2])."""
    M, K = x.shape
    N = qs.shape[0]
    _need(x, torch.float32, (M, K), "x")
    _need(qs, torch.uint8, (N, K // 2), "qs")
    _need(sm, torch.float16, (N, K // 32, 2), "sm")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need(y, torch.float32, (M, N), "y")
    ws, wsb = _workspace(q4_gemv_g32_workspace_bytes(M, N, K), workspace, x.device)
    _check(lib().q4_gemv_g32(_ptr(x), M, _ptr(qs), _ptr(sm), N, K, _ptr(y), _ptr(ws), wsb,
                             _stream(stream, x)), "q4_gemv_g32")
    return y


def q4_mmq_gemm(qa, ds, qs, sm, y=None, workspace=None, stream=None):
    """y fp32 [M][N] from Q8_1 activations (qa, ds) and packed weights (qs, sm)."""
    M, K = qa.shape
    N = qs.shape[0]
    _need(qa, torch.int8, (M, K), "qa")
    _need(ds, torch.float16, (M, K // 32, 2), "ds")
    _need(qs, torch.uint8, (N, K // 2), "qs")
    _need(sm, torch.float16, (N, K // 256, 2), "sm")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=qa.device)
    _need(y, torch.float32, (M, N), "y")
    ws, wsb = _workspace(q4_mmq_workspace_bytes(M, N, K), workspace, qa.device)
    _check(lib().q4_mmq_gemm(_ptr(qa), _ptr(ds), M, _ptr(qs), _ptr(sm), N, K, _ptr(y), _ptr(ws),
                             wsb, _stream(stream, qa)), "q4_mmq_gemm")
    return y


def q4_mmq_int8_workspace_bytes(M, N, K):
    return lib().q4_mmq_int8_workspace_bytes(int(M), int(N), int(K))


def q4_mmq_gemm_int8(qa, ds, qs, sm, y=None, workspace=None, stream=None):
    """q4_mmq_gemm on the int8 matrix-core design at any shape."""
    M, K = qa.shape
    N = qs.shape[0]
    _need(qa, torch.int8, (M, K), "qa")
    _need(ds, torch.float16, (M, K // 32, 2), "ds")
    _need(qs, torch.uint8, (N, K // 2), "qs")
    _need(sm, torch.float16, (N, K // 256, 2), "sm")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=qa.device)
    _need(y, torch.float32, (M, N), "y")
    ws, wsb = _workspace(q4_mmq_int8_workspace_bytes(M, N, K), workspace, qa.device)
    _check(lib().q4_mmq_gemm_int8(_ptr(qa), _ptr(ds), M, _ptr(qs), _ptr(sm), N, K, _ptr(y), _ptr(ws),
                                  wsb, _stream(stream, qa)), "q4_mmq_gemm_int8")
    return y


def q4_mmq_gemm_q8_1(qa, ds, qs, sm, qa_out=None, ds_out=None, workspace=None, stream=None):
    """(qa_out int8 [M][N], ds_out float16 [M][N/32][2]) = Q8_1 of the MMQ result."""
    M, K = qa.shape
    N = qs.shape[0]
    _need(qa, torch.int8, (M, K), "qa")
    _need(ds, torch.float16, (M, K // 32, 2), "ds")
    _need(qs, torch.uint8, (N, K // 2), "qs")
    _need(sm, torch.float16, (N, K // 256, 2), "sm")
    if qa_out is None:
        qa_out = torch.empty((M, N), dtype=torch.int8, device=qa.device)
    if ds_out is None:
        ds_out = torch.empty((M, N // 32, 2), dtype=torch.float16, device=qa.device)
    _need(qa_out, torch.int8, (M, N), "qa_out")
    _need(ds_out, torch.float16, (M, N // 32, 2), "ds_out")
    ws, wsb = _workspace(q4_mmq_workspace_bytes(M, N, K), workspace, qa.device)
    _check(lib().q4_mmq_gemm_q8_1(_ptr(qa), _ptr(ds), M, _ptr(qs), _ptr(sm), N, K, _ptr(qa_out),
                                  _ptr(ds_out), _ptr(ws), wsb, _stream(stream, qa)), "q4_mmq_gemm_q8_1")
    return qa_out, ds_out


def q4_mmq_gemm_g32(qa, ds, qs, sm, y=None, workspace=None, stream=None):
    """q4_mmq_gemm on group-32 weights (sm float16 [N][K/32][2])."""
    M, K = qa.shape
    N = qs.shape[0]
    _need(qa, torch.int8, (M, K), "qa")
    _need(ds, torch.float16, (M, K // 32, 2), "ds")
    _need(qs, torch.uint8, (N, K // 2), "qs")
    _need(sm, torch.float16, (N, K // 32, 2), "sm")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=qa.device)
    _need(y, torch.float32, (M, N), "y")
    ws, wsb = _workspace(q4_mmq_workspace_bytes(M, N, K), workspace, qa.device)
    _check(lib().q4_mmq_gemm_g32(_ptr(qa), _ptr(ds), M, _ptr(qs), _ptr(sm), N, K, _ptr(y), _ptr(ws),
                                 wsb, _stream(stream, qa)), "q4_mmq_gemm_g32")
    return y


def q4_mmq_block_dots(qa, qs, idot=None, stream=None):
    """idot int32 [M][N][K/32] = per-block integer dots of qa and the 4-bit codes."""
    M, K = qa.shape
    N = qs.shape[0]
    _need(qa, torch.int8, (M, K), "qa")
    _need(qs, torch.uint8, (N, K // 2), "qs")
    if idot is None:
        idot = torch.empty((M, N, K // 32), dtype=torch.int32, device=qa.device)
    _need(idot, torch.int32, (M, N, K // 32), "idot")
    _check(lib().q4_mmq_block_dots(_ptr(qa), M, _ptr(qs), N, K, _ptr(idot), _stream(stream, qa)),
           "q4_mmq_block_dots")
    return idot
