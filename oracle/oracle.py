"""Python access to the CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the library's product path never
does.  It loads ``liboracle.so`` built from ``oracle.c`` by ``build()`` below
(gcc, no GPU code) and marshals numpy arrays into the plain C calls.

Every function returns fresh numpy arrays:
    q4_pack(W, group=256)     -> (qs u8 [N][K/2], sm u16 [N][K/group][2]); group 256 or 32
    q4_dequant(qs, sm, K)     -> fp64 [N][K]
    q4_codes(qs, K)           -> u8 [N][K] codes 0..15
    q8_1_quantize(x)          -> (qa i8 [M][K], ds u16 [M][K/32][2])
    q8_1_dequant(qa, ds)      -> fp64 [M][K]
    q4_gemv(x, qs, sm, K)     -> fp64 [M][N]   (the weight functions take group= too)
    q4_block_dots(qa, qs, K)  -> i32 [M][N][K/32]
    q4_mmq(qa, ds, qs, sm, K) -> fp64 [M][N]
    f32_to_f16(a) / f16_to_f32(h) elementwise IEEE binary16 conversion
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

GROUP = 256
BLOCK = 32


def build(force=False):
    """Compile oracle.c into liboracle.so with gcc (IEEE fp32, no contraction)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    sig = {
        "orc_version": ([], ctypes.c_int),
        "orc_set_mutation": ([ctypes.c_int], None),
        "orc_get_mutation": ([], ctypes.c_int),
        "orc_set_threads": ([ctypes.c_int], None),
        "orc_get_threads": ([], ctypes.c_int),
        "orc_f32_to_f16": ([ctypes.c_float], ctypes.c_uint16),
        "orc_f16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
        "orc_q4_pack": ([P, I64, I64, P, P], ctypes.c_int),
        "orc_q4_pack_g": ([P, I64, I64, I64, P, P], ctypes.c_int),
        "orc_q4_dequant_g": ([P, P, I64, I64, I64, P], ctypes.c_int),
        "orc_q4_gemv_g": ([P, I64, P, P, I64, I64, I64, P], ctypes.c_int),
        "orc_q4_mmq_g": ([P, P, I64, P, P, I64, I64, I64, P], ctypes.c_int),
        "orc_q4_dequant": ([P, P, I64, I64, P], ctypes.c_int),
        "orc_q4_codes": ([P, I64, I64, P], ctypes.c_int),
        "orc_q8_1_quantize": ([P, I64, I64, P, P], ctypes.c_int),
        "orc_q8_1_dequant": ([P, P, I64, I64, P], ctypes.c_int),
        "orc_q4_gemv": ([P, I64, P, P, I64, I64, P], ctypes.c_int),
        "orc_q4_block_dots": ([P, I64, P, I64, I64, P], ctypes.c_int),
        "orc_q4_mmq": ([P, P, I64, P, P, I64, I64, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    # thread count: every core this process may run on
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    lib.orc_set_threads(max(1, ncpu))
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s failed (rc=%d)" % (what, rc))


def set_mutation(m):
    """Test-only: plant mistake number m (0 = none) in the oracle."""
    _load().orc_set_mutation(int(m))


def get_mutation():
    return _load().orc_get_mutation()


def set_threads(n):
    _load().orc_set_threads(int(n))


def get_threads():
    return _load().orc_get_threads()


def f32_to_f16(a):
    lib = _load()
    a = np.asarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat, fo = a.reshape(-1), out.reshape(-1)
    for i in range(flat.size):
        fo[i] = lib.orc_f32_to_f16(float(flat[i]))
    return out


def f16_to_f32(h):
    lib = _load()
    h = np.asarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    flat, fo = h.reshape(-1), out.reshape(-1)
    for i in range(flat.size):
        fo[i] = lib.orc_f16_to_f32(int(flat[i]))
    return out


def q4_pack(W, group=GROUP):
    """group = 256 (the main format) or 32 (one scale/minimum pair per 32 weights)."""
    W = _c(W, np.float32)
    N, K = W.shape
    qs = np.empty((N, K // 2), dtype=np.uint8)
    sm = np.empty((N, K // group, 2), dtype=np.uint16)
    _check(_load().orc_q4_pack_g(_ptr(W), N, K, group, _ptr(qs), _ptr(sm)), "q4_pack")
    return qs, sm


def q4_dequant(qs, sm, K, group=GROUP):
    qs = _c(qs, np.uint8)
    sm = _c(sm, np.uint16)
    N = qs.shape[0]
    out = np.empty((N, K), dtype=np.float64)
    _check(_load().orc_q4_dequant_g(_ptr(qs), _ptr(sm), N, K, group, _ptr(out)), "q4_dequant")
    return out


def q4_codes(qs, K):
    qs = _c(qs, np.uint8)
    N = qs.shape[0]
    out = np.empty((N, K), dtype=np.uint8)
    _check(_load().orc_q4_codes(_ptr(qs), N, K, _ptr(out)), "q4_codes")
    return out


def q8_1_quantize(x):
    x = _c(x, np.float32)
    M, K = x.shape
    qa = np.empty((M, K), dtype=np.int8)
    ds = np.empty((M, K // BLOCK, 2), dtype=np.uint16)
    _check(_load().orc_q8_1_quantize(_ptr(x), M, K, _ptr(qa), _ptr(ds)), "q8_1_quantize")
    return qa, ds


def q8_1_dequant(qa, ds):
    qa = _c(qa, np.int8)
    ds = _c(ds, np.uint16)
    M, K = qa.shape
    out = np.empty((M, K), dtype=np.float64)
    _check(_load().orc_q8_1_dequant(_ptr(qa), _ptr(ds), M, K, _ptr(out)), "q8_1_dequant")
    return out


def q4_gemv(x, qs, sm, K, group=GROUP):
    x = _c(x, np.float32)
    qs = _c(qs, np.uint8)
    sm = _c(sm, np.uint16)
    M, N = x.shape[0], qs.shape[0]
    assert x.shape[1] == K and qs.shape[1] == K // 2 and sm.shape[1] == K // group
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().orc_q4_gemv_g(_ptr(x), M, _ptr(qs), _ptr(sm), N, K, group, _ptr(y)), "q4_gemv")
    return y


def q4_block_dots(qa, qs, K):
    qa = _c(qa, np.int8)
    qs = _c(qs, np.uint8)
    M, N = qa.shape[0], qs.shape[0]
    out = np.empty((M, N, K // BLOCK), dtype=np.int32)
    _check(_load().orc_q4_block_dots(_ptr(qa), M, _ptr(qs), N, K, _ptr(out)), "q4_block_dots")
    return out


def q4_mmq(qa, ds, qs, sm, K, group=GROUP):
    qa = _c(qa, np.int8)
    ds = _c(ds, np.uint16)
    qs = _c(qs, np.uint8)
    sm = _c(sm, np.uint16)
    M, N = qa.shape[0], qs.shape[0]
    assert sm.shape[1] == K // group
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().orc_q4_mmq_g(_ptr(qa), _ptr(ds), M, _ptr(qs), _ptr(sm), N, K, group, _ptr(y)), "q4_mmq")
    return y
