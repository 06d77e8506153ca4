"""ctypes binding of the plain C++17 oracle (oracle/cpu_oracle.cpp).

TEST INFRASTRUCTURE (see the package docstring). `build()` compiles the
oracle with g++ -O2 -std=c++17 -ffp-contract=off (no fast-math) into
oracle/lib/libcpu_oracle.so; `lib()` loads what is built and builds it only
if nothing is. The functions take numpy arrays, marshal them, and return
numpy arrays with the same meaning as their numpy counterparts in
oracle.gemm and oracle.codecs. The HIP library is never loaded here.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpu_oracle.cpp")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libcpu_oracle.so")

FLAGS = ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle (every call)."""
    gxx = os.environ.get("CXX") or shutil.which("g++")
    if not gxx:
        raise RuntimeError("g++ not found")
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + ".tmp"
    r = subprocess.run([gxx, *FLAGS, SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int

_SIGS = {
    "orc_bf16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
    "orc_f32_to_bf16": ([ctypes.c_float], ctypes.c_uint16),
    "orc_e2m1": ([ctypes.c_uint], ctypes.c_double),
    "orc_e4m3fn": ([ctypes.c_uint], ctypes.c_double),
    "orc_bf16_to_f32_array": ([_P, _P, _I64], None),
    "orc_f32_to_bf16_array": ([_P, _P, _I64], None),
    "orc_dequant_fp4": ([_P, _P, _P, _I64, _I64], None),
    "orc_hardware_threads": ([], _INT),
    "orc_gemm_bf16_f64": ([_P, _P, _P, _I64, _I64, _I64, _INT], None),
    "orc_gemm_bf16_f64_rows": ([_P, _P, _P, _P, _I64, _I64, _I64, _INT], None),
    "orc_gemm_ordered": ([_P, _P, _P, _P, _I64, _I64, _I64, _INT], None),
    "orc_scaled_acc_epilogue": ([_P, _P, ctypes.c_float, _P, _I64], None),
    "orc_splitk_chunk": ([_I64, _I64], _I64),
    "orc_splitk_planes_f64": ([_P, _P, _P, _I64, _I64, _I64, _I64, _INT], None),
    "orc_splitk_reduce": ([_P, _I64, _I64, _P], None),
    "orc_gemm_fp4_f64": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _INT], None),
    "orc_gemm_w4a16_f64": ([_P, _P, _P, ctypes.c_float, _P, _I64, _I64, _I64, _INT], None),
}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        h = ctypes.CDLL(LIB)
        for name, (args, res) in _SIGS.items():
            f = getattr(h, name)
            f.argtypes = args
            f.restype = res
        _lib = h
    return _lib


def _c(x, dtype):
    return np.ascontiguousarray(np.asarray(x, dtype=dtype))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def hardware_threads() -> int:
    return int(lib().orc_hardware_threads())


# ---- codecs --------------------------------------------------------------------

def bf16_to_f32(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float32)
    lib().orc_bf16_to_f32_array(_p(b), _p(out), b.size)
    return out


def f32_to_bf16(x) -> np.ndarray:
    f = _c(x, np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_p(f), _p(out), f.size)
    return out


def e2m1_to_f64(codes) -> np.ndarray:
    c = _c(codes, np.uint32)
    f = lib().orc_e2m1
    return np.array([f(int(v)) for v in c.reshape(-1)], np.float64).reshape(c.shape)


def e4m3fn_to_f64(b) -> np.ndarray:
    v = _c(b, np.uint32)
    f = lib().orc_e4m3fn
    return np.array([f(int(x)) for x in v.reshape(-1)], np.float64).reshape(v.shape)


def dequant_fp4(packed, scales) -> np.ndarray:
    q = _c(packed, np.uint8)
    s = _c(scales, np.uint8)
    rows, k = q.shape[0], q.shape[1] * 2
    assert s.shape == (rows, k // 16), "one scale per 16 K elements"
    out = np.empty((rows, k), np.float64)
    lib().orc_dequant_fp4(_p(q), _p(s), _p(out), rows, k)
    return out


# ---- GEMM definitions ------------------------------------------------------------

def gemm_bf16_ref(a_bits, b_bits, threads: int = 0) -> np.ndarray:
    a, b = _c(a_bits, np.uint16), _c(b_bits, np.uint16)
    assert a.shape[1] == b.shape[1], "A and B share K"
    m, k = a.shape
    n = b.shape[0]
    c = np.empty((m, n), np.float64)
    lib().orc_gemm_bf16_f64(_p(a), _p(b), _p(c), m, n, k, threads)
    return c


def gemm_bf16_ref_rows(a_bits, b_bits, rows, threads: int = 0) -> np.ndarray:
    """gemm_bf16_ref restricted to the listed output rows."""
    a, b = _c(a_bits, np.uint16), _c(b_bits, np.uint16)
    r = _c(rows, np.int64)
    n, k = b.shape
    assert a.shape[1] == k and (r.size == 0 or (r.min() >= 0 and r.max() < a.shape[0]))
    c = np.empty((r.size, n), np.float64)
    lib().orc_gemm_bf16_f64_rows(_p(a), _p(b), _p(r), _p(c), r.size, n, k, threads)
    return c


def gemm_ordered_f32(a_bits, b_bits, threads: int = 0) -> np.ndarray:
    a, b = _c(a_bits, np.uint16), _c(b_bits, np.uint16)
    m, k = a.shape
    n = b.shape[0]
    c = np.empty((m, n), np.float32)
    lib().orc_gemm_ordered(_p(a), _p(b), _p(c), None, m, n, k, threads)
    return c


def gemm_ordered(a_bits, b_bits, threads: int = 0) -> np.ndarray:
    a, b = _c(a_bits, np.uint16), _c(b_bits, np.uint16)
    m, k = a.shape
    n = b.shape[0]
    c32 = np.empty((m, n), np.float32)
    c16 = np.empty((m, n), np.uint16)
    lib().orc_gemm_ordered(_p(a), _p(b), _p(c32), _p(c16), m, n, k, threads)
    return c16


def scaled_acc_epilogue(out_bits, delta_bf16_bits, scale) -> np.ndarray:
    o, d = _c(out_bits, np.uint16), _c(delta_bf16_bits, np.uint16)
    assert o.shape == d.shape
    res = np.empty(o.shape, np.uint16)
    lib().orc_scaled_acc_epilogue(_p(o), _p(d), float(np.float32(scale)), _p(res), o.size)
    return res


def splitk_chunk(k: int, k_splits: int) -> int:
    if k_splits <= 0:
        raise ValueError("k_splits >= 1")
    return int(lib().orc_splitk_chunk(k, k_splits))


def gemm_splitk_planes_ref(a_bits, b_bits, k_splits: int, threads: int = 0) -> np.ndarray:
    a, b = _c(a_bits, np.uint16), _c(b_bits, np.uint16)
    m, k = a.shape
    n = b.shape[0]
    planes = np.empty((k_splits, m, n), np.float64)
    lib().orc_splitk_planes_f64(_p(a), _p(b), _p(planes), m, n, k, k_splits, threads)
    return planes


def splitk_reduce(planes_f32) -> np.ndarray:
    p = _c(planes_f32, np.float32)
    ks = p.shape[0]
    count = p[0].size
    out = np.empty(p.shape[1:], np.uint16)
    lib().orc_splitk_reduce(_p(p), ks, count, _p(out))
    return out


def gemm_fp4_ref(a_packed, sfa, b_packed, sfb, k_range=None, threads: int = 0) -> np.ndarray:
    aq, sa = _c(a_packed, np.uint8), _c(sfa, np.uint8)
    bq, sb = _c(b_packed, np.uint8), _c(sfb, np.uint8)
    m, k = aq.shape[0], aq.shape[1] * 2
    n = bq.shape[0]
    assert bq.shape[1] * 2 == k and sa.shape == (m, k // 16) and sb.shape == (n, k // 16)
    k0, k1 = (0, k) if k_range is None else k_range
    c = np.empty((m, n), np.float64)
    lib().orc_gemm_fp4_f64(_p(aq), _p(sa), _p(bq), _p(sb), _p(c), m, n, k, k0, k1, threads)
    return c


def gemm_fp4_splitk_planes_ref(a_packed, sfa, b_packed, sfb, k_splits: int, threads: int = 0) -> np.ndarray:
    k = np.asarray(a_packed).shape[1] * 2
    kc = splitk_chunk(k, k_splits)
    return np.stack([gemm_fp4_ref(a_packed, sfa, b_packed, sfb, (min(k, s * kc), min(k, (s + 1) * kc)), threads)
                     for s in range(k_splits)])


def gemm_w4a16_ref(a_bits, b_packed, sfb, scale_2, threads: int = 0) -> np.ndarray:
    a = _c(a_bits, np.uint16)
    bq, sb = _c(b_packed, np.uint8), _c(sfb, np.uint8)
    m, k = a.shape
    n = bq.shape[0]
    assert bq.shape[1] * 2 == k and sb.shape == (n, k // 16)
    c = np.empty((m, n), np.float64)
    lib().orc_gemm_w4a16_f64(_p(a), _p(bq), _p(sb), float(np.float32(scale_2)), _p(c), m, n, k, threads)
    return c
