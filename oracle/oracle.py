"""ctypes wrapper around the plain-C oracle (``oracle.c``).

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the product path never does.  The wrapper only moves
arrays across the call; every step of the arithmetic is in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc -O2 (no fast-math) and OpenMP."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC",
                    "-Wall", "-Wextra", src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _declare(lib):
    c_i64, c_p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_q8_quantize.argtypes = [c_p, c_i64, c_i64, c_p, c_p]
    lib.oracle_q4k_unpack.argtypes = [c_p, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p]
    lib.oracle_blockdots.argtypes = [c_p, c_i64, c_i64, c_p, c_i64, c_p]
    lib.oracle_out_f64.argtypes = [c_p, c_i64, c_i64, c_p, c_p, c_i64, c_p]
    lib.oracle_q4k_repack.argtypes = [c_p, c_i64, c_i64, c_p]
    lib.oracle_q4k_repack.restype = ctypes.c_int
    lib.oracle_q8_tiles.argtypes = [c_p, c_i64, c_i64, c_p]
    lib.oracle_q8_tiles.restype = ctypes.c_int
    lib.oracle_silu_mul.argtypes = [c_p, c_p, c_i64, c_p]
    lib.oracle_silu_mul.restype = None
    lib.oracle_q8_quantize_silu_mul.argtypes = [c_p, c_p, c_i64, c_i64, c_p, c_p]
    lib.oracle_q6k_unpack.argtypes = [c_p, c_i64, c_i64, c_p, c_p, c_p]
    lib.oracle_q6k_dots.argtypes = [c_p, c_i64, c_i64, c_p, c_i64, c_p]
    lib.oracle_q6k_out_f64.argtypes = [c_p, c_i64, c_i64, c_p, c_p, c_i64, c_p]
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = ctypes.c_double
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_get_threads.restype = ctypes.c_int
    for fn in (lib.oracle_q8_quantize, lib.oracle_q4k_unpack, lib.oracle_blockdots,
               lib.oracle_out_f64, lib.oracle_q6k_unpack, lib.oracle_q6k_dots,
               lib.oracle_q6k_out_f64, lib.oracle_q8_quantize_silu_mul):
        fn.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load the oracle library (building it first if it is missing).

    With ``path`` given, load that build (e.g. a test's planted-mistake copy)
    and return a fresh handle instead of the shared one.
    """
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (rc=%d)" % (what, rc))


def set_threads(n: int, lib=None):
    (lib or load()).oracle_set_threads(int(n))


def get_threads(lib=None) -> int:
    return int((lib or load()).oracle_get_threads())


def quantize(x: np.ndarray, lib=None):
    """x float32 [n, k] -> (q int8 [n, k], ds uint32 [n, k/32])."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    n, k = x.shape
    q = np.empty((n, k), dtype=np.int8)
    ds = np.empty((n, k // 32), dtype=np.uint32)
    _check(lib.oracle_q8_quantize(_ptr(x), n, k, _ptr(q), _ptr(ds)), "quantize")
    return q, ds


def silu_mul(g: np.ndarray, u: np.ndarray, lib=None) -> np.ndarray:
    """h = float32(g*u / (1 + exp(-g))) evaluated in float64, elementwise."""
    lib = lib or load()
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    h = np.empty_like(g)
    lib.oracle_silu_mul(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def quantize_silu_mul(g: np.ndarray, u: np.ndarray, lib=None):
    """Fused SiLU-gate quantize: (q int8 [n, k], ds uint32 [n, k/32]) of h = SiLU(g)*u."""
    lib = lib or load()
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    n, k = g.shape
    q = np.empty((n, k), dtype=np.int8)
    ds = np.empty((n, k // 32), dtype=np.uint32)
    _check(lib.oracle_q8_quantize_silu_mul(_ptr(g), _ptr(u), n, k, _ptr(q), _ptr(ds)),
           "quantize_silu_mul")
    return q, ds


def q4k_unpack(w: np.ndarray, m: int, k: int, lib=None):
    """q4_K bytes [m, (k/256)*144] -> dict of fields (q, sc, mn, d, dmin as f16)."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.uint8)
    q = np.empty((m, k), dtype=np.uint8)
    sc = np.empty((m, k // 32), dtype=np.uint8)
    mn = np.empty((m, k // 32), dtype=np.uint8)
    d = np.empty((m, k // 256), dtype=np.uint16)
    dmin = np.empty((m, k // 256), dtype=np.uint16)
    _check(lib.oracle_q4k_unpack(_ptr(w), m, k, _ptr(q), _ptr(sc), _ptr(mn),
                                 _ptr(d), _ptr(dmin)), "q4k_unpack")
    return dict(q=q, sc=sc, mn=mn, d=d.view(np.float16), dmin=dmin.view(np.float16))


def blockdots(w: np.ndarray, m: int, k: int, q: np.ndarray, lib=None) -> np.ndarray:
    """Exact per-block dots: int32 [n, m, k/32]."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    n = q.shape[0]
    dots = np.empty((n, m, k // 32), dtype=np.int32)
    _check(lib.oracle_blockdots(_ptr(w), m, k, _ptr(q), n, _ptr(dots)), "blockdots")
    return dots


def out_f64(w: np.ndarray, m: int, k: int, q: np.ndarray, ds: np.ndarray,
            lib=None) -> np.ndarray:
    """Two-term-fold output in float64: [n, m]."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    ds = np.ascontiguousarray(ds, dtype=np.uint32)
    n = q.shape[0]
    out = np.empty((n, m), dtype=np.float64)
    _check(lib.oracle_out_f64(_ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out)), "out_f64")
    return out


def q4k_repack(w: np.ndarray, m: int, k: int, lib=None) -> np.ndarray:
    """The few-token record layout of a q4_K matrix: uint8 [ceil(m/16)*(k/256)*2368]."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.uint8)
    wr = np.empty(((m + 15) // 16) * (k // 256) * 2368, dtype=np.uint8)
    _check(lib.oracle_q4k_repack(_ptr(w), m, k, _ptr(wr)), "q4k_repack")
    return wr


def q8_tiles(q: np.ndarray, lib=None) -> np.ndarray:
    """q8 codes int8 [n, k] -> the binary16 operand-tile layout, as uint16 bits
    [ceil(n/128) * 128 * k]."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    n, k = q.shape
    qt = np.empty(((n + 127) // 128) * 128 * k, dtype=np.uint16)
    _check(lib.oracle_q8_tiles(_ptr(q), n, k, _ptr(qt)), "q8_tiles")
    return qt


def q6k_unpack(w: np.ndarray, m: int, k: int, lib=None):
    """q6_K bytes [m, (k/256)*210] -> dict of fields (q codes, sc int8, d as f16)."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.uint8)
    q = np.empty((m, k), dtype=np.uint8)
    sc = np.empty((m, k // 16), dtype=np.int8)
    d = np.empty((m, k // 256), dtype=np.uint16)
    _check(lib.oracle_q6k_unpack(_ptr(w), m, k, _ptr(q), _ptr(sc), _ptr(d)), "q6k_unpack")
    return dict(q=q, sc=sc, d=d.view(np.float16))


def q6k_dots(w: np.ndarray, m: int, k: int, q: np.ndarray, lib=None) -> np.ndarray:
    """Exact q6_K group dots: int32 [n, m, k/16]."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    n = q.shape[0]
    dots = np.empty((n, m, k // 16), dtype=np.int32)
    _check(lib.oracle_q6k_dots(_ptr(w), m, k, _ptr(q), n, _ptr(dots)), "q6k_dots")
    return dots


def q6k_out_f64(w: np.ndarray, m: int, k: int, q: np.ndarray, ds: np.ndarray,
                lib=None) -> np.ndarray:
    """q6_K output in float64: [n, m]."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    ds = np.ascontiguousarray(ds, dtype=np.uint32)
    n = q.shape[0]
    out = np.empty((n, m), dtype=np.float64)
    _check(lib.oracle_q6k_out_f64(_ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out)), "q6k_out_f64")
    return out


def f16_to_f64(bits: int, lib=None) -> float:
    return float((lib or load()).oracle_f16_to_double(int(bits) & 0xFFFF))


def f16_bits(x: float, lib=None) -> int:
    return int((lib or load()).oracle_f32_to_f16(float(np.float32(x))))
