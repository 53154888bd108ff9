"""Thin ctypes binding over the C ABI of ``include/mmq.h``.

Argument marshalling only: torch tensors give device pointers and the current
HIP stream; every step of the computation runs in the HIP kernels of
``libq4q8mmq.so``.  There is no fallback: if the library is missing or the
device is not gfx950, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4q8mmq.so")
EXPORTS = ("q8_quantize_rows", "q8_quantize_silu_mul", "mmq_q4k_q8", "mmq_q4k_q8_fp32out", "mmq_q4k_q8_f16out",
           "mmq_q6k_q8", "mmq_q6k_q8_fp32out", "mmq_q6k_q8_f16out", "q4k_repack",
           "mmq_q4kr_q8_fp32out", "q8_quantize_rows_tiled", "mmq_q4k_q8t_fp32out",
           "mmq_q4kr_q8t_fp32out", "mmq_q6k_q8t_fp32out", "q8_quantize_silu_mul_tiled",
           "mmq_status_string")
_MMQ_CALLS = ("mmq_q4k_q8", "mmq_q4k_q8_fp32out", "mmq_q4k_q8_f16out",
              "mmq_q6k_q8", "mmq_q6k_q8_fp32out", "mmq_q6k_q8_f16out", "mmq_q4kr_q8_fp32out",
              "mmq_q4k_q8t_fp32out", "mmq_q4kr_q8t_fp32out", "mmq_q6k_q8t_fp32out")
_lib = None


class MMQError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__("%s failed: %s (status %d)" % (fn, text, status))
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("HIP library %s is missing: build it with "
                           "`python -m q4_q8_integer_amd.build` (or __graft_entry__.build())" % path)
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.q8_quantize_rows.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.q8_quantize_rows.restype = ctypes.c_int
    lib.q8_quantize_rows_tiled.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.q8_quantize_rows_tiled.restype = ctypes.c_int
    lib.q8_quantize_silu_mul_tiled.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    lib.q8_quantize_silu_mul_tiled.restype = ctypes.c_int
    lib.q8_quantize_silu_mul.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    lib.q8_quantize_silu_mul.restype = ctypes.c_int
    lib.q4k_repack.argtypes = [vp, i64, i64, vp, vp]
    lib.q4k_repack.restype = ctypes.c_int
    for name in _MMQ_CALLS:
        fn = getattr(lib, name)
        fn.argtypes = [vp, i64, i64, vp, vp, i64, vp, vp]
        fn.restype = ctypes.c_int
    lib.mmq_status_string.argtypes = [ctypes.c_int]
    lib.mmq_status_string.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mmq_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise MMQError(fn, status, status_string(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise TypeError("%s must be a contiguous %s tensor on a HIP device" % (name, dtype))


# -------------------------------------------------------------- raw entries
def q8_quantize_rows(x, n, k, q, ds):
    """Enqueue the quantizer on preallocated outputs (C ABI call, same name)."""
    _check("q8_quantize_rows", load_library().q8_quantize_rows(
        _ptr(x), n, k, _ptr(q), _ptr(ds), _stream()))


def q8_quantize_rows_tiled(x, n, k, qt, ds):
    """Enqueue the quantizer with the codes as binary16 operand tiles."""
    _check("q8_quantize_rows_tiled", load_library().q8_quantize_rows_tiled(
        _ptr(x), n, k, _ptr(qt), _ptr(ds), _stream()))


def q8_quantize_silu_mul_tiled(gate, up, n, k, qt, ds):
    """Enqueue the fused SiLU-gate quantizer with the codes as operand tiles."""
    _check("q8_quantize_silu_mul_tiled", load_library().q8_quantize_silu_mul_tiled(
        _ptr(gate), _ptr(up), n, k, _ptr(qt), _ptr(ds), _stream()))


def q8_quantize_silu_mul(gate, up, n, k, q, ds):
    """Enqueue the fused SiLU-gate quantizer on preallocated outputs."""
    _check("q8_quantize_silu_mul", load_library().q8_quantize_silu_mul(
        _ptr(gate), _ptr(up), n, k, _ptr(q), _ptr(ds), _stream()))


def mmq_q4k_q8(w, m, k, q, ds, n, dots):
    _check("mmq_q4k_q8", load_library().mmq_q4k_q8(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(dots), _stream()))


def mmq_q4k_q8_fp32out(w, m, k, q, ds, n, out):
    _check("mmq_q4k_q8_fp32out", load_library().mmq_q4k_q8_fp32out(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q4k_q8_f16out(w, m, k, q, ds, n, out):
    _check("mmq_q4k_q8_f16out", load_library().mmq_q4k_q8_f16out(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out), _stream()))


def q4k_repack(w, m, k, wr):
    _check("q4k_repack", load_library().q4k_repack(_ptr(w), m, k, _ptr(wr), _stream()))


def mmq_q4kr_q8_fp32out(wr, m, k, q, ds, n, out):
    _check("mmq_q4kr_q8_fp32out", load_library().mmq_q4kr_q8_fp32out(
        _ptr(wr), m, k, _ptr(q), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q4k_q8t_fp32out(w, m, k, qt, ds, n, out):
    _check("mmq_q4k_q8t_fp32out", load_library().mmq_q4k_q8t_fp32out(
        _ptr(w), m, k, _ptr(qt), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q4kr_q8t_fp32out(wr, m, k, qt, ds, n, out):
    _check("mmq_q4kr_q8t_fp32out", load_library().mmq_q4kr_q8t_fp32out(
        _ptr(wr), m, k, _ptr(qt), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q6k_q8t_fp32out(w, m, k, qt, ds, n, out):
    _check("mmq_q6k_q8t_fp32out", load_library().mmq_q6k_q8t_fp32out(
        _ptr(w), m, k, _ptr(qt), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q6k_q8(w, m, k, q, ds, n, dots):
    _check("mmq_q6k_q8", load_library().mmq_q6k_q8(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(dots), _stream()))


def mmq_q6k_q8_fp32out(w, m, k, q, ds, n, out):
    _check("mmq_q6k_q8_fp32out", load_library().mmq_q6k_q8_fp32out(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q6k_q8_f16out(w, m, k, q, ds, n, out):
    _check("mmq_q6k_q8_f16out", load_library().mmq_q6k_q8_f16out(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out), _stream()))


# --------------------------------------------------------- tensor helpers
def quantize(x: torch.Tensor):
    """x float32 [n, k] -> (q int8 [n, k], ds int32 [n, k/32] holding the uint32 words)."""
    _need(x, torch.float32, "x")
    n, k = x.shape
    q = torch.empty((n, k), dtype=torch.int8, device=x.device)
    ds = torch.empty((n, k // 32 if k % 32 == 0 else 0), dtype=torch.int32, device=x.device)
    q8_quantize_rows(x, n, k, q, ds)
    return q, ds


def tiles_elems(n: int, k: int) -> int:
    """binary16 values in q8_quantize_rows_tiled's output for n tokens of k."""
    return (n + 127) // 128 * 128 * k


def quantize_tiled(x: torch.Tensor):
    """x float32 [n, k] -> (qt int16 [tiles_elems(n, k)] holding the binary16
    operand tiles, ds int32 [n, k/32])."""
    _need(x, torch.float32, "x")
    n, k = x.shape
    qt = torch.empty(tiles_elems(n, k), dtype=torch.int16, device=x.device)
    ds = torch.empty((n, k // 32 if k % 32 == 0 else 0), dtype=torch.int32, device=x.device)
    q8_quantize_rows_tiled(x, n, k, qt, ds)
    return qt, ds


def quantize_silu_mul_tiled(gate: torch.Tensor, up: torch.Tensor):
    """Operand tiles of q8(SiLU(gate) * up): (qt int16 [tiles_elems(n, k)], ds int32 [n, k/32])."""
    _need(gate, torch.float32, "gate")
    _need(up, torch.float32, "up")
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    n, k = gate.shape
    qt = torch.empty(tiles_elems(n, k), dtype=torch.int16, device=gate.device)
    ds = torch.empty((n, k // 32 if k % 32 == 0 else 0), dtype=torch.int32, device=gate.device)
    q8_quantize_silu_mul_tiled(gate, up, n, k, qt, ds)
    return qt, ds


def quantize_silu_mul(gate: torch.Tensor, up: torch.Tensor):
    """q8 of SiLU(gate) * up: (q int8 [n, k], ds int32 [n, k/32])."""
    _need(gate, torch.float32, "gate")
    _need(up, torch.float32, "up")
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    n, k = gate.shape
    q = torch.empty((n, k), dtype=torch.int8, device=gate.device)
    ds = torch.empty((n, k // 32 if k % 32 == 0 else 0), dtype=torch.int32, device=gate.device)
    q8_quantize_silu_mul(gate, up, n, k, q, ds)
    return q, ds


def blockdots(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds=None):
    """Exact int32 block dots [n, m, k/32]."""
    _need(w, torch.uint8, "w")
    _need(q, torch.int8, "q")
    n = q.shape[0]
    dots = torch.empty((n, m, k // 32), dtype=torch.int32, device=q.device)
    mmq_q4k_q8(w, m, k, q, ds, n, dots)
    return dots


def fp32(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, out=None):
    """Two-term-fold output float32 [n, m]."""
    _need(w, torch.uint8, "w")
    _need(q, torch.int8, "q")
    _need(ds, torch.int32, "ds")
    n = q.shape[0]
    if out is None:
        out = torch.empty((n, m), dtype=torch.float32, device=q.device)
    else:
        _need(out, torch.float32, "out")
    mmq_q4k_q8_fp32out(w, m, k, q, ds, n, out)
    return out


def fp16(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, out=None):
    """Two-term-fold output as binary16 [n, m] (the float32 result, rounded to nearest-even)."""
    _need(w, torch.uint8, "w")
    _need(q, torch.int8, "q")
    _need(ds, torch.int32, "ds")
    n = q.shape[0]
    if out is None:
        out = torch.empty((n, m), dtype=torch.float16, device=q.device)
    else:
        _need(out, torch.float16, "out")
    mmq_q4k_q8_f16out(w, m, k, q, ds, n, out)
    return out


def q6k_dots(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds=None):
    """Exact int32 q6_K group dots [n, m, k/16]."""
    _need(w, torch.uint8, "w")
    _need(q, torch.int8, "q")
    n = q.shape[0]
    dots = torch.empty((n, m, k // 16), dtype=torch.int32, device=q.device)
    mmq_q6k_q8(w, m, k, q, ds, n, dots)
    return dots


def q6k_fp32(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, out=None):
    """q6_K output float32 [n, m]."""
    _need(w, torch.uint8, "w")
    _need(q, torch.int8, "q")
    _need(ds, torch.int32, "ds")
    n = q.shape[0]
    if out is None:
        out = torch.empty((n, m), dtype=torch.float32, device=q.device)
    else:
        _need(out, torch.float32, "out")
    mmq_q6k_q8_fp32out(w, m, k, q, ds, n, out)
    return out


def q6k_fp16(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, out=None):
    """q6_K output as binary16 [n, m] (the float32 result, rounded to nearest-even)."""
    _need(w, torch.uint8, "w")
    _need(q, torch.int8, "q")
    _need(ds, torch.int32, "ds")
    n = q.shape[0]
    if out is None:
        out = torch.empty((n, m), dtype=torch.float16, device=q.device)
    else:
        _need(out, torch.float16, "out")
    mmq_q6k_q8_f16out(w, m, k, q, ds, n, out)
    return out


def fp32_tiles(w: torch.Tensor, m: int, k: int, qt: torch.Tensor, ds: torch.Tensor, out=None,
               repacked: bool = False):
    """The fold on q8 operand tiles (from quantize_tiled): float32 [n, m]; w is
    q4_K rows, or q4k_repack records with repacked=True."""
    _need(w, torch.uint8, "w")
    _need(qt, torch.int16, "qt")
    _need(ds, torch.int32, "ds")
    n = ds.shape[0]
    if out is None:
        out = torch.empty((n, m), dtype=torch.float32, device=ds.device)
    else:
        _need(out, torch.float32, "out")
    (mmq_q4kr_q8t_fp32out if repacked else mmq_q4k_q8t_fp32out)(w, m, k, qt, ds, n, out)
    return out


def q6k_fp32_tiles(w: torch.Tensor, m: int, k: int, qt: torch.Tensor, ds: torch.Tensor, out=None):
    """The q6_K fold on q8 operand tiles (from quantize_tiled): float32 [n, m]."""
    _need(w, torch.uint8, "w")
    _need(qt, torch.int16, "qt")
    _need(ds, torch.int32, "ds")
    n = ds.shape[0]
    if out is None:
        out = torch.empty((n, m), dtype=torch.float32, device=ds.device)
    else:
        _need(out, torch.float32, "out")
    mmq_q6k_q8t_fp32out(w, m, k, qt, ds, n, out)
    return out


def repack_bytes(m: int, k: int) -> int:
    """Size of q4k_repack's output for an m x k matrix."""
    return (m + 15) // 16 * (k // 256) * 2368


def repack(w: torch.Tensor, m: int, k: int):
    """Load-time repack of q4_K weights: uint8 tensor of repack_bytes(m, k)."""
    _need(w, torch.uint8, "w")
    wr = torch.empty(repack_bytes(m, k), dtype=torch.uint8, device=w.device)
    q4k_repack(w, m, k, wr)
    return wr


def fp32_repacked(wr: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, out=None):
    """mmq_q4k_q8_fp32out on repacked weights: float32 [n, m]."""
    _need(wr, torch.uint8, "wr")
    _need(q, torch.int8, "q")
    _need(ds, torch.int32, "ds")
    n = q.shape[0]
    if out is None:
        out = torch.empty((n, m), dtype=torch.float32, device=q.device)
    else:
        _need(out, torch.float32, "out")
    mmq_q4kr_q8_fp32out(wr, m, k, q, ds, n, out)
    return out
