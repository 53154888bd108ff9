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
           "mmq_q4k_q8_fold", "mmq_q6k_q8", "mmq_q6k_q8_fp32out", "mmq_q6k_q8_f16out", "mmq_q6k_q8_fold",
           "q4k_repack", "mmq_q4kr_q8_fp32out", "q8_quantize_rows_tiled", "mmq_q4k_q8t_fp32out",
           "mmq_q4kr_q8t_fp32out", "mmq_q6k_q8t_fp32out", "q8_quantize_silu_mul_tiled",
           "mmq_kernel_choice", "mmq_status_string")

# enum mmq_kernel / enum mmq_format of include/mmq.h
KERNEL_AUTO, KERNEL_DOT4, KERNEL_FEW, KERNEL_F16, KERNEL_I8, KERNEL_NARROW, KERNEL_STREAM = 0, 1, 2, 3, 4, 5, 6
KERNEL_NAMES = {KERNEL_DOT4: "dot4", KERNEL_FEW: "few", KERNEL_F16: "f16", KERNEL_I8: "i8",
                KERNEL_NARROW: "narrow", KERNEL_STREAM: "stream"}
(FORMAT_Q4K, FORMAT_Q4K_REPACKED, FORMAT_Q6K, FORMAT_Q4K_TILES, FORMAT_Q4K_REPACKED_TILES,
 FORMAT_Q6K_TILES) = range(6)
Q4K_BLOCK_BYTES, Q6K_BLOCK_BYTES, REPACK_RECORD_BYTES = 144, 210, 2368
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
    for name in ("mmq_q4k_q8_fold", "mmq_q6k_q8_fold"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, i64, i64, vp, vp, i64, vp, ctypes.c_int, ctypes.c_int, vp]
        fn.restype = ctypes.c_int
    lib.mmq_kernel_choice.argtypes = [ctypes.c_int, i64, i64, i64]
    lib.mmq_kernel_choice.restype = ctypes.c_int
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


# Size checks.  The C ABI sees pointers only, so a wrong m, k or n would make
# the kernels read or write past a tensor; every wrapper below checks that
# each tensor holds what the sizes say (and that all sit on one device)
# before it calls the library, and raises ValueError otherwise.
def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _fits(t, nbytes: int, name: str):
    """A tensor argument (None passes through as NULL) holds >= nbytes bytes."""
    if t is not None and isinstance(t, torch.Tensor) and _nbytes(t) < nbytes:
        raise ValueError("%s holds %d bytes, the sizes given need %d" % (name, _nbytes(t), nbytes))


def _same_device(*ts):
    devs = {t.device for t in ts if isinstance(t, torch.Tensor)}
    if len(devs) > 1:
        raise ValueError("all tensors must be on one device, got %s" % sorted(str(d) for d in devs))


def _mmq_sizes(m: int, k: int, n: int):
    if m < 0 or n < 0 or k <= 0 or k % 256:
        raise ValueError("need m, n >= 0 and k a positive multiple of 256 (m=%d k=%d n=%d)" % (m, k, n))


def _check_fold_args(w, wbytes, m, k, q, qbytes, ds, n, out, outbytes):
    _mmq_sizes(m, k, n)
    _fits(w, wbytes, "w")
    _fits(q, qbytes, "q")
    _fits(ds, n * (k // 32) * 4, "ds")
    _fits(out, outbytes, "out")
    _same_device(w, q, ds, out)


def _w_bytes(m: int, k: int, fmt: str) -> int:
    if fmt == "q6k":
        return m * (k // 256) * Q6K_BLOCK_BYTES
    if fmt == "repacked":
        return (m + 15) // 16 * (k // 256) * REPACK_RECORD_BYTES
    return m * (k // 256) * Q4K_BLOCK_BYTES


# -------------------------------------------------------------- raw entries
# Same names and arguments as the C ABI (tensors for pointers); each checks
# that its tensors hold what the sizes say before the call.
def q8_quantize_rows(x, n, k, q, ds):
    """Enqueue the quantizer on preallocated outputs (C ABI call, same name)."""
    if n >= 0 and k > 0 and k % 32 == 0:
        _fits(x, n * k * 4, "x")
        _fits(q, n * k, "q")
        _fits(ds, n * (k // 32) * 4, "ds")
        _same_device(x, q, ds)
    _check("q8_quantize_rows", load_library().q8_quantize_rows(
        _ptr(x), n, k, _ptr(q), _ptr(ds), _stream()))


def q8_quantize_rows_tiled(x, n, k, qt, ds):
    """Enqueue the quantizer with the codes as binary16 operand tiles."""
    if n >= 0 and k > 0 and k % 256 == 0:
        _fits(x, n * k * 4, "x")
        _fits(qt, tiles_elems(n, k) * 2, "qt")
        _fits(ds, n * (k // 32) * 4, "ds")
        _same_device(x, qt, ds)
    _check("q8_quantize_rows_tiled", load_library().q8_quantize_rows_tiled(
        _ptr(x), n, k, _ptr(qt), _ptr(ds), _stream()))


def q8_quantize_silu_mul_tiled(gate, up, n, k, qt, ds):
    """Enqueue the fused SiLU-gate quantizer with the codes as operand tiles."""
    if n >= 0 and k > 0 and k % 256 == 0:
        _fits(gate, n * k * 4, "gate")
        _fits(up, n * k * 4, "up")
        _fits(qt, tiles_elems(n, k) * 2, "qt")
        _fits(ds, n * (k // 32) * 4, "ds")
        _same_device(gate, up, qt, ds)
    _check("q8_quantize_silu_mul_tiled", load_library().q8_quantize_silu_mul_tiled(
        _ptr(gate), _ptr(up), n, k, _ptr(qt), _ptr(ds), _stream()))


def q8_quantize_silu_mul(gate, up, n, k, q, ds):
    """Enqueue the fused SiLU-gate quantizer on preallocated outputs."""
    if n >= 0 and k > 0 and k % 32 == 0:
        _fits(gate, n * k * 4, "gate")
        _fits(up, n * k * 4, "up")
        _fits(q, n * k, "q")
        _fits(ds, n * (k // 32) * 4, "ds")
        _same_device(gate, up, q, ds)
    _check("q8_quantize_silu_mul", load_library().q8_quantize_silu_mul(
        _ptr(gate), _ptr(up), n, k, _ptr(q), _ptr(ds), _stream()))


def _sized(m, k, n):
    return m >= 0 and n >= 0 and k > 0 and k % 256 == 0


def mmq_q4k_q8(w, m, k, q, ds, n, dots):
    if _sized(m, k, n):
        _check_fold_args(w, _w_bytes(m, k, "q4k"), m, k, q, n * k, None, n, dots, n * m * (k // 32) * 4)
        _fits(ds, n * (k // 32) * 4, "ds")
    _check("mmq_q4k_q8", load_library().mmq_q4k_q8(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(dots), _stream()))


def mmq_q4k_q8_fp32out(w, m, k, q, ds, n, out):
    if _sized(m, k, n):
        _check_fold_args(w, _w_bytes(m, k, "q4k"), m, k, q, n * k, ds, n, out, n * m * 4)
    _check("mmq_q4k_q8_fp32out", load_library().mmq_q4k_q8_fp32out(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q4k_q8_f16out(w, m, k, q, ds, n, out):
    if _sized(m, k, n):
        _check_fold_args(w, _w_bytes(m, k, "q4k"), m, k, q, n * k, ds, n, out, n * m * 2)
    _check("mmq_q4k_q8_f16out", load_library().mmq_q4k_q8_f16out(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q4k_q8_fold(w, m, k, q, ds, n, out, out_f16, kernel):
    if _sized(m, k, n):
        _check_fold_args(w, _w_bytes(m, k, "q4k"), m, k, q, n * k, ds, n, out, n * m * (2 if out_f16 else 4))
    _check("mmq_q4k_q8_fold", load_library().mmq_q4k_q8_fold(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out), int(out_f16), int(kernel), _stream()))


def q4k_repack(w, m, k, wr):
    if m >= 0 and k > 0 and k % 256 == 0:
        _fits(w, _w_bytes(m, k, "q4k"), "w")
        _fits(wr, _w_bytes(m, k, "repacked"), "wr")
        _same_device(w, wr)
    _check("q4k_repack", load_library().q4k_repack(_ptr(w), m, k, _ptr(wr), _stream()))


def mmq_q4kr_q8_fp32out(wr, m, k, q, ds, n, out):
    if _sized(m, k, n):
        _check_fold_args(wr, _w_bytes(m, k, "repacked"), m, k, q, n * k, ds, n, out, n * m * 4)
    _check("mmq_q4kr_q8_fp32out", load_library().mmq_q4kr_q8_fp32out(
        _ptr(wr), m, k, _ptr(q), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q4k_q8t_fp32out(w, m, k, qt, ds, n, out):
    if _sized(m, k, n):
        _check_fold_args(w, _w_bytes(m, k, "q4k"), m, k, qt, tiles_elems(n, k) * 2, ds, n, out, n * m * 4)
    _check("mmq_q4k_q8t_fp32out", load_library().mmq_q4k_q8t_fp32out(
        _ptr(w), m, k, _ptr(qt), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q4kr_q8t_fp32out(wr, m, k, qt, ds, n, out):
    if _sized(m, k, n):
        _check_fold_args(wr, _w_bytes(m, k, "repacked"), m, k, qt, tiles_elems(n, k) * 2, ds, n, out, n * m * 4)
    _check("mmq_q4kr_q8t_fp32out", load_library().mmq_q4kr_q8t_fp32out(
        _ptr(wr), m, k, _ptr(qt), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q6k_q8t_fp32out(w, m, k, qt, ds, n, out):
    if _sized(m, k, n):
        _check_fold_args(w, _w_bytes(m, k, "q6k"), m, k, qt, tiles_elems(n, k) * 2, ds, n, out, n * m * 4)
    _check("mmq_q6k_q8t_fp32out", load_library().mmq_q6k_q8t_fp32out(
        _ptr(w), m, k, _ptr(qt), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q6k_q8(w, m, k, q, ds, n, dots):
    if _sized(m, k, n):
        _check_fold_args(w, _w_bytes(m, k, "q6k"), m, k, q, n * k, None, n, dots, n * m * (k // 16) * 4)
        _fits(ds, n * (k // 32) * 4, "ds")
    _check("mmq_q6k_q8", load_library().mmq_q6k_q8(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(dots), _stream()))


def mmq_q6k_q8_fp32out(w, m, k, q, ds, n, out):
    if _sized(m, k, n):
        _check_fold_args(w, _w_bytes(m, k, "q6k"), m, k, q, n * k, ds, n, out, n * m * 4)
    _check("mmq_q6k_q8_fp32out", load_library().mmq_q6k_q8_fp32out(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q6k_q8_f16out(w, m, k, q, ds, n, out):
    if _sized(m, k, n):
        _check_fold_args(w, _w_bytes(m, k, "q6k"), m, k, q, n * k, ds, n, out, n * m * 2)
    _check("mmq_q6k_q8_f16out", load_library().mmq_q6k_q8_f16out(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out), _stream()))


def mmq_q6k_q8_fold(w, m, k, q, ds, n, out, out_f16, kernel):
    if _sized(m, k, n):
        _check_fold_args(w, _w_bytes(m, k, "q6k"), m, k, q, n * k, ds, n, out, n * m * (2 if out_f16 else 4))
    _check("mmq_q6k_q8_fold", load_library().mmq_q6k_q8_fold(
        _ptr(w), m, k, _ptr(q), _ptr(ds), n, _ptr(out), int(out_f16), int(kernel), _stream()))


def mmq_kernel_choice(fmt: int, m: int, k: int, n: int) -> int:
    """The kernel id (KERNEL_*) a fold entry point of format fmt runs for an
    m x k weight and n tokens (host logic only; raises on a bad argument)."""
    r = load_library().mmq_kernel_choice(int(fmt), m, k, n)
    _check("mmq_kernel_choice", r if r < 0 else 0)
    return r


# --------------------------------------------------------- tensor helpers
def _tokens(q, k, name="q"):
    """Token count of a q8 code tensor [n, k] (raises unless its rows are k long)."""
    if q.dim() != 2 or q.shape[1] != k:
        raise ValueError("%s must be [n, %d], got %s" % (name, k, tuple(q.shape)))
    return q.shape[0]


def _scale_words(ds, n, k):
    if tuple(ds.shape) != (n, k // 32):
        raise ValueError("ds must be [%d, %d], got %s" % (n, k // 32, tuple(ds.shape)))


def _out_tensor(out, n, m, dtype, dev):
    if out is None:
        return torch.empty((n, m), dtype=dtype, device=dev)
    _need(out, dtype, "out")
    if tuple(out.shape) != (n, m):
        raise ValueError("out must be [%d, %d], got %s" % (n, m, tuple(out.shape)))
    return out


def _weights(w, m, k, fmt, name="w"):
    _need(w, torch.uint8, name)
    _mmq_sizes(m, k, 0)
    if w.numel() != _w_bytes(m, k, fmt):
        raise ValueError("%s must hold %d bytes for a %d x %d %s matrix, got %d"
                         % (name, _w_bytes(m, k, fmt), m, k, fmt, w.numel()))


def quantize(x: torch.Tensor):
    """x float32 [n, k] -> (q int8 [n, k], ds int32 [n, k/32] holding the uint32 words)."""
    _need(x, torch.float32, "x")
    if x.dim() != 2:
        raise ValueError("x must be [n, k]")
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
    if x.dim() != 2:
        raise ValueError("x must be [n, k]")
    n, k = x.shape
    qt = torch.empty(tiles_elems(n, k), dtype=torch.int16, device=x.device)
    ds = torch.empty((n, k // 32 if k % 32 == 0 else 0), dtype=torch.int32, device=x.device)
    q8_quantize_rows_tiled(x, n, k, qt, ds)
    return qt, ds


def quantize_silu_mul_tiled(gate: torch.Tensor, up: torch.Tensor):
    """Operand tiles of q8(SiLU(gate) * up): (qt int16 [tiles_elems(n, k)], ds int32 [n, k/32])."""
    _need(gate, torch.float32, "gate")
    _need(up, torch.float32, "up")
    if gate.shape != up.shape or gate.dim() != 2:
        raise ValueError("gate and up must have the same shape [n, k]")
    n, k = gate.shape
    qt = torch.empty(tiles_elems(n, k), dtype=torch.int16, device=gate.device)
    ds = torch.empty((n, k // 32 if k % 32 == 0 else 0), dtype=torch.int32, device=gate.device)
    q8_quantize_silu_mul_tiled(gate, up, n, k, qt, ds)
    return qt, ds


def quantize_silu_mul(gate: torch.Tensor, up: torch.Tensor):
    """q8 of SiLU(gate) * up: (q int8 [n, k], ds int32 [n, k/32])."""
    _need(gate, torch.float32, "gate")
    _need(up, torch.float32, "up")
    if gate.shape != up.shape or gate.dim() != 2:
        raise ValueError("gate and up must have the same shape [n, k]")
    n, k = gate.shape
    q = torch.empty((n, k), dtype=torch.int8, device=gate.device)
    ds = torch.empty((n, k // 32 if k % 32 == 0 else 0), dtype=torch.int32, device=gate.device)
    q8_quantize_silu_mul(gate, up, n, k, q, ds)
    return q, ds


def blockdots(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds=None):
    """Exact int32 block dots [n, m, k/32]."""
    _weights(w, m, k, "q4k")
    _need(q, torch.int8, "q")
    n = _tokens(q, k)
    dots = torch.empty((n, m, k // 32), dtype=torch.int32, device=q.device)
    mmq_q4k_q8(w, m, k, q, ds, n, dots)
    return dots


def _fold(w, m, k, q, ds, out, fmt, out_dtype, call):
    _weights(w, m, k, fmt)
    _need(q, torch.int8, "q")
    _need(ds, torch.int32, "ds")
    n = _tokens(q, k)
    _scale_words(ds, n, k)
    out = _out_tensor(out, n, m, out_dtype, q.device)
    call(w, m, k, q, ds, n, out)
    return out


def fp32(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, out=None):
    """Two-term-fold output float32 [n, m]."""
    return _fold(w, m, k, q, ds, out, "q4k", torch.float32, mmq_q4k_q8_fp32out)


def fp16(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, out=None):
    """Two-term-fold output as binary16 [n, m] (the float32 result, rounded to nearest-even)."""
    return _fold(w, m, k, q, ds, out, "q4k", torch.float16, mmq_q4k_q8_f16out)


def fold_kernel(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, kernel: int,
                f16: bool = False, out=None):
    """The q4_K fold on a named kernel (KERNEL_*): float32 or binary16 [n, m]."""
    return _fold(w, m, k, q, ds, out, "q4k", torch.float16 if f16 else torch.float32,
                 lambda *a: mmq_q4k_q8_fold(*a, int(f16), kernel))


def q6k_dots(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds=None):
    """Exact int32 q6_K group dots [n, m, k/16]."""
    _weights(w, m, k, "q6k")
    _need(q, torch.int8, "q")
    n = _tokens(q, k)
    dots = torch.empty((n, m, k // 16), dtype=torch.int32, device=q.device)
    mmq_q6k_q8(w, m, k, q, ds, n, dots)
    return dots


def q6k_fp32(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, out=None):
    """q6_K output float32 [n, m]."""
    return _fold(w, m, k, q, ds, out, "q6k", torch.float32, mmq_q6k_q8_fp32out)


def q6k_fp16(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, out=None):
    """q6_K output as binary16 [n, m] (the float32 result, rounded to nearest-even)."""
    return _fold(w, m, k, q, ds, out, "q6k", torch.float16, mmq_q6k_q8_f16out)


def q6k_fold_kernel(w: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, kernel: int,
                    f16: bool = False, out=None):
    """The q6_K fold on a named kernel (KERNEL_*): float32 or binary16 [n, m]."""
    return _fold(w, m, k, q, ds, out, "q6k", torch.float16 if f16 else torch.float32,
                 lambda *a: mmq_q6k_q8_fold(*a, int(f16), kernel))


def _tiles_fold(w, m, k, qt, ds, out, fmt, call):
    _weights(w, m, k, fmt)
    _need(qt, torch.int16, "qt")
    _need(ds, torch.int32, "ds")
    if ds.dim() != 2:
        raise ValueError("ds must be [n, k/32]")
    n = ds.shape[0]
    _scale_words(ds, n, k)
    if qt.numel() != tiles_elems(n, k):
        raise ValueError("qt must hold tiles_elems(%d, %d) = %d values, got %d"
                         % (n, k, tiles_elems(n, k), qt.numel()))
    out = _out_tensor(out, n, m, torch.float32, ds.device)
    call(w, m, k, qt, ds, n, out)
    return out


def fp32_tiles(w: torch.Tensor, m: int, k: int, qt: torch.Tensor, ds: torch.Tensor, out=None,
               repacked: bool = False):
    """The fold on q8 operand tiles (from quantize_tiled): float32 [n, m]; w is
    q4_K rows, or q4k_repack records with repacked=True."""
    return _tiles_fold(w, m, k, qt, ds, out, "repacked" if repacked else "q4k",
                       mmq_q4kr_q8t_fp32out if repacked else mmq_q4k_q8t_fp32out)


def q6k_fp32_tiles(w: torch.Tensor, m: int, k: int, qt: torch.Tensor, ds: torch.Tensor, out=None):
    """The q6_K fold on q8 operand tiles (from quantize_tiled): float32 [n, m]."""
    return _tiles_fold(w, m, k, qt, ds, out, "q6k", mmq_q6k_q8t_fp32out)


def repack_bytes(m: int, k: int) -> int:
    """Size of q4k_repack's output for an m x k matrix."""
    return _w_bytes(m, k, "repacked")


def repack(w: torch.Tensor, m: int, k: int):
    """Load-time repack of q4_K weights: uint8 tensor of repack_bytes(m, k)."""
    _weights(w, m, k, "q4k")
    wr = torch.empty(repack_bytes(m, k), dtype=torch.uint8, device=w.device)
    q4k_repack(w, m, k, wr)
    return wr


def fp32_repacked(wr: torch.Tensor, m: int, k: int, q: torch.Tensor, ds: torch.Tensor, out=None):
    """mmq_q4k_q8_fp32out on repacked weights: float32 [n, m]."""
    return _fold(wr, m, k, q, ds, out, "repacked", torch.float32, mmq_q4kr_q8_fp32out)
