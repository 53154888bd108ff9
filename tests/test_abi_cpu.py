"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

from q4_q8_integer_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmq.h")

OK, NULL, SHAPE, ALIGN, OVERFLOW, DEVICE = 0, -1, -2, -3, -4, -5
A = 0x10000          # a fake, 16-byte aligned address; never dereferenced by these calls
MIS = A + 4          # misaligned


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:int|const char \*)\s*(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from q4_q8_integer_amd.build import build_library
        build_library()
    return binding.load_library()


def test_header_declares_every_exported_call():
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS), names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen("nm -D --defined-only %s" % binding.LIB_PATH).read()
    for name in declared_functions():
        assert re.search(r"\bT %s\b" % name, out), name


def test_status_strings(lib):
    for code in (OK, NULL, SHAPE, ALIGN, OVERFLOW, DEVICE, -6, 12345):
        assert isinstance(lib.mmq_status_string(code), bytes)
    assert b"ALIGN" in lib.mmq_status_string(ALIGN)


@pytest.mark.parametrize("args,want", [
    ((A, -1, 64, A, A), SHAPE),
    ((A, 4, 0, A, A), SHAPE),
    ((A, 4, 48, A, A), SHAPE),
    ((A, 4, (1 << 24) + 32, A, A), OVERFLOW),
    ((A, 1 << 31, 32, A, A), OVERFLOW),
    ((0, 4, 64, A, A), NULL),
    ((A, 4, 64, 0, A), NULL),
    ((A, 4, 64, A, 0), NULL),
    ((MIS, 4, 64, A, A), ALIGN),
    ((A, 4, 64, MIS, A), ALIGN),
    ((A, 0, 64, 0, 0), OK),            # empty: no pointer is needed, nothing runs
])
def test_quantize_validation(lib, args, want):
    assert lib.q8_quantize_rows(*args, None) == want
    # the fused SiLU-gate quantizer checks the same, with `up` beside `gate`
    x, n, k, q, ds = args
    assert lib.q8_quantize_silu_mul(x, A, n, k, q, ds, None) == want


@pytest.mark.parametrize("args,want", [
    ((A, -1, 256, A, A), SHAPE),
    ((A, 4, 0, A, A), SHAPE),
    ((A, 4, 64, A, A), SHAPE),           # the tiled codes need k % 256 == 0
    ((A, 4, (1 << 24) + 256, A, A), OVERFLOW),
    ((A, (1 << 31) - 127, 256, A, A), OVERFLOW),
    ((0, 4, 256, A, A), NULL),
    ((A, 4, 256, 0, A), NULL),
    ((A, 4, 256, A, 0), NULL),
    ((MIS, 4, 256, A, A), ALIGN),
    ((A, 4, 256, MIS, A), ALIGN),
    ((A, 4, 256, A, MIS), ALIGN),
    ((A, 0, 256, 0, 0), OK),
])
def test_quantize_tiled_validation(lib, args, want):
    assert lib.q8_quantize_rows_tiled(*args, None) == want
    x, n, k, qt, ds = args
    assert lib.q8_quantize_silu_mul_tiled(x, A, n, k, qt, ds, None) == want


def test_silu_quantize_tiled_checks_up(lib):
    assert lib.q8_quantize_silu_mul_tiled(A, 0, 4, 256, A, A, None) == NULL
    assert lib.q8_quantize_silu_mul_tiled(A, MIS, 4, 256, A, A, None) == ALIGN


def test_silu_quantize_checks_up(lib):
    assert lib.q8_quantize_silu_mul(A, 0, 4, 64, A, A, None) == NULL
    assert lib.q8_quantize_silu_mul(A, MIS, 4, 64, A, A, None) == ALIGN


MMQ_CALLS = ["mmq_q4k_q8", "mmq_q4k_q8_fp32out", "mmq_q4k_q8_f16out",
             "mmq_q6k_q8", "mmq_q6k_q8_fp32out", "mmq_q6k_q8_f16out", "mmq_q4kr_q8_fp32out",
             "mmq_q4k_q8t_fp32out", "mmq_q4kr_q8t_fp32out", "mmq_q6k_q8t_fp32out"]


@pytest.mark.parametrize("fn", MMQ_CALLS)
@pytest.mark.parametrize("args,want", [
    ((A, 8, 512, A, A, -3, A), SHAPE),
    ((A, -8, 512, A, A, 3, A), SHAPE),
    ((A, 8, 0, A, A, 3, A), SHAPE),
    ((A, 8, 288, A, A, 3, A), SHAPE),
    ((A, 8, 1 << 25, A, A, 3, A), OVERFLOW),
    ((A, 1 << 31, 512, A, A, 3, A), OVERFLOW),
    ((A, 1 << 30, 512, A, A, 1 << 30, A), OVERFLOW),
    ((0, 8, 512, A, A, 3, A), NULL),
    ((A, 8, 512, 0, A, 3, A), NULL),
    ((A, 8, 512, A, A, 3, 0), NULL),
    ((MIS, 8, 512, A, A, 3, A), ALIGN),
    ((A, 8, 512, MIS, A, 3, A), ALIGN),
    ((A, 8, 512, A, A, 3, MIS), ALIGN),
    ((A, 8, 512, A, A, 0, A), OK),
    ((0, 0, 512, 0, 0, 5, 0), OK),
])
def test_mmq_validation(lib, fn, args, want):
    assert getattr(lib, fn)(*args, None) == want


@pytest.mark.parametrize("fn", ["mmq_q4k_q8_fp32out", "mmq_q4k_q8_f16out",
                                "mmq_q6k_q8_fp32out", "mmq_q6k_q8_f16out", "mmq_q4kr_q8_fp32out",
                                "mmq_q4k_q8t_fp32out", "mmq_q4kr_q8t_fp32out", "mmq_q6k_q8t_fp32out"])
def test_fold_needs_scales(lib, fn):
    assert getattr(lib, fn)(A, 8, 512, A, 0, 3, A, None) == NULL
    assert getattr(lib, fn)(A, 8, 512, A, MIS, 3, A, None) == ALIGN


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="needs a host without a HIP device")
def test_valid_arguments_without_device_report_device_error(lib):
    # Arguments pass validation, so the next step is the device check, which
    # fails here before anything could be launched on the fake pointers.
    assert lib.q8_quantize_rows(A, 4, 64, A, A, None) == DEVICE
    assert lib.q8_quantize_silu_mul(A, A, 4, 64, A, A, None) == DEVICE
    assert lib.mmq_q4k_q8_fp32out(A, 8, 512, A, A, 3, A, None) == DEVICE
    assert lib.mmq_q4k_q8_f16out(A, 8, 512, A, A, 3, A, None) == DEVICE
    assert lib.mmq_q4k_q8(A, 8, 512, A, 0, 3, A, None) == DEVICE
    assert lib.mmq_q6k_q8(A, 8, 512, A, 0, 3, A, None) == DEVICE
    assert lib.mmq_q6k_q8_fp32out(A, 8, 512, A, A, 3, A, None) == DEVICE
    assert lib.mmq_q6k_q8_f16out(A, 8, 512, A, A, 3, A, None) == DEVICE
    assert lib.q4k_repack(A, 8, 512, A, None) == DEVICE
    assert lib.mmq_q4kr_q8_fp32out(A, 8, 512, A, A, 3, A, None) == DEVICE
    assert lib.q8_quantize_rows_tiled(A, 4, 256, A, A, None) == DEVICE
    assert lib.q8_quantize_silu_mul_tiled(A, A, 4, 256, A, A, None) == DEVICE
    assert lib.mmq_q4k_q8t_fp32out(A, 8, 512, A, A, 3, A, None) == DEVICE
    assert lib.mmq_q4kr_q8t_fp32out(A, 8, 512, A, A, 3, A, None) == DEVICE
    assert lib.mmq_q6k_q8t_fp32out(A, 8, 512, A, A, 3, A, None) == DEVICE


def test_tiled_fold_token_limit(lib):
    # the operand tiles round n up to 128 tokens: n within 127 of 2^31 is
    # rejected (n*k and n*m are inside the other limits here)
    n = (1 << 31) - 100
    assert lib.mmq_q4k_q8t_fp32out(A, 8, 256, A, A, n, A, None) == OVERFLOW
    assert lib.mmq_q4kr_q8t_fp32out(A, 8, 256, A, A, n, A, None) == OVERFLOW
    assert lib.mmq_q6k_q8t_fp32out(A, 8, 256, A, A, n, A, None) == OVERFLOW


@pytest.mark.parametrize("args,want", [
    ((A, -1, 512, A), SHAPE),
    ((A, 8, 0, A), SHAPE),
    ((A, 8, 288, A), SHAPE),
    ((A, 8, 1 << 25, A), OVERFLOW),
    ((A, 1 << 31, 512, A), OVERFLOW),
    ((0, 8, 512, A), NULL),
    ((A, 8, 512, 0), NULL),
    ((MIS, 8, 512, A), ALIGN),
    ((A, 8, 512, MIS), ALIGN),
    ((0, 0, 512, 0), OK),
])
def test_repack_validation(lib, args, want):
    assert lib.q4k_repack(*args, None) == want


def test_q6k_weight_bytes_limit(lib):
    # m*(k/256) blocks with 144*blocks < 2^40 <= 210*blocks: an empty q4_K
    # call passes, the q6_K one is rejected for its larger blocks.
    m, k = 6_000_000, 1 << 18
    assert m * (k // 256) * 144 < 1 << 40 <= m * (k // 256) * 210
    assert lib.mmq_q4k_q8_fp32out(A, m, k, A, A, 0, A, None) == OK
    assert lib.mmq_q6k_q8_fp32out(A, m, k, A, A, 0, A, None) == OVERFLOW


def test_binding_raises_on_error_status(lib):
    with pytest.raises(binding.MMQError):
        binding._check("q8_quantize_rows", SHAPE)


KERNEL = -7
K_AUTO, K_DOT4, K_FEW, K_F16, K_I8, K_NARROW, K_STREAM = 0, 1, 2, 3, 4, 5, 6


@pytest.mark.parametrize("fn", ["mmq_q4k_q8_fold", "mmq_q6k_q8_fold"])
@pytest.mark.parametrize("args,want", [
    ((A, 8, 512, A, A, -3, A, 0, K_AUTO), SHAPE),
    ((A, 8, 288, A, A, 3, A, 0, K_F16), SHAPE),
    ((A, 8, 1 << 25, A, A, 3, A, 0, K_F16), OVERFLOW),
    ((0, 8, 512, A, A, 3, A, 0, K_F16), NULL),
    ((A, 8, 512, A, 0, 3, A, 0, K_F16), NULL),
    ((A, 8, 512, A, A, 3, MIS, 1, K_F16), ALIGN),
    ((A, 8, 512, A, A, 3, A, 0, 9), KERNEL),          # unknown kernel id
    ((A, 8, 512, A, A, 3, A, 0, 7), KERNEL),
    ((A, 8, 512, A, A, 3, A, 0, -1), KERNEL),
    ((A, 8, 512, A, A, 9, A, 0, K_DOT4), KERNEL),     # dot4 takes at most 8 tokens
    ((A, 8, 512, A, A, 0, A, 0, 9), OK),              # empty calls succeed before the kernel check
])
def test_fold_kernel_validation(lib, fn, args, want):
    assert getattr(lib, fn)(*args, None) == want


def test_fold_kernel_token_ranges(lib):
    # the few-token MFMA kernel takes at most 64 tokens, the narrow kernel at
    # most 16, and neither has a q6_K form
    assert lib.mmq_q4k_q8_fold(A, 8, 512, A, A, 65, A, 0, K_FEW, None) == KERNEL
    assert lib.mmq_q6k_q8_fold(A, 8, 512, A, A, 5, A, 0, K_FEW, None) == KERNEL
    assert lib.mmq_q4k_q8_fold(A, 8, 512, A, A, 17, A, 0, K_NARROW, None) == KERNEL
    assert lib.mmq_q6k_q8_fold(A, 8, 512, A, A, 5, A, 0, K_NARROW, None) == KERNEL
    # the stream kernel takes at most 16 tokens, q4_K only
    assert lib.mmq_q4k_q8_fold(A, 8, 512, A, A, 17, A, 0, K_STREAM, None) == KERNEL
    assert lib.mmq_q6k_q8_fold(A, 8, 512, A, A, 5, A, 0, K_STREAM, None) == KERNEL


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="needs a host without a HIP device")
def test_fold_kernel_valid_arguments_reach_device_check(lib):
    for k in (K_AUTO, K_DOT4, K_FEW, K_F16, K_I8, K_NARROW, K_STREAM):
        assert lib.mmq_q4k_q8_fold(A, 8, 512, A, A, 3, A, 0, k, None) == DEVICE
    for k in (K_AUTO, K_DOT4, K_F16, K_I8):
        assert lib.mmq_q6k_q8_fold(A, 8, 512, A, A, 3, A, 1, k, None) == DEVICE


def test_grid_limits_are_overflow_errors(lib):
    """Sizes inside the element limits whose launch would exceed HIP's 2^32
    work-items per grid are MMQ_ERR_OVERFLOW, before any HIP call."""
    # quantizer: 4 lanes per 32-block, n*k/8 work-items
    n, k = 1 << 20, 1 << 15
    assert n * k < 1 << 40 and n * k // 8 >= 1 << 32
    assert lib.q8_quantize_rows(A, n, k, A, A, None) == OVERFLOW
    assert lib.q8_quantize_silu_mul(A, A, n, k, A, A, None) == OVERFLOW
    assert lib.q8_quantize_rows_tiled(A, n, k, A, A, None) == OVERFLOW
    assert lib.q8_quantize_silu_mul_tiled(A, A, n, k, A, A, None) == OVERFLOW
    # binary16-MFMA kernel: 1024 work-items per 128 x 64 tile
    m, n, k = 1 << 19, 1 << 16, 256
    assert n * m < 1 << 40 and (m // 128) * (n // 64) * 1024 >= 1 << 32
    for fn in ("mmq_q4k_q8_fp32out", "mmq_q4k_q8_f16out", "mmq_q4kr_q8_fp32out", "mmq_q4k_q8t_fp32out",
               "mmq_q4kr_q8t_fp32out"):
        assert getattr(lib, fn)(A, m, k, A, A, n, A, None) == OVERFLOW, fn
    # the q6_K binary16 kernel: 1024 work-items per 128 x 128 tile
    n = 1 << 17
    assert (m // 128) * (n // 128) * 1024 >= 1 << 32
    for fn in ("mmq_q6k_q8_fp32out", "mmq_q6k_q8t_fp32out"):
        assert getattr(lib, fn)(A, m, k, A, A, n, A, None) == OVERFLOW, fn
    # dot4 kernel at one token: 256 work-items per 16 rows
    m = 1 << 28
    assert lib.mmq_q4k_q8_fp32out(A, m, 256, A, A, 1, A, None) == OVERFLOW
    assert lib.mmq_q6k_q8_fp32out(A, m, 256, A, A, 1, A, None) == OVERFLOW
    assert lib.mmq_q4kr_q8_fp32out(A, m, 256, A, A, 1, A, None) == OVERFLOW
    # repack: 64 work-items per record of 16 rows
    assert lib.q4k_repack(A, (1 << 31) - 1, 256, A, None) == OVERFLOW


@pytest.mark.parametrize("m,n,want", [
    # up to 4096 rows the narrow kernel takes 1-16 tokens (dot4's 16-row
    # workgroups do not fill the chip there)
    (4096, 1, K_NARROW), (4096, 5, K_NARROW), (4096, 6, K_NARROW), (4096, 8, K_NARROW), (4096, 9, K_NARROW),
    (4096, 16, K_NARROW), (4096, 17, K_FEW), (10240, 1, K_DOT4), (10232, 1, K_NARROW),
    # 17-32 tokens: the binary16 kernel where its 64-token tiles fill 224-255 CUs in one round
    (28672, 32, K_F16), (28672, 17, K_F16), (28544, 17, K_FEW), (24576, 17, K_FEW), (32768, 32, K_FEW),
    (28672, 33, K_F16),            # 224 x 1 tiles of 128 x 128: enough for the chip
    (20480, 33, K_F16),            # 160 tiles: the threshold
    (20352, 33, K_FEW),            # 159 tiles
    (8192, 33, K_FEW), (8192, 64, K_FEW), (8192, 65, K_F16), (4096, 2630, K_F16),
])
def test_kernel_choice_q4k(lib, m, n, want):
    assert lib.mmq_kernel_choice(0, m, 4096, n) == want


@pytest.mark.parametrize("m,k,n,want", [
    # 9-16 tokens: the narrow kernel where its 32-row tiles (at least 256 of
    # them, 4 waves each from 512 on, else 8) give each wave at least 11
    # super-blocks of 256
    (8192, 28672, 9, K_NARROW), (8192, 28672, 16, K_NARROW), (8192, 28672, 17, K_FEW),
    (8160, 28672, 13, K_FEW),       # 255 tiles of 32 rows: not the narrow kernel
    (8160, 28672, 12, K_STREAM),    # the stream kernel's 9-12-token rule for long rows
    (28672, 8192, 17, K_F16),       # 224 tiles of 64 tokens
    (13824, 5120, 1, K_NARROW),     # 20 super-blocks per row: not dot4's multiple of 16
    (8192, 28672, 1, K_DOT4), (8192, 8192, 1, K_NARROW),   # 8192 rows: dot4 only with >= 64 super-blocks
    (16384, 16384, 7, K_NARROW),
    (16384, 16384, 16, K_NARROW),   # 512 tiles: 4 waves x 16 super-blocks
    (8192, 8192, 12, K_FEW),        # 256 tiles but 8 waves x 4 super-blocks
    (8192, 24576, 12, K_NARROW),    # 8 waves x 12
    (8192, 22528, 12, K_NARROW),    # 8 waves x 11
    (8192, 20480, 13, K_FEW),       # 8 waves x 10: not the narrow kernel
    (8192, 20480, 12, K_STREAM),    # the stream kernel's 9-12-token rule for long rows
])
def test_kernel_choice_q4k_by_k(lib, m, k, n, want):
    assert lib.mmq_kernel_choice(0, m, k, n) == want


@pytest.mark.parametrize("m,k,n,want", [
    # 3-4 and 6-16 tokens: the stream kernel where it has at least 7 x 256
    # tiles of 8 rows, k <= 8192 in whole token phases, and up to 8 tokens 7
    # or 8 waves per workgroup, above 8 k > 4096 or at least 14 tiles per
    # workgroup; dot4 at 1-2 and 5 tokens; the narrow kernel elsewhere up to 8
    (28672, 8192, 1, K_DOT4), (28672, 8192, 2, K_DOT4), (28672, 8192, 3, K_STREAM),
    (28672, 8192, 4, K_STREAM), (28672, 8192, 5, K_DOT4), (28672, 8192, 6, K_STREAM),
    (28672, 8192, 8, K_STREAM), (14336, 4096, 7, K_STREAM), (14336, 4096, 3, K_STREAM),
    (14328, 4096, 7, K_NARROW),     # 1791 tiles of 8
    (16384, 4096, 7, K_STREAM),     # 8 tiles and waves per workgroup
    (18432, 4096, 7, K_NARROW),     # 9 tiles: 5 waves of two
    (26624, 4096, 7, K_STREAM),     # 13 tiles: 7 waves
    (24576, 6144, 7, K_NARROW),     # 24 super-blocks: a ragged 16-block phase
    (24576, 6144, 12, K_STREAM),    # three 8-block phases
    (28672, 8448, 7, K_NARROW),     # 33 super-blocks: three token phases
    (8192, 28672, 7, K_NARROW), (8192, 28672, 4, K_NARROW), (8192, 28672, 5, K_NARROW),
    (28672, 8192, 9, K_STREAM), (28672, 8192, 12, K_STREAM), (28672, 8192, 13, K_STREAM),
    (28672, 8192, 16, K_STREAM), (28672, 4096, 12, K_STREAM), (20480, 4096, 12, K_FEW),
    (14336, 4096, 9, K_FEW),        # one phase over 7 tiles
    (6144, 16384, 12, K_STREAM),    # 9-12 tokens on rows of >= 64 super-blocks
    (6144, 16384, 13, K_FEW), (8192, 8192, 9, K_FEW), (8192, 28672, 12, K_NARROW),
    (28672, 4352, 12, K_FEW),       # 17 super-blocks
])
def test_kernel_choice_stream(lib, m, k, n, want):
    assert lib.mmq_kernel_choice(0, m, k, n) == want


@pytest.mark.parametrize("m,n,want", [
    (4096, 8, K_DOT4), (4096, 16, K_DOT4), (28672, 17, K_F16), (8192, 17, K_DOT4),
    (8192, 40, K_DOT4), (8192, 41, K_F16), (4096, 2630, K_F16),
])
def test_kernel_choice_repacked(lib, m, n, want):
    assert lib.mmq_kernel_choice(1, m, 4096, n) == want


def test_kernel_choice_other_formats(lib):
    assert [lib.mmq_kernel_choice(2, 4096, 4096, n) for n in (1, 8, 9, 2630)] == [K_DOT4, K_DOT4, K_F16, K_F16]
    for fmt in (3, 4, 5):
        assert lib.mmq_kernel_choice(fmt, 4096, 4096, 1) == K_F16
    assert lib.mmq_kernel_choice(6, 4096, 4096, 1) == KERNEL
    assert lib.mmq_kernel_choice(0, 4096, 300, 1) == SHAPE
    assert lib.mmq_kernel_choice(0, -1, 4096, 1) == SHAPE
    assert binding.mmq_kernel_choice(binding.FORMAT_Q4K, 4096, 4096, 2630) == binding.KERNEL_F16
    with pytest.raises(binding.MMQError):
        binding.mmq_kernel_choice(0, 4096, 300, 1)


# ------------------------------------------------ binding size checks (no GPU)
# The C ABI sees only pointers; the binding checks every tensor's size (and
# that all tensors share a device) against m, k, n before the call, so a
# wrong size raises ValueError instead of reaching a kernel.  CPU tensors
# stand in for device tensors here: the checks run before any library call.
def _t(nbytes, dtype=torch.uint8, device="cpu"):
    item = torch.empty((), dtype=dtype).element_size()
    return torch.empty((nbytes + item - 1) // item, dtype=dtype, device=device)


M_, K_, N_ = 40, 512, 3
GOOD = dict(w=M_ * (K_ // 256) * 144, q=N_ * K_, ds=N_ * (K_ // 32) * 4, out=N_ * M_ * 4)


@pytest.mark.parametrize("short", ["w", "q", "ds", "out"])
def test_binding_rejects_short_tensors(short):
    sizes = dict(GOOD)
    sizes[short] -= 1
    w, q, ds, out = _t(sizes["w"]), _t(sizes["q"], torch.int8), _t(sizes["ds"]), _t(sizes["out"])
    with pytest.raises(ValueError, match=short):
        binding.mmq_q4k_q8_fp32out(w, M_, K_, q, ds, N_, out)


def test_binding_size_checks_cover_every_fold_call():
    w, q, ds = _t(GOOD["w"]), _t(GOOD["q"], torch.int8), _t(GOOD["ds"])
    small = _t(16)
    calls = [
        lambda: binding.mmq_q4k_q8(w, M_, K_, q, ds, N_, small),
        lambda: binding.mmq_q4k_q8_f16out(w, M_, K_, q, ds, N_, small),
        lambda: binding.mmq_q4k_q8_fold(w, M_, K_, q, ds, N_, small, 0, 0),
        lambda: binding.mmq_q4kr_q8_fp32out(w, M_, K_, q, ds, N_, _t(GOOD["out"])),   # records are larger
        lambda: binding.mmq_q4k_q8t_fp32out(w, M_, K_, q, ds, N_, _t(GOOD["out"])),   # tiles are 128 tokens
        lambda: binding.mmq_q6k_q8_fp32out(w, M_, K_, q, ds, N_, _t(GOOD["out"])),    # q6_K blocks are 210 B
        lambda: binding.mmq_q6k_q8(w, M_, K_, q, ds, N_, small),
        lambda: binding.q4k_repack(w, M_, K_, small),
        lambda: binding.q8_quantize_rows(_t(N_ * K_ * 4 - 4), N_, K_, q, ds),
        lambda: binding.q8_quantize_rows_tiled(_t(N_ * K_ * 4), N_, K_, small, ds),
    ]
    for call in calls:
        with pytest.raises(ValueError):
            call()


def test_binding_rejects_mixed_devices():
    w, q, ds = _t(GOOD["w"]), _t(GOOD["q"], torch.int8), _t(GOOD["ds"])
    out = _t(GOOD["out"], device="meta")
    with pytest.raises(ValueError, match="one device"):
        binding.mmq_q4k_q8_fp32out(w, M_, K_, q, ds, N_, out)


def test_binding_tensor_shape_helpers():
    with pytest.raises(ValueError):
        binding._tokens(torch.empty((3, 256), dtype=torch.int8), 512)
    with pytest.raises(ValueError):
        binding._scale_words(torch.empty((3, 8), dtype=torch.int32), 3, 512)
    with pytest.raises(ValueError):
        binding._mmq_sizes(4, 300, 1)
    assert binding._tokens(torch.empty((3, 512), dtype=torch.int8), 512) == 3
