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
