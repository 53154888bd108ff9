"""Every q4_K float32 kernel meets the same bar on shapes outside its
default range, named through mmq_q4k_q8_fold: i8 (the int8-MFMA kernel with a
three-operation fold, kept for comparison), f16 (the binary16-MFMA kernel,
default above 64 tokens and from 33 where the matrix gives it enough tiles,
here also on few tokens), few (the few-token int8-MFMA kernels, one tile up
to 16 tokens and more above, default from 9 tokens, here also on fewer),
dot4 (the vector-ALU kernel, default up to 5 tokens), narrow (the 4x4x4
int8-MFMA kernel on LDS-staged weights, up to 16 tokens, default from 6) and
stream (the narrow kernel's arithmetic with token operands shared in LDS by a
workgroup of many 8-row tiles, up to 16 tokens).  Each kernel's binary16
output must equal its float32 output rounded to nearest-even, bit for bit,
and the automatic choice must equal the kernel mmq_kernel_choice names."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_fp32, gpu_quantize, note, to_dev
from q4_q8_integer_amd import binding, synth

pytestmark = pytest.mark.gpu

SHAPES = {
    binding.KERNEL_I8: [(64, 256, 512), (77, 200, 768), (130, 129, 512), (5, 131, 2304)],
    # k = 256 .. 2304: the producers' three-set loop leaves after 2, 4, 6 (whole), 10 and 18
    # (whole) stages of 128 k
    binding.KERNEL_F16: [(1, 256, 512), (7, 200, 768), (33, 129, 512), (64, 131, 2304), (65, 130, 256),
                         (80, 96, 1280)],
    binding.KERNEL_FEW: [(1, 1, 256), (7, 31, 1280), (16, 17, 2304), (17, 200, 768), (48, 129, 512),
                         (64, 256, 11008)],
    binding.KERNEL_DOT4: [(1, 1, 256), (2, 17, 2304), (3, 33, 512), (4, 200, 768), (5, 129, 4352),
                          (6, 16, 256), (7, 131, 2304), (8, 256, 11008)],
    binding.KERNEL_NARROW: [(1, 1, 256), (2, 65, 2304), (3, 33, 512), (4, 200, 768), (5, 129, 4352),
                            (6, 17, 1280), (7, 131, 2304), (8, 256, 11008), (8, 48, 3584), (9, 70, 1280),
                            (12, 33, 2304), (13, 17, 4352), (16, 130, 768)],
    # k of 1, 2 and 3 token phases of 16 super-blocks (the last ragged), 1-8 tokens; rows
    # giving 4 waves per tile (1 or 2 tiles per workgroup), 2 (3 tiles) and 1 (5 tiles)
    binding.KERNEL_STREAM: [(1, 1, 256), (2, 9, 2304), (3, 33, 4352), (4, 200, 768), (5, 131, 11008),
                            (6, 17, 8192), (3, 2100, 1280), (7, 4111, 4352), (8, 5121, 1280),
                            (4, 9000, 2304), (8, 64, 4096),
                            # 9-16 tokens: three and four groups, token phases of 8 super-blocks
                            (9, 1, 256), (12, 9, 2304), (13, 33, 4352), (16, 200, 768), (10, 131, 11008),
                            (11, 2100, 1280), (14, 4111, 4352), (16, 9000, 2304)],
}


@pytest.mark.parametrize("kernel", sorted(SHAPES), ids=lambda k: binding.KERNEL_NAMES[k])
def test_named_fp32_kernel_matches_oracle(kernel):
    for seed, (n, m, k) in enumerate(SHAPES[kernel]):
        note("named kernel %s n=%d m=%d k=%d" % (binding.KERNEL_NAMES[kernel], n, m, k))
        f = synth.random_fields(500 + seed, m, k, sc_zero_frac=0.1)
        x = synth.random_activations(500 + seed, n, k, "outliers")
        w = synth.pack_q4k(f)
        q, ds = gpu_quantize(x)
        wd = to_dev(w)
        got = binding.fold_kernel(wd, m, k, q, ds, kernel)
        got16 = binding.fold_kernel(wd, m, k, q, ds, kernel, f16=True)
        torch.cuda.synchronize()
        assert np.array_equal(got16.cpu().numpy().view(np.uint16),
                              got.cpu().numpy().astype(np.float16).view(np.uint16)), "f16 != rounded fp32"
        rq, rds = oracle.quantize(x)
        check_fp32(got.cpu().numpy(), oracle.out_f64(w, m, k, rq, rds), "named kernel")


@pytest.mark.parametrize("n,m,k", [(1, 64, 512), (5, 64, 512), (6, 64, 512), (7, 300, 512), (8, 300, 512),
                                   (9, 64, 512), (12, 8200, 16384), (33, 129, 512), (33, 20480, 512),
                                   (48, 20352, 512), (65, 96, 512)])
def test_auto_equals_the_named_choice(n, m, k):
    """The entry point's own choice is bitwise the kernel mmq_kernel_choice
    names for the shape (the 33-token rows at 20480 take the binary16 kernel
    at its 160-tile threshold; 20352 rows stay on the few-token kernel; 12
    tokens on 8200 x 16384 take the narrow kernel's 32-row tiles)."""
    note("auto choice n=%d m=%d k=%d" % (n, m, k))
    f = synth.random_fields(530 + n, m, k)
    x = synth.random_activations(530 + n, n, k)
    wd = to_dev(synth.pack_q4k(f))
    q, ds = gpu_quantize(x)
    choice = binding.mmq_kernel_choice(binding.FORMAT_Q4K, m, k, n)
    a = binding.fp32(wd, m, k, q, ds)
    b = binding.fold_kernel(wd, m, k, q, ds, choice)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


def test_named_kernel_outside_its_range_raises():
    wd = torch.zeros(256 * 144 // 256 * 4, dtype=torch.uint8, device="cuda:0")
    q = torch.zeros((9, 256), dtype=torch.int8, device="cuda:0")
    ds = torch.zeros((9, 8), dtype=torch.int32, device="cuda:0")
    with pytest.raises(binding.MMQError):
        binding.fold_kernel(wd, 4, 256, q, ds, binding.KERNEL_DOT4)


def test_tensor_wrappers_check_sizes_on_device():
    """The tensor wrappers refuse tensors whose sizes disagree with m, k and
    the token count, before anything is launched."""
    m, k, n = 40, 512, 3
    dev = "cuda:0"
    w = torch.zeros(m * (k // 256) * 144, dtype=torch.uint8, device=dev)
    q = torch.zeros((n, k), dtype=torch.int8, device=dev)
    ds = torch.zeros((n, k // 32), dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        binding.fp32(w[:-1], m, k, q, ds)
    with pytest.raises(ValueError):
        binding.fp32(w, m, k, q[:, :256].contiguous(), ds)
    with pytest.raises(ValueError):
        binding.fp32(w, m, k, q, ds[:2].contiguous())
    with pytest.raises(ValueError):
        binding.fp32(w, m, k, q, ds, out=torch.empty((n, m - 1), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        binding.fp32_repacked(w, m, k, q, ds)          # records are 2368 bytes per 16 rows
    with pytest.raises(ValueError):
        binding.q6k_fp32(w, m, k, q, ds)                # q6_K blocks are 210 bytes
    qt = torch.zeros(binding.tiles_elems(n, k) - 8, dtype=torch.int16, device=dev)
    with pytest.raises(ValueError):
        binding.fp32_tiles(w, m, k, qt, ds)


@pytest.mark.parametrize("kernel", [binding.KERNEL_DOT4, binding.KERNEL_NARROW, binding.KERNEL_STREAM,
                                    binding.KERNEL_FEW], ids=lambda k: binding.KERNEL_NAMES[k])
def test_weight_streaming_kernels_run_to_run_and_token_slice_bitwise(kernel):
    """The weight-streaming kernels sum every output in an order fixed by m
    and k alone (waves, steps and partial sums in index order): a repeated
    call, and a call on a slice of the tokens, give the same bits."""
    m, k, n = 300, 9216, 8
    note("run-to-run %s n=%d m=%d k=%d" % (binding.KERNEL_NAMES[kernel], n, m, k))
    f = synth.random_fields(541, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(541, n, k, "outliers")
    wd = to_dev(synth.pack_q4k(f))
    q, ds = gpu_quantize(x)
    a = binding.fold_kernel(wd, m, k, q, ds, kernel)
    b = binding.fold_kernel(wd, m, k, q, ds, kernel)
    s = binding.fold_kernel(wd, m, k, q[3:8].contiguous(), ds[3:8].contiguous(), kernel)
    torch.cuda.synchronize()
    a, b, s = (t.cpu().numpy().view(np.uint32) for t in (a, b, s))
    assert np.array_equal(a, b)
    assert np.array_equal(a[3:8], s)


@pytest.mark.parametrize("n,m,k", [(7, 8200, 16384), (16, 8200, 16384), (9, 16400, 8192), (6, 16400, 8192)])
def test_narrow_32_row_tiles(n, m, k):
    """The narrow kernel's 32-row tiles, run by 8 waves per workgroup (257
    tiles, 64 super-blocks per row) and by 4 (513 tiles, 32 super-blocks),
    the last tile ragged: every output against the oracle, and the binary16
    output bitwise the rounded float32 one."""
    note("narrow 32-row tiles n=%d m=%d k=%d" % (n, m, k))
    f = synth.random_fields(560 + n, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(560 + n, n, k, "outliers")
    w = synth.pack_q4k(f)
    q, ds = gpu_quantize(x)
    wd = to_dev(w)
    got = binding.fold_kernel(wd, m, k, q, ds, binding.KERNEL_NARROW)
    got16 = binding.fold_kernel(wd, m, k, q, ds, binding.KERNEL_NARROW, f16=True)
    torch.cuda.synchronize()
    assert np.array_equal(got16.cpu().numpy().view(np.uint16),
                          got.cpu().numpy().astype(np.float16).view(np.uint16)), "f16 != rounded fp32"
    rq, rds = oracle.quantize(x)
    check_fp32(got.cpu().numpy(), oracle.out_f64(w, m, k, rq, rds), "narrow 32-row tiles")


def test_narrow_32_row_tiles_run_to_run_and_token_slice_bitwise():
    """The 32-row tiles sum in an order fixed by m and k alone too: a repeated
    call and calls on token slices (other token-group counts) give the same
    bits."""
    m, k, n = 8200, 16384, 12
    note("run-to-run narrow 32-row tiles n=%d m=%d k=%d" % (n, m, k))
    f = synth.random_fields(561, m, k)
    x = synth.random_activations(561, n, k, "outliers")
    wd = to_dev(synth.pack_q4k(f))
    q, ds = gpu_quantize(x)
    a = binding.fold_kernel(wd, m, k, q, ds, binding.KERNEL_NARROW)
    b = binding.fold_kernel(wd, m, k, q, ds, binding.KERNEL_NARROW)
    s1 = binding.fold_kernel(wd, m, k, q[2:12].contiguous(), ds[2:12].contiguous(), binding.KERNEL_NARROW)
    s2 = binding.fold_kernel(wd, m, k, q[5:8].contiguous(), ds[5:8].contiguous(), binding.KERNEL_NARROW)
    torch.cuda.synchronize()
    a, b, s1, s2 = (t.cpu().numpy().view(np.uint32) for t in (a, b, s1, s2))
    assert np.array_equal(a, b)
    assert np.array_equal(a[2:12], s1)
    assert np.array_equal(a[5:8], s2)


@pytest.mark.parametrize("n,m,k", [(7, 16392, 4352), (5, 20000, 512), (8, 24583, 8448), (15, 20000, 512),
                                   (16, 16392, 2304)])
def test_stream_two_tiles_per_wave(n, m, k):
    """The stream kernel with two 8-row tiles per wave (from 2049 tiles on:
    10 to 16 tiles per workgroup), ragged in rows and in the last phase:
    every output against the oracle, and the binary16 output bitwise the
    rounded float32 one."""
    note("stream two tiles per wave n=%d m=%d k=%d" % (n, m, k))
    f = synth.random_fields(570 + n, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(570 + n, n, k, "outliers")
    w = synth.pack_q4k(f)
    q, ds = gpu_quantize(x)
    wd = to_dev(w)
    got = binding.fold_kernel(wd, m, k, q, ds, binding.KERNEL_STREAM)
    got16 = binding.fold_kernel(wd, m, k, q, ds, binding.KERNEL_STREAM, f16=True)
    torch.cuda.synchronize()
    assert np.array_equal(got16.cpu().numpy().view(np.uint16),
                          got.cpu().numpy().astype(np.float16).view(np.uint16)), "f16 != rounded fp32"
    rq, rds = oracle.quantize(x)
    check_fp32(got.cpu().numpy(), oracle.out_f64(w, m, k, rq, rds), "stream two tiles per wave")


def test_f16_row_split_launch():
    """A binary16-kernel call whose 128-token tiles overshoot whole rounds of
    256 runs in two launches cut by rows: 4220 rows (33 row tiles, the last
    ragged) x 1024 tokens = 264 tiles -> 32 x 8 tiles of 128 tokens, then the
    last row tile in 16 tiles of 64.  Sampled tokens against the oracle (every
    token tile, both parts), the binary16 output bitwise the rounded float32
    one, and the first 512 tokens (132 tiles of 64, one launch) bitwise equal
    to the same rows of the split call."""
    n, m, k = 1024, 4220, 512
    note("f16 row split n=%d m=%d k=%d" % (n, m, k))
    f = synth.random_fields(580, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(580, n, k, "outliers")
    w = synth.pack_q4k(f)
    wd = to_dev(w)
    q, ds = gpu_quantize(x)
    got = binding.fold_kernel(wd, m, k, q, ds, binding.KERNEL_F16)
    got16 = binding.fold_kernel(wd, m, k, q, ds, binding.KERNEL_F16, f16=True)
    part = binding.fold_kernel(wd, m, k, q[:512].contiguous(), ds[:512].contiguous(), binding.KERNEL_F16)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.array_equal(got16.cpu().numpy().view(np.uint16), got.astype(np.float16).view(np.uint16))
    assert np.array_equal(got[:512].view(np.uint32), part.cpu().numpy().view(np.uint32))
    toks = np.r_[0:4, 127:130, 500:503, 1020:1024]
    rq, rds = oracle.quantize(x[toks])
    check_fp32(got[toks], oracle.out_f64(w, m, k, rq, rds), "f16 row split")
