"""q6_K weights on the GPU (mmq_q6k_q8, mmq_q6k_q8_fp32out, mmq_q6k_q8_f16out)
against the oracle: bit-exact group dots, the float32 bar, binary16 output
equal to the rounded float32 output bit for bit, ragged shapes (odd
super-block counts put blocks at both 2- and 4-byte alignments), both
kernels (the dot4 kernel by default up to 8 tokens, the binary16-MFMA kernel
above that, the int8-MFMA tile kernel behind the dots entry; each also named
outside its range through mmq_q6k_q8_fold), the hand-worked
super-block, full-size workloads, and metamorphic properties."""
import numpy as np
import pytest
import torch

import oracle
import pins
from gpu_helpers import check_fp32, gpu_quantize, host_ds, note, sample_tokens, to_dev
from q4_q8_integer_amd import binding, synth

pytestmark = pytest.mark.gpu



def run_case(f, x, what, dots=True):
    m, k = f.q.shape
    n = x.shape[0]
    note("q6k: %s n=%d m=%d k=%d" % (what, n, m, k))
    w = synth.pack_q6k(f)
    wg = to_dev(w)
    q, ds = gpu_quantize(x)
    rq, rds = oracle.quantize(x)
    assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(host_ds(ds), rds)
    if dots:
        got = binding.q6k_dots(wg, m, k, q)
        torch.cuda.synchronize()
        ref = oracle.q6k_dots(w, m, k, rq)
        got = got.cpu().numpy()
        assert np.array_equal(got, ref), "%s: group dots differ at %d places" % (what, int((got != ref).sum()))
    o32 = binding.q6k_fp32(wg, m, k, q, ds)
    o16 = binding.q6k_fp16(wg, m, k, q, ds)
    torch.cuda.synchronize()
    o32 = o32.cpu().numpy()
    assert np.array_equal(o16.cpu().numpy().view(np.uint16), o32.astype(np.float16).view(np.uint16))
    return check_fp32(o32, oracle.q6k_out_f64(w, m, k, rq, rds), what)


@pytest.mark.parametrize("n,m,k", [(1, 1, 256), (2, 17, 768), (3, 33, 512), (5, 131, 2304),
                                   (7, 16, 256), (8, 200, 1280), (9, 129, 768), (64, 127, 256),
                                   (130, 257, 512), (200, 300, 1280)])
def test_q6k_ragged_shapes(n, m, k):
    f = synth.random_q6k_fields(n * 11 + m, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(n * 11 + m, n, k, "outliers")
    run_case(f, x, "ragged")


@pytest.mark.parametrize("k", [2304, 16640])
@pytest.mark.parametrize("n", range(1, 9))
def test_q6k_few_token_layouts(n, k):
    """Every token count of the dot4 kernel with and without the second LDS
    area: 9 super-blocks per row (one area) and 65 (the next step's copy in
    flight up to 4 tokens; each wave's last step runs past its range).  37
    rows leave a 5-row tile whose bytes end inside a 16-byte piece."""
    m = 37
    f = synth.random_q6k_fields(740 + 10 * n + k % 7, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(740 + 10 * n + k % 7, n, k, "outliers")
    run_case(f, x, "few-token layouts", dots=False)


def test_q6k_hand_worked_superblock():
    f, x, dots, out = pins.golden_q6k_one_superblock()
    wg = to_dev(synth.pack_q6k(f))
    q, ds = gpu_quantize(x)
    d = binding.q6k_dots(wg, 1, 256, q)
    o = binding.q6k_fp32(wg, 1, 256, q, ds)
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy()[0, 0], dots)
    assert o.cpu().numpy()[0, 0] == np.float32(out)


@pytest.mark.parametrize("n", [3, 40])
def test_q6k_zero_scale_group_is_exactly_zero(n):
    """A group with sc = 0 adds exactly 0: scrambling its codes leaves the
    output bit-identical (both kernels)."""
    m, k = 70, 768
    note("q6k zero-scale group n=%d" % n)
    f = synth.random_q6k_fields(800 + n, m, k)
    x = synth.random_activations(800 + n, n, k)
    q, ds = gpu_quantize(x)
    f.sc[:, 21] = 0
    a = binding.q6k_fp32(to_dev(synth.pack_q6k(f)), m, k, q, ds)
    f.q[:, 336:352] = (f.q[:, 336:352] + 17) % 64
    b = binding.q6k_fp32(to_dev(synth.pack_q6k(f)), m, k, q, ds)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("n", [1, 6, 100])
def test_q6k_repeats_are_bitwise_identical(n):
    m, k = 300, 1024
    note("q6k repeat n=%d" % n)
    f = synth.random_q6k_fields(810 + n, m, k)
    x = synth.random_activations(810 + n, n, k)
    wg = to_dev(synth.pack_q6k(f))
    q, ds = gpu_quantize(x)
    a = binding.q6k_fp32(wg, m, k, q, ds)
    b = binding.q6k_fp32(wg, m, k, q, ds)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


# ------------------------------------------------------- full-size workloads
@pytest.mark.parametrize("n", [1, 7])
def test_q6k_wide_in_full(n):
    """W[28672 x 8192] q6_K at 1 and 7 tokens (the dot4 kernel), every output
    against the oracle."""
    f = synth.q6k_weights("wide_in")
    x = synth.q6k_activation("wide_in", n)
    run_case(f, x, "wide_in full", dots=False)


def test_q6k_qproj_full_sampled():
    """W[4096 x 4096] q6_K at 2630 tokens (the binary16-MFMA kernel): sampled
    tokens x all rows in float32, exact group dots (the tile kernel) for
    sampled tokens x a row window."""
    f = synth.q6k_weights("qproj")
    m, k = f.q.shape
    n = 2630
    x = synth.q6k_activation("qproj", n)
    note("q6k full: qproj n=%d m=%d k=%d" % (n, m, k))
    w = synth.pack_q6k(f)
    wg = to_dev(w)
    q, ds = binding.quantize(to_dev(x))
    out = binding.q6k_fp32(wg, m, k, q, ds)
    torch.cuda.synchronize()
    toks = sample_tokens(n, 40)
    rq, rds = oracle.quantize(x[toks])
    assert np.array_equal(q.cpu().numpy()[toks], rq)
    check_fp32(out.cpu().numpy()[toks], oracle.q6k_out_f64(w, m, k, rq, rds), "qproj q6k sampled")
    r0, r1 = 1000, 1160
    wwin = np.ascontiguousarray(w[r0:r1])
    dg = binding.q6k_dots(to_dev(wwin), r1 - r0, k, q[torch.from_numpy(toks).to(q.device)].contiguous())
    torch.cuda.synchronize()
    assert np.array_equal(dg.cpu().numpy(), oracle.q6k_dots(wwin, r1 - r0, k, rq))


FORCED = {
    binding.KERNEL_I8: [(1, 1, 256), (3, 33, 768), (5, 131, 2304), (8, 200, 1280), (40, 96, 512), (130, 129, 768)],
    binding.KERNEL_F16: [(1, 1, 256), (3, 33, 768), (8, 200, 1280), (9, 17, 512), (64, 127, 256), (200, 300, 1280)],
    binding.KERNEL_DOT4: [(1, 40, 512), (4, 16, 256), (8, 129, 2304)],
}


@pytest.mark.parametrize("kernel", sorted(FORCED), ids=lambda k: binding.KERNEL_NAMES[k])
def test_q6k_named_kernel(kernel):
    """Every q6_K fold kernel meets the bar outside its default range (named
    through mmq_q6k_q8_fold), and its binary16 output is its float32 output
    rounded to nearest-even."""
    for seed, (n, m, k) in enumerate(FORCED[kernel]):
        note("q6k named kernel %s n=%d m=%d k=%d" % (binding.KERNEL_NAMES[kernel], n, m, k))
        f = synth.random_q6k_fields(600 + seed, m, k, sc_zero_frac=0.1)
        x = synth.random_activations(600 + seed, n, k, "outliers")
        w = synth.pack_q6k(f)
        q, ds = gpu_quantize(x)
        wd = to_dev(w)
        got = binding.q6k_fold_kernel(wd, m, k, q, ds, kernel)
        got16 = binding.q6k_fold_kernel(wd, m, k, q, ds, kernel, f16=True)
        torch.cuda.synchronize()
        assert np.array_equal(got16.cpu().numpy().view(np.uint16),
                              got.cpu().numpy().astype(np.float16).view(np.uint16))
        rq, rds = oracle.quantize(x)
        check_fp32(got.cpu().numpy(), oracle.q6k_out_f64(w, m, k, rq, rds), "named q6k kernel")


# ------------------------------------------------------------- metamorphic
@pytest.mark.parametrize("n", [5, 70])
def test_q6k_outputs_fully_written_and_guard_bands_untouched(n):
    """NaN-poisoned outputs are fully overwritten (both fold kernels, and the
    dots kernel) and the bytes on either side are untouched."""
    m, k = 100, 512
    note("q6k guard bands n=%d" % n)
    f = synth.random_q6k_fields(820 + n, m, k)
    x = synth.random_activations(820 + n, n, k)
    w = synth.pack_q6k(f)
    wg = to_dev(w)
    q, ds = gpu_quantize(x)
    pad = 64
    buf = torch.full((n * m + 2 * pad,), float("nan"), dtype=torch.float32, device=q.device)
    buf[:pad] = 12345.0
    buf[-pad:] = -6789.0
    binding.mmq_q6k_q8_fp32out(wg, m, k, q, ds, n, buf[pad:pad + n * m])
    dbuf = torch.full((n * m * (k // 16) + 2 * pad,), -77, dtype=torch.int32, device=q.device)
    binding.mmq_q6k_q8(wg, m, k, q, ds, n, dbuf[pad:pad + n * m * (k // 16)])
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert not np.isnan(h[pad:-pad]).any()
    assert (h[:pad] == 12345.0).all() and (h[-pad:] == -6789.0).all()
    hd = dbuf.cpu().numpy()
    assert (hd[:pad] == -77).all() and (hd[-pad:] == -77).all()
    rq, _ = oracle.quantize(x)
    assert np.array_equal(hd[pad:-pad].reshape(n, m, k // 16), oracle.q6k_dots(w, m, k, rq))


def test_q6k_token_slice_bitwise():
    """Above 8 tokens, a token's output row does not depend on the other
    tokens of the call (same kernel, same summation order)."""
    m, k = 150, 1024
    f = synth.random_q6k_fields(830, m, k)
    x = synth.random_activations(830, 200, k)
    wg = to_dev(synth.pack_q6k(f))
    q, ds = gpu_quantize(x)
    a = binding.q6k_fp32(wg, m, k, q, ds)
    s = binding.q6k_fp32(wg, m, k, q[37:151].contiguous(), ds[37:151].contiguous())
    d1 = binding.q6k_dots(wg, m, k, q)
    d2 = binding.q6k_dots(wg, m, k, q[37:151].contiguous())
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy()[37:151].view(np.uint32), s.cpu().numpy().view(np.uint32))
    assert np.array_equal(d1.cpu().numpy()[37:151], d2.cpu().numpy())


def test_q6k_empty_calls_touch_nothing():
    q = torch.zeros((0, 256), dtype=torch.int8, device="cuda:0")
    ds = torch.zeros((0, 8), dtype=torch.int32, device="cuda:0")
    w = torch.zeros((4, 210), dtype=torch.uint8, device="cuda:0")
    assert binding.q6k_fp32(w, 4, 256, q, ds).shape == (0, 4)
    assert binding.q6k_dots(w, 4, 256, q).shape == (0, 4, 16)
