"""The load-time repack (q4k_repack) and the MMQ on repacked weights
(mmq_q4kr_q8_fp32out) on the GPU: repacked bytes equal the oracle's bit for
bit.  The result meets the float32 bar against the oracle for every n, and
equals mmq_q4k_q8_fp32out's bit for bit where both run the same arithmetic
on the two layouts: n <= 8 (the dot4 kernel) and n > 64 (the binary16-MFMA
kernel, which the repacked entry takes above 16 tokens where its tiles fill
the CUs or above 40 tokens; other counts run as slices of 8)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_fp32, gpu_quantize, note, sample_tokens, to_dev
from q4_q8_integer_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,k", [(1, 256), (16, 512), (33, 768), (200, 2304), (257, 11008)])
def test_repack_bytes_match_oracle(m, k):
    note("repack m=%d k=%d" % (m, k))
    f = synth.random_fields(600 + m, m, k)
    w = synth.pack_q4k(f)
    wr = binding.repack(to_dev(w), m, k)
    torch.cuda.synchronize()
    assert np.array_equal(wr.cpu().numpy(), oracle.q4k_repack(w, m, k))


@pytest.mark.parametrize("n,m,k", [(1, 1, 256), (2, 17, 2304), (3, 33, 512), (5, 129, 4352),
                                   (7, 131, 2304), (8, 256, 11008), (9, 40, 768), (16, 33, 512),
                                   (17, 100, 1024), (20, 100, 1024), (64, 129, 2304), (65, 129, 512),
                                   (130, 257, 1024), (300, 200, 2304), (200, 40, 16640)])
def test_repacked_mmq(n, m, k):
    note("repacked mmq n=%d m=%d k=%d" % (n, m, k))
    f = synth.random_fields(610 + n, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(610 + n, n, k, "outliers")
    w = synth.pack_q4k(f)
    wd = to_dev(w)
    q, ds = gpu_quantize(x)
    wr = binding.repack(wd, m, k)
    got = binding.fp32_repacked(wr, m, k, q, ds)
    # the repacked records run the dot4 kernel up to 8 tokens and the
    # binary16 kernel above 64: the same summation order as those kernels on
    # the q4_K rows
    base = binding.fold_kernel(wd, m, k, q, ds, binding.KERNEL_DOT4 if n <= 8 else binding.KERNEL_F16)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    if n <= 8 or n > 64:
        assert np.array_equal(got.view(np.uint32), base.cpu().numpy().view(np.uint32))
    rq, rds = oracle.quantize(x)
    check_fp32(got, oracle.out_f64(w, m, k, rq, rds), "repacked")


@pytest.mark.parametrize("n", [1, 7])
def test_repacked_wide_in_full(n):
    f = synth.weight_bound_weights("wide_in")
    x = synth.weight_bound_activation("wide_in", n)
    m, k = f.q.shape
    note("repacked wide_in full n=%d" % n)
    w = synth.pack_q4k(f)
    wd = to_dev(w)
    q, ds = binding.quantize(to_dev(x))
    wr = binding.repack(wd, m, k)
    got = binding.fp32_repacked(wr, m, k, q, ds)
    base = binding.fold_kernel(wd, m, k, q, ds, binding.KERNEL_DOT4)   # the records' kernel, on q4_K rows
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint32), base.cpu().numpy().view(np.uint32))
    assert np.array_equal(wr.cpu().numpy()[:4 * 2368 * 32], oracle.q4k_repack(w[:64], 64, k))


def test_repacked_qproj_full():
    """The 7B q-proj prefill on repacked weights: bit for bit the GGUF-layout
    result, and the float32 bar on sampled tokens."""
    f, x = synth.qproj_inputs()
    m, k = f.q.shape
    n = x.shape[0]
    note("repacked q-proj full n=%d" % n)
    w = synth.pack_q4k(f)
    wd = to_dev(w)
    q, ds = binding.quantize(to_dev(x))
    got = binding.fp32_repacked(binding.repack(wd, m, k), m, k, q, ds)
    base = binding.fp32(wd, m, k, q, ds)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), base.view(torch.int32))
    toks = sample_tokens(n, 24)
    rq, rds = oracle.quantize(x[toks])
    check_fp32(got[torch.from_numpy(toks).to(got.device)].cpu().numpy(),
               oracle.out_f64(w, m, k, rq, rds), "repacked q-proj")


def test_repack_guard_bands_and_empty():
    m, k = 21, 512
    f = synth.random_fields(620, m, k)
    w = synth.pack_q4k(f)
    size = binding.repack_bytes(m, k)
    pad = 64
    buf = torch.full((size + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda:0")
    binding.q4k_repack(to_dev(w), m, k, buf[pad:pad + size])
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert (h[:pad] == 0xA5).all() and (h[-pad:] == 0xA5).all()
    assert np.array_equal(h[pad:-pad], oracle.q4k_repack(w, m, k))
    empty = torch.zeros(0, dtype=torch.uint8, device="cuda:0")
    binding.q4k_repack(empty, 0, k, empty)
