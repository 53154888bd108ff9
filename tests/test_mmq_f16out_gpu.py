"""Binary16 output (mmq_q4k_q8_f16out): the same fold as the float32 entry
point, stored as binary16.

Two bars:
  * bit for bit, out16 == binary16(out32) rounded to nearest-even (numpy's
    float32 -> float16 conversion), for the same inputs and binary, including
    overflow to +-inf and binary16 subnormals;
  * against the float64 oracle, every element within one binary16 ulp of the
    exact value plus the float32 bar's row tolerance.
Shapes cover every kernel's default range (n <= 8, 9..64, > 64); the forced
kernels are covered in test_mmq_kernel_variants_gpu.py."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import MAX_ABS_ROW, gpu_quantize, note, sample_tokens, to_dev
from q4_q8_integer_amd import binding, synth

pytestmark = pytest.mark.gpu


def _both(f, x):
    w = synth.pack_q4k(f)
    q, ds = gpu_quantize(x)
    wd = to_dev(w)
    out32 = binding.fp32(wd, f.m, f.k, q, ds)
    out16 = binding.fp16(wd, f.m, f.k, q, ds)
    torch.cuda.synchronize()
    return w, out32.cpu().numpy(), out16.cpu().numpy()


def _ulp16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v.astype(np.float16)).astype(np.float64)
    nxt = np.nextafter(np.abs(v.astype(np.float16)), np.float16(np.inf)).astype(np.float64)
    return np.maximum(nxt - a, 2.0 ** -24)


@pytest.mark.parametrize("n,m,k", [(1, 33, 512), (5, 131, 2304), (8, 64, 256), (9, 17, 768),
                                   (33, 200, 1024), (64, 96, 512), (65, 129, 512),
                                   (130, 257, 1024), (300, 64, 2304)])
def test_f16out_is_rounded_fp32out(n, m, k):
    note("f16out n=%d m=%d k=%d" % (n, m, k))
    f = synth.random_fields(700 + n, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(700 + n, n, k, "outliers")
    w, o32, o16 = _both(f, x)
    want = o32.astype(np.float16)
    assert np.array_equal(o16.view(np.uint16), want.view(np.uint16))
    rq, rds = oracle.quantize(x)
    ref = oracle.out_f64(w, m, k, rq, rds)
    rowscale = np.abs(ref).max(axis=1, keepdims=True)
    err = np.abs(o16.astype(np.float64) - ref)
    assert np.all(err <= _ulp16(ref) + MAX_ABS_ROW * rowscale)


@pytest.mark.parametrize("n", [3, 40, 150])
def test_f16out_overflows_to_inf(n):
    # d scaled up so that outputs pass 65504 and round to +-inf.
    m, k = 80, 1024
    note("f16out overflow n=%d" % n)
    f = synth.random_fields(710 + n, m, k)
    big = dataclasses.replace(f, d=(f.d.astype(np.float32) * 4000).astype(np.float16))
    x = synth.random_activations(710 + n, n, k)
    _, o32, o16 = _both(big, x)
    with np.errstate(over="ignore"):
        want = o32.astype(np.float16)   # numpy's own overflow to +-inf is the expectation
    assert np.isinf(want).any() and np.isfinite(want).any()
    assert np.array_equal(o16.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("n", [3, 40, 150])
def test_f16out_subnormal_outputs(n):
    # d and dmin near the bottom of binary16 and small activations: outputs
    # around 1e-5, inside the binary16 subnormal range (< 2^-14).
    m, k = 80, 1024
    note("f16out subnormal n=%d" % n)
    f = synth.random_fields(720 + n, m, k)
    tiny = dataclasses.replace(f, d=(f.d.astype(np.float32) * 1e-5).astype(np.float16),
                               dmin=(f.dmin.astype(np.float32) * 1e-5).astype(np.float16))
    x = synth.random_activations(720 + n, n, k) * np.float32(1e-2)
    _, o32, o16 = _both(tiny, x)
    want = o32.astype(np.float16)
    sub = (want != 0) & (np.abs(want) < np.float16(2.0 ** -14))
    assert sub.mean() > 0.1
    assert np.array_equal(o16.view(np.uint16), want.view(np.uint16))


def test_f16out_qproj_full_size():
    """The full 7B q-proj (2630 tokens): bit for bit the rounded float32
    output everywhere, and on sampled tokens within one binary16 ulp of the
    float64 oracle plus the row bar."""
    f, x = synth.qproj_inputs()
    note("f16out q-proj full size")
    w, o32, o16 = _both(f, x)
    assert np.array_equal(o16.view(np.uint16), o32.astype(np.float16).view(np.uint16))
    toks = sample_tokens(x.shape[0], 32)
    rq, rds = oracle.quantize(x[toks])
    ref = oracle.out_f64(w, f.m, f.k, rq, rds)
    rowscale = np.abs(ref).max(axis=1, keepdims=True)
    err = np.abs(o16[toks].astype(np.float64) - ref)
    assert np.all(err <= _ulp16(ref) + MAX_ABS_ROW * rowscale)
