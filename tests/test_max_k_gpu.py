"""The largest k the ABI accepts, 2^24, through every fold kernel: a q4_K row
is 9.4 MB, a q6_K row 13.8 MB, and 128 tokens of q8 are 2^31 bytes, so the
kernels' byte offsets and buffer extents run up to their limits.  The
activations are three distinct token rows repeated over n tokens (every row
still sits at its own address), so the oracle computes three rows; every
output row is checked against the oracle row of its token.

The accuracy bar is the workloads' one (relative L2 <= 1e-5, max-abs <=
1e-3 x row scale) for the kernels that split k over several waves.  The
binary16-MFMA kernel (more than 64 tokens) keeps one float32 accumulator
per output over all S = k/256 = 65536 super-block folds; serial float32
summation of S terms has a typical relative error of about sqrt(S) * 2^-24
(1.5e-5 here), so for it this test takes 4 * sqrt(S) * 2^-24 = 6.1e-5 as its
relative-L2 bar (the max-abs bar is unchanged)."""
import functools

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_fp32, note, to_dev
from q4_q8_integer_amd import binding, synth

pytestmark = pytest.mark.gpu

K = 1 << 24
M = 20          # a full and a 4-row tile of 16


@functools.lru_cache(maxsize=1)
def case_inputs(fmt):
    """Weights, three token rows, their q8 and the oracle output (shared by
    the token counts of one format)."""
    if fmt == "q4k":
        w = synth.pack_q4k(synth.random_fields(950, M, K, sc_zero_frac=0.1))
        ref_fn = oracle.out_f64
    else:
        w = synth.pack_q6k(synth.random_q6k_fields(960, M, K, sc_zero_frac=0.1))
        ref_fn = oracle.q6k_out_f64
    base = synth.random_activations(970, 3, K, "outliers")
    rq, rds = oracle.quantize(base)
    return w, base, rq, rds, ref_fn(w, M, K, rq, rds)


def run_max_k(fmt, n):
    note("max k: %s n=%d m=%d k=%d" % (fmt, n, M, K))
    w, base, rq, rds, ref = case_inputs(fmt)
    fold = binding.fp32 if fmt == "q4k" else binding.q6k_fp32
    idx = np.arange(n) % 3
    wd = to_dev(w)
    x = to_dev(base)[torch.from_numpy(idx).to("cuda:0")]
    q, ds = binding.quantize(x)
    del x
    out = fold(wd, M, K, q, ds)
    torch.cuda.synchronize()
    for r in range(min(n, 3)):
        assert np.array_equal(q[r].cpu().numpy(), rq[r])
        assert np.array_equal(ds[r].cpu().numpy().view(np.uint32), rds[r])
    rel_l2 = 4 * np.sqrt(K // 256) * 2.0 ** -24 if n > 64 else 1e-5
    check_fp32(out.cpu().numpy(), ref[idx], "max k %s n=%d" % (fmt, n), rel_l2=rel_l2)
    del wd, q, ds, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [1, 9, 33, 128])
def test_max_k_q4k(n):
    run_max_k("q4k", n)


@pytest.mark.parametrize("n", [1, 128])
def test_max_k_q6k(n):
    run_max_k("q6k", n)
