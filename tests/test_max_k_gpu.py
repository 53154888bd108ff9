"""The largest k the ABI accepts, 2^24, through every fold kernel: a q4_K row
is 9.4 MB, a q6_K row 13.8 MB, and 128 tokens of q8 are 2^31 bytes, so the
kernels' byte offsets and buffer extents run up to their limits.  The
activations are three distinct token rows repeated over n tokens (every row
still sits at its own address), so the oracle computes three rows; every
output row is checked against the oracle row of its token.

The accuracy bar is the workloads' one (relative L2 <= 1e-5, max-abs <=
1e-3 x row scale) for every kernel.  The dot4 and few-token kernels split k
over several waves; the narrow kernel (7 tokens here) and the stream kernel
(named, 7 tokens) move their float32 partials into a second accumulator
every 32 super-blocks; the binary16-MFMA
kernels (more than 64 tokens) restart their
float32 partial every 256 super-blocks into a second accumulator, so no
float32 sum runs over more than 256 terms (one sum over all S = k/256 =
65536 super-block folds would reach about sqrt(S) * 2^-24 = 1.5e-5)."""
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
    check_fp32(out.cpu().numpy(), ref[idx], "max k %s n=%d" % (fmt, n))
    del wd, q, ds, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [1, 7, 9, 33, 128])
def test_max_k_q4k(n):
    run_max_k("q4k", n)


@pytest.mark.parametrize("n", [1, 128])
def test_max_k_q6k(n):
    run_max_k("q6k", n)


def test_max_k_stream_kernel():
    """The stream kernel (named: its automatic range has k <= 8192) at the
    largest k: 4096 token phases of 16 super-blocks, 7 tokens, 20 rows (three
    tiles of 8, the last partial, one per workgroup, four waves per tile each
    taking every fourth step)."""
    n = 7
    note("max k: stream kernel n=%d" % n)
    w, base, rq, rds, ref = case_inputs("q4k")
    idx = np.arange(n) % 3
    x = to_dev(base)[torch.from_numpy(idx).to("cuda:0")]
    q, ds = binding.quantize(x)
    del x
    out = binding.fold_kernel(to_dev(w), M, K, q, ds, binding.KERNEL_STREAM)
    torch.cuda.synchronize()
    check_fp32(out.cpu().numpy(), ref[idx], "max k stream")
    del q, ds, out
    torch.cuda.empty_cache()


def test_max_k_operand_tiles():
    """The tiled entry points run the binary16 kernels at every n; at the
    largest k they keep the same bar (4 tokens, 20 rows)."""
    n = 4
    note("max k: operand tiles n=%d" % n)
    w, base, rq, rds, ref = case_inputs("q4k")
    idx = np.arange(n) % 3
    x = to_dev(base)[torch.from_numpy(idx).to("cuda:0")]
    qt, ds = binding.quantize_tiled(x)
    del x
    out = binding.fp32_tiles(to_dev(w), M, K, qt, ds)
    torch.cuda.synchronize()
    check_fp32(out.cpu().numpy(), ref[idx], "max k tiles")
    del qt, ds, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [20480, 20352])
def test_33_tokens_on_many_rows(m):
    """33 tokens on a matrix with 160 row tiles of 128 take the binary16
    kernel, with 159 the few-token kernel (the automatic choice's
    threshold): both at the float32 bar on a k of 8192 (32 super-blocks),
    checked on a window of 256 rows at each end of the matrix."""
    k, n = 8192, 33
    note("33 tokens on %d rows" % m)
    f = synth.random_fields(990 + m % 7, m, k, sc_zero_frac=0.1)
    w = synth.pack_q4k(f)
    x = synth.random_activations(991, n, k, "outliers")
    q, ds = binding.quantize(to_dev(x))
    out = binding.fp32(to_dev(w), m, k, q, ds)
    torch.cuda.synchronize()
    rq, rds = oracle.quantize(x)
    rows = np.r_[0:256, m - 256:m]
    wsub = np.ascontiguousarray(w.reshape(m, -1)[rows])
    ref = oracle.out_f64(wsub, len(rows), k, rq, rds)
    check_fp32(out.cpu().numpy()[:, rows], ref, "33 tokens, %d rows" % m)
