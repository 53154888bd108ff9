"""q8_quantize_rows on the GPU: bit-exact q and scale words against the oracle
on every workload's activation kind, ragged token counts and crafted blocks."""
import numpy as np
import pytest

import oracle
import pins
from gpu_helpers import gpu_quantize, host_ds, note
from q4_q8_integer_amd import synth

pytestmark = pytest.mark.gpu


def check(x, what):
    note("quantize: %s %s" % (what, x.shape))
    q, ds = gpu_quantize(x)
    rq, rds = oracle.quantize(x)
    gq = q.cpu().numpy()
    gds = host_ds(ds)
    bad = np.nonzero((gq != rq).any(axis=1))[0]
    assert bad.size == 0, "%s: q differs in rows %s" % (what, bad[:5])
    assert np.array_equal(gds, rds), "%s: scale words differ" % what


def test_tiny():
    check(synth.tiny_inputs()[1], "tiny 64x512")


def test_qproj_full():
    check(synth.gen_normal(synth.rng_for(1, 1), 2630, 4096), "q-proj 2630x4096")


def test_ffn_silu_full():
    check(synth.ffn_inputs("x_down"), "ffn down input SiLU 2630x11008")


@pytest.mark.parametrize("which", ["attn_in", "down_in"])
def test_layer_outliers(which):
    check(synth.layer_activation(which, 512), "layer %s N=512" % which)


@pytest.mark.parametrize("n", [1, 7, 33])
def test_weight_bound_ragged(n):
    check(synth.weight_bound_activation("wide_out", n), "wide_out N=%d" % n)


@pytest.mark.parametrize("n,k", [(1, 32), (3, 96), (5, 4096 + 32)])
def test_odd_block_counts(n, k):
    check(synth.random_activations(n + k, n, k, "outliers"), "random %dx%d" % (n, k))


def test_crafted_blocks():
    blocks = pins.golden_q8_blocks()
    x = np.stack([b[0] for b in blocks.values()]).reshape(1, -1)
    check(x, "golden blocks")
    q, ds = gpu_quantize(x)
    words = host_ds(ds)[0]
    for i, (xb, qb, ssum, word) in enumerate(blocks.values()):
        assert words[i] == word
        assert np.array_equal(q.cpu().numpy()[0, 32 * i:32 * i + 32], qb)


def test_zero_tiny_and_huge_blocks():
    x = np.zeros((3, 128), dtype=np.float32)
    x[1, 32:64] = np.float32(1e-30) * np.arange(32, dtype=np.float32)   # da underflows binary16
    x[1, 64:96] = np.float32(3e-6)                                      # subnormal binary16 da
    x[2, 0:32] = np.float32(1e30)
    x[2, 96:128] = -np.float32(7.0)
    check(x, "zero / subnormal / huge blocks")
