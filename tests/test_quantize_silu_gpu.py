"""q8_quantize_silu_mul on the GPU: bit-exact against the oracle (q and the
scale words) on ragged shapes, extreme gates and the full FFN down-projection
input, and equal to q8_quantize_rows applied to the oracle's h; its tiled
output (q8_quantize_silu_mul_tiled) is the oracle's operand tiles of those codes."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import host_ds, note, to_dev
from q4_q8_integer_amd import binding, synth

pytestmark = pytest.mark.gpu


def _inputs(seed, n, k, scale=2.0):
    rng = np.random.default_rng([960, seed])
    g = (rng.standard_normal((n, k)) * scale).astype(np.float32)
    u = rng.standard_normal((n, k)).astype(np.float32)
    return g, u


def _check(g, u, what):
    n, k = g.shape
    note("silu quantize: %s n=%d k=%d" % (what, n, k))
    q, ds = binding.quantize_silu_mul(to_dev(g), to_dev(u))
    torch.cuda.synchronize()
    rq, rds = oracle.quantize_silu_mul(g, u)
    gq = q.cpu().numpy()
    assert np.array_equal(gq, rq), "%s: %d q values differ" % (what, int((gq != rq).sum()))
    assert np.array_equal(host_ds(ds), rds), "%s: scale words differ" % what
    return q, ds


@pytest.mark.parametrize("n,k", [(1, 32), (3, 96), (5, 4096), (77, 11008), (130, 2048)])
def test_silu_quantize_matches_oracle(n, k):
    g, u = _inputs(n * 3 + k, n, k)
    _check(g, u, "ragged")


def test_silu_quantize_extreme_gates():
    # saturated sigmoid both ways, exact zeros, tiny and huge products
    n, k = 8, 1024
    g, u = _inputs(7, n, k, scale=40.0)
    g[0, :32] = 0.0
    u[1, :64] = 0.0
    g[2] = np.linspace(-200, 200, k, dtype=np.float32)
    u[3] *= np.float32(1e-30)
    u[4] *= np.float32(1e30)
    g[5, :32] = -1e4
    _check(g, u, "extreme")


def test_silu_quantize_equals_plain_quantize_of_h():
    g, u = _inputs(11, 64, 2048)
    q, ds = _check(g, u, "vs plain")
    h = oracle.silu_mul(g, u)
    q2, ds2 = binding.quantize(to_dev(h))
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(ds, ds2)


def test_silu_quantize_ffn_down_full_size():
    g, u = synth.ffn_gate_up_outputs()
    _check(g, u, "FFN down input 2630x11008")


def test_silu_quantize_guard_bands_and_empty():
    n, k = 9, 320
    g, u = _inputs(13, n, k)
    pad = 64
    qbuf = torch.full((n * k + 2 * pad,), 99, dtype=torch.int8, device="cuda:0")
    dbuf = torch.full((n * k // 32 + 2 * pad,), -5, dtype=torch.int32, device="cuda:0")
    binding.q8_quantize_silu_mul(to_dev(g), to_dev(u), n, k, qbuf[pad:pad + n * k], dbuf[pad:pad + n * k // 32])
    torch.cuda.synchronize()
    hq, hd = qbuf.cpu().numpy(), dbuf.cpu().numpy()
    assert (hq[:pad] == 99).all() and (hq[-pad:] == 99).all()
    assert (hd[:pad] == -5).all() and (hd[-pad:] == -5).all()
    rq, rds = oracle.quantize_silu_mul(g, u)
    assert np.array_equal(hq[pad:-pad].reshape(n, k), rq)
    assert np.array_equal(hd[pad:-pad].view(np.uint32).reshape(n, k // 32), rds)
    z = torch.zeros((0, 64), device="cuda:0")
    q0, ds0 = binding.quantize_silu_mul(z, z)
    assert q0.shape == (0, 64) and ds0.shape == (0, 2)


@pytest.mark.parametrize("n,k", [(1, 256), (77, 11008), (130, 2048), (2630, 11008)])
def test_silu_quantize_tiled_matches_oracle(n, k):
    """The tiled output: the oracle's operand tiles of the oracle's codes, and
    its scale words, bit for bit."""
    g, u = _inputs(n * 5 + k, n, k)
    note("silu quantize tiled n=%d k=%d" % (n, k))
    qt, ds = binding.quantize_silu_mul_tiled(to_dev(g), to_dev(u))
    torch.cuda.synchronize()
    rq, rds = oracle.quantize_silu_mul(g, u)
    assert np.array_equal(qt.cpu().numpy().view(np.uint16), oracle.q8_tiles(rq))
    assert np.array_equal(host_ds(ds), rds)
