"""The q8 operand tiles on the GPU: q8_quantize_rows_tiled writes the
oracle's tile layout bit for bit (and the scale words of q8_quantize_rows),
touching nothing outside its buffers; the folds on the tiles
(mmq_q4k_q8t_fp32out on q4_K rows, mmq_q4kr_q8t_fp32out on repacked records,
mmq_q6k_q8t_fp32out on q6_K rows) meet the float32 bar against the oracle for
every n, and equal the int8-code entry point bit for bit wherever that runs
the same binary16-MFMA kernel (q4_K n > 64, q6_K n > 8)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_fp32, note, sample_tokens, to_dev
from q4_q8_integer_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,k", [(1, 256), (37, 512), (128, 256), (131, 768), (300, 2304),
                                 (1100, 4096)])
def test_quantize_tiled_matches_oracle(n, k):
    note("quantize tiled n=%d k=%d" % (n, k))
    x = synth.random_activations(900 + n, n, k, "outliers")
    x[0, :32] = 0.0                       # an all-zero block: code 0, word 0
    xd = to_dev(x)
    pad = 64
    size = binding.tiles_elems(n, k)
    buf = torch.full((size + 2 * pad,), 0x5A5A, dtype=torch.int16, device="cuda:0")
    ds = torch.empty((n, k // 32), dtype=torch.int32, device="cuda:0")
    binding.q8_quantize_rows_tiled(xd, n, k, buf[pad:pad + size], ds)
    q_rows, ds_rows = binding.quantize(xd)
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(np.uint16)
    assert (h[:pad] == 0x5A5A).all() and (h[-pad:] == 0x5A5A).all()
    rq, rds = oracle.quantize(x)
    assert np.array_equal(h[pad:-pad], oracle.q8_tiles(rq))
    assert np.array_equal(ds.cpu().numpy().view(np.uint32), rds)
    assert torch.equal(ds, ds_rows)
    assert np.array_equal(q_rows.cpu().numpy(), rq)


# (n, m, k): 64-token tiles (fewer than 256 tiles of 128) and 128-token tiles
# (32 x 9 = 288), ragged rows and tokens, one token, the longest k here.
CASES = [(1, 33, 512), (37, 300, 768), (65, 129, 512), (130, 257, 1024), (300, 200, 2304),
         (200, 40, 16640), (1100, 4096, 512)]


@pytest.mark.parametrize("repacked", [False, True], ids=["q4k", "repacked"])
@pytest.mark.parametrize("n,m,k", CASES)
def test_tiles_fold(n, m, k, repacked):
    note("tiles fold n=%d m=%d k=%d repacked=%s" % (n, m, k, repacked))
    f = synth.random_fields(910 + n, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(910 + n, n, k, "outliers")
    w = synth.pack_q4k(f)
    wd = to_dev(w)
    xd = to_dev(x)
    qt, ds = binding.quantize_tiled(xd)
    wt = binding.repack(wd, m, k) if repacked else wd
    got = binding.fp32_tiles(wt, m, k, qt, ds, repacked=repacked)
    q, ds_rows = binding.quantize(xd)
    base = binding.fp32(wd, m, k, q, ds_rows)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    if n > 64:
        assert np.array_equal(got.view(np.uint32), base.cpu().numpy().view(np.uint32))
    toks = sample_tokens(n, 24)
    rq, rds = oracle.quantize(x[toks])
    check_fp32(got[toks], oracle.out_f64(w, m, k, rq, rds), "tiles fold")


def test_tiles_qproj_full():
    """The 7B q-proj prefill through the tiles, on both weight layouts: bit
    for bit the int8-activation path's result."""
    f, x = synth.qproj_inputs()
    m, k = f.q.shape
    note("tiles q-proj full n=%d" % x.shape[0])
    wd = to_dev(synth.pack_q4k(f))
    xd = to_dev(x)
    qt, ds = binding.quantize_tiled(xd)
    got = binding.fp32_tiles(wd, m, k, qt, ds)
    got_r = binding.fp32_tiles(binding.repack(wd, m, k), m, k, qt, ds, repacked=True)
    q, ds_rows = binding.quantize(xd)
    base = binding.fp32(wd, m, k, q, ds_rows)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), base.view(torch.int32))
    assert torch.equal(got_r.view(torch.int32), base.view(torch.int32))


# q6_K on the same tiles: 9 tokens and more take the binary16 kernel on both
# sides (bitwise equal); one token checks the bar only.
@pytest.mark.parametrize("n,m,k", [(1, 33, 512), (9, 40, 768), (65, 129, 512), (300, 200, 2304),
                                   (200, 40, 16640), (1100, 4096, 512)])
def test_q6k_tiles_fold(n, m, k):
    note("q6k tiles fold n=%d m=%d k=%d" % (n, m, k))
    f = synth.random_q6k_fields(930 + n, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(930 + n, n, k, "outliers")
    w = synth.pack_q6k(f)
    wd = to_dev(w)
    xd = to_dev(x)
    qt, ds = binding.quantize_tiled(xd)
    got = binding.q6k_fp32_tiles(wd, m, k, qt, ds)
    q, ds_rows = binding.quantize(xd)
    base = binding.q6k_fp32(wd, m, k, q, ds_rows)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    if n > 8:
        assert np.array_equal(got.view(np.uint32), base.cpu().numpy().view(np.uint32))
    toks = sample_tokens(n, 24)
    rq, rds = oracle.quantize(x[toks])
    check_fp32(got[toks], oracle.q6k_out_f64(w, m, k, rq, rds), "q6k tiles fold")
