"""mmq_q4k_q8 (exact int32 block dots) and mmq_q4k_q8_fp32out on the GPU
against the oracle: bit-exact dots, the float32 bar on every workload (full
sizes, launched exactly as the benchmark launches them, with sampled tokens
checked), ragged shapes, and metamorphic properties."""
import numpy as np
import pytest
import torch

import oracle
import pins
from gpu_helpers import check_fp32, gpu_quantize, host_ds, note, sample_tokens, to_dev
from q4_q8_integer_amd import binding, synth

pytestmark = pytest.mark.gpu


def gpu_dots(w, m, k, q):
    d = binding.blockdots(w, m, k, q)
    torch.cuda.synchronize()
    return d.cpu().numpy()


def gpu_fp32(w, m, k, q, ds):
    o = binding.fp32(w, m, k, q, ds)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def run_case(f, x, what, dots=True):
    """Full comparison for a shape small enough for the oracle."""
    m, k = f.q.shape
    note("mmq: %s n=%d m=%d k=%d" % (what, x.shape[0], m, k))
    w = synth.pack_q4k(f)
    wg = to_dev(w)
    q, ds = gpu_quantize(x)
    rq, rds = oracle.quantize(x)
    assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(host_ds(ds), rds)
    if dots:
        got = gpu_dots(wg, m, k, q)
        ref = oracle.blockdots(w, m, k, rq)
        assert np.array_equal(got, ref), "%s: block dots differ at %d places" % (
            what, int((got != ref).sum()))
    check_fp32(gpu_fp32(wg, m, k, q, ds), oracle.out_f64(w, m, k, rq, rds), what)


def test_tiny():
    f, x = synth.tiny_inputs()
    run_case(f, x, "tiny")


@pytest.mark.parametrize("n,m,k", [(1, 1, 256), (3, 33, 256), (77, 200, 768), (130, 129, 512),
                                   (129, 256, 1024), (5, 131, 2304), (64, 127, 256)])
def test_ragged_shapes(n, m, k):
    f = synth.random_fields(n * 7 + m, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(n * 7 + m, n, k, "outliers")
    run_case(f, x, "ragged")


@pytest.mark.parametrize("k", [2304, 16640])
@pytest.mark.parametrize("n", range(1, 9))
def test_few_token_weight_layouts(n, k):
    """Every token count of the dot4 kernel on both sides of its layout
    choices: 9 super-blocks per row (weights staged through one LDS area up
    to 5 tokens, loaded into registers from 6) and 65 (staged with the next
    step in flight up to 6 tokens: 4 waves of 16-17 super-blocks, so each
    wave's last step runs past its range and the last row's past the
    matrix).  40 rows leave a half tile.  The dot4 result also equals the
    repacked-layout path bit for bit (same summation order); the entry
    point's own choice (the narrow kernel at 6-8 tokens on these 40 rows)
    meets the same bar."""
    m = 40
    note("few-token layouts n=%d m=%d k=%d" % (n, m, k))
    f = synth.random_fields(700 + 10 * n + k % 7, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(700 + 10 * n + k % 7, n, k, "outliers")
    w = synth.pack_q4k(f)
    wd = to_dev(w)
    q, ds = gpu_quantize(x)
    dot4 = binding.fold_kernel(wd, m, k, q, ds, binding.KERNEL_DOT4)
    auto = binding.fp32(wd, m, k, q, ds)
    rep = binding.fp32_repacked(binding.repack(wd, m, k), m, k, q, ds)
    torch.cuda.synchronize()
    dot4 = dot4.cpu().numpy()
    assert np.array_equal(dot4.view(np.uint32), rep.cpu().numpy().view(np.uint32))
    rq, rds = oracle.quantize(x)
    ref = oracle.out_f64(w, m, k, rq, rds)
    check_fp32(dot4, ref, "few-token layouts")
    check_fp32(auto.cpu().numpy(), ref, "few-token auto choice")


@pytest.mark.parametrize("k", [2304, 16640])
@pytest.mark.parametrize("n", [9, 13, 16])
def test_one_tile_mfma_kernel(n, k):
    """9-16 tokens (one 16-token tile of the few-token MFMA path) with 9
    super-blocks per row (one copy area per wave) and 65 (the next step's
    copies in flight; 16-17 per wave); 37 rows leave a 5-row tile."""
    f = synth.random_fields(760 + n + k % 7, 37, k, sc_zero_frac=0.1)
    x = synth.random_activations(760 + n + k % 7, n, k, "outliers")
    run_case(f, x, "one-tile MFMA")


def test_hand_worked_superblock():
    f, x, dots, ssum, out = pins.golden_one_superblock()
    wg = to_dev(synth.pack_q4k(f))
    q, ds = gpu_quantize(x)
    assert np.array_equal(gpu_dots(wg, 1, 256, q)[0, 0], dots)
    assert gpu_fp32(wg, 1, 256, q, ds)[0, 0] == np.float32(out)


# ------------------------------------------------------- full-size workloads
def sampled_check(f, x, what, w=None, count=48, dots_rows=160):
    """Run the GPU path at full size; check sampled tokens x all rows in fp32,
    and exact dots for a window of rows at the real K."""
    m, k = f.q.shape
    n = x.shape[0]
    note("mmq full: %s n=%d m=%d k=%d" % (what, n, m, k))
    w = synth.pack_q4k(f) if w is None else w
    wg = to_dev(w)
    xg = to_dev(x)
    q, ds = binding.quantize(xg)
    out = binding.fp32(wg, m, k, q, ds)
    torch.cuda.synchronize()
    toks = sample_tokens(n, count)
    rq, rds = oracle.quantize(x[toks])
    assert np.array_equal(q[torch.from_numpy(toks).to(q.device)].cpu().numpy(), rq)
    ref = oracle.out_f64(w, m, k, rq, rds)
    got = out[torch.from_numpy(toks).to(out.device)].cpu().numpy()
    check_fp32(got, ref, what)
    if dots_rows:
        rows = np.r_[0:min(dots_rows, m) - 32, m - 32:m]
        wsub = np.ascontiguousarray(w[rows])
        tq = q[torch.from_numpy(toks[:24]).to(q.device)].contiguous()
        got = gpu_dots(to_dev(wsub), len(rows), k, tq)
        assert np.array_equal(got, oracle.blockdots(wsub, len(rows), k, rq[:24])), what + " dots"
    del wg, xg, q, ds, out
    torch.cuda.empty_cache()


def test_qproj_full():
    f, x = synth.qproj_inputs()
    sampled_check(f, x, "7B q-proj N=2630")


@pytest.mark.parametrize("which", ["gate", "up", "down"])
def test_ffn_full(which):
    f = synth.ffn_inputs(which)
    x = synth.ffn_inputs("x_down" if which == "down" else "x")
    sampled_check(f, x, "7B FFN %s N=2630" % which)


@pytest.mark.parametrize("n", [512, 2048, 8192])
def test_layer_set(n):
    inputs = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "o_in",
              "gate": "ffn_in", "up": "ffn_in", "down": "down_in"}
    cache = {}
    for name in ("q", "k", "v", "o", "gate", "up", "down"):
        src = inputs[name]
        if src not in cache:
            cache[src] = synth.layer_activation(src, n)
        sampled_check(synth.layer_weights(name), cache[src], "layer %s N=%d" % (name, n),
                      count=24 if n == 8192 else 32, dots_rows=96 if name in ("q", "down") else 0)


@pytest.mark.parametrize("name", ["wide_in", "wide_out"])
@pytest.mark.parametrize("n", [1, 7, 33, 2051])
def test_weight_bound(name, n):
    f = synth.weight_bound_weights(name)
    x = synth.weight_bound_activation(name, n)
    sampled_check(f, x, "weight-bound %s N=%d" % (name, n), count=16 if n > 33 else n,
                  dots_rows=96)


# ------------------------------------------------------------- metamorphic
@pytest.mark.parametrize("n", [1, 4, 7, 9, 16, 33, 130])
def test_negative_super_block_scales(n):
    """d and dmin are signed binary16 fields: with the sign set on a random
    half of each, every kernel (dot4, the few-token MFMA kernels, the binary16
    kernel) on every weight layout and activation format meets the float32
    bar against the oracle."""
    m, k = 40, 768
    note("negative scales n=%d" % n)
    f = synth.random_fields(970 + n, m, k, sc_zero_frac=0.1)
    rng = np.random.default_rng([970, n])
    f.d = np.where(rng.random(f.d.shape) < 0.5, -f.d, f.d).astype(np.float16)
    f.dmin = np.where(rng.random(f.dmin.shape) < 0.5, -f.dmin, f.dmin).astype(np.float16)
    assert (f.d < 0).any() and (f.dmin < 0).any()
    x = synth.random_activations(970 + n, n, k, "outliers")
    w = synth.pack_q4k(f)
    wd = to_dev(w)
    q, ds = gpu_quantize(x)
    rq, rds = oracle.quantize(x)
    ref = oracle.out_f64(w, m, k, rq, rds)
    check_fp32(gpu_fp32(wd, m, k, q, ds), ref, "negative scales, q4_K rows")
    wr = binding.repack(wd, m, k)
    got_r = binding.fp32_repacked(wr, m, k, q, ds)
    qt, dst = binding.quantize_tiled(to_dev(x))
    got_t = binding.fp32_tiles(wd, m, k, qt, dst)
    torch.cuda.synchronize()
    check_fp32(got_r.cpu().numpy(), ref, "negative scales, repacked")
    check_fp32(got_t.cpu().numpy(), ref, "negative scales, operand tiles")
    # q6_K: d is a signed binary16 field as well (its 8-bit scales are signed
    # already)
    f6 = synth.random_q6k_fields(970 + n, m, k, sc_zero_frac=0.1)
    f6.d = np.where(rng.random(f6.d.shape) < 0.5, -f6.d, f6.d).astype(np.float16)
    w6 = synth.pack_q6k(f6)
    w6d = to_dev(w6)
    ref6 = oracle.q6k_out_f64(w6, m, k, rq, rds)
    got6 = binding.q6k_fp32(w6d, m, k, q, ds)
    got6t = binding.q6k_fp32_tiles(w6d, m, k, qt, dst)
    torch.cuda.synchronize()
    check_fp32(got6.cpu().numpy(), ref6, "negative scales, q6_K")
    check_fp32(got6t.cpu().numpy(), ref6, "negative scales, q6_K on operand tiles")


def test_run_to_run_and_token_slice_bitwise():
    f = synth.random_fields(61, 300, 1024)
    x = synth.random_activations(61, 200, 1024)
    wg = to_dev(synth.pack_q4k(f))
    q, ds = gpu_quantize(x)
    a = gpu_fp32(wg, 300, 1024, q, ds)
    b = gpu_fp32(wg, 300, 1024, q, ds)
    assert np.array_equal(a, b)
    s = gpu_fp32(wg, 300, 1024, q[37:151].contiguous(), ds[37:151].contiguous())
    assert np.array_equal(a[37:151], s)
    d1 = gpu_dots(wg, 300, 1024, q)
    d2 = gpu_dots(wg, 300, 1024, q[37:151].contiguous())
    assert np.array_equal(d1[37:151], d2)


def test_zero_scale_subblock_nibbles_do_not_matter():
    """With sc = 0 the main term of that sub-block is exactly 0, so its nibbles
    cannot change the float32 output at all."""
    f = synth.random_fields(62, 96, 512, sc_zero_frac=0.25)
    x = synth.random_activations(62, 40, 512)
    q, ds = gpu_quantize(x)
    base = gpu_fp32(to_dev(synth.pack_q4k(f)), 96, 512, q, ds)
    zero = np.repeat(f.sc == 0, 32, axis=1)
    f.q[zero] = (f.q[zero] + 5) % 16
    assert np.array_equal(base, gpu_fp32(to_dev(synth.pack_q4k(f)), 96, 512, q, ds))


def test_outputs_fully_written_and_guard_bands_untouched():
    n, m, k = 70, 100, 512
    f = synth.random_fields(63, m, k)
    x = synth.random_activations(63, n, k)
    wg = to_dev(synth.pack_q4k(f))
    q, ds = gpu_quantize(x)
    pad = 64
    buf = torch.full((n * m + 2 * pad,), float("nan"), dtype=torch.float32, device=q.device)
    buf[:pad] = 12345.0
    buf[-pad:] = -6789.0
    out = buf[pad:pad + n * m].view(n, m)
    binding.mmq_q4k_q8_fp32out(wg, m, k, q, ds, n, out)
    dbuf = torch.full((n * m * (k // 32) + 2 * pad,), -77, dtype=torch.int32, device=q.device)
    dots = dbuf[pad:pad + n * m * (k // 32)]
    binding.mmq_q4k_q8(wg, m, k, q, ds, n, dots)
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert not np.isnan(h[pad:-pad]).any()
    assert (h[:pad] == 12345.0).all() and (h[-pad:] == -6789.0).all()
    hd = dbuf.cpu().numpy()
    assert (hd[:pad] == -77).all() and (hd[-pad:] == -77).all()
    rq, rds = oracle.quantize(x)
    w = synth.pack_q4k(f)
    assert np.array_equal(hd[pad:-pad].reshape(n, m, k // 32), oracle.blockdots(w, m, k, rq))


def test_empty_calls_touch_nothing():
    q = torch.zeros((0, 256), dtype=torch.int8, device="cuda:0")
    ds = torch.zeros((0, 8), dtype=torch.int32, device="cuda:0")
    w = torch.zeros((4, 144), dtype=torch.uint8, device="cuda:0")
    out = binding.fp32(w, 4, 256, q, ds)
    assert out.shape == (0, 4)
    binding.q8_quantize_rows(torch.zeros((0, 64), device="cuda:0"), 0, 64, q, ds)
