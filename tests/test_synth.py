"""The seeded input generators: determinism, shapes, value ranges, structure."""
import numpy as np

from q4_q8_integer_amd import synth


def test_streams_are_deterministic_and_distinct():
    a = synth.random_fields(3, 4, 256)
    b = synth.random_fields(3, 4, 256)
    c = synth.random_fields(4, 4, 256)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.d, b.d)
    assert not np.array_equal(a.q, c.q)


def test_tiny_workload_fields():
    f, x = synth.tiny_inputs()
    assert f.q.shape == (256, 512) and x.shape == (64, 512) and x.dtype == np.float32
    assert f.q.max() == 15 and f.q.min() == 0
    assert f.sc.max() == 63 and f.mn.max() == 63
    assert f.d.dtype == np.float16 and (f.d >= 0).all()
    w = synth.pack_q4k(f)
    assert w.shape == (256, 2 * 144) and w.dtype == np.uint8


def test_sc_zero_mask_fraction():
    f = synth.random_fields(5, 512, 1024, sc_zero_frac=0.1)
    frac = (f.sc == 0).mean()
    assert 0.09 < frac < 0.12          # 10% forced + 1/64 natural zeros


def test_outlier_and_silu_structure():
    x = synth.random_activations(1, 64, 4096, "outliers")
    assert (np.abs(x) > 8).mean() > 0.004    # N(0,1) alone almost never exceeds 8
    s = synth.random_activations(1, 64, 4096, "silu")
    assert s.min() > -0.2785 and s.dtype == np.float32   # SiLU minimum is about -0.2785


def test_layer_and_weight_bound_shapes():
    x = synth.layer_activation("down_in", 512)
    assert x.shape == (512, 11008)
    x = synth.weight_bound_activation("wide_out", 7)
    assert x.shape == (7, 28672)


def test_q6k_fields_and_block_bytes():
    f = synth.random_q6k_fields(7, 64, 768, sc_zero_frac=0.1)
    assert f.q.min() == 0 and f.q.max() == 63
    assert f.sc.dtype == np.int8 and f.sc.min() == -128 and f.sc.max() == 127
    assert 0.09 < (f.sc == 0).mean() < 0.12
    assert f.d.dtype == np.float16 and (f.d >= 0).all()
    w = synth.pack_q6k(f)
    assert w.shape == (64, 3 * 210) and w.dtype == np.uint8
    # scales and d sit at fixed offsets of each 210-byte block
    blk = w.reshape(64, 3, 210)
    assert np.array_equal(blk[:, :, 192:208].view(np.int8).reshape(64, 48), f.sc)
    assert np.array_equal(blk[:, :, 208:210].copy().view("<f2").reshape(64, 3), f.d)


def test_q6k_workload_shapes():
    x = synth.q6k_activation("wide_in", 1)
    assert x.shape == (1, 8192) and x.dtype == np.float32
    assert np.array_equal(x, synth.q6k_activation("wide_in", 1))
