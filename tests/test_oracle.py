"""The CPU oracle against what the pages, the mathematics and library routines
fix (see pins.py for what each pin checks)."""
import numpy as np
import pytest

import oracle
import pins
from q4_q8_integer_amd import synth


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_token_slice_invariance(lib):
    """Rows of the output do not depend on which other tokens are in the call."""
    f, x = synth.tiny_inputs()
    q, ds = oracle.quantize(x)
    qs, dss = oracle.quantize(x[17:29])
    assert np.array_equal(q[17:29], qs) and np.array_equal(ds[17:29], dss)
    w = synth.pack_q4k(f)
    assert np.array_equal(oracle.out_f64(w, 256, 512, q, ds)[17:29],
                          oracle.out_f64(w, 256, 512, qs, dss))


def test_thread_count_does_not_change_results(lib):
    f, x = synth.tiny_inputs()
    q, ds = oracle.quantize(x)
    w = synth.pack_q4k(f)
    nt = oracle.get_threads()
    oracle.set_threads(1)
    a = oracle.out_f64(w, 256, 512, q, ds)
    oracle.set_threads(max(2, nt))
    b = oracle.out_f64(w, 256, 512, q, ds)
    oracle.set_threads(nt)
    assert np.array_equal(a, b)


def test_rejects_bad_shapes(lib):
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 33), dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.out_f64(np.zeros((1, 144), np.uint8), 1, 300, np.zeros((1, 300), np.int8),
                       np.zeros((1, 9), np.uint32))
