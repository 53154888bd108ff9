"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` function takes an oracle library handle and raises
AssertionError when the oracle disagrees with what the pages, the mathematics
or a library routine fixes.  ``test_oracle.py`` runs them on the oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes and expects each mistake to fail at least one of them.

Independent references used here (none calls the oracle's own helpers):
* numpy's IEEE binary16 conversions and float32 division;
* numpy float64 / int64 matrix products on dequantized values built from the
  generator's unpacked fields (never from the oracle's byte decoder);
* hand-derived fixtures under ``tests/golden/``;
* closed forms and invariants of the definition.
"""
from __future__ import annotations

import os

import numpy as np

import oracle
from q4_q8_integer_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ readers
def read_kv(name):
    """Parse a golden file of ``key: value`` / ``key = value`` lines."""
    out, blocks, cur = {}, {}, None
    with open(os.path.join(GOLDEN, name)) as fh:
        for raw in fh:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("block "):
                cur = blocks.setdefault(line.split()[1], {})
                continue
            sep = ":" if ":" in line else "="
            key, val = (s.strip() for s in line.split(sep, 1))
            (cur if cur is not None else out)[key] = val
    return out, blocks


def golden_q4k_block():
    kv, _ = read_kv("q4k_block.txt")
    sc = np.array([int(v) for v in kv["sc"].split()], dtype=np.uint8)
    mn = np.array([int(v) for v in kv["m"].split()], dtype=np.uint8)
    e = np.arange(256)
    q = ((2 * (e // 32) + (e % 32)) % 16).astype(np.uint8)
    f = synth.Q4KFields(
        q=q[None, :], sc=sc[None, :], mn=mn[None, :],
        d=np.array([[int(kv["d_f16"], 16)]], dtype=np.uint16).view(np.float16),
        dmin=np.array([[int(kv["dmin_f16"], 16)]], dtype=np.uint16).view(np.float16))
    expected = {int(k): int(v, 16) for k, v in kv.items() if k.isdigit()}
    return f, expected


def golden_q8_blocks():
    _, blocks = read_kv("q8_blocks.txt")
    out = {}
    for name, b in blocks.items():
        x = np.zeros(32, dtype=np.float32)
        q = np.zeros(32, dtype=np.int8)
        for tok in b.get("x", "").split():
            i, v = tok.split("=")
            x[int(i)] = np.float32(v)
        for tok in b.get("q", "").split():
            i, v = tok.split("=")
            q[int(i)] = int(v)
        out[name] = (x, q, int(b["ssum"]), int(b["word"], 16))
    return out


def golden_one_superblock():
    kv, _ = read_kv("one_superblock.txt")
    f, _ = golden_q4k_block()
    x = np.zeros((1, 256), dtype=np.float32)
    for c in range(8):
        x[0, 32 * c] = 127.0
        x[0, 32 * c + 1] = -(c + 1)
    dots = np.array([int(v) for v in kv["dots"].split()], dtype=np.int32)
    ssum = np.array([int(v) for v in kv["ssum"].split()], dtype=np.int32)
    return f, x, dots, ssum, float(kv["out"])


# ---------------------------------------------------- independent references
def deq_weights(f: synth.Q4KFields) -> np.ndarray:
    """d*sc*q - dmin*m in float64 from the generator's unpacked fields."""
    d = f.d.astype(np.float64).repeat(256, axis=1)
    dmin = f.dmin.astype(np.float64).repeat(256, axis=1)
    sc = f.sc.astype(np.float64).repeat(32, axis=1)
    mn = f.mn.astype(np.float64).repeat(32, axis=1)
    return d * sc * f.q.astype(np.float64) - dmin * mn


def deq_acts(q: np.ndarray, ds: np.ndarray) -> np.ndarray:
    """da16*q8 in float64 with da16 decoded by numpy's binary16."""
    da = (ds & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    return q.astype(np.float64) * da.repeat(32, axis=1)


def brute_dots(f: synth.Q4KFields, q8: np.ndarray) -> np.ndarray:
    """int64 per-32 block dots from the unpacked nibbles: [n, m, k/32]."""
    m, k = f.q.shape
    a = f.q.astype(np.int64).reshape(m, k // 32, 32)
    b = q8.astype(np.int64).reshape(q8.shape[0], k // 32, 32)
    return np.einsum("oci,tci->toc", a, b)


def ssum_of(ds):
    return ((ds >> 16) & 0xFFFF).astype(np.uint16).view(np.int16).astype(np.int64)


# --------------------------------------------------------------------- pins
def pin_f16_encode(lib):
    """Binary16 rounding (nearest, ties to even, subnormals kept) = numpy's."""
    rng = np.random.default_rng(7)
    mant = rng.random(3000) + 1.0
    expo = rng.integers(-30, 17, 3000)
    vals = (mant * np.exp2(expo)).astype(np.float32)
    # exact binary16 midpoints (ties) in normal and subnormal ranges
    grid = np.arange(1, 2047, dtype=np.float64)
    ties = np.concatenate([(grid + 0.5) * 2.0**-24, (1024 + grid[:1000] + 0.5) * 2.0**-13,
                           (1024 + grid[:1000] + 0.5) * 2.0**-5]).astype(np.float32)
    vals = np.concatenate([vals, -vals, ties, -ties,
                           np.array([0.0, -0.0, 65504.0, 65519.0, 65520.0, 1e6, 6.0e-8,
                                     2.9e-8, 3.0e-8], dtype=np.float32)])
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    got = np.array([lib.oracle_f32_to_f16(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "f16 encode differs at %r" % (vals[bad[:5]],)


def pin_f16_decode(lib):
    """Binary16 decoding of every finite bit pattern = numpy's."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    got = np.array([lib.oracle_f16_to_double(int(b)) for b in bits[fin]])
    assert np.array_equal(got, ref[fin])


def pin_q4k_golden_block(lib):
    """Unpacking the hand-derived block gives back the hand-chosen fields."""
    f, expected = golden_q4k_block()
    w = synth.pack_q4k(f)
    for off, byte in expected.items():
        assert w[0, off] == byte, "packer byte %d: %02x != %02x" % (off, w[0, off], byte)
    u = oracle.q4k_unpack(w, 1, 256, lib=lib)
    assert np.array_equal(u["q"], f.q)
    assert np.array_equal(u["sc"], f.sc)
    assert np.array_equal(u["mn"], f.mn)
    assert np.array_equal(u["d"].view(np.uint16), f.d.view(np.uint16))
    assert np.array_equal(u["dmin"].view(np.uint16), f.dmin.view(np.uint16))


def pin_q4k_roundtrip(lib):
    """Unpack(pack(fields)) == fields on random matrices."""
    for seed, (m, k) in enumerate([(3, 256), (5, 512), (2, 1024)]):
        f = synth.random_fields(seed, m, k)
        u = oracle.q4k_unpack(synth.pack_q4k(f), m, k, lib=lib)
        for name in ("q", "sc", "mn"):
            assert np.array_equal(u[name], getattr(f, name)), name
        assert np.array_equal(u["d"].view(np.uint16), f.d.view(np.uint16))
        assert np.array_equal(u["dmin"].view(np.uint16), f.dmin.view(np.uint16))


def pin_q8_golden(lib):
    """Hand-derived q8 blocks (ties, negative ssum, zero block, non-exact da)."""
    for name, (x, q, ssum, word) in golden_q8_blocks().items():
        gq, gds = oracle.quantize(x[None, :], lib=lib)
        assert np.array_equal(gq[0], q), "block %s q" % name
        assert int(gds[0, 0]) == word, "block %s word %08x != %08x" % (name, gds[0, 0], word)
        assert int(ssum_of(gds)[0, 0]) == ssum


def pin_q8_invariants(lib):
    """On N(0,1), x20-outlier and SiLU data: |q| <= 127; ssum = sum q; the
    largest |x| maps to |q| = 127; the scale is binary16(fp32(amax)/127); every
    q is the nearest integer to fp32(x)/fp32(da) with ties away from zero."""
    for kind in ("normal", "outliers", "silu"):
        x = synth.random_activations(3, 24, 1024, kind)
        q, ds = oracle.quantize(x, lib=lib)
        xb = x.reshape(24, 32, 32)
        qb = q.reshape(24, 32, 32).astype(np.int64)
        assert np.abs(qb).max() <= 127
        assert np.array_equal(qb.sum(axis=2), ssum_of(ds))
        amax = np.abs(xb).max(axis=2)
        da32 = amax.astype(np.float32) / np.float32(127.0)
        assert np.array_equal((ds & 0xFFFF).astype(np.uint16), da32.astype(np.float16).view(np.uint16))
        arg = np.abs(xb).argmax(axis=2)
        assert np.all(np.abs(np.take_along_axis(qb, arg[..., None], 2)) == 127)
        r = (xb / da32[..., None]).astype(np.float64)  # numpy fp32 divide
        err = np.abs(r - qb)
        assert err.max() <= 0.5
        tie = err == 0.5
        assert np.all(np.abs(qb[tie]) > np.abs(r[tie]))


def pin_q8_zero_block(lib):
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 40] = -3.0
    q, ds = oracle.quantize(x, lib=lib)
    assert not q[0].any() and ds[0, 0] == 0 and ds[0, 1] == 0 and ds[1, 0] == 0
    assert q[1, 40] == -127


def pin_dots_bruteforce(lib):
    """Block dots = int64 dot products over the generator's unpacked nibbles."""
    for seed, (n, m, k) in enumerate([(3, 4, 256), (5, 7, 512), (1, 1, 768), (9, 2, 256)]):
        f = synth.random_fields(10 + seed, m, k)
        x = synth.random_activations(10 + seed, n, k)
        q, _ = oracle.quantize(x, lib=lib)
        got = oracle.blockdots(synth.pack_q4k(f), m, k, q, lib=lib)
        assert np.array_equal(got, brute_dots(f, q))


def pin_dots_closed_forms(lib):
    """q4 = 15 with q8 = 127 gives 15*127*32 = 60960; q4 = const k gives
    k*ssum; q8 = 0 gives 0."""
    f = synth.random_fields(20, 3, 256)
    f.q[:] = 15
    x = np.full((2, 256), 5.0, dtype=np.float32)
    q, _ = oracle.quantize(x, lib=lib)
    assert (q == 127).all()
    assert (oracle.blockdots(synth.pack_q4k(f), 3, 256, q, lib=lib) == 60960).all()
    x = synth.random_activations(21, 4, 256)
    q, ds = oracle.quantize(x, lib=lib)
    for kc in (0, 1, 9):
        f.q[:] = kc
        got = oracle.blockdots(synth.pack_q4k(f), 3, 256, q, lib=lib)
        assert np.array_equal(got, np.broadcast_to(kc * ssum_of(ds)[:, None, :], got.shape))
    f = synth.random_fields(22, 3, 256)
    q0 = np.zeros((2, 256), dtype=np.int8)
    assert not oracle.blockdots(synth.pack_q4k(f), 3, 256, q0, lib=lib).any()


def pin_out_bruteforce(lib):
    """fp64 output = numpy float64 matmul of the dequantized operands (the two
    forms are algebraically equal; every product is exact in float64)."""
    cases = [(64, 256, 512)] + [(1 + 3 * s, 1 + 5 * s, 256 * (1 + s % 3)) for s in range(12)]
    for seed, (n, m, k) in enumerate(cases):
        if seed == 0:
            f, x = synth.tiny_inputs()
        else:
            f = synth.random_fields(30 + seed, m, k, sc_zero_frac=0.1 * (seed % 2))
            x = synth.random_activations(30 + seed, n, k, ("normal", "outliers", "silu")[seed % 3])
        q, ds = oracle.quantize(x, lib=lib)
        got = oracle.out_f64(synth.pack_q4k(f), m, k, q, ds, lib=lib)
        ref = deq_acts(q, ds) @ deq_weights(f).T
        scale = np.abs(ref).max()
        assert np.abs(got - ref).max() <= 1e-12 * scale, "case %d" % seed


def pin_out_negative_scales(lib):
    """The super-block scales d and dmin are signed binary16 fields: with the
    sign set on a random half of each, the fp64 output still equals the numpy
    float64 matmul of the dequantized operands."""
    for seed, (n, m, k) in enumerate([(5, 9, 512), (33, 17, 768)]):
        f = synth.random_fields(60 + seed, m, k, sc_zero_frac=0.1)
        rng = np.random.default_rng([60, seed])
        f.d = np.where(rng.random(f.d.shape) < 0.5, -f.d, f.d).astype(np.float16)
        f.dmin = np.where(rng.random(f.dmin.shape) < 0.5, -f.dmin, f.dmin).astype(np.float16)
        assert (f.d < 0).any() and (f.dmin < 0).any()
        x = synth.random_activations(60 + seed, n, k, "outliers")
        q, ds = oracle.quantize(x, lib=lib)
        got = oracle.out_f64(synth.pack_q4k(f), m, k, q, ds, lib=lib)
        ref = deq_acts(q, ds) @ deq_weights(f).T
        assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max(), "case %d" % seed


def pin_out_special_cases(lib):
    """q4 = 0 leaves only the min term; m = 0 leaves only the main term;
    d = dmin = 0 gives exactly 0."""
    n, m, k = 5, 6, 512
    x = synth.random_activations(40, n, k)
    q, ds = oracle.quantize(x, lib=lib)
    da = (ds & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    f = synth.random_fields(40, m, k)
    f.q[:] = 0
    got = oracle.out_f64(synth.pack_q4k(f), m, k, q, ds, lib=lib)
    dmm = f.dmin.astype(np.float64).repeat(8, axis=1) * f.mn
    ref = -(da * ssum_of(ds)) @ dmm.T
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    f = synth.random_fields(41, m, k)
    f.mn[:] = 0
    got = oracle.out_f64(synth.pack_q4k(f), m, k, q, ds, lib=lib)
    w = f.d.astype(np.float64).repeat(256, axis=1) * f.sc.astype(np.float64).repeat(32, axis=1) * f.q
    ref = deq_acts(q, ds) @ w.T
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    f.d[:] = 0
    f.dmin[:] = 0
    assert not oracle.out_f64(synth.pack_q4k(f), m, k, q, ds, lib=lib).any()


def pin_out_zero_scale_block(lib):
    """A sub-block with sc = m = 0 contributes exactly 0: scrambling its
    nibbles leaves the output bit-identical, and so does zeroing them."""
    n, m, k = 4, 5, 512
    f = synth.random_fields(50, m, k)
    x = synth.random_activations(50, n, k)
    q, ds = oracle.quantize(x, lib=lib)
    f.sc[:, 3] = 0
    f.mn[:, 3] = 0
    base = oracle.out_f64(synth.pack_q4k(f), m, k, q, ds, lib=lib)
    f.q[:, 96:128] = (f.q[:, 96:128] + 7) % 16
    assert np.array_equal(base, oracle.out_f64(synth.pack_q4k(f), m, k, q, ds, lib=lib))
    f.q[:, 96:128] = 0
    assert np.array_equal(base, oracle.out_f64(synth.pack_q4k(f), m, k, q, ds, lib=lib))


def pin_one_superblock(lib):
    """The hand-worked single super-block example."""
    f, x, dots, ssum, out = golden_one_superblock()
    q, ds = oracle.quantize(x, lib=lib)
    assert np.array_equal(ssum_of(ds)[0], ssum)
    w = synth.pack_q4k(f)
    assert np.array_equal(oracle.blockdots(w, 1, 256, q, lib=lib)[0, 0], dots)
    assert oracle.out_f64(w, 1, 256, q, ds, lib=lib)[0, 0] == out


# ------------------------------------------------------------------ q6_K
def golden_q6k_block():
    kv, _ = read_kv("q6k_block.txt")
    sc = np.array([int(v) for v in kv["sc"].split()], dtype=np.int8)
    e = np.arange(256)
    h, g, l = e // 128, (e // 32) % 4, e % 32
    q = ((3 * l + 7 * g + 11 * h) % 64).astype(np.uint8)
    f = synth.Q6KFields(q=q[None, :], sc=sc[None, :],
                        d=np.array([[int(kv["d_f16"], 16)]], dtype=np.uint16).view(np.float16))
    expected = {int(k): int(v, 16) for k, v in kv.items() if k.isdigit()}
    return f, expected


def golden_q6k_one_superblock():
    kv, _ = read_kv("q6k_one_superblock.txt")
    f, _ = golden_q6k_block()
    x = np.zeros((1, 256), dtype=np.float32)
    for j in range(16):
        x[0, 16 * j] = 127.0
        x[0, 16 * j + 1] = -(j + 1)
    dots = np.array([int(v) for v in kv["dots"].split()], dtype=np.int32)
    return f, x, dots, float(kv["out"])


def deq_q6k_weights(f: synth.Q6KFields) -> np.ndarray:
    """d*sc*(q - 32) in float64 from the generator's unpacked fields."""
    d = f.d.astype(np.float64).repeat(256, axis=1)
    sc = f.sc.astype(np.float64).repeat(16, axis=1)
    return d * sc * (f.q.astype(np.float64) - 32.0)


def brute_q6k_dots(f: synth.Q6KFields, q8: np.ndarray) -> np.ndarray:
    """int64 per-16 group dots of the offset codes: [n, m, k/16]."""
    m, k = f.q.shape
    a = f.q.astype(np.int64).reshape(m, k // 16, 16) - 32
    b = q8.astype(np.int64).reshape(q8.shape[0], k // 16, 16)
    return np.einsum("ogi,tgi->tog", a, b)


def pin_q6k_golden_block(lib):
    """Packing the hand-chosen fields gives the hand-derived bytes, and the
    oracle's decoder gives the fields back."""
    f, expected = golden_q6k_block()
    w = synth.pack_q6k(f)
    assert w.shape == (1, 210)
    for off, byte in expected.items():
        assert w[0, off] == byte, "packer byte %d: %02x != %02x" % (off, w[0, off], byte)
    u = oracle.q6k_unpack(w, 1, 256, lib=lib)
    assert np.array_equal(u["q"], f.q)
    assert np.array_equal(u["sc"], f.sc)
    assert np.array_equal(u["d"].view(np.uint16), f.d.view(np.uint16))


def pin_q6k_roundtrip(lib):
    """Unpack(pack(fields)) == fields on random matrices (odd super-block
    counts included, so blocks start at every alignment)."""
    for seed, (m, k) in enumerate([(3, 256), (5, 768), (2, 1024)]):
        f = synth.random_q6k_fields(seed, m, k)
        u = oracle.q6k_unpack(synth.pack_q6k(f), m, k, lib=lib)
        assert np.array_equal(u["q"], f.q)
        assert np.array_equal(u["sc"], f.sc)
        assert np.array_equal(u["d"].view(np.uint16), f.d.view(np.uint16))


def pin_q6k_dots_bruteforce(lib):
    """Group dots = int64 dot products of (code - 32) with q8 from the
    generator's unpacked codes."""
    for seed, (n, m, k) in enumerate([(3, 4, 256), (5, 7, 512), (1, 1, 768), (9, 2, 256)]):
        f = synth.random_q6k_fields(10 + seed, m, k)
        x = synth.random_activations(60 + seed, n, k)
        q, _ = oracle.quantize(x, lib=lib)
        got = oracle.q6k_dots(synth.pack_q6k(f), m, k, q, lib=lib)
        assert np.array_equal(got, brute_q6k_dots(f, q))


def pin_q6k_dots_closed_forms(lib):
    """Code 32 (weight 0) gives 0; code 63 with q8 = 127 gives 31*127*16 =
    62992; code 0 with q8 = -127 gives 32*127*16 = 65024 (the largest
    magnitude); code c gives (c - 32) times the q8 sum over the 16 weights."""
    f = synth.random_q6k_fields(20, 3, 256)
    x = synth.random_activations(21, 4, 256, "outliers")
    q, _ = oracle.quantize(x, lib=lib)
    f.q[:] = 32
    assert not oracle.q6k_dots(synth.pack_q6k(f), 3, 256, q, lib=lib).any()
    s16 = q.astype(np.int64).reshape(4, 16, 16).sum(axis=2)
    for c in (0, 1, 31, 33, 63):
        f.q[:] = c
        got = oracle.q6k_dots(synth.pack_q6k(f), 3, 256, q, lib=lib)
        assert np.array_equal(got, np.broadcast_to((c - 32) * s16[:, None, :], got.shape))
    f.q[:] = 63
    qp = np.full((2, 256), 127, dtype=np.int8)
    assert (oracle.q6k_dots(synth.pack_q6k(f), 3, 256, qp, lib=lib) == 62992).all()
    f.q[:] = 0
    assert (oracle.q6k_dots(synth.pack_q6k(f), 3, 256, -qp, lib=lib) == 65024).all()


def pin_q6k_out_bruteforce(lib):
    """fp64 output = numpy float64 matmul of the dequantized operands."""
    cases = [(1 + 3 * s, 1 + 5 * s, 256 * (1 + s % 3)) for s in range(10)]
    for seed, (n, m, k) in enumerate(cases):
        f = synth.random_q6k_fields(30 + seed, m, k, sc_zero_frac=0.1 * (seed % 2))
        x = synth.random_activations(70 + seed, n, k, ("normal", "outliers", "silu")[seed % 3])
        q, ds = oracle.quantize(x, lib=lib)
        got = oracle.q6k_out_f64(synth.pack_q6k(f), m, k, q, ds, lib=lib)
        ref = deq_acts(q, ds) @ deq_q6k_weights(f).T
        scale = np.abs(ref).max()
        assert np.abs(got - ref).max() <= 1e-12 * scale, "case %d" % seed


def pin_q6k_out_special_cases(lib):
    """A group with sc = 0 contributes exactly 0 (scrambling its codes leaves
    the output bit-identical); negating every scale negates the output
    exactly; d = 0 or every code = 32 gives exactly 0."""
    n, m, k = 4, 5, 512
    f = synth.random_q6k_fields(50, m, k)
    f.sc[f.sc == -128] = -127
    x = synth.random_activations(50, n, k)
    q, ds = oracle.quantize(x, lib=lib)
    f.sc[:, 5] = 0
    base = oracle.q6k_out_f64(synth.pack_q6k(f), m, k, q, ds, lib=lib)
    f.q[:, 80:96] = (f.q[:, 80:96] + 29) % 64
    assert np.array_equal(base, oracle.q6k_out_f64(synth.pack_q6k(f), m, k, q, ds, lib=lib))
    neg = synth.Q6KFields(q=f.q, sc=-f.sc, d=f.d)
    assert np.array_equal(-base, oracle.q6k_out_f64(synth.pack_q6k(neg), m, k, q, ds, lib=lib))
    zero_d = synth.Q6KFields(q=f.q, sc=f.sc, d=np.zeros_like(f.d))
    assert not oracle.q6k_out_f64(synth.pack_q6k(zero_d), m, k, q, ds, lib=lib).any()
    mid = synth.Q6KFields(q=np.full_like(f.q, 32), sc=f.sc, d=f.d)
    assert not oracle.q6k_out_f64(synth.pack_q6k(mid), m, k, q, ds, lib=lib).any()


def pin_q6k_one_superblock(lib):
    """The hand-worked single q6_K super-block example."""
    f, x, dots, out = golden_q6k_one_superblock()
    q, ds = oracle.quantize(x, lib=lib)
    assert np.array_equal(q, x.astype(np.int8))
    w = synth.pack_q6k(f)
    assert np.array_equal(oracle.q6k_dots(w, 1, 256, q, lib=lib)[0, 0], dots)
    assert oracle.q6k_out_f64(w, 1, 256, q, ds, lib=lib)[0, 0] == out


# --------------------------------------------------- fused SiLU-gate quantize
def _gate_inputs(seed, n, k):
    rng = np.random.default_rng([950, seed])
    g = (rng.standard_normal((n, k)) * 3).astype(np.float32)
    u = rng.standard_normal((n, k)).astype(np.float32)
    g[0, :64] = np.linspace(-120, 120, 64, dtype=np.float32)   # saturated sigmoid both ways
    g[0, 64:96] = 0.0
    u[0, 96:128] = 0.0
    return g, u


def _silu_mul_f64(g, u):
    gd = g.astype(np.float64)
    return (gd * u.astype(np.float64) / (1.0 + np.exp(-gd))).astype(np.float32)


def pin_silu_mul_float64(lib):
    """h = float32 of g*u/(1 + exp(-g)) in float64: equal to numpy's float64
    evaluation (a different exp) on all but a vanishing fraction, and never
    more than one float32 ulp away."""
    g, u = _gate_inputs(1, 40, 4096)
    h = oracle.silu_mul(g, u, lib=lib)
    ref = _silu_mul_f64(g, u)
    diff = h != ref
    assert diff.mean() <= 1e-4, "h differs from the float64 definition at %d places" % diff.sum()
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(h.astype(np.float64) - ref) <= ulp)


def pin_silu_mul_closed_forms(lib):
    """g = 0 gives 0; g >= 40 gives float32(g*u) exactly (exp(-g) vanishes
    next to 1); g <= -800 gives 0; SiLU(g) - SiLU(-g) = g."""
    g = np.array([0.0, 40.0, 55.5, 1e4, -800.0, -1e4], dtype=np.float32)
    u = np.array([3.0, 1.5, -2.25, 7.0, 5.0, -3.0], dtype=np.float32)
    h = oracle.silu_mul(g, u, lib=lib)
    assert h[0] == 0.0
    assert np.array_equal(h[1:4], (g[1:4] * u[1:4]).astype(np.float32))
    assert h[4] == 0.0 and h[5] == 0.0
    x = np.linspace(-9, 9, 1001, dtype=np.float32)
    one = np.ones_like(x)
    d = oracle.silu_mul(x, one, lib=lib).astype(np.float64) - oracle.silu_mul(-x, one, lib=lib)
    assert np.all(np.abs(d - x) <= 4 * np.spacing(np.abs(x) + 1).astype(np.float64))


def pin_quantize_silu_mul(lib):
    """The fused quantizer = the (pinned) quantizer applied to the float64
    definition of h, bit for bit, on rows where numpy's h agrees."""
    g, u = _gate_inputs(2, 24, 2048)
    q, ds = oracle.quantize_silu_mul(g, u, lib=lib)
    ref = _silu_mul_f64(g, u)
    same = np.all(oracle.silu_mul(g, u, lib=lib) == ref, axis=1)
    assert same.mean() > 0.9
    rq, rds = oracle.quantize(ref[same], lib=lib)
    assert np.array_equal(q[same], rq) and np.array_equal(ds[same], rds)


# -------------------------------------------------------- load-time repack
def expected_repack(f: synth.Q4KFields) -> np.ndarray:
    """The record layout built with numpy from the generator's unpacked fields
    (never from the oracle's decoder or the packer's scale packing)."""
    m, k = f.q.shape
    S, T = k // 256, (m + 15) // 16
    rec = np.zeros((T, S, 2368), dtype=np.uint8)
    mp = T * 16
    d = np.zeros((mp, S), dtype=np.uint16)
    dm = np.zeros((mp, S), dtype=np.uint16)
    d[:m] = f.d.view(np.uint16)
    dm[:m] = f.dmin.view(np.uint16)
    hdr = (d.astype(np.uint32) | (dm.astype(np.uint32) << 16)).reshape(T, 16, S).transpose(0, 2, 1)
    rec[:, :, 0:64] = hdr.copy().view(np.uint8).reshape(T, S, 64)
    sc = np.zeros((mp, S, 8), dtype=np.uint8)
    mn = np.zeros((mp, S, 8), dtype=np.uint8)
    sc[:m] = f.sc.reshape(m, S, 8)
    mn[:m] = f.mn.reshape(m, S, 8)
    sw = np.stack([sc[:, :, 0::2], sc[:, :, 1::2], mn[:, :, 0::2], mn[:, :, 1::2]], axis=-1)  # [row, S, p, 4]
    sw = sw.reshape(T, 16, S, 4, 4).transpose(0, 2, 3, 1, 4)                                 # [T, S, p, r, 4]
    rec[:, :, 64:320] = sw.reshape(T, S, 256)
    q = np.zeros((mp, k), dtype=np.uint8)
    q[:m] = f.q
    q = q.reshape(T, 16, S, 4, 2, 32)                  # [T, r, S, pair p, chunk in pair, i]
    qs = q[:, :, :, :, 0, :] | (q[:, :, :, :, 1, :] << 4)   # qs byte 32p + i: [T, r, S, p, 32]
    qs = qs.reshape(T, 16, S, 4, 2, 16).transpose(0, 2, 3, 4, 1, 5)   # [T, S, p, h, r, 16]
    rec[:, :, 320:] = qs.reshape(T, S, 2048)
    return rec.reshape(-1)


def pin_q4k_repack(lib):
    """The oracle's repack equals the record layout built from the fields,
    on row counts that fill the last 16-row tile and ones that do not."""
    for seed, (m, k) in enumerate([(16, 256), (5, 512), (33, 768), (48, 256)]):
        f = synth.random_fields(70 + seed, m, k)
        got = oracle.q4k_repack(synth.pack_q4k(f), m, k, lib=lib)
        assert np.array_equal(got, expected_repack(f)), "repack differs (m=%d k=%d)" % (m, k)


# ------------------------------------------------------ q8 operand tiles
def expected_q8_tiles(q: np.ndarray) -> np.ndarray:
    """The operand-tile layout built with numpy reshapes from the codes (not
    the oracle's loops): k = 128 s + 32 c + 16 g + 8 h + e', tokens padded
    with zeros to 128, slots ordered (T, s, c, h, g, tt), a slot's element e
    taking e' = 0, 2, 1, 3, 4, 6, 5, 7."""
    n, k = q.shape
    T = (n + 127) // 128
    qp = np.zeros((T * 128, k), dtype=np.float16)
    qp[:n] = q
    a = qp.reshape(T, 128, k // 128, 4, 2, 2, 8)          # [T, tt, s, c, g, h, e']
    a = a[..., [0, 2, 1, 3, 4, 6, 5, 7]]
    a = a.transpose(0, 2, 3, 5, 4, 1, 6)                   # [T, s, c, h, g, tt, e]
    return np.ascontiguousarray(a).reshape(-1).view(np.uint16)


def pin_q8_tiles(lib):
    """The oracle's operand tiles equal the numpy-built layout, for token
    counts below one tile, at a tile boundary and past it."""
    for seed, (n, k) in enumerate([(1, 256), (37, 512), (128, 256), (131, 768)]):
        rng = np.random.default_rng(90 + seed)
        q = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
        got = oracle.q8_tiles(q, lib=lib)
        assert np.array_equal(got, expected_q8_tiles(q)), "q8 tiles differ (n=%d k=%d)" % (n, k)


ALL_PINS = [pin_f16_encode, pin_f16_decode, pin_q4k_golden_block, pin_q4k_roundtrip,
            pin_q8_golden, pin_q8_invariants, pin_q8_zero_block, pin_dots_bruteforce,
            pin_dots_closed_forms, pin_out_bruteforce, pin_out_negative_scales, pin_out_special_cases,
            pin_out_zero_scale_block, pin_one_superblock,
            pin_q6k_golden_block, pin_q6k_roundtrip, pin_q6k_dots_bruteforce,
            pin_q6k_dots_closed_forms, pin_q6k_out_bruteforce, pin_q6k_out_special_cases,
            pin_q6k_one_superblock, pin_silu_mul_float64, pin_silu_mul_closed_forms,
            pin_quantize_silu_mul, pin_q4k_repack, pin_q8_tiles]
