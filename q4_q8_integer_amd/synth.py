"""Seeded synthetic inputs for the q4_K x q8 quantized matmul.

This module only draws random numbers and lays them out in the q4_K byte
format; it holds none of the method's arithmetic (no quantization, no dot
products, no rescale).  Both the HIP path's tests and the CPU oracle's tests
take their inputs from here, and from nowhere else.

Every tensor comes from its own ``numpy.random.default_rng([config_id,
tensor_id])`` stream, so each can be regenerated alone.

Weight fields (all workloads): nibble q ~ U{0..15}; 6-bit sub-block scale sc and
min m ~ U{0..63}; super-block scales d, dmin = binary16(|N(0,1)| * 1e-2),
rounded to nearest-even from the float64 draw.  Activations: X ~ N(0,1) in
float32, with the per-workload variants below.

q4_K super-block byte layout (256 weights in 144 bytes).  The pages name the
format (the r31 page's result line: a "7B q4_K" model) and the roles of its
fields (the r31 page, section 2: the weight-side pair d*sc and -dmin*m per
32-weight sub-block), but not the bytes; the layout below is the k-quant
super-block of the GGUF ecosystem the pages work in (the r17 page, section 1,
compares against that ecosystem's Q4_K kernel):

* bytes 0-1   d     (binary16, little endian)
* bytes 2-3   dmin  (binary16)
* bytes 4-15  twelve bytes holding eight 6-bit sc and eight 6-bit m:
    for j < 4:  sc[j] = low 6 bits of byte j,  m[j] = low 6 bits of byte j+4;
    for j >= 4: sc[j] = low nibble of byte j+4 | (top 2 bits of byte j-4) << 4,
                m[j]  = high nibble of byte j+4 | (top 2 bits of byte j) << 4
* bytes 16-143 qs: weight 64p+i (i < 32) of the super-block is the low nibble
  of qs[32p+i]; weight 64p+32+i is its high nibble (p = 0..3).

Dequantized weight = d*sc[j]*q - dmin*m[j] for sub-block j = (index // 32).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QK_K = 256          # weights per super-block
QK = 32             # weights per sub-block (and activations per q8 block)
BLOCK_BYTES = 144   # bytes per q4_K super-block


def rng_for(config_id: int, tensor_id: int) -> np.random.Generator:
    """The one seeded stream of tensor ``tensor_id`` of workload ``config_id``."""
    return np.random.default_rng([int(config_id), int(tensor_id)])


@dataclass
class Q4KFields:
    """Unpacked q4_K fields of an ``m x k`` weight matrix (rows = outputs)."""

    q: np.ndarray      # uint8 [m, k], 0..15
    sc: np.ndarray     # uint8 [m, k/32], 0..63
    mn: np.ndarray     # uint8 [m, k/32], 0..63
    d: np.ndarray      # float16 [m, k/256]
    dmin: np.ndarray   # float16 [m, k/256]

    @property
    def m(self) -> int:
        return self.q.shape[0]

    @property
    def k(self) -> int:
        return self.q.shape[1]


def gen_q4k_fields(rng: np.random.Generator, m: int, k: int,
                   sc_zero_frac: float = 0.0) -> Q4KFields:
    """Draw q4_K fields in a fixed order: q, sc, m, d, dmin, then the sc=0 mask."""
    if k % QK_K:
        raise ValueError("k must be a multiple of 256")
    c, s = k // QK, k // QK_K
    q = rng.integers(0, 16, size=(m, k), dtype=np.uint8)
    sc = rng.integers(0, 64, size=(m, c), dtype=np.uint8)
    mn = rng.integers(0, 64, size=(m, c), dtype=np.uint8)
    d = (np.abs(rng.standard_normal((m, s))) * 1e-2).astype(np.float16)
    dmin = (np.abs(rng.standard_normal((m, s))) * 1e-2).astype(np.float16)
    if sc_zero_frac > 0.0:
        mask = rng.random((m, c)) < sc_zero_frac
        sc[mask] = 0
    return Q4KFields(q=q, sc=sc, mn=mn, d=d, dmin=dmin)


def pack_q4k(f: Q4KFields) -> np.ndarray:
    """Lay the fields out as q4_K super-blocks: uint8 [m, (k/256)*144]."""
    m, k = f.q.shape
    s = k // QK_K
    out = np.empty((m, s, BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = f.d.astype("<f2").view(np.uint8).reshape(m, s, 2)
    out[:, :, 2:4] = f.dmin.astype("<f2").view(np.uint8).reshape(m, s, 2)
    sc = f.sc.reshape(m, s, 8).astype(np.uint16)
    mn = f.mn.reshape(m, s, 8).astype(np.uint16)
    scales = np.empty((m, s, 12), dtype=np.uint16)
    scales[:, :, 0:4] = (sc[:, :, 0:4] & 63) | ((sc[:, :, 4:8] >> 4) << 6)
    scales[:, :, 4:8] = (mn[:, :, 0:4] & 63) | ((mn[:, :, 4:8] >> 4) << 6)
    scales[:, :, 8:12] = (sc[:, :, 4:8] & 15) | ((mn[:, :, 4:8] & 15) << 4)
    out[:, :, 4:16] = scales.astype(np.uint8)
    q = f.q.reshape(m, s, 4, 2, 32)          # [row, sb, pair p, half, i]
    out[:, :, 16:144] = (q[:, :, :, 0, :] | (q[:, :, :, 1, :] << 4)).reshape(m, s, 128)
    return out.reshape(m, s * BLOCK_BYTES)


# ------------------------------------------------------------------ q6_K
# q6_K super-block byte layout (256 weights in 210 bytes).  The pages only
# name the format (the r31 page's closing notes speak of a "q6_K line" of
# rounds); the layout is the GGUF k-quant one, written out here:
#
# * bytes 0-127    ql: low 4 bits of the quants
# * bytes 128-191  qh: high 2 bits of the quants
# * bytes 192-207  sc: sixteen signed 8-bit scales, one per 16 weights
# * bytes 208-209  d:  binary16 super-block scale
#
# Weight e = 128h + 32g + l of the super-block (h = 0..1, g = 0..3, l = 0..31)
# has the 6-bit code q = lo | hi << 4 with
#   lo = nibble g // 2 (0 = low, 1 = high) of ql[64h + 32(g % 2) + l],
#   hi = bits 2g, 2g+1 of qh[32h + l],
# and the dequantized weight is d * sc[e // 16] * (q - 32).
Q6K_BLOCK_BYTES = 210
QK6 = 16            # weights per q6_K scale group


@dataclass
class Q6KFields:
    """Unpacked q6_K fields of an ``m x k`` weight matrix (rows = outputs)."""

    q: np.ndarray      # uint8 [m, k], 0..63 (the stored code; the weight uses q - 32)
    sc: np.ndarray     # int8 [m, k/16]
    d: np.ndarray      # float16 [m, k/256]

    @property
    def m(self) -> int:
        return self.q.shape[0]

    @property
    def k(self) -> int:
        return self.q.shape[1]


def gen_q6k_fields(rng: np.random.Generator, m: int, k: int,
                   sc_zero_frac: float = 0.0) -> Q6KFields:
    """Draw q6_K fields in a fixed order: q ~ U{0..63}, sc ~ U{-128..127},
    d = binary16(|N(0,1)| * 1e-3), then the sc=0 mask."""
    if k % QK_K:
        raise ValueError("k must be a multiple of 256")
    g, s = k // QK6, k // QK_K
    q = rng.integers(0, 64, size=(m, k), dtype=np.uint8)
    sc = rng.integers(-128, 128, size=(m, g), dtype=np.int16).astype(np.int8)
    d = (np.abs(rng.standard_normal((m, s))) * 1e-3).astype(np.float16)
    if sc_zero_frac > 0.0:
        mask = rng.random((m, g)) < sc_zero_frac
        sc[mask] = 0
    return Q6KFields(q=q, sc=sc, d=d)


def pack_q6k(f: Q6KFields) -> np.ndarray:
    """Lay the fields out as q6_K super-blocks: uint8 [m, (k/256)*210]."""
    m, k = f.q.shape
    s = k // QK_K
    out = np.empty((m, s, Q6K_BLOCK_BYTES), dtype=np.uint8)
    q = f.q.reshape(m, s, 2, 4, 32)          # [row, sb, half h, group g, l]
    lo, hi = q & 15, q >> 4
    ql = np.empty((m, s, 2, 2, 32), dtype=np.uint8)   # [row, sb, h, g % 2, l]
    ql[:, :, :, 0, :] = lo[:, :, :, 0, :] | (lo[:, :, :, 2, :] << 4)
    ql[:, :, :, 1, :] = lo[:, :, :, 1, :] | (lo[:, :, :, 3, :] << 4)
    out[:, :, 0:128] = ql.reshape(m, s, 128)
    qh = hi[:, :, :, 0, :] | (hi[:, :, :, 1, :] << 2) | (hi[:, :, :, 2, :] << 4) | (hi[:, :, :, 3, :] << 6)
    out[:, :, 128:192] = qh.reshape(m, s, 64)
    out[:, :, 192:208] = f.sc.reshape(m, s, 16).view(np.uint8)
    out[:, :, 208:210] = f.d.astype("<f2").view(np.uint8).reshape(m, s, 2)
    return out.reshape(m, s * Q6K_BLOCK_BYTES)


def gen_normal(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """X ~ N(0,1), float32 [n, k]."""
    return rng.standard_normal((n, k), dtype=np.float32)


def gen_silu(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """SiLU(z) for z ~ N(0,1), evaluated in float64 then cast to float32."""
    z = rng.standard_normal((n, k))
    return (z / (1.0 + np.exp(-z))).astype(np.float32)


def gen_outliers(rng: np.random.Generator, n: int, k: int,
                 frac: float = 0.01, scale: float = 20.0) -> np.ndarray:
    """X ~ N(0,1) float32 with a Bernoulli(frac) mask of entries scaled by ``scale``."""
    x = rng.standard_normal((n, k), dtype=np.float32)
    mask = rng.random((n, k)) < frac
    x[mask] *= np.float32(scale)
    return x


# ---------------------------------------------------------------- workloads
# Shapes of the five workloads (rows x input features, token counts).
TINY = dict(m=256, k=512, n=64)
QPROJ = dict(m=4096, k=4096, n=2630)
FFN = dict(d_model=4096, d_ff=11008, n=2630)
LAYER_TOKENS = (512, 2048, 8192)
LAYER_MATS = (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096),
              ("o", 4096, 4096), ("gate", 11008, 4096), ("up", 11008, 4096),
              ("down", 4096, 11008))
WEIGHT_BOUND_MATS = (("wide_in", 28672, 8192), ("wide_out", 8192, 28672))
WEIGHT_BOUND_TOKENS = (1, 7, 33, 2051)


def tiny_inputs():
    """Tiny case: W[256 x 512] q4_K, X[64 x 512] ~ N(0,1); seed stream 0."""
    f = gen_q4k_fields(rng_for(0, 0), TINY["m"], TINY["k"])
    x = gen_normal(rng_for(0, 1), TINY["n"], TINY["k"])
    return f, x


def qproj_inputs(n: int | None = None):
    """7B q-projection prefill: W[4096 x 4096], X[2630 x 4096]."""
    f = gen_q4k_fields(rng_for(1, 0), QPROJ["m"], QPROJ["k"])
    x = gen_normal(rng_for(1, 1), QPROJ["n"] if n is None else n, QPROJ["k"])
    return f, x


def ffn_inputs(which: str, n: int | None = None):
    """7B FFN prefill: gate/up [11008 x 4096] on X[2630 x 4096]; down [4096 x 11008]
    on SiLU(N(0,1)) [2630 x 11008]."""
    n = FFN["n"] if n is None else n
    if which == "gate":
        return gen_q4k_fields(rng_for(2, 0), FFN["d_ff"], FFN["d_model"])
    if which == "up":
        return gen_q4k_fields(rng_for(2, 1), FFN["d_ff"], FFN["d_model"])
    if which == "down":
        return gen_q4k_fields(rng_for(2, 2), FFN["d_model"], FFN["d_ff"])
    if which == "x":
        return gen_normal(rng_for(2, 3), n, FFN["d_model"])
    if which == "x_down":
        return gen_silu(rng_for(2, 4), n, FFN["d_ff"])
    raise ValueError(which)


def ffn_gate_up_outputs(n: int | None = None):
    """The FFN's gate and up projection outputs [n x 11008] (the fused
    SiLU-gate quantizer's inputs): gate ~ 2 N(0,1) (so the SiLU sees both its
    linear and its saturated range), up ~ N(0,1), float32, streams (2, 5) and
    (2, 6)."""
    n = FFN["n"] if n is None else n
    g = (rng_for(2, 5).standard_normal((n, FFN["d_ff"]), dtype=np.float32) * np.float32(2.0))
    u = rng_for(2, 6).standard_normal((n, FFN["d_ff"]), dtype=np.float32)
    return g, u


def layer_weights(name: str) -> Q4KFields:
    """One projection of the full 7B layer set (tensor ids 0..6 in LAYER_MATS order)."""
    for tid, (nm, m, k) in enumerate(LAYER_MATS):
        if nm == name:
            return gen_q4k_fields(rng_for(3, tid), m, k)
    raise ValueError(name)


def layer_activation(which: str, n: int) -> np.ndarray:
    """Layer-set inputs with 1% of entries scaled x20: attn_in, o_in, ffn_in
    [n x 4096] and down_in [n x 11008]."""
    names = ("attn_in", "o_in", "ffn_in", "down_in")
    ni = LAYER_TOKENS.index(n) if n in LAYER_TOKENS else 3 + n
    j = names.index(which)
    k = 11008 if which == "down_in" else 4096
    return gen_outliers(rng_for(3, 7 + 4 * ni + j), n, k)


def weight_bound_weights(name: str) -> Q4KFields:
    """W[28672 x 8192] ("wide_in") or W[8192 x 28672] ("wide_out"); 10% of
    sub-blocks have sc = 0."""
    for tid, (nm, m, k) in enumerate(WEIGHT_BOUND_MATS):
        if nm == name:
            return gen_q4k_fields(rng_for(4, tid), m, k, sc_zero_frac=0.1)
    raise ValueError(name)


def weight_bound_activation(name: str, n: int) -> np.ndarray:
    """X ~ N(0,1) [n x K] for the weight-bound matrix ``name``."""
    k = dict((nm, kk) for nm, _, kk in WEIGHT_BOUND_MATS)[name]
    mi = [nm for nm, _, _ in WEIGHT_BOUND_MATS].index(name)
    ni = WEIGHT_BOUND_TOKENS.index(n) if n in WEIGHT_BOUND_TOKENS else 4 + n
    return gen_normal(rng_for(4, 2 + 16 * mi + ni), n, k)


# q6_K workloads (stream 5): the q-projection shape at prefill and the
# weight-bound wide matrix, with q6_K weights in place of q4_K.
Q6K_MATS = (("qproj", 4096, 4096), ("wide_in", 28672, 8192))


def q6k_weights(name: str) -> Q6KFields:
    """q6_K W[4096 x 4096] ("qproj") or W[28672 x 8192] ("wide_in", 10% of
    scale groups with sc = 0)."""
    for tid, (nm, m, k) in enumerate(Q6K_MATS):
        if nm == name:
            return gen_q6k_fields(rng_for(5, tid), m, k, sc_zero_frac=0.1 if nm == "wide_in" else 0.0)
    raise ValueError(name)


def q6k_activation(name: str, n: int) -> np.ndarray:
    """X ~ N(0,1) [n x K] for the q6_K matrix ``name``."""
    k = dict((nm, kk) for nm, _, kk in Q6K_MATS)[name]
    mi = [nm for nm, _, _ in Q6K_MATS].index(name)
    return gen_normal(rng_for(5, 2 + (1 << 20) * mi + n), n, k)


def random_q6k_fields(seed: int, m: int, k: int, sc_zero_frac: float = 0.0) -> Q6KFields:
    """q6_K fields for ad-hoc test shapes, from stream [102, seed]."""
    return gen_q6k_fields(rng_for(102, seed), m, k, sc_zero_frac)


def random_fields(seed: int, m: int, k: int, sc_zero_frac: float = 0.0) -> Q4KFields:
    """Fields for ad-hoc test shapes, from stream [100, seed]."""
    return gen_q4k_fields(rng_for(100, seed), m, k, sc_zero_frac)


def random_activations(seed: int, n: int, k: int, kind: str = "normal") -> np.ndarray:
    """Activations for ad-hoc test shapes, from stream [101, seed]."""
    rng = rng_for(101, seed)
    if kind == "normal":
        return gen_normal(rng, n, k)
    if kind == "silu":
        return gen_silu(rng, n, k)
    if kind == "outliers":
        return gen_outliers(rng, n, k)
    raise ValueError(kind)
