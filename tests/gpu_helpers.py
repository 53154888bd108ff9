"""Helpers shared by the GPU parity tests: device transfer, the parity
tolerance, and token sampling for full-size workloads."""
from __future__ import annotations

import sys

import numpy as np
import torch

from q4_q8_integer_amd import binding

# float32 output bar: relative L2 <= 1e-5 and every element within 1e-3 of
# its token row's largest |value| (both against the float64 oracle).
REL_L2 = 1e-5
MAX_ABS_ROW = 1e-3


def dev():
    return torch.device("cuda:0")


def note(msg: str):
    """Name the case on stdout before a GPU step (flushed)."""
    print(msg, file=sys.stdout, flush=True)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def gpu_quantize(x: np.ndarray):
    q, ds = binding.quantize(to_dev(x))
    torch.cuda.synchronize()
    return q, ds


def host_ds(ds: torch.Tensor) -> np.ndarray:
    return ds.cpu().numpy().view(np.uint32)


def check_fp32(got: np.ndarray, ref: np.ndarray, what: str = "", rel_l2: float = REL_L2):
    got = got.astype(np.float64)
    err = got - ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= rel_l2, "%s: relative L2 error %.3g > %g" % (what, rel, rel_l2)
    rowscale = np.abs(ref).max(axis=1, keepdims=True)
    worst = (np.abs(err) / np.maximum(rowscale, 1e-300)).max()
    assert worst <= MAX_ABS_ROW, "%s: max |err| / row scale %.3g > %g" % (what, worst, MAX_ABS_ROW)
    return rel, worst


def sample_tokens(n: int, count: int = 48, seed: int = 0, tile: int = 128) -> np.ndarray:
    """First, last and tail-tile tokens plus ``count`` random ones (sorted, unique)."""
    rng = np.random.default_rng([900, seed, n])
    pick = {0, 1, n - 1, n - 2}
    tail0 = (n // tile) * tile
    pick.update(range(tail0, min(n, tail0 + 8)))
    pick.update(rng.integers(0, n, size=min(count, n)).tolist())
    return np.array(sorted(t for t in pick if 0 <= t < n), dtype=np.int64)
