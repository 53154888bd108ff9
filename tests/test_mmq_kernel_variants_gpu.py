"""Every float32 kernel meets the same bar on shapes outside its default
range: MMQ_FP32_KERNEL=i8 (int8-MFMA kernel, kept for comparison), f16 (the
binary16-MFMA kernel, default above 64 tokens and from 49 where the matrix
gives it enough tiles, here also on few tokens), small (the few-token
int8-MFMA kernels, one-tile up to 16 tokens and multi-tile above, default
from 9 tokens, here also on fewer), pair (the
chunk-pair int8-MFMA kernel, kept for comparison) and gemv (the vector-ALU
dot4 kernel, default up to 8 tokens).  Each forced kernel's binary16 output
must equal its float32 output rounded to nearest-even, bit for bit.  The
switch is read once per process, so each runs in one child process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, %(root)r)
sys.path.insert(0, %(tests)r)
import numpy as np
import oracle
from gpu_helpers import check_fp32, gpu_quantize, to_dev
from q4_q8_integer_amd import binding, synth
import torch
for seed, (n, m, k) in enumerate(%(shapes)s):
    f = synth.random_fields(500 + seed, m, k, sc_zero_frac=0.1)
    x = synth.random_activations(500 + seed, n, k, "outliers")
    w = synth.pack_q4k(f)
    q, ds = gpu_quantize(x)
    wd = to_dev(w)
    got = binding.fp32(wd, m, k, q, ds)
    got16 = binding.fp16(wd, m, k, q, ds)
    torch.cuda.synchronize()
    assert np.array_equal(got16.cpu().numpy().view(np.uint16),
                          got.cpu().numpy().astype(np.float16).view(np.uint16)), "f16out != rounded fp32out"
    rq, rds = oracle.quantize(x)
    rel, worst = check_fp32(got.cpu().numpy(), oracle.out_f64(w, m, k, rq, rds), "forced kernel")
    print("case", n, m, k, "rel %%.2e" %% rel, flush=True)
print("ok")
"""


SHAPES = {
    "i8": [(64, 256, 512), (77, 200, 768), (130, 129, 512), (5, 131, 2304)],
    "f16": [(1, 256, 512), (7, 200, 768), (33, 129, 512), (64, 131, 2304)],
    "small": [(1, 1, 256), (7, 31, 1280), (16, 17, 2304), (17, 200, 768), (48, 129, 512),
              (64, 256, 11008)],
    "gemv": [(1, 1, 256), (2, 17, 2304), (3, 33, 512), (4, 200, 768), (5, 129, 4352),
             (6, 16, 256), (7, 131, 2304), (8, 256, 11008)],
    "pair": [(1, 1, 256), (2, 17, 2304), (4, 33, 512), (5, 200, 768), (7, 129, 4352),
             (8, 16, 256), (9, 131, 2304), (12, 64, 1280), (16, 256, 11008)],
}


@pytest.mark.parametrize("kernel", sorted(SHAPES))
def test_forced_fp32_kernel_matches_oracle(kernel):
    env = dict(os.environ, MMQ_FP32_KERNEL=kernel)
    code = CHILD % {"root": ROOT, "tests": os.path.join(ROOT, "tests"), "shapes": repr(SHAPES[kernel])}
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    print(r.stdout, r.stderr[-2000:])
    assert r.returncode == 0 and r.stdout.strip().endswith("ok")
