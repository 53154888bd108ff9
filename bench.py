"""Benchmark of the q4_K x q8 MMQ hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
q8-quantize each activation matrix (q8_quantize_rows) and run every
projection's MMQ with the two-term fold (mmq_q4k_q8_fp32out).  Inputs are
resident in HBM before timing starts; several copies of the weights and
activations are rotated so that the 256 MB last-level cache cannot hold a
step's working set.

Default workload: the 7B layer projection set at N = 2048 tokens (q, k, v, o
4096 x 4096; gate, up 11008 x 4096; down 4096 x 11008; 4 quantizes and 7
MMQs per step), the configuration the metric's "prefill tok/s over 7B
projections" is quoted on: tok/s = N / (32 * t_step) for 32 layers.  Beside
it: the same set at N = 512 and 8192, and the N = 2048 step on the
library's fastest calls (weights repacked at load time, activations
quantized to binary16 operand tiles) under "fastest_path".  Prints one JSON
line (see the keys in ``main``).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload layer2048]
"""
from __future__ import annotations

import argparse
import math
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MMQ int8 TOPS (+% MFMA peak) and prefill tok/s over 7B projections"
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA, published
F16_PEAK_TFLOPS = 2500.0   # MI355X dense binary16 MFMA, published
DEFAULT_WORKLOAD = "layer2048"
FASTEST = "t_r_layer2048"  # the default workload on the fastest calls
BESIDE = ("layer512", "layer8192")   # the other token counts of the layer set
LAYERS = 32                # layers of a 7B model (the pages do not state it)
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published


def build_workload(name: str):
    """-> (description dict, inputs {name: X}, mats [(label, fields, input name)])."""
    from q4_q8_integer_amd import synth
    if name == "qproj":
        f, x = synth.qproj_inputs()
        return ({"workload": "7B q-proj prefill: q4_K W[4096x4096] x q8 X[2630x4096] -> fp32 [2630x4096]",
                 "m": 4096, "k": 4096, "n": 2630},
                {"x": x}, [("q", f, "x")])
    if name == "ffn":
        return ({"workload": "7B FFN prefill: gate,up q4_K [11008x4096] on X[2630x4096], "
                             "down [4096x11008] on SiLU input [2630x11008]", "n": 2630},
                {"x": synth.ffn_inputs("x"), "x_down": synth.ffn_inputs("x_down")},
                [("gate", synth.ffn_inputs("gate"), "x"), ("up", synth.ffn_inputs("up"), "x"),
                 ("down", synth.ffn_inputs("down"), "x_down")])
    if name.startswith("layer"):
        n = int(name[5:])
        src = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "o_in",
               "gate": "ffn_in", "up": "ffn_in", "down": "down_in"}
        inputs = {s: synth.layer_activation(s, n) for s in sorted(set(src.values()))}
        mats = [(nm, synth.layer_weights(nm), src[nm]) for nm, _, _ in synth.LAYER_MATS]
        return ({"workload": "7B layer projection set q,k,v,o,gate,up,down at N=%d "
                             "(4 quantizes + 7 MMQs; 1%% of inputs x20)" % n, "n": n},
                inputs, mats)
    if name == "q6k_qproj":
        f = synth.q6k_weights("qproj")
        return ({"workload": "q-proj prefill with q6_K weights: q6_K W[4096x4096] x q8 X[2630x4096] "
                             "-> fp32 [2630x4096]", "m": 4096, "k": 4096, "n": 2630},
                {"x": synth.q6k_activation("qproj", 2630)}, [("q", f, "x")])
    if name.startswith("q6k_wide_in_n"):
        n = int(name.rsplit("_n", 1)[1])
        f = synth.q6k_weights("wide_in")
        return ({"workload": "weight-bound q6_K W[%dx%d] at N=%d (10%% of scale groups sc=0)"
                             % (f.m, f.k, n), "m": f.m, "k": f.k, "n": n},
                {"x": synth.q6k_activation("wide_in", n)}, [("wide_in", f, "x")])
    if name.startswith("t_"):
        desc, inputs, mats = build_workload(name[2:])
        return (dict(desc, tiles=True, workload=desc["workload"] +
                     ", activations quantized to binary16 operand tiles (q8_quantize_rows_tiled)"),
                inputs, mats)
    if name.startswith("r_"):
        desc, inputs, mats = build_workload(name[2:])
        if any(not isinstance(f, synth.Q4KFields) for _, f, _ in mats):
            raise SystemExit("the repacked layout is for q4_K weights")
        desc = dict(desc, repacked=True,
                    workload=desc["workload"] + ", weights repacked at load time (q4k_repack)")
        return desc, inputs, mats
    if name.startswith("wide_in") or name.startswith("wide_out"):
        wname, n = name.rsplit("_n", 1)
        n = int(n)
        f = synth.weight_bound_weights(wname)
        return ({"workload": "weight-bound q4_K W[%dx%d] at N=%d (10%% of sub-blocks sc=0)"
                             % (f.m, f.k, n), "m": f.m, "k": f.k, "n": n},
                {"x": synth.weight_bound_activation(wname, n)}, [(wname, f, "x")])
    raise SystemExit("unknown workload %r" % name)


def kernel_choice(desc, f, n):
    """(format, kernel id) the library's own dispatch (mmq_kernel_choice)
    runs for this call, or the kernel named with --kernel."""
    from q4_q8_integer_amd import binding, synth
    q6 = isinstance(f, synth.Q6KFields)
    if desc.get("kernel"):
        ids = {v: k for k, v in binding.KERNEL_NAMES.items()}
        return (binding.FORMAT_Q6K if q6 else binding.FORMAT_Q4K), ids[desc["kernel"]]
    if desc.get("tiles"):
        fmt = binding.FORMAT_Q6K_TILES if q6 else (
            binding.FORMAT_Q4K_REPACKED_TILES if desc.get("repacked") else binding.FORMAT_Q4K_TILES)
    else:
        fmt = binding.FORMAT_Q6K if q6 else (
            binding.FORMAT_Q4K_REPACKED if desc.get("repacked") else binding.FORMAT_Q4K)
    return fmt, binding.mmq_kernel_choice(fmt, f.m, f.k, n)


def compute_dtype(desc, f, n):
    """Arithmetic type of the kernel the library runs for this call: "f16"
    for the binary16-MFMA kernels (exact integer operands in binary16,
    float32 accumulation), "int8" for the dot4, narrow, stream, few-token
    and int8-MFMA kernels."""
    from q4_q8_integer_amd import binding
    return "f16" if kernel_choice(desc, f, n)[1] == binding.KERNEL_F16 else "int8"


def kernel_source(desc, f, n):
    """The csrc file of the kernel the library runs for this call."""
    from q4_q8_integer_amd import binding
    fmt, kid = kernel_choice(desc, f, n)
    q6 = fmt in (binding.FORMAT_Q6K, binding.FORMAT_Q6K_TILES)
    names = ({binding.KERNEL_DOT4: "mmq_q6k_gemv.hip", binding.KERNEL_F16: "mmq_q6k_f16.hip",
              binding.KERNEL_I8: "mmq_q6k_i8.hip"} if q6 else
             {binding.KERNEL_DOT4: "mmq_gemv.hip", binding.KERNEL_NARROW: "mmq_narrow.hip",
              binding.KERNEL_STREAM: "mmq_stream.hip", binding.KERNEL_FEW: "mmq_small.hip", binding.KERNEL_F16: "mmq_f16.hip",
              binding.KERNEL_I8: "mmq_i8.hip"})
    return "q4_q8_integer_amd/csrc/" + names[kid]


def raw_call(name, args):
    """The C-ABI entry point `name` with its arguments marshalled once (tensors
    to device pointers, the current stream appended): a callable that repeats
    the call with no per-call Python work, for the event-timed loop, where the
    host must enqueue launches faster than the GPU runs them.  The arguments
    were checked by the binding's own wrapper in the timed steps before."""
    import ctypes
    import torch
    from q4_q8_integer_amd import binding
    fn = getattr(binding.load_library(), name)
    cargs = tuple(ctypes.c_void_p(a.data_ptr()) if isinstance(a, torch.Tensor) else a for a in args)
    cargs += (ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),)

    def call():
        status = fn(*cargs)
        if status != 0:
            raise RuntimeError("%s: %s" % (name, binding.status_string(status)))
    return call


def weight_format(f):
    """'q6k' for q6_K fields, 'q4k' for q4_K: (packer, weight bytes per weight,
    C-ABI name prefix, oracle output function name)."""
    from q4_q8_integer_amd import synth
    if isinstance(f, synth.Q6KFields):
        return synth.pack_q6k, 210.0 / 256.0, "mmq_q6k_q8", "q6k_out_f64"
    return synth.pack_q4k, 144.0 / 256.0, "mmq_q4k_q8", "out_f64"


def source_digest(src: str) -> str:
    """sha256 prefix (16 hex digits) over a kernel source file and, depth
    first in include order, every local header it includes with
    `#include "..."`, each file once: a change in a shared header changes
    the digest of every source that includes it."""
    import hashlib
    import re
    files = []

    def walk(path):
        path = os.path.normpath(path)
        if path in files:
            return
        files.append(path)
        for line in open(path, encoding="utf-8", errors="replace"):
            m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
            if m:
                walk(os.path.join(os.path.dirname(path), m.group(1)))

    walk(os.path.join(ROOT, src))
    h = hashlib.sha256()
    for path in files:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(key: str, src: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    record (profiles/traffic.txt), already scaled by the copy-probe factors;
    None unless the record was taken on the kernel the library runs now
    (src, its csrc file) with that source and the headers it includes as
    they are now (source_digest)."""
    try:
        rec = json.loads(open(os.path.join(ROOT, "profiles", "traffic.txt")).read())[key]
        digest = source_digest(rec["src"])
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("src") != src or rec.get("sha256_16") != digest:
        return None
    return int(rec["read_bytes"] + rec["write_bytes"])


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo), with the CPU
    family, model and the cores lscpu reports (virtual machines often give
    only a generic name)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        f = {}
        for line in out.splitlines():
            if ":" in line:
                key, val = line.split(":", 1)
                f[key.strip()] = val.strip()
        if "Model name" in f:
            extra = ", ".join("%s %s" % (lbl, f[key]) for key, lbl in
                              (("CPU family", "family"), ("Model", "model"), ("Core(s) per socket", "cores/socket"),
                               ("Socket(s)", "sockets"), ("Thread(s) per core", "threads/core")) if key in f)
            return "%s (%s)" % (f["Model name"], extra) if extra else f["Model name"]
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(mats, inputs, budget_s: float = 12.0):
    """Time the oracle (as it stands) on a bounded token sample of the same
    workload: quantize + float64 fold for every projection, with all host
    threads (about budget_s seconds) and with one thread (about 2/3 of
    that).  Its cost is a fixed part per call (the weight decode) plus a
    part linear in the tokens; two short probes fit both, and the sample is
    sized from the fit.  The rate at the sample extends to the whole
    workload (the fixed part only shrinks with more tokens)."""
    import oracle

    packed = [(weight_format(f)[0](f), f.m, f.k, src, getattr(oracle, weight_format(f)[3]))
              for _, f, src in mats]
    n_full = min(x.shape[0] for x in inputs.values())

    def run(nt):
        t0 = time.perf_counter()
        qs = {s: oracle.quantize(x[:nt]) for s, x in inputs.items()}
        for w, m, k, src, out_f64 in packed:
            q, ds = qs[src]
            out_f64(w, m, k, q, ds)
        return time.perf_counter() - t0

    def timed(budget):
        n0, n1 = min(2, n_full), min(10, n_full)
        t0, t1 = run(n0), run(n1)
        per_tok = max((t1 - t0) / max(n1 - n0, 1), 1e-6)
        fixed = max(t0 - n0 * per_tok, 0.0)
        nt = int(max(n1, min(n_full, (budget - fixed) / per_tok)))
        return nt, run(nt)

    all_threads = oracle.get_threads()
    nt, t = timed(budget_s)
    oracle.set_threads(1)
    try:
        nt1, t1 = timed(budget_s * 2 / 3)
    finally:
        oracle.set_threads(all_threads)
    flops = sum(2.0 * m * k for _, m, k, _, _ in packed)   # per token
    return {"value": flops * nt / t / 1e12, "unit": "TOPS", "cores": all_threads,
            "kind": "oracle", "tok_per_s": nt / t,
            "one_thread": {"value": flops * nt1 / t1 / 1e12, "tok_per_s": nt1 / t1, "cores": 1,
                           "sample": "first %d tokens (%.1f s)" % (nt1, t1)},
            "cpu_model": cpu_model(),
            "sample": "first %d tokens of every input, all rows, quantize + float64 fold "
                      "(%.1f s)" % (nt, t)}


def run_silu_q8(args):
    """The fused SiLU-gate quantizer (q8_quantize_silu_mul) on the FFN down
    projection's input, 2630 x 11008: a step is one fused quantize.  The
    unfused equivalent (torch's SiLU and product, then q8_quantize_rows) is
    timed beside it for context."""
    import torch
    from q4_q8_integer_amd import binding, synth

    dev = torch.device("cuda:0")
    binding.load_library()
    g, u = synth.ffn_gate_up_outputs()
    n, k = g.shape
    sets = []
    for _ in range(max(1, args.copies)):
        sets.append((torch.from_numpy(g).to(dev), torch.from_numpy(u).to(dev),
                     torch.empty((n, k), dtype=torch.int8, device=dev),
                     torch.empty((n, k // 32), dtype=torch.int32, device=dev)))
    h = torch.empty((n, k), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(i):
        gd, ud, q, ds = sets[i % len(sets)]
        binding.q8_quantize_silu_mul(gd, ud, n, k, q, ds)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stream = torch.cuda.current_stream()
    # about 25 ms of GPU time each way, as for the MMQ below
    rounds = int(min(4000, max(args.steps, 10, math.ceil(25.0 / max(wall * 1e3 / args.steps, 1e-3)))))

    def event_time(fn):
        # behind untimed rounds of the same work, as for the MMQ below
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(rounds):
            fn(i)
        e0.record(stream)
        for i in range(rounds):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / rounds

    fused_ms = event_time(step)

    def unfused(i):
        gd, ud, q, ds = sets[i % len(sets)]
        torch.mul(torch.nn.functional.silu(gd), ud, out=h)
        binding.q8_quantize_rows(h, n, k, q, ds)

    unfused(0)
    unfused_ms = event_time(unfused)

    alg = 9.125 * n * k     # 4 + 4 B read, 1 + 4/32 B written per element
    gbs = alg / (fused_ms * 1e-3) / 1e9
    ms_step = wall * 1e3 / args.steps
    res = {
        "metric": "fused SiLU-gate q8 quantize throughput (FFN down input)",
        "value": round(alg / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64->f32->i8",
        "data": "synthetic",
        "config": {"workload": "q8_quantize_silu_mul of SiLU(gate)*up, gate/up fp32 [%dx%d]" % (n, k),
                   "n": n, "k": k, "copies": len(sets)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": "q8_quantize_silu_mul",
                     "traffic": measured_traffic("q8_quantize_silu_mul|silu_q8", "q4_q8_integer_amd/csrc/quantize.hip"),
                     "avg_launch_us": round(fused_ms * 1e3, 2), "launches_timed": rounds,
                     "alg_bytes_per_step": alg},
        "unfused_us": round(unfused_ms * 1e3, 2),
    }
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = 2 * src.numel() * 4
    if not args.no_cpu_baseline:
        import oracle
        rows = 8
        t0 = time.perf_counter()
        oracle.quantize_silu_mul(g[:rows], u[:rows])
        t = time.perf_counter() - t0
        rows = int(min(n, max(rows, rows * 12.0 / max(t, 1e-6))))
        t0 = time.perf_counter()
        oracle.quantize_silu_mul(g[:rows], u[:rows])
        t = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(9.125 * rows * k / t / 1e9, 3), "unit": "GB/s",
                               "cores": oracle.get_threads(), "kind": "oracle",
                               "sample": "first %d of %d rows (%.1f s)" % (rows, n, t)}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first (the GPU reaches its working clocks over some tens of ms)")
    ap.add_argument("--workload", default=None,
                    help="default: %s, with %s and the fastest path (%s) measured beside it"
                         % (DEFAULT_WORKLOAD, ", ".join(BESIDE), FASTEST))
    ap.add_argument("--copies", type=int, default=3, help="rotated input copies (cache defeat)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--f16-out", action="store_true",
                    help="time the binary16-output entry point (mmq_*_f16out) instead of the float32 one")
    ap.add_argument("--kernel", default=None,
                    help="run the MMQ on this named kernel through the fold entry point "
                         "(mmq_q4k_q8_fold / mmq_q6k_q8_fold: dot4, narrow, stream, few, f16 or i8) instead "
                         "of the library's own choice; GGUF-layout, int8-code workloads only")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run one 1 GiB device copy (known bytes) so that "
                         "profiler byte counters can be calibrated against it")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sharding is described in the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    default_run = args.workload is None
    if default_run:
        args.workload = DEFAULT_WORKLOAD
    host_cpu = cpu_model()   # before the GPU is touched (lscpu runs as a child process)
    if args.workload == "silu_q8":
        return run_silu_q8(args)

    res, mats, inputs = measure(args, args.workload)
    if args.copy_probe:
        import torch
        dev = torch.device("cuda:0")
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = 2 * src.numel() * 4
    if default_run and not args.f16_out:
        # The layer set at the other token counts, and the same N = 2048 step
        # through the library's fastest calls: weights repacked at load time,
        # activations quantized to the binary16 operand tiles (same codes,
        # scale words and output as the headline calls).  Reported beside the
        # headline, which stays on the calls the boundary names.
        res["layer_set"] = {str(res["config"]["n"]): summary(res)}
        for wl in BESIDE:
            alt, _, _ = measure(args, wl)
            res["layer_set"][str(alt["config"]["n"])] = summary(alt)
        alt, _, _ = measure(args, FASTEST)
        res["fastest_path"] = dict(summary(alt), workload=FASTEST, step=alt["config"]["step"],
                                   roofline=alt["roofline"])
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = dict(cpu_baseline(mats, inputs), cpu_model=host_cpu)
    print(json.dumps(res), flush=True)


def summary(r):
    """The figures of one measured workload that the default line repeats."""
    keys = ("value", "unit", "ms_per_step", "tok_per_s", "tok_per_s_7b_projections", "pct_int8_peak", "dtype")
    out = {k: r[k] for k in keys if k in r}
    out["mmq_us_per_projection"] = r["roofline"]["avg_launch_us"]
    out["mmq_int8_tops"] = r["roofline"]["int8_tops"]
    return out


def measure(args, workload):
    """Time one workload: -> (result dict without cpu_baseline, mats, inputs)."""
    import torch
    from q4_q8_integer_amd import binding, synth

    desc, inputs, mats = build_workload(workload)
    if getattr(args, "kernel", None):
        if desc.get("repacked") or desc.get("tiles"):
            raise SystemExit("--kernel applies to GGUF-layout workloads with int8 codes")
        if args.kernel not in binding.KERNEL_NAMES.values():
            raise SystemExit("--kernel: one of %s" % ", ".join(sorted(binding.KERNEL_NAMES.values())))
        desc = dict(desc, kernel=args.kernel)
    dev = torch.device("cuda:0")
    binding.load_library()

    # resident inputs, several copies
    sets = []
    for _ in range(max(1, args.copies)):
        xs = {s: torch.from_numpy(x).to(dev) for s, x in inputs.items()}
        ws = [(lbl, torch.from_numpy(weight_format(f)[0](f)).to(dev), f.m, f.k, src)
              for lbl, f, src in mats]
        if desc.get("repacked"):   # load-time step, outside the timed region
            ws = [(lbl, binding.repack(w, m, k), m, k, src) for lbl, w, m, k, src in ws]
        if desc.get("tiles"):
            qs = {s: (torch.empty(binding.tiles_elems(*x.shape), dtype=torch.int16, device=dev),
                      torch.empty((x.shape[0], x.shape[1] // 32), dtype=torch.int32, device=dev))
                  for s, x in xs.items()}
        else:
            qs = {s: (torch.empty(x.shape, dtype=torch.int8, device=dev),
                      torch.empty((x.shape[0], x.shape[1] // 32), dtype=torch.int32, device=dev))
                  for s, x in xs.items()}
        odt = torch.float16 if args.f16_out else torch.float32
        outs = [torch.empty((xs[src].shape[0], m), dtype=odt, device=dev)
                for _, _, m, _, src in ws]
        sets.append((xs, ws, qs, outs))
    torch.cuda.synchronize()

    n_tok = max(x.shape[0] for x in inputs.values())
    mmq_ops = sum(2.0 * inputs[src].shape[0] * f.m * f.k for _, f, src in mats)
    out_bytes = 2.0 if args.f16_out else 4.0
    wbytes = (lambda f: 2368.0 / 4096.0) if desc.get("repacked") else (lambda f: weight_format(f)[1])
    act_bytes = 2.125 if desc.get("tiles") else 1.125   # binary16 tiles or int8 codes, + scale words
    mmq_alg_bytes = sum(wbytes(f) * f.m * f.k + act_bytes * inputs[src].shape[0] * f.k
                        + out_bytes * inputs[src].shape[0] * f.m for _, f, src in mats)
    suffix = "_f16out" if args.f16_out else "_fp32out"
    names = sorted({weight_format(f)[2] + suffix for _, f, _ in mats})
    if desc.get("repacked"):
        if args.f16_out:
            raise SystemExit("the repacked layout has a float32 entry point only")
        names = ["mmq_q4kr_q8_fp32out"]
    if desc.get("tiles"):
        if args.f16_out:
            raise SystemExit("the operand-tile entry points are float32 only")
        names = ["mmq_q4kr_q8t_fp32out" if desc.get("repacked") else
                 "mmq_q6k_q8t_fp32out" if isinstance(mats[0][1], synth.Q6KFields) else "mmq_q4k_q8t_fp32out"]
    mmq_name = "+".join(names)
    calls = [getattr(binding, names[0] if desc.get("repacked") or desc.get("tiles")
                     else weight_format(f)[2] + suffix)
             for _, f, _ in mats]
    raw_names = [names[0] if desc.get("repacked") or desc.get("tiles") else weight_format(f)[2] + suffix
                 for _, f, _ in mats]
    raw_extra = [() for _ in mats]
    if desc.get("kernel"):   # the named kernel through the fold entry point
        kid = {v: k for k, v in binding.KERNEL_NAMES.items()}[desc["kernel"]]
        raw_names = [weight_format(f)[2] + "_fold" for _, f, _ in mats]
        raw_extra = [(int(args.f16_out), kid) for _ in mats]

        def named(fold):
            return lambda w, m, k, q, ds, n, out: fold(w, m, k, q, ds, kid, f16=args.f16_out, out=out)
        calls = [named(binding.q6k_fold_kernel if isinstance(f, synth.Q6KFields) else binding.fold_kernel)
                 for _, f, _ in mats]
        mmq_name = "+".join(sorted({weight_format(f)[2] + "_fold" for _, f, _ in mats})) + ":" + desc["kernel"]
    quantize = binding.q8_quantize_rows_tiled if desc.get("tiles") else binding.q8_quantize_rows
    quantize_name = "q8_quantize_rows_tiled" if desc.get("tiles") else "q8_quantize_rows"

    def step(i):
        xs, ws, qs, outs = sets[i % len(sets)]
        for s, x in xs.items():
            q, ds = qs[s]
            quantize(x, x.shape[0], x.shape[1], q, ds)
        for (lbl, w, m, k, src), out, mmq in zip(ws, outs, calls):
            q, ds = qs[src]
            mmq(w, m, k, q, ds, ds.shape[0], out)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Duration of the dominant kernel (the MMQ entry point) with HIP events on
    # the stream it runs on: R rounds of every projection's MMQ, back to back,
    # enqueued behind R untimed rounds of the same launches, R sized to about
    # 25 ms of GPU time each way.  The clocks settle over some 10-20 ms of
    # sustained load after an idle gap (a one-wave spin before the events, or
    # too few rounds, measured the ramp: q-proj 206-209 us per launch over
    # 20 rounds after a spin, 175-177 us after 200 warm rounds).  The calls
    # are marshalled once, so the host enqueues a launch faster than the GPU
    # runs one and host launch latency is not counted.
    ms_step = wall * 1e3 / args.steps
    rounds = int(min(4000, max(args.steps, 10, math.ceil(25.0 / max(ms_step, 1e-3)))))
    stream = torch.cuda.current_stream()

    raw = []
    for xs, ws, qs, outs in sets:
        raw.append([raw_call(nm, (w, m, k, qs[src][0], qs[src][1], qs[src][1].shape[0], out) + ex)
                    for (lbl, w, m, k, src), out, nm, ex in zip(ws, outs, raw_names, raw_extra)])

    def mmq_round(i):
        for call in raw[i % len(raw)]:
            call()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(rounds):
        mmq_round(i)
    e0.record(stream)
    for i in range(rounds):
        mmq_round(i)
    e1.record(stream)
    torch.cuda.synchronize()
    mmq_ms = e0.elapsed_time(e1) / rounds          # all projections of one step

    value = mmq_ops / (ms_step * 1e-3) / 1e12
    achieved_tops = mmq_ops / (mmq_ms * 1e-3) / 1e12
    alg_gbs = mmq_alg_bytes / (mmq_ms * 1e-3) / 1e9
    few_tokens = n_tok <= 64
    dtypes = sorted({compute_dtype(desc, f, inputs[src].shape[0]) for _, f, src in mats})
    dtype = "+".join(dtypes)
    kernels = {lbl: compute_dtype(desc, f, inputs[src].shape[0]) for lbl, f, src in mats}
    srcs = sorted({kernel_source(desc, f, inputs[src].shape[0]) for _, f, src in mats})
    if few_tokens:   # weights streamed once: HBM roofline
        roof = {"bound": "hbm", "achieved": round(alg_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(alg_gbs / HBM_PEAK_GBS, 4)}
    else:
        # the method's int8 MACs (2 N M K ops) against the dense int8 MFMA
        # peak; above 64 tokens the contraction runs on binary16 MFMA with
        # exact integer operands, whose own peak is half that: its fraction
        # is reported beside it
        roof = {"bound": "mfma", "achieved": round(achieved_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                "frac": round(achieved_tops / INT8_PEAK_TOPS, 4),
                "f16_peak_frac": round(achieved_tops / F16_PEAK_TFLOPS, 4)}
    roof.update({
        "kernel": mmq_name,
        "traffic": measured_traffic(mmq_name + "|" + workload, srcs[0]) if len(srcs) == 1 else None,
        "avg_launch_us": round(mmq_ms * 1e3 / len(mats), 2),
        "launches_timed": rounds * len(mats),
        "alg_bytes_per_step": mmq_alg_bytes,
        "alg_gbs": round(alg_gbs, 1),
        "int8_tops": round(achieved_tops, 2)})
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": dict(desc, step="%s + %s per projection" % (quantize_name, mmq_name),
                       copies=len(sets)),
        "tok_per_s": round(n_tok / (ms_step * 1e-3), 1),
        "pct_int8_peak": round(100.0 * value / INT8_PEAK_TOPS, 2),
        "kernels": kernels,
        "roofline": roof,
    }
    base = workload
    while base[:2] in ("t_", "r_"):
        base = base[2:]
    if base.startswith("layer"):
        # prefill tok/s over the projections of a 7B model: N tokens through
        # 32 layers' steps
        res["tok_per_s_7b_projections"] = round(n_tok / (LAYERS * ms_step * 1e-3), 1)
    del sets
    torch.cuda.empty_cache()
    return res, mats, inputs


if __name__ == "__main__":
    main()
