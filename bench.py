"""Benchmark of the attention hot path on one MI355X.

Headline: attention TFLOP/s (4*B*H*Sq*Skv*d / time) of the bf16 forward pass on
the FLUX-like workload (B1 H24 S16896 d128), with inputs already resident in
HBM.  A step is one dit_attn_fwd_ws call over the whole workload: the forward
kernel, whose last partial wave of query tiles is split over the keys, and the
small kernel that merges those pieces (workspace allocated once, before timing).
The step's average duration is measured with HIP events on the stream it runs
on, and compared with MI355X's dense bf16 MFMA peak (2.5 PFLOP/s).  The fp64 CPU
oracle is timed on a bounded sample of the same workload (cpu_baseline).

Extra lines of the hot path (fp8 forward with its quantiser, the SD3-like and
tiny shapes, and one ring rank's share: four chunk forwards + the LSE-merge) are
timed the same way and reported under "extras".

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
# rocprofv3 summary of the dominant kernel and the sources it was taken from;
# its traffic figure is reported only while those sources are unchanged
PROFILE = os.path.join(ROOT, "profiles", "fwd_bf16_d128_flux.md")
PROFILE_SOURCES = ("attention_non_causal_amd/csrc/fwd_bf16_d128.hip",
                   "attention_non_causal_amd/csrc/common.hpp")
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def to_dev(bits, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def host_info():
    """Host CPU model, ROCm version and HIP runtime of this run."""
    import torch
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    return {"cpu_model": cpu, "host_threads": len(os.sched_getaffinity(0)),
            "rocm_version": rocm, "hip_runtime": torch.version.hip}


def _smi_market_name():
    """The GPU's product name from amd-smi (torch reports a generic one), or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "static", "-g", "0", "-a", "--json"], capture_output=True,
                           text=True, timeout=10)
        data = json.loads(r.stdout) if r.returncode == 0 else None
    except (OSError, subprocess.TimeoutExpired, ValueError):
        return None
    found = []

    def walk(x):
        if isinstance(x, dict):
            for k, v in x.items():
                if k == "market_name" and isinstance(v, str) and v.strip():
                    found.append(v.strip())
                walk(v)
        elif isinstance(x, list):
            for v in x:
                walk(v)
    walk(data)
    return found[0] if found else None


def _smi_gfx_clock_mhz():
    """The GPU's current shader (gfx) clock in MHz from amd-smi, or None."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True,
                           text=True, timeout=10)
    except (OSError, subprocess.TimeoutExpired):
        return None
    if r.returncode != 0:
        return None
    try:
        data = json.loads(r.stdout)
    except ValueError:
        return None
    # the "gfx_*" entries of the clock section; each has a current clock value
    vals = []

    def walk(x, key=""):
        if isinstance(x, dict):
            for k, v in x.items():
                walk(v, f"{key}/{k}")
        elif isinstance(x, list):
            for v in x:
                walk(v, key)
        elif re.search(r"gfx_?\d*/clk$", key) and isinstance(x, (int, float)):
            vals.append(float(x))
        elif re.search(r"gfx_?\d*/clk/value$", key) and isinstance(x, (int, float)):
            vals.append(float(x))
    walk(data)
    return float(sum(vals) / len(vals)) if vals else None


def sustained_clock(fn, seconds):
    """Run fn() back to back for `seconds` (untimed, after the measurement)
    while a host thread samples the shader clock with amd-smi; returns
    (median MHz over the samples, number of samples) or (None, 0)."""
    import threading
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        time.sleep(0.2)  # let the load start
        while not stop.is_set():
            c = _smi_gfx_clock_mhz()
            if c is None:
                return
            samples.append(c)
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if not samples:
        return None, 0
    samples.sort()
    return samples[len(samples) // 2], len(samples)


def settle(fn, seconds):
    """Keep calling fn() for `seconds` of wall time (in batches of 8 between
    synchronisations).  After a pause -- input generation on the host -- the
    shader clock takes ~0.1 s of load to settle, longer than a few warmup
    calls of a short kernel."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_launches(fn, steps, warmup, min_warm_s=0.0):
    """Run fn() warmup times, then time `steps` calls: returns (wall ms per call
    between two synchronisations, list of per-call event ms on torch's current
    stream, which is the stream the library launches on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    settle(fn, min_warm_s)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, [a.elapsed_time(b) for a, b in ev]


def time_batched(fn, steps, warmup, min_warm_s=0.0):
    """ms per call of a short launch: one event pair around `steps` back-to-back
    calls on torch's current stream (per-call event pairs would mostly measure
    launch gaps for kernels of a few tens of microseconds)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    settle(fn, min_warm_s)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def time_graph(fn, calls, replays, settle_s):
    """ms per call of `calls` back-to-back fn() captured once into a HIP graph
    (torch.cuda.CUDAGraph captures the stream the library launches on) and
    replayed `replays` times between two events."""
    import torch
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    settle(graph.replay, settle_s)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (replays * calls)


def cpu_baseline(W, g, budget_s):
    """Time the fp64 oracle on a bounded sample of query rows (all heads, all
    keys) of the same workload; report its TFLOP/s."""
    import oracle
    from attention_non_causal_amd import workloads as wl
    # two-point calibration: a call has a fixed cost (decoding the bf16
    # tensors) plus a cost per query row
    t0 = time.perf_counter()
    oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=[0])
    t1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=list(range(1, 17)))
    t16 = time.perf_counter() - t0
    per_row = max((t16 - t1) / 15, 1e-4)
    fixed = max(t1 - per_row, 0.0)
    n = int(max(1, min(W.Sq, (budget_s - fixed) / per_row)))
    rows = wl.sample_rows(W.Sq, n)
    t0 = time.perf_counter()
    oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * W.B * W.H * len(rows) * W.Skv * W.d
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{len(rows)} of {W.Sq} query rows x all {W.H} heads x {W.Skv} keys "
                      f"(d{W.d}, fp64) in {dt:.1f} s"}


def profiled_traffic():
    """HBM bytes per launch from the committed rocprofv3 summary (FETCH_SIZE +
    WRITE_SIZE, each scaled by a plain-copy calibration), or None when the
    kernel sources have changed since it was taken."""
    import hashlib
    import re
    try:
        text = open(PROFILE).read()
    except OSError:
        return None
    h = hashlib.sha256()
    for src in PROFILE_SOURCES:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    m_sha = re.search(r"source_sha256: ([0-9a-f]+)", text)
    m_tr = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    if not m_sha or not m_tr or not h.hexdigest().startswith(m_sha.group(1)):
        return None
    return int(m_tr.group(1))


def bench_fwd(W, g, dev, steps, warmup):
    import torch
    from attention_non_causal_amd import functional as F
    q, k, v = to_dev(g["q"], dev), to_dev(g["k"], dev), to_dev(g["v"], dev)
    o = torch.empty_like(q)
    lse = torch.empty((W.B, W.H, W.Sq), dtype=torch.float32, device=dev)
    ws = F.workspace_for(q, k)  # scratch of the split launch, allocated before timing
    fn = lambda: F.attention(q, k, v, W.scale, out=o, lse=lse, workspace=ws)
    # the first launch on the fresh inputs (code object load, cold caches), timed alone
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    fn()
    b.record(stream)
    torch.cuda.synchronize()
    cold = a.elapsed_time(b)
    wall, evs = time_launches(fn, steps, warmup)
    return wall, evs, cold, fn


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="flux")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for cpu_baseline (0: skip)")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of back-to-back calls before each extra is timed, so the "
                         "shader clock has settled (0: only the warmup calls)")
    ap.add_argument("--clock-seconds", type=float, default=1.5,
                    help="seconds of back-to-back steps after the timed ones while amd-smi "
                         "samples the shader clock (0: skip, and run no amd-smi at all: "
                         "under rocprofv3 --pmc the GPU is initialised before the program "
                         "starts, and amd-smi re-executes itself)")
    ap.add_argument("--fp8-rows", type=int, default=64,
                    help="query rows of the fp8 workloads compared with the oracle in the "
                         "cpu_baseline leg")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the benchmark: the dense matrix-core throughput this GPU "
                         "sustains (bf16 and e4m3, random and all-zero operands; "
                         "libditprobe.so) and its shader clock meanwhile; one JSON line")
    ap.add_argument("--valu-issue", action="store_true",
                    help="instead of the benchmark: shader-clock cycles per wave64 vector "
                         "instruction of the softmax's kinds (exponential, FMA, addition, "
                         "bf16 and e4m3 packs) at one and two waves per SIMD "
                         "(libditprobe.so); one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain device-to-device copy of 1 GiB, whose HBM "
                         "counters calibrate FETCH_SIZE / WRITE_SIZE in a --pmc profile")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design, not a build", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from attention_non_causal_amd import workloads as wl
    from attention_non_causal_amd import functional as F

    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    if args.mfma_ceiling:
        print(json.dumps(mfma_ceiling(dev, props, clock_s=args.clock_seconds)), flush=True)
        return
    if args.valu_issue:
        print(json.dumps(valu_issue(dev, props)), flush=True)
        return
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: one 1 GiB device-to-device copy done")
        del src, dst
    W = wl.WORKLOADS[args.workload]
    log(f"{props.name}: {props.multi_processor_count} CUs; workload {W.name}: generating inputs")
    g = wl.generate(W)
    wall, evs, cold_ms, step_fn = bench_fwd(W, g, dev, args.steps, args.warmup)
    kern_ms = float(np.mean(evs))
    value = W.flops / (wall * 1e-3) / 1e12
    achieved = W.flops / (kern_ms * 1e-3) / 1e12
    log(f"fwd {W.name}: wall {wall:.3f} ms/step, event mean {kern_ms:.3f} ms "
        f"(median {float(np.median(evs)):.3f}, min {min(evs):.3f}, first launch "
        f"{cold_ms:.3f}) -> {achieved:.1f} TFLOP/s")

    # the shader clock this step sustains (after the timed steps; amd-smi
    # sampled from a host thread while the step runs back to back)
    clock_mhz, clock_n = (None, 0)
    if args.clock_seconds > 0:
        clock_mhz, clock_n = sustained_clock(step_fn, args.clock_seconds)
        log(f"sustained shader clock: {clock_mhz} MHz ({clock_n} amd-smi samples)")

    extras = {}
    fp8_outputs = None
    if not args.no_extras:
        extras, fp8_outputs = run_extras(dev, max(3, args.steps // 4), 2, args.settle)

    cpu = None
    if args.cpu_budget > 0:
        log("cpu_baseline: timing the oracle on a row sample")
        cpu = cpu_baseline(W, g, args.cpu_budget)
        log(f"cpu_baseline: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")
        if fp8_outputs is not None:
            extras["flux_fp8"].update(fp8_errors(fp8_outputs, args.fp8_rows))
            extras["flux_fp8_unit_normal"] = fp8_unit_normal_error(W, g, dev, args.fp8_rows)

    out = {
        "metric": "attention TFLOP/s & % of MFMA peak, B1 H24 S=16896 d128 bf16",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), Q/K RMS-normalised), no dataset or weights",
        "config": {"workload": W.description, "B": W.B, "H": W.H, "Sq": W.Sq, "Skv": W.Skv,
                   "d": W.d, "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic(), "traffic_unit": "bytes/launch",
                     "algorithmic_bytes": W.algorithmic_bytes,
                     "kernel": "fwd_bf16_d128_kernel (+ split_merge_kernel<128>, a few us)",
                     "kernel_ms": round(kern_ms, 4),
                     "kernel_ms_median": round(float(np.median(evs)), 4),
                     "kernel_ms_min": round(float(min(evs)), 4),
                     "first_launch_ms": round(cold_ms, 4)},
        "cpu_baseline": cpu,
        "device": {"name": (_smi_market_name() if args.clock_seconds > 0 else None) or props.name,
                   "torch_name": props.name,
                   "arch": getattr(props, "gcnArchName", None),
                   "cus": props.multi_processor_count,
                   "sustained_sclk_mhz": clock_mhz, "sclk_samples": clock_n,
                   "peak_basis": "2.5 PFLOP/s bf16 / 5.0 PFLOP/s fp8 dense at 2.4 GHz, "
                                 "256 CUs",
                   # context only (roofline.frac stays against the 2.4 GHz peak): the
                   # dense bf16 peak at the clock the part sustained under this load,
                   # and the achieved rate's fraction of it
                   "bf16_peak_at_sustained_sclk": (round(PEAK_BF16_TFLOPS * clock_mhz / 2400.0, 1)
                                                   if clock_mhz else None),
                   "frac_at_sustained_sclk": (round(achieved / (PEAK_BF16_TFLOPS * clock_mhz
                                                                / 2400.0), 4)
                                              if clock_mhz else None)},
        "host": host_info(),
        "extras": extras,
    }
    print(json.dumps(out), flush=True)


def mfma_ceiling(dev, props, launch_ms=100.0, timed=5, clock_s=1.5):
    """The matrix cores' sustained throughput on this GPU: the probe kernel
    (attention_non_causal_amd/probe/mfma_ceiling.hip, two waves per SIMD, 16
    MFMAs per loop turn, operands changing every instruction) for bf16
    32x32x16 and e4m3 32x32x64 on N(0,1) data and on zeros, and bf16 16x16x32
    on N(0,1) data, in rotation and in chains of four dependent instructions.  Each case:
    0.3 s of launches to settle the clock, then `timed` launches of about
    launch_ms each between events, then clock_s seconds more while amd-smi
    samples the shader clock (0: none)."""
    import ctypes
    import numpy as np
    import torch
    from attention_non_causal_amd import build as libbuild
    from attention_non_causal_amd import functional as F
    if not os.path.exists(libbuild.PROBE_LIB_PATH):
        raise SystemExit(f"{libbuild.PROBE_LIB_PATH} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(libbuild.PROBE_LIB_PATH)
    lib.dit_probe_mfma_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.dit_probe_mfma_ceiling.restype = ctypes.c_int
    n_blocks = 2 * props.multi_processor_count
    out = torch.empty(n_blocks * 256, dtype=torch.float32, device=dev)
    rng = np.random.default_rng(42)
    # operand data: 4096 words; bf16 N(0,1) bits, or e4m3 codes of N(0,1)
    # values from the library's own quantiser (per-128-token-block scaled)
    bf = torch.from_numpy(rng.standard_normal(8192).astype(np.float32)).to(torch.bfloat16)
    src_bf16 = bf.view(torch.int16).to(dev).view(torch.int32).contiguous()
    x = torch.from_numpy(rng.standard_normal(16384).astype(np.float32)).to(torch.bfloat16)
    x8, _ = F.quantize_fp8(x.reshape(1, 128, 1, 128).to(dev))
    src_fp8 = x8.reshape(-1).view(torch.int32).contiguous()
    zeros = torch.zeros(4096, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    res = {"n_blocks": n_blocks, "waves_per_simd": 2}
    for name, kind, src, flop in (("bf16_random", 0, src_bf16, 2 * 32 * 32 * 16),
                                  ("bf16_zeros", 0, zeros, 2 * 32 * 32 * 16),
                                  ("bf16_16x16x32_random", 2, src_bf16, 2 * 16 * 16 * 32),
                                  ("bf16_16x16x32_chains_random", 3, src_bf16, 2 * 16 * 16 * 32),
                                  ("fp8_random", 1, src_fp8, 2 * 32 * 32 * 64),
                                  ("fp8_zeros", 1, zeros, 2 * 32 * 32 * 64)):
        def launch(iters):
            st = lib.dit_probe_mfma_ceiling(src.data_ptr(), out.data_ptr(), n_blocks, iters,
                                            kind, stream)
            assert st == 0, f"probe launch failed: HIP status {st}"
        # size the launch: time a short one after the clock has settled
        settle(lambda: launch(2000), 0.3)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch(2000)
        b.record()
        torch.cuda.synchronize()
        iters = max(1, int(2000 * launch_ms / a.elapsed_time(b)))
        settle(lambda: launch(iters), 0.3)
        evs = []
        for _ in range(timed):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            launch(iters)
            b.record()
            torch.cuda.synchronize()
            evs.append(a.elapsed_time(b))
        ms = float(np.median(evs))
        flops = n_blocks * 4 * 16 * iters * flop
        mhz, n = (sustained_clock(lambda: launch(iters // 10 or 1), clock_s) if clock_s > 0
                  else (None, 0))
        res[name] = {"tflops": round(flops / ms / 1e9, 1), "launch_ms": round(ms, 3),
                     "iters": iters, "sustained_sclk_mhz": mhz, "sclk_samples": n}
        log(f"mfma ceiling {name}: {res[name]['tflops']} TFLOP/s ({ms:.3f} ms per launch of "
            f"{iters} loop turns), shader clock {mhz} MHz")
    return {"mfma_ceiling": res, "device": {"name": props.name,
                                            "arch": getattr(props, "gcnArchName", None),
                                            "cus": props.multi_processor_count}}


def valu_issue(dev, props, iters=512):
    """Cycles a SIMD spends per wave64 vector instruction, by kind, at one and
    two waves per SIMD: the probe kernel (attention_non_causal_amd/probe/
    valu_issue.hip) runs `iters` turns of 16 independent instructions per wave
    and times them with s_memtime; the figure is the median wave's cycles /
    (instructions per wave x waves per SIMD).  One warm launch per case, then
    the measured one."""
    import ctypes
    import numpy as np
    import torch
    from attention_non_causal_amd import build as libbuild
    if not os.path.exists(libbuild.PROBE_LIB_PATH):
        raise SystemExit(f"{libbuild.PROBE_LIB_PATH} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(libbuild.PROBE_LIB_PATH)
    lib.dit_probe_valu_issue.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.dit_probe_valu_issue.restype = ctypes.c_int
    n_blocks = props.multi_processor_count
    out = torch.zeros(n_blocks * 8, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    res = {"n_blocks": n_blocks, "instructions_per_wave": 16 * iters,
           "unit": "shader-clock cycles per wave64 instruction per SIMD"}
    for name, kind in (("v_exp_f32", 0), ("v_fma_f32", 1), ("v_add_f32", 2),
                       ("v_cvt_pk_bf16_f32", 3), ("v_cvt_pk_fp8_f32", 4),
                       ("v_exp_f32+v_fma_f32 alternating", 5)):
        res[name] = {}
        for waves in (4, 8):
            for _ in range(2):
                st = lib.dit_probe_valu_issue(out.data_ptr(), n_blocks, waves, iters, kind, stream)
                assert st == 0, f"probe launch failed: HIP status {st}"
            torch.cuda.synchronize()
            cyc = out[: n_blocks * waves].cpu().numpy()
            per_simd = waves // 4
            res[name][f"{per_simd}_wave_per_simd"] = round(
                float(np.median(cyc)) / (16 * iters * per_simd), 2)
        log(f"valu issue {name}: {res[name]}")
    return {"valu_issue": res, "device": {"name": props.name,
                                          "arch": getattr(props, "gcnArchName", None),
                                          "cus": props.multi_processor_count}}


def run_extras(dev, steps, warmup, settle_s):
    import numpy as np
    import torch
    from attention_non_causal_amd import _lib, functional as F
    from attention_non_causal_amd import workloads as wl
    res = {}
    for name in ("tiny", "sd3", "flux_h3"):
        W = wl.WORKLOADS[name]
        g = wl.generate(W)
        q, k, v = to_dev(g["q"], dev), to_dev(g["k"], dev), to_dev(g["v"], dev)
        o = torch.empty_like(q)
        lse = torch.empty((W.B, W.H, W.Sq), dtype=torch.float32, device=dev)
        ws = F.workspace_for(q, k)
        ms = time_batched(lambda: F.attention(q, k, v, W.scale, out=o, lse=lse, workspace=ws),
                          4 * steps, warmup, settle_s)
        res[name] = {"kernel_ms": round(ms, 4), "tflops": round(W.flops / ms / 1e9, 1)}
        log(f"extra {name}: {ms:.3f} ms, {res[name]['tflops']} TFLOP/s")
        if name == "tiny":
            # a launch-bound shape: the same calls replayed from one captured
            # HIP graph (no host work per call) against issuing them eagerly
            gms = time_graph(lambda: F.attention(q, k, v, W.scale, out=o, lse=lse, workspace=ws),
                             16, max(1, steps // 4), settle_s)
            res[name]["graph_ms_per_call"] = round(gms, 4)
            log(f"extra {name}: {gms:.4f} ms per call replayed from a graph of 16 calls")

    W = wl.WORKLOADS["wan_ring"]
    g = wl.generate(W)
    q, k, v = to_dev(g["q"], dev), to_dev(g["k"], dev), to_dev(g["v"], dev)
    del g
    parts = ([torch.empty_like(q) for _ in range(W.n_chunks)],
             [torch.empty((1, W.H, W.Sq), dtype=torch.float32, device=dev)
              for _ in range(W.n_chunks)])
    o = torch.empty_like(q)
    lse = torch.empty((1, W.H, W.Sq), dtype=torch.float32, device=dev)
    wall, evs = time_launches(
        lambda: F.ring_share_attention(q, k, v, W.n_chunks, W.scale, parts=parts, out=o, lse=lse),
        steps, warmup, settle_s)
    # medians: one slow call (a clock dip, a page of the inputs faulting in)
    # moves a mean of a handful of calls by several percent
    ms = float(np.median(evs))
    mms = time_batched(lambda: F.merge(parts[0], parts[1], out=o, lse=lse), 4 * steps, warmup,
                       settle_s)
    merge_bytes = W.n_chunks * (W.Sq * W.H * W.d * 2 + W.H * W.Sq * 4) + W.Sq * W.H * W.d * 2 \
        + W.H * W.Sq * 4
    # the same share as a ring loop runs it: each chunk merged into the running
    # result by dit_attn_fwd_acc (no partial outputs, no separate merge)
    nws = _lib.dit_attn_fwd_workspace_size(1, W.H, W.Sq, W.chunk, W.d)
    aws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    _, aevs = time_launches(
        lambda: F.ring_share_attention_acc(q, k, v, W.n_chunks, W.scale, out=o, lse=lse,
                                           workspace=aws),
        steps, warmup, settle_s)
    ams = float(np.median(aevs))
    res["wan_ring"] = {"total_ms": round(ms, 4), "tflops": round(W.flops / ms / 1e9, 1),
                       "merge_ms": round(mms, 4),
                       "merge_GBs": round(merge_bytes / mms / 1e6, 1),
                       "acc_total_ms": round(ams, 4), "acc_tflops": round(W.flops / ams / 1e9, 1)}
    log(f"extra wan_ring: {ms:.3f} ms total ({res['wan_ring']['tflops']} TFLOP/s), merge "
        f"{mms:.3f} ms = {res['wan_ring']['merge_GBs']} GB/s; merged as it runs "
        f"(dit_attn_fwd_acc) {ams:.3f} ms ({res['wan_ring']['acc_tflops']} TFLOP/s)")
    del q, k, v, parts, o, lse

    # fp8: the FLUX-like shape with 1% x8 outlier channels, quantised per
    # (head, 128-token block); attention alone vs the fp8 peak, and the layer
    # (three quantiser launches + attention)
    W = wl.WORKLOADS["flux_fp8"]
    g = wl.generate(W)
    q, k, v = to_dev(g["q"], dev), to_dev(g["k"], dev), to_dev(g["v"], dev)
    nblk = (W.Skv + 127) // 128
    bufs = {n: (torch.empty(t.shape, dtype=torch.uint8, device=dev),
                torch.empty((W.B, W.H, nblk), dtype=torch.float32, device=dev))
            for n, t in (("q", q), ("k", k), ("v", v))}
    o = torch.empty_like(q)
    lse = torch.empty((W.B, W.H, W.Sq), dtype=torch.float32, device=dev)

    def quant_all():
        for n, t in (("q", q), ("k", k), ("v", v)):
            _lib.dit_quant_fp8(t, bufs[n][0], bufs[n][1], W.B, W.H, t.shape[1], W.d)

    ws8 = F.workspace_for(bufs["q"][0], bufs["k"][0], _lib.DIT_DTYPE_FP8_E4M3)

    def attn_fp8():  # the split launch, scratch allocated before timing
        F.attention_fp8(bufs["q"][0], bufs["q"][1], bufs["k"][0], bufs["k"][1], bufs["v"][0],
                        bufs["v"][1], W.scale, out=o, lse=lse, workspace=ws8)

    quant_all()
    torch.cuda.synchronize()
    qms = time_batched(lambda: _lib.dit_quant_fp8(k, bufs["k"][0], bufs["k"][1], W.B, W.H,
                                                   W.Skv, W.d), 4 * steps, warmup, settle_s)
    qbytes = W.B * W.Skv * W.H * W.d * 3 + nblk * W.B * W.H * 4
    res["quant_fp8"] = {"kernel_ms": round(qms, 4), "GBs": round(qbytes / qms / 1e6, 1)}
    log(f"extra quant_fp8 (one tensor): {qms:.4f} ms = {res['quant_fp8']['GBs']} GB/s")
    _, aevs = time_launches(attn_fp8, steps, warmup, settle_s)
    ams = float(np.median(aevs))
    _, levs = time_launches(lambda: (quant_all(), attn_fp8()), steps, warmup, settle_s)
    lms = float(np.median(levs))
    res["flux_fp8"] = {"kernel_ms": round(ams, 4), "tflops": round(W.flops / ams / 1e9, 1),
                       "pct_of_fp8_peak": round(100 * W.flops / ams / 1e9 / PEAK_FP8_TFLOPS, 2),
                       "layer_ms_with_quant": round(lms, 4),
                       "layer_tflops_with_quant": round(W.flops / lms / 1e9, 1)}
    log(f"extra flux_fp8: attention {ams:.3f} ms = {res['flux_fp8']['tflops']} TFLOP/s "
        f"({res['flux_fp8']['pct_of_fp8_peak']}% of fp8 peak); with 3 quantiser launches "
        f"{lms:.3f} ms")
    # the outputs of the last timed call (the path is deterministic), kept for
    # the comparison with the oracle in the cpu_baseline leg
    torch.cuda.synchronize()
    fp8_out = {"W": W, "g": g, "o": o.float().cpu().numpy(), "lse": lse.cpu().numpy(),
               "q8": bufs["q"][0].cpu().numpy(), "qs": bufs["q"][1].cpu().numpy(),
               "k8": bufs["k"][0].cpu().numpy(), "ks": bufs["k"][1].cpu().numpy(),
               "v8": bufs["v"][0].cpu().numpy(), "vs": bufs["v"][1].cpu().numpy()}
    return res, fp8_out


def fp8_errors(out, n_rows):
    """cpu_baseline leg, outside any timed region: the fp8 path's output on the
    x8-outlier FLUX-like workload against the oracle on sampled query rows (all
    heads and keys) -- max|dO| and max|dLSE| against the oracle on the
    unquantised bf16 inputs (the path's total error), against the oracle on
    the dequantised inputs (the kernel's own error), and the quantisation
    floor (the two oracles against each other)."""
    import numpy as np
    import oracle
    from attention_non_causal_amd import workloads as wl
    W, g = out["W"], out["g"]
    rows = wl.sample_rows(W.Sq, n_rows)
    log(f"flux_fp8 vs oracle on {len(rows)} rows")
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=rows)
    deq = [oracle.dequant_fp8(out[n + "8"], out[n + "s"]) for n in "qkv"]
    o_dq, l_dq = oracle.attn_fwd(deq[0], deq[1], deq[2], W.scale, rows=rows)
    o, l = out["o"][:, rows].astype(np.float64), out["lse"][:, :, rows].astype(np.float64)
    r = {"oracle_rows": int(len(rows)),
         "max_dO_vs_unquantised": float(np.abs(o - o_ref).max()),
         "max_dLSE_vs_unquantised": float(np.abs(l - l_ref).max()),
         "max_dO_vs_dequantised": float(np.abs(o - o_dq).max()),
         "max_dLSE_vs_dequantised": float(np.abs(l - l_dq).max()),
         "floor_max_dO": float(np.abs(o_dq - o_ref).max()),
         "floor_max_dLSE": float(np.abs(l_dq - l_ref).max())}
    log(f"flux_fp8 errors: {r}")
    return r


def fp8_unit_normal_error(W, g, dev, n_rows):
    """cpu_baseline leg: the fp8 path (quantiser + split forward) on the
    unit-normal FLUX-like inputs against the oracle on the unquantised inputs
    -- the 6e-2 gate -- on sampled rows, with the quantisation floor."""
    import numpy as np
    import oracle
    import torch
    from attention_non_causal_amd import functional as F
    from attention_non_causal_amd import workloads as wl
    q, k, v = to_dev(g["q"], dev), to_dev(g["k"], dev), to_dev(g["v"], dev)
    q8, qs = F.quantize_fp8(q)
    k8, ks = F.quantize_fp8(k)
    v8, vs = F.quantize_fp8(v)
    o, lse = F.attention_fp8(q8, qs, k8, ks, v8, vs, W.scale)
    torch.cuda.synchronize()
    rows = wl.sample_rows(W.Sq, n_rows)
    log(f"flux fp8 unit-normal vs oracle on {len(rows)} rows")
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=rows)
    deq = [oracle.dequant_fp8(a.cpu().numpy(), b.cpu().numpy())
           for a, b in ((q8, qs), (k8, ks), (v8, vs))]
    o_dq, _ = oracle.attn_fwd(deq[0], deq[1], deq[2], W.scale, rows=rows)
    og = o.float().cpu().numpy()[:, rows].astype(np.float64)
    lg = lse.cpu().numpy()[:, :, rows].astype(np.float64)
    r = {"oracle_rows": int(len(rows)), "max_dO_vs_unquantised": float(np.abs(og - o_ref).max()),
         "max_dLSE_vs_unquantised": float(np.abs(lg - l_ref).max()),
         "floor_max_dO": float(np.abs(o_dq - o_ref).max()), "gate_max_dO": 6e-2}
    log(f"flux fp8 unit-normal errors: {r}")
    return r


if __name__ == "__main__":
    main()
