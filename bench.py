#!/usr/bin/env python3
"""Benchmark of fused exact attention on one MI355X.

A step is one pass of the whole hot path over one batch: fa_fwd (O, LSE)
followed by fa_bwd (dQ, dK, dV) on the fwd+bwd workload (B=2, H=16, N=2048,
d=128, causal; the only workload with a backward pass). ``--workload 1..4``
times the forward-only workloads instead (the causal d=128 long-sequence
forwards are 3 and 4).

Prints ONE JSON line. ``value`` is algorithmic TFLOP/s over the timed steps
(forward 4*B*H*N^2*d, backward 10*B*H*N^2*d, each halved when causal) with
inputs resident in HBM. ``roofline`` describes the dominant launch, timed with
HIP events on the stream the kernels run on (on every fourth timed step by
default: events on every step add 4-6 % to the step time). ``cpu_baseline`` times the fp64
oracle on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOP/s (bf16, d=128) and % of MI355X bf16 MFMA peak"


# Child process that polls the GPU clock (amdsmi, per-XCD current gfxclk) every
# ~0.3 ms until its stdin closes, then prints the samples as JSON. It is
# started before this process touches the GPU and never touches it itself.
_CLOCK_POLLER = r"""
import json, select, sys, time
try:
    import amdsmi
    amdsmi.amdsmi_init()
    h = amdsmi.amdsmi_get_processor_handles()[0]
except Exception as e:
    print(json.dumps({"error": repr(e)}), flush=True)
    sys.exit(0)
print("ready", flush=True)
samples = []
while True:
    r, _, _ = select.select([sys.stdin], [], [], 0)
    if r:
        break
    try:
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        c = [x for x in m.get("current_gfxclks", []) if isinstance(x, (int, float))]
        if not c and isinstance(m.get("current_gfxclk"), (int, float)):
            c = [m["current_gfxclk"]]
        if c:
            samples.append((time.monotonic(), sum(c) / len(c)))
    except Exception:
        pass
    time.sleep(0.0002)
amdsmi.amdsmi_shut_down()
print(json.dumps({"samples": samples}), flush=True)
"""


class ClockPoller:
    """GPU shader-clock samples in named time windows (time.monotonic).

    ``mark(name, t0, t1)`` records a window; ``finish()`` stops the poller and
    returns {name: {"mean", "min", "max", "samples"}} for each window (None
    when the clock cannot be read)."""

    def __init__(self):
        import subprocess
        self.windows = []
        self.proc = None
        try:
            self.proc = subprocess.Popen([sys.executable, "-c", _CLOCK_POLLER],
                                         stdin=subprocess.PIPE, stdout=subprocess.PIPE,
                                         stderr=subprocess.DEVNULL, text=True)
            line = self.proc.stdout.readline().strip()
            if line != "ready":
                self.proc.wait(timeout=10)
                self.proc = None
        except Exception:
            self.proc = None

    def mark(self, name, t0, t1):
        self.windows.append((name, t0, t1))

    def finish(self):
        if self.proc is None:
            return {name: None for name, _, _ in self.windows}
        try:
            out, _ = self.proc.communicate(input="stop\n", timeout=30)
            samples = json.loads(out.strip().splitlines()[-1]).get("samples", [])
        except Exception:
            return {name: None for name, _, _ in self.windows}
        res = {}
        for name, t0, t1 in self.windows:
            xs = [c for t, c in samples if t0 <= t <= t1]
            res[name] = ({"mean": round(sum(xs) / len(xs), 1), "min": min(xs), "max": max(xs),
                          "samples": len(xs)} if xs else None)
        return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--warmup-min-s", type=float, default=0.25,
                   help="after the --warmup steps, keep warming up (whole steps, untimed) "
                        "until this much wall time has passed (0 disables)")
    p.add_argument("--event-every", type=int, default=4,
                   help="record the per-launch HIP events on every n-th timed step only "
                        "(default 4; 1 = every step, which adds 4-6 %% to the step time)")
    p.add_argument("--no-clock-soak", action="store_true",
                   help="skip the untimed runs after each timed loop that let the SMU's clock "
                        "reading settle (for profiler runs: the trace then holds only the "
                        "warm-up, timed and cold calls; sclk fields become null)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate CPU time budget of the oracle sample")
    p.add_argument("--copy-calib-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration)")
    p.add_argument("--fwd-shape", default=None, metavar="B,H,N,d,causal",
                   help="instead of the fused step, time the forward alone on seeded N(0,1) "
                        "bf16 inputs of this shape (scale 1/sqrt(d)) and print one JSON line")
    p.add_argument("--decode", choices=["d1", "d8"], default=None,
                   help="instead of the fused step, time decode attention (Nq query rows "
                        "against a KV cache) on this decode workload; HBM-bound")
    p.add_argument("--unfused", action="store_true",
                   help="also time the unfused comparator (S and P in device memory) on the "
                        "same forward inputs and report the fused forward's speedup over it")
    p.add_argument("--fa1", action="store_true",
                   help="also time the loop-order comparator (outer loop over key/value "
                        "tiles, one workgroup per head) on the same forward inputs")
    p.add_argument("--persistent", action="store_true",
                   help="also time the persistent-grid comparator (at most two resident "
                        "workgroups per CU looping over the query tiles in a static snake "
                        "order) on the same forward inputs")
    p.add_argument("--oracle-all", action="store_true",
                   help="instead of the GPU step, time the oracle (as it stands) on every "
                        "workload in full on the host cores: median of 3 runs for workloads "
                        "1-2, one run for 3-5; one JSON line")
    p.add_argument("--no-long-fwd", action="store_true",
                   help="skip the causal d=128 long-sequence forwards (workloads 3 and 4) "
                        "that the default fwd+bwd run also times")
    return p.parse_args()


def fwd_bytes(w):
    n = w.B * w.H * w.N
    return 4 * n * w.d * 2 + 4 * n


def bwd_bytes(w):
    n = w.B * w.H * w.N
    return 5 * n * w.d * 2 + 4 * n + 8 * n + 3 * n * w.d * 2


def recorded_traffic(workload_idx, launch):
    """HBM bytes per launch from the committed counter record, or None when the
    kernel sources changed since the counters were taken (hash mismatch)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{launch}_workload{workload_idx}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    csrc = os.path.join(ROOT, "exact_io_aware_12_amd", "csrc")
    srcs = "".join(open(os.path.join(csrc, f)).read()
                   for f in ("fa_common.h", "fa_fwd.hip", "fa_bwd.hip"))
    if hashlib.sha256(srcs.encode()).hexdigest()[:16] != rec.get("sources_sha256_16"):
        return None
    return rec["read_bytes"] + rec["write_bytes"]


def median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def clock_soak(clock, name, fn, torch, seconds):
    """Run `fn` back to back, untimed, for `seconds` and mark the last half as
    window `name`. The SMU's clock reading (amdsmi) lags the load by up to about
    a second and updates in steps, so a timed loop of a few tens of ms reads
    the level of whatever ran before it; the soak gives it time to settle on
    the clock this work runs at."""
    s0 = time.monotonic()
    while time.monotonic() - s0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    clock.mark(name, s0 + seconds / 2, time.monotonic())


def long_forwards(fa, torch, fi, dev, clock, soak, warmup=20, calls=50, warmup_min_s=0.25):
    """The causal d=128 forwards at N >= 4096 (workloads 3 and 4), where the
    >= 50 %-of-peak forward target is stated, on the seeded inputs: `calls`
    back-to-back calls on the launch stream between one pair of HIP events,
    after `warmup` calls extended to at least `warmup_min_s` of wall time.
    (Events around every call cost a few per cent of these ~0.3-1 ms calls.)"""
    import numpy as np
    out = []
    stream = torch.cuda.current_stream(dev)
    for idx in (3, 4):
        w = fi.WORKLOADS[idx]
        inp = fi.make_inputs(idx)
        q, k, v = (torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)
                   .to(dev) for b in (inp.q, inp.k, inp.v))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), device=dev, dtype=torch.float32)

        def call():
            fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

        w0 = time.perf_counter()
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        while time.perf_counter() - w0 < warmup_min_s:
            for _ in range(5):
                call()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(calls):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        if soak:
            clock_soak(clock, w.name, call, torch, 2.0)
        avg = e0.elapsed_time(e1) / calls
        tf = w.fwd_flops() / (avg * 1e-3) / 1e12
        out.append({"workload": w.name, "kernel": fa.fa_fwd_kernel_name(w.B, w.H, w.N, w.d, w.causal),
                    "avg_ms": round(avg, 4), "calls": calls,
                    "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                    "target_frac": 0.5})
        del q, k, v, o, lse
    return out


# Stated parity bounds (max abs error against the fp64 oracle), per output.
TOLS = {"O": 2e-2, "LSE": 1e-3, "dQ": 5e-2, "dK": 5e-2, "dV": 5e-2}


def cpu_baseline(w, inp, budget_s, gpu_out=None):
    """Time the oracle (as it stands) on a bounded sample of heads. With the
    GPU's outputs of the same inputs (`gpu_out`: name -> float64 array of the
    whole [B,H,...] output), also report their max / mean abs error against
    the oracle's on the sampled heads (compared after each head's timing)."""
    import numpy as np
    import oracle
    from exact_io_aware_12_amd.inputs import bf16_bits_to_f64
    cores = blas_threads()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, flops, t_total = 0, 0.0, 0.0
    per_head_fwd = w.fwd_flops() / len(heads)
    per_head_bwd = w.bwd_flops() / len(heads) if w.backward else 0.0
    err = {}
    for b, h in heads:
        q = bf16_bits_to_f64(inp.q[b, h]); k = bf16_bits_to_f64(inp.k[b, h])
        v = bf16_bits_to_f64(inp.v[b, h])
        t0 = time.perf_counter()
        outs = oracle.attention_fwd(q, k, v, w.scale, w.causal)
        if w.backward:
            outs = tuple(outs) + tuple(oracle.attention_bwd(
                q, k, v, bf16_bits_to_f64(inp.do[b, h]), w.scale, w.causal))
        t_total += time.perf_counter() - t0
        done += 1
        flops += per_head_fwd + per_head_bwd
        if gpu_out is not None:
            for name, ref in zip(("O", "LSE", "dQ", "dK", "dV"), outs):
                e = np.abs(gpu_out[name][b, h] - np.asarray(ref))
                m, s_, n = err.get(name, (0.0, 0.0, 0))
                err[name] = (max(m, float(e.max())), s_ + float(e.sum()), n + e.size)
        if t_total >= budget_s:
            break
    rec = {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} heads, {'fwd+bwd' if w.backward else 'fwd'} in fp64 "
                  f"(numpy/OpenBLAS, one head at a time), {t_total:.1f} s",
        "seconds_per_step_extrapolated": t_total / done * len(heads),
        "cpu_model": cpu_model(),
        "host_cpus": len(os.sched_getaffinity(0)),
    }
    if inp.q32 is not None:
        rec["fp32_input_context"] = fp32_input_context(w, inp)
    if err:
        rec["parity_vs_oracle"] = {
            "heads": f"{done} of {len(heads)}",
            **{name: {"max_abs": m, "mean_abs": s_ / n, "tol": TOLS[name], "pass": m <= TOLS[name]}
               for name, (m, s_, n) in err.items()}}
    return rec


def versions(torch) -> dict:
    """ROCm (from the install's version file), torch and its HIP runtime."""
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"rocm": rocm, "torch": torch.__version__, "torch_hip": torch.version.hip}


def blas_threads() -> int:
    """Threads the oracle's BLAS calls use (the threads it actually runs on)."""
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            return max(int(x.get("num_threads", 1)) for x in info)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def fp32_input_context(w, inp):
    """How far the oracle's O and LSE move when it sees the fp32 draws instead
    of their bf16 roundings (the inputs both sides are compared on): input
    quantization, reported as context, not a parity figure."""
    import numpy as np
    import oracle
    from exact_io_aware_12_amd.inputs import bf16_bits_to_f64
    o32, l32 = oracle.attention_fwd(inp.q32.astype(np.float64), inp.k32.astype(np.float64),
                                    inp.v32.astype(np.float64), w.scale, w.causal)
    o16, l16 = oracle.attention_fwd(bf16_bits_to_f64(inp.q), bf16_bits_to_f64(inp.k),
                                    bf16_bits_to_f64(inp.v), w.scale, w.causal)
    return {"O_max_abs_shift": float(np.abs(o32 - o16).max()),
            "LSE_max_abs_shift": float(np.abs(l32 - l16).max()),
            "note": "oracle on the fp32 draws vs on their bf16 roundings"}


def run_oracle_all(args):
    """The oracle, as it stands, on every workload in full on the host cores:
    median of 3 runs for the small workloads 1-2, one run for 3-5."""
    import oracle
    from exact_io_aware_12_amd import inputs as fi
    from exact_io_aware_12_amd.inputs import bf16_bits_to_f64
    out = []
    for idx in (1, 2, 3, 4, 5):
        w = fi.WORKLOADS[idx]
        inp = fi.make_inputs(idx)
        q, k, v = (bf16_bits_to_f64(x) for x in (inp.q, inp.k, inp.v))
        do = bf16_bits_to_f64(inp.do) if w.backward else None
        runs = 3 if idx <= 2 else 1
        ts = []
        for _ in range(runs):
            # One head per call (the oracle loops over heads the same way);
            # the sum of the calls' times is the run's time.
            total, last = 0.0, time.perf_counter()
            for b in range(w.B):
                for h in range(w.H):
                    t0 = time.perf_counter()
                    oracle.attention_fwd(q[b, h], k[b, h], v[b, h], w.scale, w.causal)
                    if w.backward:
                        oracle.attention_bwd(q[b, h], k[b, h], v[b, h], do[b, h], w.scale,
                                             w.causal)
                    total += time.perf_counter() - t0
                    if time.perf_counter() - last > 10:
                        last = time.perf_counter()
                        print(f"[oracle] {w.name}: head {b},{h}, {total:.1f} s so far",
                              file=sys.stderr, flush=True)
            ts.append(total)
        sec = median(ts)
        flops = w.fwd_flops() + (w.bwd_flops() if w.backward else 0.0)
        out.append({"workload": w.name, "pass": "fwd+bwd" if w.backward else "fwd",
                    "runs": runs, "seconds": round(sec, 4),
                    "GFLOP_per_s": round(flops / sec / 1e9, 2)})
        print(f"[oracle] {w.name}: {sec:.3f} s", file=sys.stderr, flush=True)
    print(json.dumps({"oracle_times": out, "cores": blas_threads(),
                      "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
                      "kind": "oracle", "note": "fp64 NumPy/OpenBLAS, heads one at a time, "
                      "all heads of each workload"}), flush=True)


def run_fwd_shape(args):
    """Forward alone on one shape: HIP events around each call, on the launch stream."""
    import numpy as np
    import torch
    from exact_io_aware_12_amd import fa
    from exact_io_aware_12_amd import inputs as fi
    B, H, N, d, causal = (int(x) for x in args.fwd_shape.split(","))
    causal = bool(causal)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.library()
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(fi.random_bf16((B, H, N, d), 9100 + i).view(np.int16)).view(torch.bfloat16).to(dev)
               for i in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in ev:
        e[0].record(stream)
        fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    avg = sum(ms) / len(ms)
    flops = 4.0 * B * H * N * N * d / (2 if causal else 1)
    tf = flops / (avg * 1e-3) / 1e12
    print(json.dumps({"metric": "attention fwd TFLOP/s (bf16)", "value": round(tf, 2), "unit": "TFLOP/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(avg, 4),
                      "median_ms": round(median(ms), 4), "min_ms": round(min(ms), 4),
                      "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": f"fwd_b{B}h{H}n{N}d{d}{'_causal' if causal else ''}",
                                 "B": B, "H": H, "N": N, "d": d, "causal": causal},
                      "kernel": fa.fa_fwd_kernel_name(B, H, N, d, causal),
                      "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}), flush=True)


def run_decode(args):
    """Decode attention: value = K/V bytes read per call / call time (GB/s)."""
    import numpy as np
    import torch
    from exact_io_aware_12_amd import fa
    from exact_io_aware_12_amd import inputs as fi

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.library()
    dev = torch.device("cuda:0")
    w = fi.DECODE_WORKLOADS[args.decode]
    qb, kb, vb = fi.make_decode_inputs(w)

    def gpu(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = gpu(qb), gpu(kb), gpu(vb)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), device=dev, dtype=torch.float32)
    ws = torch.empty(fa.fa_decode_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d), device=dev,
                     dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)

    def call():
        fa.decode_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    gbs = w.kv_bytes() / (ms * 1e-3) / 1e9
    rec = {
        "metric": "decode attention K/V read bandwidth (bf16, d=128)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "pass": "decode"},
        "decode": {"avg_ms": round(ms, 4), "tflops": round(w.flops() / (ms * 1e-3) / 1e12, 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "fa_decode_fwd (kernels fa_decode_kernel, fa_decode_merge_kernel)",
                     "avg_launch_ms": round(ms, 4)},
    }
    if not args.no_cpu_baseline:
        import oracle
        from exact_io_aware_12_amd.inputs import bf16_bits_to_f64
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
        done, t_total = 0, 0.0
        for b, h in heads:
            qq, kk, vv = (bf16_bits_to_f64(x[b, h]) for x in (qb, kb, vb))
            t_s = time.perf_counter()
            oracle.attention_decode(qq, kk, vv, w.scale, w.causal)
            t_total += time.perf_counter() - t_s
            done += 1
            if t_total >= args.cpu_seconds:
                break
        per_head = w.kv_bytes() / len(heads)
        rec["cpu_baseline"] = {"value": round(per_head * done / t_total / 1e9, 3), "unit": "GB/s",
                               "cores": os.cpu_count() or 1, "kind": "oracle",
                               "sample": f"{done} of {len(heads)} heads in fp64 (numpy), "
                                         f"{t_total:.2f} s"}
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(attention shards by head with no exchange, so each GPU would run the "
              "same kernels on its share of the heads). "
              f"Asked for --gpus {args.gpus} (WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    if args.oracle_all:
        run_oracle_all(args)
        return
    if args.decode is not None:
        run_decode(args)
        return
    if args.fwd_shape is not None:
        run_fwd_shape(args)
        return

    import numpy as np
    import torch
    from exact_io_aware_12_amd import fa
    from exact_io_aware_12_amd import inputs as fi

    clock = ClockPoller()   # before anything touches the GPU
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.library()
    dev = torch.device("cuda:0")
    w = fi.WORKLOADS[args.workload]
    inp = fi.make_inputs(args.workload, keep_f32=(args.workload == 1))

    def gpu(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = gpu(inp.q), gpu(inp.k), gpu(inp.v)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), device=dev, dtype=torch.float32)
    if w.backward:
        do = gpu(inp.do)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N, w.d), device=dev,
                         dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        if w.backward:
            fa.bwd(q, k, v, o, do, lse, causal=w.causal, scale=w.scale, workspace=ws,
                   dq=dq, dk=dk, dv=dv)
            if ev is not None:
                ev[2].record(stream)

    w0 = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The warm-up lasts at least --warmup-min-s of wall time: after idle the
    # GPU needs on the order of 0.1 s of load to leave its low clock, and a
    # handful of warm-up steps (a few ms) leave the timed steps on the ramp
    # (workload 5, 20 timed steps: 0.222 ms per step after 5 warm-up steps,
    # 0.189 after 500). The extra steps are counted in the line.
    warm_extra = 0
    while time.perf_counter() - w0 < args.warmup_min_s:
        for _ in range(5):
            step()
        warm_extra += 5
        torch.cuda.synchronize()

    # Per-launch HIP events on every `event_every`-th timed step: a record
    # before and after each launch on the launch stream. Events on every step
    # cost 4-6 % of the workload-5 step time (measured in one process), on
    # every fourth step about 1 %.
    every = max(1, args.event_every)
    events = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)]
              for i in range(0, args.steps, every)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    m0 = time.monotonic()
    for i in range(args.steps):
        step(events.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock.mark("step", m0, time.monotonic())

    fwd_ms = [e[0].elapsed_time(e[1]) for e in events.values()]
    bwd_ms = ([e[1].elapsed_time(e[2]) for e in events.values()] if w.backward
              else [0.0] * len(events))

    # One cold step: a 512 MiB write first evicts the inputs from the L2s and
    # the memory-side cache.
    flush = torch.empty(512 * 2 ** 20, device=dev, dtype=torch.uint8)
    flush.fill_(1)
    cold = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    step(cold)
    torch.cuda.synchronize()
    cold_fwd_ms = cold[0].elapsed_time(cold[1])
    cold_bwd_ms = cold[1].elapsed_time(cold[2]) if w.backward else None
    del flush

    if not args.no_clock_soak:
        clock_soak(clock, "step_soak", step, torch, 3.0)
    ms_step = wall * 1e3 / args.steps
    flops = w.fwd_flops() + (w.bwd_flops() if w.backward else 0.0)
    value = flops / (ms_step * 1e-3) / 1e12

    f_avg = sum(fwd_ms) / len(fwd_ms)
    b_avg = sum(bwd_ms) / len(bwd_ms)
    fwd_tf = w.fwd_flops() / (f_avg * 1e-3) / 1e12
    bwd_tf = (w.bwd_flops() / (b_avg * 1e-3) / 1e12) if w.backward else None
    if w.backward and b_avg > f_avg:
        dom = {"launch": "fa_bwd (kernels fa_bwd_dq, fa_bwd_dkdv back to back)",
               "achieved": bwd_tf, "avg_ms": b_avg,
               "traffic": recorded_traffic(args.workload, "fa_bwd")}
    else:
        kname = fa.fa_fwd_kernel_name(w.B, w.H, w.N, w.d, w.causal)
        dom = {"launch": f"fa_fwd (kernel {kname})", "achieved": fwd_tf, "avg_ms": f_avg,
               "traffic": recorded_traffic(args.workload, "fa_fwd")}
    roofline = {"bound": "mfma", "achieved": round(dom["achieved"], 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom["achieved"] / PEAK_BF16_TFLOPS, 4),
                "traffic": dom["traffic"],
                "kernel": dom["launch"], "avg_launch_ms": round(dom["avg_ms"], 4)}
    if dom["traffic"] is not None:
        # Counter-based HBM rate of the dominant launch (recorded bytes per
        # launch over this run's average launch time).
        roofline["traffic_GBs"] = round(dom["traffic"] / (dom["avg_ms"] * 1e-3) / 1e9, 1)

    unfused = None
    if args.unfused:
        ws_u = torch.empty(fa.fa_unfused_workspace_bytes(w.B, w.H, w.N, w.d), device=dev,
                           dtype=torch.uint8)
        o_u = torch.empty_like(q)
        lse_u = torch.empty_like(lse)

        def ufwd():
            fa.unfused_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o_u, lse=lse_u,
                           workspace=ws_u)

        for _ in range(3):
            ufwd()
        torch.cuda.synchronize()
        n_u = max(3, min(args.steps, 30))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_u):
            ufwd()
        e1.record(stream)
        torch.cuda.synchronize()
        u_ms = e0.elapsed_time(e1) / n_u
        unfused = {"avg_ms": round(u_ms, 4), "calls": n_u,
                   "fwd_tflops_equiv": round(w.fwd_flops() / (u_ms * 1e-3) / 1e12, 2),
                   "fused_fwd_speedup": round(u_ms / f_avg, 2),
                   "workspace_GB": round(ws_u.numel() / 1e9, 3),
                   "note": "S = scale*QK^T (fp32) and P (bf16) round-trip device memory; "
                           "library GEMMs for QK^T and PV, hand-written row softmax; the "
                           "full N x N is computed also when causal"}
        del ws_u

    fa1 = None
    if args.fa1:
        ws_1 = torch.empty(fa.fa_fa1_workspace_bytes(w.B, w.H, w.N, w.d), device=dev,
                           dtype=torch.uint8)
        o_1 = torch.empty_like(q)
        lse_1 = torch.empty_like(lse)

        def fwd1():
            fa.fa1_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o_1, lse=lse_1,
                       workspace=ws_1)

        fwd1()
        torch.cuda.synchronize()
        n_1 = max(2, min(args.steps, 10))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_1):
            fwd1()
        e1.record(stream)
        torch.cuda.synchronize()
        a_ms = e0.elapsed_time(e1) / n_1
        fa1 = {"avg_ms": round(a_ms, 4), "calls": n_1,
               "fwd_tflops_equiv": round(w.fwd_flops() / (a_ms * 1e-3) / 1e12, 2),
               "fused_fwd_speedup": round(a_ms / f_avg, 2),
               "workgroups": w.B * w.H,
               "workspace_GB": round(ws_1.numel() / 1e9, 3),
               "note": "outer loop over 64-key tiles, inner over 128-row query tiles; the "
                       "running O, max and sum of every query tile round-trip device memory "
                       "once per (key tile, query tile) pair"}
        del ws_1

    persistent = None
    if args.persistent:
        o_p = torch.empty_like(q)
        lse_p = torch.empty_like(lse)

        def fwdp():
            fa.fwd_persistent(q, k, v, causal=w.causal, scale=w.scale, out=o_p, lse=lse_p)

        for _ in range(3):
            fwdp()
        torch.cuda.synchronize()
        n_p = max(3, min(args.steps, 50))
        # Back to back, as the fused forward's steps are timed.
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_p)]
        for e in pev:
            e[0].record(stream)
            fwdp()
            e[1].record(stream)
        torch.cuda.synchronize()
        pms = [e[0].elapsed_time(e[1]) for e in pev]
        p_ms = sum(pms) / len(pms)
        persistent = {"avg_ms": round(p_ms, 4), "median_ms": round(median(pms), 4),
                      "calls": n_p,
                      "fwd_tflops": round(w.fwd_flops() / (p_ms * 1e-3) / 1e12, 2),
                      "fused_fwd_speedup": round(p_ms / f_avg, 3),
                      "workgroups": min(512, ((w.N + 127) // 128) * w.B * w.H),
                      "note": "128-row forward kernel on a persistent grid, static snake order "
                              "within each XCD's heads; fa_fwd launches one workgroup per query "
                              "tile and its kernel is named in roofline.kernel"}

    if args.copy_calib_mib > 0:
        src = torch.empty(args.copy_calib_mib * 2 ** 20, device=dev, dtype=torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "key_scale": w.key_scale,
                   "pass": "fwd+bwd" if w.backward else "fwd"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "seed": w.seed,
        "flops": {"fwd": w.fwd_flops(), "bwd": w.bwd_flops() if w.backward else 0.0},
        "bytes_alg": {"fwd": fwd_bytes(w), "bwd": bwd_bytes(w) if w.backward else 0},
        "versions": versions(torch),
        "event_steps": len(events),
        "warmup_extra_steps": warm_extra,
        "fwd": {"avg_ms": round(f_avg, 4), "median_ms": round(median(fwd_ms), 4),
                "min_ms": round(min(fwd_ms), 4), "cold_ms": round(cold_fwd_ms, 4),
                "tflops": round(fwd_tf, 2),
                "hbm_alg_GBs": round(fwd_bytes(w) / (f_avg * 1e-3) / 1e9, 1)},
        "roofline": roofline,
    }
    if w.backward:
        rec["bwd"] = {"avg_ms": round(b_avg, 4), "median_ms": round(median(bwd_ms), 4),
                      "min_ms": round(min(bwd_ms), 4), "cold_ms": round(cold_bwd_ms, 4),
                      "tflops": round(bwd_tf, 2),
                      "hbm_alg_GBs": round(bwd_bytes(w) / (b_avg * 1e-3) / 1e9, 1)}
    if unfused is not None:
        rec["unfused"] = unfused
    if fa1 is not None:
        rec["fa1_order"] = fa1
    if persistent is not None:
        rec["persistent"] = persistent
    if w.N * w.B * w.H <= 128:
        # A single 128-row tile: one workgroup on 256 CUs, launch-latency
        # bound; reported in microseconds with no fraction-of-peak claim.
        rec["latency_us"] = {"avg": round(f_avg * 1e3, 2), "median": round(median(fwd_ms) * 1e3, 2),
                             "min": round(min(fwd_ms) * 1e3, 2)}
        rec["roofline"]["note"] = ("launch-latency bound (one workgroup); the fraction is not "
                                   "a throughput claim")
    if w.backward and not args.no_long_fwd:
        rec["fwd_causal_long"] = long_forwards(fa, torch, fi, dev, clock, not args.no_clock_soak)
    clocks = clock.finish()
    rec["sclk_mhz"] = dict(clocks.get("step_soak") or {}, source=(
        "amdsmi current_gfxclks (the SMU's clock reading), mean of the 8 XCDs, polled every "
        "~0.5 ms over the last 1.5 s of a 3 s untimed run of the same step right after the "
        "timed loop: the reading lags the load by up to about a second (during the timed loop "
        f"itself it showed {(clocks.get('step') or {}).get('mean')} MHz). The counter-based "
        "clock (GRBM_GUI_ACTIVE per dispatch) is in profiles/fa_kernels_clock_under_load.md")) \
        if clocks.get("step_soak") else None
    for ent in rec.get("fwd_causal_long", []):
        c = clocks.get(ent["workload"])
        ent["sclk_mhz_mean"] = c["mean"] if c else None
    if not args.no_cpu_baseline:
        def f64(t):
            return t.float().cpu().numpy().astype("float64")
        gpu_out = {"O": f64(o), "LSE": f64(lse)}
        if w.backward:
            gpu_out.update({"dQ": f64(dq), "dK": f64(dk), "dV": f64(dv)})
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds, gpu_out)
        par = rec["cpu_baseline"].pop("parity_vs_oracle", None)
        if par is not None:
            rec["parity_vs_oracle"] = par
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
