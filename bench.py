#!/usr/bin/env python3
"""Benchmark of the gfx950 FlashAttention-2 forward (one GPU).

A step is one fa_fwd call over the whole batch of the headline workload,
[B=4, H=16, N=4096, D=128] bf16, non-causal, inputs resident in HBM. Prints
one JSON line: attention TFLOP/s (4*B*H*N^2*D FLOPs, halved for causal, the
count of "FlashAttention 2 from PyTorch to Triton", Step 4), the fraction of
the MI355X dense bf16 MFMA peak, the same figures for the causal mask and the
other N=4096 workload in "extra", and the fp64 CPU oracle timed on a bounded
sample of the same workload as "cpu_baseline" (with every other benchmarked
workload and mask sampled the same way). "extra" also holds per-launch
percentiles (back to back, and with the caches scrubbed before each call),
the split-KV and backward timings; "clock" holds the graphics clock and
socket power read while the headline call runs back to back, and the
roofline adds the fraction of the peak scaled to that clock.

Every timed line follows `--warmup` calls and at least `--settle` seconds
(default 1) of untimed back-to-back calls, so that the board has reached the
clock it holds under sustained load; "timing" records the settle.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle S] [--no-cpu-baseline]
                       [--no-extra] [--no-clock] [--counters-run REPS]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fa_inputs  # noqa: E402

# MI355X published dense MFMA peak for bf16/fp16 (256 CUs x 4096 FLOP/clk x 2.4 GHz)
PEAK_BF16_TFLOPS = 2516.6
METRIC = "attention fwd TFLOP/s and % of MFMA bf16 peak at N=4096 (causal/non-causal)"


def attention_flops(B, H, N, D, causal):
    """4*B*H*N^2*D, halved for causal (two N x N x D matmuls, 2 FLOPs per MAC)."""
    f = 4 * B * H * N * N * D
    return f / 2 if causal else f


def attention_bytes(B, H, N, D, esize, with_lse=True):
    """Algorithmic HBM bytes: Q, K, V read once and O written once, plus the
    fp32 LSE ("A09 - Advanced Triton & FlashAttention", section 2: fused
    traffic per head is 4*N*d elements)."""
    return 4 * B * H * N * D * esize + (4 * B * H * N if with_lse else 0)


PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "fa_fwd_twogroup_bf16_d128_b4h16_n4096_hbm_traffic.txt")


# the sources that make up the headline forward kernel and its launch
FORWARD_SOURCES = ("fa_kernel.hpp", "fa_kernel_pp.hpp", "fa_kernel_pp16.hpp", "fa_inst_pp.hip", "fa_launch.hpp",
                   "fa_api.hip", "fa.h")


def kernel_sources_digest():
    """sha256 over the sources and build flags of the headline forward kernel,
    so a stored counter reading is only used for the kernel it was taken on."""
    import hashlib
    from exact_attention_10_amd import build as fa_build
    h = hashlib.sha256()
    for path in sorted(fa_build.DEPENDS):
        name = os.path.basename(path)
        if name not in FORWARD_SOURCES:
            continue
        h.update(name.encode())
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(" ".join(fa_build.FILE_FLAGS.get(name, [])).encode())
    h.update(" ".join(fa_build.HIPCC_FLAGS).encode())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch of the headline kernel from the committed
    FETCH_SIZE / WRITE_SIZE summary, or None when the kernel sources changed
    since the counters were taken (or no summary exists)."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_sources_sha256") != kernel_sources_digest():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


_BITS = {}


def workload_bits(w):
    """The workload's seeded input bits, drawn once per process."""
    if w.name not in _BITS:
        _BITS[w.name] = fa_inputs.workload_inputs(w)
    return _BITS[w.name]


def _device_inputs(w, torch):
    qb, kb, vb = workload_bits(w)
    dt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]

    def dev(b):
        t = torch.from_numpy(b)
        if w.dtype != "fp32":
            t = t.view(torch.int16).view(dt)
        return t.cuda()
    return (dev(qb), dev(kb), dev(vb)), (qb, kb, vb)


def settle(call, stream, torch, seconds, probes=10):
    """Run `call` back to back for at least `seconds` of wall time, so that the
    board reaches the clock and power state it holds under sustained load
    ("How to profile and optimise kernels", How I profile: warm up for about a
    second before timing). Returns the time spent, the number of calls and
    the per-launch durations (ms) of `probes` calls made at the end."""
    t0 = time.perf_counter()
    n, batch = 0, 4
    while True:
        for _ in range(batch):
            call()
        torch.cuda.synchronize()
        n += batch
        elapsed = time.perf_counter() - t0
        if elapsed >= seconds:
            break
        batch = min(batch * 2, 512)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(probes)]
    for e0, e1 in ev:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    return elapsed, n, [round(e0.elapsed_time(e1), 5) for e0, e1 in ev]


def time_gpu(w, causal, steps, warmup, torch, fa, variant=None, splitkv=False, settle_s=1.0):
    """Whole-run timing: `warmup` untimed calls, then at least `settle_s`
    seconds of untimed back-to-back calls, then `steps` calls bracketed by
    synchronisation and events on the launch stream (fa_fwd, kernel variant
    `variant` through fa_fwd_variant, or fa_fwd_splitkv with the library's
    split choice and a workspace allocated before timing)."""
    (q, k, v), _ = _device_inputs(w, torch)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    ws = None
    if splitkv:
        need = fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.N, w.N, w.D, 0)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)

    def call():
        if splitkv:
            fa.fa_fwd_splitkv(q, k, v, o, lse, causal=causal, scale=w.scale, stream=stream,
                              num_splits=0, workspace=ws)
        elif variant is None:
            fa.fa_fwd(q, k, v, o, lse, causal=causal, scale=w.scale, stream=stream)
        else:
            fa.fa_fwd_variant(q, k, v, o, lse, causal=causal, scale=w.scale, stream=stream,
                              variant=variant)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    settled_s, settle_calls, settle_last = settle(call, stream, torch, settle_s)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    flops = attention_flops(w.B, w.H, w.N, w.D, causal)
    return {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12, "wall_s": wall,
            "flops": flops, "settle_s": round(settled_s, 3), "settle_calls": settle_calls,
            "settle_last_ms": settle_last}


class ClockSampler:
    """Reads the GPU's graphics clock (MHz, mean over its XCDs) and socket
    power from amdsmi's GPU metrics in a background thread. The metrics table
    refreshes about once a second, so a reading needs a window of sustained
    load of a few seconds (measure_clock). Reports nothing (None) where
    amdsmi or the device's metrics are not available."""

    def __init__(self, torch, period_s=0.05):
        self.period = period_s
        self.samples = []
        self.handle = None
        self._stop = None
        self._thread = None
        self._t0 = 0.0
        try:
            import amdsmi
            props = torch.cuda.get_device_properties(torch.cuda.current_device())
            amdsmi.amdsmi_init()
            for h in amdsmi.amdsmi_get_processor_handles():
                dom, bus, _ = amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")
                if int(bus, 16) == props.pci_bus_id and int(dom, 16) == props.pci_domain_id:
                    self.handle = h
            self._smi = amdsmi
        except Exception:
            self.handle = None

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self.handle)
        clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, (int, float)) and 0 < c < 10000]
        if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
            clks = [m["current_gfxclk"]]
        power = m.get("current_socket_power")
        return (time.perf_counter() - self._t0, sum(clks) / len(clks) if clks else None,
                power if isinstance(power, (int, float)) else None)

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception:
                return
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        self._t0 = time.perf_counter()
        if self.handle is not None:
            self._stop = threading.Event()
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False


def measure_clock(w, torch, fa, seconds=3.0, settle_s=1.2):
    """The graphics clock and socket power while the headline call runs back
    to back for `seconds`: the median of the readings taken after `settle_s`
    (the metrics refresh about once a second). None where unavailable."""
    (q, k, v), _ = _device_inputs(w, torch)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    sampler = ClockSampler(torch)
    if sampler.handle is None:
        return None
    with sampler:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(200):
                fa.fa_fwd(q, k, v, o, lse, causal=False, scale=w.scale)
            torch.cuda.synchronize()
    late = [(c, p) for t, c, p in sampler.samples if t >= settle_s and c is not None]
    if not late:
        return None
    clk = sorted(c for c, _ in late)
    pw = sorted(p for _, p in late if p is not None)
    return {"sclk_mhz_median": round(clk[len(clk) // 2], 1), "sclk_mhz_min": round(clk[0], 1),
            "sclk_mhz_max": round(clk[-1], 1), "readings": len(clk),
            "socket_power_w_median": pw[len(pw) // 2] if pw else None,
            "source": f"amdsmi GPU metrics (graphics clock averaged over the XCDs), read every "
                      f"{sampler.period * 1e3:.0f} ms while {w.name} non-causal ran back to back for "
                      f"{seconds:.0f} s, readings after the first {settle_s:.1f} s"}


def time_per_launch(w, causal, reps, torch, fa, scrub_mib=0, settle_s=1.0):
    """Per-launch durations (median, p10, p90 in ms) from one event pair
    around each fa_fwd call; with scrub_mib > 0 each call is preceded by an
    untimed read of a buffer of that many MiB, so that Q, K and V start
    outside the L2 and the memory-side cache. The sweep only reads (a sum into
    a preallocated scalar): a write sweep would leave that many MiB of dirty
    lines, whose write-back would then compete with the timed call for HBM.
    The calls follow `settle_s` seconds of back-to-back calls."""
    (q, k, v), _ = _device_inputs(w, torch)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    scrub = (torch.ones(scrub_mib << 18, dtype=torch.float32, device=q.device)
             if scrub_mib else None)
    scrub_out = torch.empty((), dtype=torch.float32, device=q.device)
    settle(lambda: fa.fa_fwd(q, k, v, o, lse, causal=causal, scale=w.scale, stream=stream),
           stream, torch, settle_s)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
    for e0, e1 in events:
        if scrub is not None:
            torch.sum(scrub, dim=0, out=scrub_out)
        e0.record(stream)
        fa.fa_fwd(q, k, v, o, lse, causal=causal, scale=w.scale, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in events)
    pick = lambda f: ms[min(len(ms) - 1, int(f * len(ms)))]   # noqa: E731
    return {"median_ms": round(pick(0.5), 5), "p10_ms": round(pick(0.1), 5),
            "p90_ms": round(pick(0.9), 5), "reps": reps,
            "scrub_mib": scrub_mib}


def time_bwd(w, causal, steps, warmup, torch, fa, settle_s=1.0):
    """Backward timing: the forward runs once untimed for O and LSE, then
    `warmup` calls, `settle_s` seconds of calls and `steps` timed fa_bwd
    calls, timed like time_gpu."""
    (q, k, v), _ = _device_inputs(w, torch)
    g = torch.Generator(device=q.device)
    g.manual_seed(w.seed + 1000)
    dout = torch.randn(q.shape, device=q.device, generator=g).to(q.dtype)
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=w.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()

    def call():
        fa.fa_bwd(q, k, v, o, dout, lse, causal=causal, scale=w.scale, dq=dq, dk=dk, dv=dv,
                  delta=delta, stream=stream)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    settle(call, stream, torch, settle_s)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    flops = 2.5 * attention_flops(w.B, w.H, w.N, w.D, causal)
    return {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12}


def cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_one(w, causal, target_s, rng):
    """The fp64 oracle (as it stands) on a bounded random sample of query rows
    of one workload and mask: a probe of 256 rows sizes the sample to about
    `target_s` seconds. Returns oracle TFLOP/s with the benchmark's FLOP count
    per row (4*D per visible key), rows, seconds."""
    import oracle
    qb, kb, vb = workload_bits(w)
    q, k, v = (fa_inputs.to_f32(x, w.dtype) for x in (qb, kb, vb))
    BH = w.B * w.H

    def run(n_rows):
        rows = np.stack([rng.integers(0, BH, n_rows), rng.integers(0, w.N, n_rows)], 1)
        flops = float(sum(4 * ((int(i) + 1) if causal else w.N) * w.D for i in rows[:, 1]))
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, w.scale, causal, rows)
        return time.perf_counter() - t0, flops

    probe = min(256, BH * w.N)
    t, f = run(probe)
    n_rows = int(min(BH * w.N, max(probe, probe * target_s / max(t, 1e-4))))
    t, f = run(n_rows)
    return {"tflops": f / t / 1e12, "rows": n_rows, "seconds": round(t, 2),
            "gflop": round(f / 1e9, 2)}


def cpu_baseline(cases, headline, gpu_tflops, target_s=2.5):
    """The fp64 oracle timed on the host cores on a bounded sample of every
    benchmarked workload and mask, next to the GPU's rate on the same case.
    The headline case is the reported value."""
    threads = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    rng = np.random.default_rng(123)
    per = {}
    for name, causal in cases:
        key = f"{name}_{'causal' if causal else 'noncausal'}"
        r = cpu_baseline_one(fa_inputs.WORKLOADS[name], causal, target_s, rng)
        if key in gpu_tflops:
            r["gpu_tflops"] = round(gpu_tflops[key], 2)
            r["gpu_over_oracle"] = round(gpu_tflops[key] / r["tflops"], 1)
        r["tflops"] = round(r["tflops"], 5)
        per[key] = r
        print(f"[bench] cpu oracle {key}: {r['tflops'] * 1e3:.2f} GFLOP/s "
              f"({r['rows']} rows, {r['seconds']} s)", file=sys.stderr, flush=True)
    head = per[headline]
    return {"value": head["tflops"], "unit": "TFLOP/s", "cores": int(os.environ["OMP_NUM_THREADS"]),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{head['rows']} random query rows of {headline}, explicit fp64 attention "
                      f"per row (the oracle as it stands, C + OpenMP), {head['seconds']} s, "
                      f"{head['gflop']} GFLOP; every other benchmarked workload and mask sampled "
                      f"the same way in per_workload",
            "per_workload": per}


def run_each_kernel_once(torch, fa, reps):
    """Run every benchmarked kernel `reps` times with nothing else in between
    (no timing, no clock sampling), for hardware-counter collection: the
    forward on every workload and mask, split-KV (split and combine kernels)
    on the two small grids, and the backward (dQ and dK/dV kernels) at the
    headline shape, both masks."""
    for name, w in fa_inputs.WORKLOADS.items():
        (q, k, v), _ = _device_inputs(w, torch)
        for causal in w.masks:
            o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=w.scale)
            for _ in range(reps):
                fa.fa_fwd(q, k, v, o, lse, causal=causal, scale=w.scale)
            torch.cuda.synchronize()
            print(f"[counters] forward {name} causal={causal}", file=sys.stderr, flush=True)
    for small in SMALL_GRIDS:
        (q, k, v), _ = _device_inputs(small, torch)
        need = fa.fa_fwd_splitkv_workspace_size(small.B, small.H, small.N, small.N, small.D, 4)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        o, lse = torch.empty_like(q), torch.empty((small.B, small.H, small.N), device=q.device)
        for _ in range(reps):
            fa.fa_fwd_splitkv(q, k, v, o, lse, causal=False, scale=small.scale, num_splits=4,
                              workspace=ws)
        torch.cuda.synchronize()
        print(f"[counters] split-KV {small.name} (4 splits)", file=sys.stderr, flush=True)
    w = fa_inputs.WORKLOADS[fa_inputs.HEADLINE]
    (q, k, v), _ = _device_inputs(w, torch)
    dout = torch.randn(q.shape, device=q.device).to(q.dtype)
    for causal in (False, True):
        o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=w.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
        for _ in range(reps):
            fa.fa_bwd(q, k, v, o, dout, lse, causal=causal, scale=w.scale, dq=dq, dk=dk, dv=dv,
                      delta=delta)
        torch.cuda.synchronize()
        print(f"[counters] backward {w.name} causal={causal}", file=sys.stderr, flush=True)


# the small grids of the split-KV lines: the [B=8, N=1024, D=64] workload (64
# workgroups of 128 query rows) and a [B=1, H=8, N=2048, D=128] one (128)
SMALL_GRIDS = (fa_inputs.WORKLOADS["b8h1_n1024_d64_bf16"],
               fa_inputs.Workload("b1h8_n2048_d128_bf16", 1, 8, 2048, 128, "bf16", 7, (False,)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle", type=float, default=1.0, metavar="SECONDS",
                    help="back-to-back untimed calls for at least this long before every timed "
                         "line, on top of --warmup (default 1 s)")
    ap.add_argument("--workload", default=fa_inputs.HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the 3 s clock reading under sustained load")
    ap.add_argument("--sweep-variants", action="store_true",
                    help="time every kernel variant on the N=4096 workloads and exit")
    ap.add_argument("--counters-run", type=int, default=0, metavar="REPS",
                    help="only run every benchmarked kernel REPS times (for hardware counters), "
                         "then exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times) to calibrate "
                         "HBM byte counters, then exit")
    a = ap.parse_args()

    if a.copy_calibration:
        import torch
        n = a.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 4 * n, "launches": 5}), flush=True)
        return

    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}): the attention "
              "forward shards over (batch, head) with no communication, so the "
              "per-GPU figure is the one that matters; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_10_amd as fa
    fa.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if a.counters_run:
        run_each_kernel_once(torch, fa, a.counters_run)
        return

    w = fa_inputs.WORKLOADS[a.workload]
    if a.sweep_variants:
        for name in (w.name, "b4h16_n4096_d64_bf16", "b1h32_n16384_d128_bf16_q8"):
            wl = fa_inputs.WORKLOADS[name]
            for causal in wl.masks:
                for var in range(fa.fa_num_variants()):
                    try:
                        r = time_gpu(wl, causal, a.steps, a.warmup, torch, fa, variant=var,
                                     settle_s=a.settle)
                    except fa.FAError as e:
                        print(f"[sweep] {name} causal={causal} {fa.fa_variant_name(var)}: {e}",
                              flush=True)
                        continue
                    print(f"[sweep] {name} causal={int(causal)} {fa.fa_variant_name(var):28s} "
                          f"{r['ms']:.4f} ms {r['tflops']:7.1f} TFLOP/s", flush=True)
        return
    head = time_gpu(w, False, a.steps, a.warmup, torch, fa, settle_s=a.settle)
    print(f"[bench] {w.name} non-causal: {head['ms']:.4f} ms/step {head['tflops']:.1f} TFLOP/s "
          f"(after {head['settle_s']} s / {head['settle_calls']} settle calls)",
          file=sys.stderr, flush=True)
    head_key = f"{w.name}_noncausal"
    gpu_rates = {head_key: head["tflops"]}
    timing = {"headline": "mean of the timed back-to-back calls",
              "warmup_calls": a.warmup, "settle_s": head["settle_s"],
              "settle_calls": head["settle_calls"], "settle_last_ms": head["settle_last_ms"],
              "timed_calls": a.steps, "timed_wall_s": round(head["wall_s"], 4)}

    extra = {}
    if not a.no_extra:
        for name, causal in ((w.name, True), ("b4h16_n4096_d64_bf16", False),
                             ("b4h16_n4096_d64_bf16", True), ("b2h16_n4000_d128_fp16", False),
                             ("b2h16_n4000_d128_fp16", True), ("b1h32_n16384_d128_bf16_q8", True)):
            r = time_gpu(fa_inputs.WORKLOADS[name], causal, max(10, a.steps // 2),
                         max(5, a.warmup // 2), torch, fa, settle_s=a.settle)
            key = f"{name}_{'causal' if causal else 'noncausal'}"
            gpu_rates[key] = r["tflops"]
            extra[key] = {"ms": round(r["ms"], 5), "tflops": round(r["tflops"], 2),
                          "frac_of_peak": round(r["tflops"] / PEAK_BF16_TFLOPS, 4),
                          "settle_s": r["settle_s"]}
            print(f"[bench] {key}: {r['ms']:.4f} ms {r['tflops']:.1f} TFLOP/s", file=sys.stderr,
                  flush=True)
        # small grids, single pass against split-KV with the library's split choice
        for small in SMALL_GRIDS:
            for causal in small.masks:
                for split in (False, True):
                    r = time_gpu(small, causal, max(20, a.steps), max(10, a.warmup), torch, fa,
                                 splitkv=split, settle_s=a.settle)
                    key = (f"{small.name}_{'causal' if causal else 'noncausal'}"
                           f"_{'splitkv' if split else 'single_pass'}")
                    if not split:
                        gpu_rates[f"{small.name}_{'causal' if causal else 'noncausal'}"] = r["tflops"]
                    extra[key] = {"ms": round(r["ms"], 5), "tflops": round(r["tflops"], 2),
                                  "frac_of_peak": round(r["tflops"] / PEAK_BF16_TFLOPS, 4)}
                    if split:
                        extra[key]["num_splits"] = fa.fa_splitkv_auto_splits(
                            small.B, small.H, small.N, small.N, small.D)
                    print(f"[bench] {key}: {r['ms']:.4f} ms {r['tflops']:.1f} TFLOP/s",
                          file=sys.stderr, flush=True)

        # per-launch distribution of the headline call, back to back and with
        # the caches scrubbed before each call (512 MiB read, untimed)
        for scrub in (0, 512):
            r = time_per_launch(w, False, max(20, a.steps), torch, fa, scrub_mib=scrub,
                                settle_s=a.settle)
            r["tflops_at_median"] = round(head["flops"] / (r["median_ms"] * 1e-3) / 1e12, 2)
            key = f"{w.name}_noncausal_per_launch{'_scrubbed' if scrub else ''}"
            extra[key] = r
            timing["per_launch_scrubbed_median_ms" if scrub else "per_launch_median_ms"] = \
                r["median_ms"]
            print(f"[bench] {key}: median {r['median_ms']:.4f} ms (p10 {r['p10_ms']:.4f}, "
                  f"p90 {r['p90_ms']:.4f})", file=sys.stderr, flush=True)

        # the backward at the headline shape (fa_bwd: dQ kernel then dK/dV
        # kernel), FLOPs counted as 2.5x the forward's (five N x N x D products)
        for causal in (False, True):
            r = time_bwd(w, causal, max(10, a.steps // 2), max(5, a.warmup // 2), torch, fa,
                         settle_s=a.settle)
            key = f"{w.name}_{'causal' if causal else 'noncausal'}_backward"
            extra[key] = {"ms": round(r["ms"], 5), "tflops": round(r["tflops"], 2),
                          "frac_of_peak": round(r["tflops"] / PEAK_BF16_TFLOPS, 4),
                          "flops_counted": "2.5x forward"}
            print(f"[bench] {key}: {r['ms']:.4f} ms {r['tflops']:.1f} TFLOP/s", file=sys.stderr,
                  flush=True)

    clock_summary = measure_clock(w, torch, fa) if not a.no_clock else None
    if clock_summary is not None:
        print(f"[bench] graphics clock under sustained load: {clock_summary['sclk_mhz_median']} MHz, "
              f"{clock_summary['socket_power_w_median']} W", file=sys.stderr, flush=True)

    esize = fa_inputs.ESIZE[w.dtype]
    roofline = {
        "bound": "mfma",
        "achieved": round(head["tflops"], 3),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(head["tflops"] / PEAK_BF16_TFLOPS, 4),
        "traffic": stored_traffic(),
        "algorithmic_flops_per_launch": head["flops"],
        "algorithmic_bytes_per_launch": attention_bytes(w.B, w.H, w.N, w.D, esize),
        "kernel": "fa_fwd_pp16_kernel<bf16, D=128> (two-group schedule on 16x16x32 MFMAs, non-causal)",
    }
    if clock_summary is not None:
        # the same fraction against the peak scaled to the clock the GPU ran at
        roofline["sclk_mhz_measured"] = clock_summary["sclk_mhz_median"]
        roofline["frac_at_measured_sclk"] = round(
            head["tflops"] / (PEAK_BF16_TFLOPS * clock_summary["sclk_mhz_median"] / 2400.0), 4)
    cpu = None
    if not a.no_cpu_baseline:
        cases = [(w.name, False)]
        if not a.no_extra:
            cases += [(w.name, True), ("b4h16_n4096_d64_bf16", False),
                      ("b4h16_n4096_d64_bf16", True), ("b2h16_n4000_d128_fp16", False),
                      ("b2h16_n4000_d128_fp16", True), ("b1h32_n16384_d128_bf16_q8", True),
                      ("b8h1_n1024_d64_bf16", False), ("b8h1_n1024_d64_bf16", True)]
        cpu = cpu_baseline(cases, head_key, gpu_rates, target_s=10.0 if a.no_extra else 2.5)
        print(f"[bench] cpu oracle: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads "
              f"({cpu['cpu_model']})", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(head["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D,
                   "dtype": w.dtype, "causal": False, "scale": w.scale,
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "timing": timing,
        "clock": clock_summary,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
