"""Benchmark of the sparse long-sequence attention forward pass on one MI355X.

A step is one la_attn_forward call on the Longformer-base workload (B=2, H=12,
N=4096, D=64, bf16, window radius 256, 64 global tokens with separate global
projections): band tiles, global-column fold, online softmax, PV, epilogue,
the global-row pass over key chunks and the merge of each global-row tile's
chunk partials by its last-finishing chunk workgroup, all in one launch.
Inputs are seeded synthetic N(0,1) tensors already resident in device memory.

Prints one JSON line. `value` is useful TFLOP/s (4*D FLOPs per allowed
(query, key) pair) on that workload; `roofline` relates the call's single
kernel launch, its average duration taken from HIP events around the timed
region on the stream it runs on, to the bf16 MFMA peak, and reports the HBM
traffic that rocprofv3's FETCH_SIZE/WRITE_SIZE counters measured for that
kernel (read from profiles/, and null when the kernel sources changed since);
`workloads` times every workload the same way; `cpu_baseline` times the fp64
CPU oracle on a bounded row sample of the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only NAME]
                       [--copy-probe] [--settle SECONDS] [--backward]

Each workload: W untimed warm-up calls, then untimed calls until the GPU has
been busy for 0.25 s (its clocks ramp up under load), then exactly K calls
timed as one region between two events, then K calls with an event pair each,
then K cold calls: before each, a 512 MiB buffer is written (more than the
L2 caches and the 256 MiB MALL hold), and an event pair times the call alone.

--backward times la_attn_backward on the Longformer-base and ETC (scalar bias
table) workloads and la_dilated_backward on the LongNet workload instead (same
method; the forward's out and lse are computed once, untimed) and prints their
JSON line.

--copy-probe also runs a plain device copy of 256 MiB (torch.neg, fp32) a few
times: under rocprofv3 --pmc its FETCH_SIZE and WRITE_SIZE give the factor that
turns those counters into bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3     # MI355X fp32 matrix
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
METRIC = "effective TFLOP/s & ms/call, window+global attn n=4096 r=256 (frac of MFMA peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Call:
    """Device-resident inputs and preallocated outputs of one workload."""

    def __init__(self, w, dev):
        import torch
        import sparse_long_sequence_amd as la
        from sparse_long_sequence_amd import workloads as W

        self.w = w
        inp = W.make_inputs(w)
        d = lambda t: None if t is None else t.to(dev).contiguous()
        self.q, self.k, self.v = d(inp.q), d(inp.k), d(inp.v)
        self.qg, self.kg, self.vg = d(inp.qg), d(inp.kg), d(inp.vg)
        self.rb = d(inp.rel_bias)
        self.rv = d(inp.rel_vec)
        self.seg = d(inp.seg)
        self.lab = {}
        if inp.glabel is not None or inp.llabel is not None or inp.seg_pieces:
            self.lab = dict(glabel=d(inp.glabel), llabel=d(inp.llabel),
                            seg_pieces=inp.seg_pieces, rel_k=inp.rel_k)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=dev)
        self.g = (torch.tensor(w.global_idx, dtype=torch.int32, device=dev)
                  if w.global_idx else None)
        dims = la.LaDims(w.B, w.H, w.N, w.D, la.LA_BF16 if w.dtype == "bf16" else la.LA_F32)
        if w.kind == "fixed":
            nb = la.la_fixed_workspace_size(dims, w.fixed[0], w.fixed[1])
        elif w.kind == "dilated":
            nb = la.la_dilated_workspace_size(dims, [p[0] for p in w.pairs], [p[1] for p in w.pairs])
        else:
            nb = la.la_attn_workspace_size(dims, len(w.global_idx), w.separate_global)
        self.ws = torch.zeros(max(nb, 1), dtype=torch.uint8, device=dev)
        if w.kind == "fixed":
            self.bound = la.bind_fixed(self.q, self.k, self.v, w.fixed[0], w.fixed[1], w.causal,
                                       out=self.out, lse=self.lse, workspace=self.ws)
        elif w.kind == "dilated":
            self.bound = la.bind_dilated(self.q, self.k, self.v, [p[0] for p in w.pairs],
                                         [p[1] for p in w.pairs], w.causal, out=self.out,
                                         lse=self.lse, workspace=self.ws)
        else:
            self.bound = la.bind_attn(self.q, self.k, self.v, self.g, w.radius, w.dilation,
                                      w.causal, self.rb, out=self.out, lse=self.lse, qg=self.qg,
                                      rel_vec=self.rv, seg_ids=self.seg,
                                      kg=self.kg, vg=self.vg, workspace=self.ws, **self.lab)

    def __call__(self):
        self.bound()


# After the warm-up steps, untimed calls continue until the GPU has been busy
# this long: its clocks ramp up under load over some tens of milliseconds, and
# a region timed straight after a short warm-up runs partly below speed.
SETTLE_S = 0.25


FLUSH_BYTES = 512 << 20
_flush = None


def flush_caches(dev):
    """Write a 512 MiB buffer: evicts the inputs from the L2 caches and the MALL."""
    import torch

    global _flush
    if _flush is None:
        _flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    _flush.fill_(1.0)


def time_calls(call, steps, warmup, settle_s=SETTLE_S, cold=True):
    """(ms per step over the timed region, mean and median ms of per-call event
    pairs, median ms of cold calls or None)."""
    import torch

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(16):
            call()
        torch.cuda.synchronize()
    # region timing: K back-to-back calls
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    region_ms = t0.elapsed_time(t1) / steps
    # per-launch timing: an event pair around every call (same stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    cold_ms = None
    if cold:
        dev = torch.device("cuda", torch.cuda.current_device())
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            flush_caches(dev)
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        cl = sorted(a.elapsed_time(b) for a, b in ev)
        cold_ms = cl[len(cl) // 2]
    return region_ms, sum(per) / len(per), per[len(per) // 2], cold_ms


def cgroup_cpu_quota():
    """CPUs' worth of time the job's cgroup allows (cpu.max quota / period), or None."""
    try:
        with open("/sys/fs/cgroup/cpu.max") as fh:
            quota, period = fh.read().split()[:2]
        if quota != "max":
            return max(1, int(int(quota) / int(period)))
    except (OSError, ValueError):
        pass
    return None


def host_cores() -> int:
    """Every core this process may use: its affinity mask, capped by the cgroup's
    CPU quota when one is set (threads beyond it would only be throttled)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    q = cgroup_cpu_quota()
    return min(n, q) if q else n


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, min_s=10.0, max_s=30.0):
    """Time the fp64 oracle on a bounded sample of the workload's rows.

    The sample grows from 2048 rows until one pass takes a quarter of max_s or
    covers every row; passes over it then repeat until min_s has elapsed (the
    whole workload takes well under a second on 16 cores, too short to time
    alone). The rate is the sampled rows' share of the useful FLOPs over the
    time of all passes."""
    import numpy as np
    import torch

    import oracle
    from sparse_long_sequence_amd import flops as F
    from sparse_long_sequence_amd import workloads as W

    cores = host_cores()
    inp = W.make_inputs(w)
    f = lambda t: None if t is None else t.to(torch.float64).numpy()
    q, k, v, qg, kg, vg, rb, rv = (f(x) for x in (inp.q, inp.k, inp.v, inp.qg, inp.kg, inp.vg,
                                                  inp.rel_bias, inp.rel_vec))
    seg = None if inp.seg is None else inp.seg.numpy()
    total_rows = w.B * w.H * w.N

    def run(sel):
        t = time.perf_counter()
        if w.kind == "dilated":
            oracle.longnet_rows(q, k, v, w.pairs, w.causal, sel=sel, n_threads=cores)
        else:
            oracle.attn_rows(q, k, v, w.global_idx, w.radius, w.dilation, w.causal, rb, qg, kg, vg,
                             sel=sel, n_threads=cores, rel_vec=rv, seg=seg)
        return time.perf_counter() - t

    n = min(total_rows, 2048)
    while True:
        sel = None if n >= total_rows else W.sample_rows(w, n, seed=3).numpy()[:n]
        elapsed = run(sel)
        if elapsed >= max_s / 4 or n >= total_rows:
            break
        n = min(total_rows, int(n * max(2.0, max_s / 8 / max(elapsed, 1e-3))))
    passes = 1
    while elapsed < min_s:
        elapsed += run(sel)
        passes += 1
    # useful FLOPs of the sampled rows: the per-row share of the whole call
    flops_per_row = F.useful_flops(w) / total_rows
    value = flops_per_row * n * passes / elapsed / 1e12
    return {"value": round(value, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {total_rows} rows of {w.name} (fp64, masked dense softmax per row), "
                      f"{passes} passes",
            "seconds": round(elapsed, 3), "nproc": os.cpu_count(),
            "affinity_cores": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
            else None, "cgroup_cpu_quota": cgroup_cpu_quota(), "cpu_model": cpu_model()}


COPY_PROBE_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_longformer_base_traffic.txt")


# The sources the band + global forward kernel and its launch geometry are
# built from, and the build flags: the measured traffic stands while they do.
TRAFFIC_SOURCES = ("csrc/attn_fwd.hip", "csrc/tile_core.h", "csrc/kernels.h", "csrc/api.hip",
                   "csrc/entry.h", "build.py")


def kernel_sources_digest() -> str:
    """sha256 over TRAFFIC_SOURCES (paths and contents)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "sparse_long_sequence_amd")
    files = [os.path.join(pkg, f) for f in TRAFFIC_SOURCES]
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per call from the committed counter summary, or None.

    The summary holds `key = value` lines: sources_sha256, fetch_kib and
    write_kib (average per call, all kernels of the call) and copy_fetch_kib /
    copy_write_kib of the copy probe. Counters are scaled by known/measured of
    the probe. None if the file is missing or the kernel sources changed.
    """
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(ln.split("=", 1) for ln in fh.read().splitlines()
                      if "=" in ln and not ln.lstrip().startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("sources_sha256") != kernel_sources_digest():
        return None
    known_kib = COPY_PROBE_BYTES / 1024
    f_fetch = known_kib / float(kv["copy_fetch_kib"])
    f_write = known_kib / float(kv["copy_write_kib"])
    return (float(kv["fetch_kib"]) * f_fetch + float(kv["write_kib"]) * f_write) * 1024


def copy_probe(dev, reps=3):
    import torch

    x = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()


def bench_backward(dev, args):
    """Backward calls, timed like the forward: the Longformer-base band + global
    backward (dq, dk, dv and the separate global projections' gradients), the
    LongNet mixture's backward, the ETC shape's (with its bias table, with
    key-side label vectors, and with the structured inputs' label matrices and
    piece masks) and the packed-documents one (segment masks). Useful work: 10*D FLOPs per allowed
    pair (q.k and dO.v recomputed, then dV, dQ and dK, 2*D each)."""
    import torch

    import sparse_long_sequence_amd as la
    from sparse_long_sequence_amd import flops as F
    from sparse_long_sequence_amd import workloads as W

    res = {}
    for w in (W.LONGFORMER_BASE, W.LONGNET_SHARE, W.WORKLOADS["etc-ng256-nl4096-r84-relk12"],
              W.PACKED, W.ETC_VECTORS, W.ETC_STRUCTURED):
        log(f"bench backward: {w.name}")
        c = Call(w, dev)
        c()
        dout = torch.randn(c.q.shape, generator=torch.Generator().manual_seed(7)).to(
            c.q.dtype).to(dev)
        if w.kind == "dilated":
            call = la.bind_dilated_backward(c.q, c.k, c.v, c.out, c.lse, dout,
                                            [p[0] for p in w.pairs], [p[1] for p in w.pairs],
                                            w.causal)
        else:
            call = la.bind_attn_backward(c.q, c.k, c.v, c.out, c.lse, dout, c.g, w.radius,
                                         w.dilation, w.causal, qg=c.qg, kg=c.kg, vg=c.vg,
                                         rel_bias=c.rb, rel_vec=c.rv, seg_ids=c.seg,
                                         **{"rel_k": w.rel_k or None, **c.lab})
        steps = max(3, min(args.steps, 20))
        region_ms, mean_ms, med_ms, _ = time_calls(call, steps, min(args.warmup, 3), args.settle,
                                                   cold=False)
        fl = 10 * w.D * F.useful_pairs(w)
        res[w.name] = {"ms_per_call": round(region_ms, 4),
                       "ms_per_call_event_pair_median": round(med_ms, 4),
                       "useful_tflops": round(fl / (region_ms * 1e-3) / 1e12, 3),
                       "useful_flop": fl, "steps": steps}
        log(f"  {res[w.name]}")
        del c, call
        torch.cuda.empty_cache()
    h = res[W.LONGFORMER_BASE.name]
    return {"metric": "backward ms/call and useful TFLOP/s (10*D FLOPs per allowed pair)",
            "value": h["useful_tflops"], "unit": "TFLOP/s", "n_gpus": 1,
            "ms_per_step": h["ms_per_call"], "higher_is_better": True, "dtype": "bf16",
            "data": "synthetic (seeded iid N(0,1), cast to bf16)",
            "config": {"workload": W.LONGFORMER_BASE.name, "pass": "backward"},
            "workloads": res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default=None, help="time only this workload name")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed calls after the warm-up (0 for counter runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 256 MiB device copy (counter scaling under rocprofv3)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward calls instead of the forward workloads")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_long_sequence_amd import flops as F
    from sparse_long_sequence_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.backward:
        print(json.dumps(bench_backward(dev, args)), flush=True)
        return
    if args.copy_probe:
        log("bench: copy probe (torch.neg, 256 MiB fp32)")
        copy_probe(dev)
    head = W.LONGFORMER_BASE
    results = {}
    for w in W.ORDERED:
        if args.only and w.name != args.only and w is not head:
            continue
        log(f"bench: {w.name} (B={w.B} H={w.H} N={w.N} {w.dtype})")
        call = Call(w, dev)
        steps = args.steps
        region_ms, mean_ms, med_ms, cold_ms = time_calls(call, steps, args.warmup, args.settle)
        fl = F.useful_flops(w)
        by = F.algorithmic_bytes(w)
        peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
        # throughput figures from the timed region of back-to-back calls; the
        # event-pair figures (one pair around each call) add the events' cost
        results[w.name] = {
            "ms_per_call": round(region_ms, 5),
            "ms_per_call_event_pair_mean": round(mean_ms, 5),
            "ms_per_call_event_pair_median": round(med_ms, 5),
            "ms_per_call_cold_median": round(cold_ms, 5),
            "useful_tflops_cold": round(fl / (cold_ms * 1e-3) / 1e12, 3),
            "useful_tflops": round(fl / (region_ms * 1e-3) / 1e12, 3),
            "frac_mfma_peak": round(fl / (region_ms * 1e-3) / 1e12 / peak, 4),
            "hbm_gbs_algorithmic": round(by / (region_ms * 1e-3) / 1e9, 1),
            "useful_flop": fl, "algorithmic_bytes": by,
        }
        log(f"  {results[w.name]}")
        del call
        torch.cuda.empty_cache()

    r = results[head.name]
    fl = F.useful_flops(head)
    by = F.algorithmic_bytes(head)
    # the call is one launch of attn_fwd_kernel: the timed region over K
    # back-to-back calls gives its average launch duration (gaps included)
    achieved = fl / (r["ms_per_call"] * 1e-3) / 1e12
    traffic = measured_traffic()
    line = {
        "metric": METRIC,
        "value": round(fl / (r["ms_per_call"] * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_call"],
        "ms_per_step_cold": r["ms_per_call_cold_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1) Q/K/V, cast to bf16)",
        "config": {"workload": head.name, "B": head.B, "H": head.H, "N": head.N, "D": head.D,
                   "radius": head.radius, "n_global": len(head.global_idx),
                   "separate_global": head.separate_global, "causal": head.causal},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "traffic_unit": "HBM bytes per call (FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                     "algorithmic_bytes": by,
                     "kernel": "attn_fwd_kernel<bf16> (one launch per call)",
                     "hbm_gbs_algorithmic": round(by / (r["ms_per_call"] * 1e-3) / 1e9, 1),
                     "hbm_peak_gbs": HBM_PEAK_GBS},
        "workloads": results,
    }
    if not args.no_cpu:
        log("bench: cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(head)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
