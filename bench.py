#!/usr/bin/env python3
"""Throughput of fused causal attention, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path on resident inputs: attn_fwd (forward
with LSE) then attn_bwd (dQ with Delta, then dK/dV), called on a stream of
the workload's own.  Throughput counts the causal FLOPs actually allowed by
the mask: 4*D per allowed (query, key) pair forward and 10*D backward (the
five products of the FlashAttention-2 accounting), divided by the measured
time.  One JSON line is printed.

Timing.  W untimed steps, then exactly K steps between two device
synchronisations with nothing else on the stream: `ms_per_step` and `value`
come from the host clock around those K steps.  A second loop of K steps
records HIP events on the launch stream around every step's forward and
backward, giving per-iteration median, p10 and p90 (`events_ms`; its own
host-clock time per step, which includes the event records, is
`ms_per_step_with_events`).  A third loop writes a 512 MiB buffer before
each step (more than the 256 MiB last-level cache holds), so every step
starts cold (`cold`).  The graphics clock is measured while steps run back to back
(`sclk_mhz`: the library's clock probe on a side stream).

Besides the headline workload the line carries:
  kernels       per-kernel median/p10/p90 from HIP events, each kernel run
                through its own entry point: the forward, the two stages
                attn_bwd runs (dQ with Delta fused, then dK/dV) and the
                standalone Delta preprocess (fp32 inputs and staged callers);
  rooflines     each of those kernels against its binding roof,
                min(matrix-core peak, arithmetic intensity x HBM peak), from
                its counted flops and algorithmic HBM bytes;
  roofline      the dominant kernel's entry, with the rocprofv3-measured HBM
                traffic when it was taken on the current sources;
  by_workload   the same measurement at the other full-size workloads
                (context 512, 8192, packed documents, grouped-query heads,
                RoPE on q and k, bf16 outputs), and one decode step against a
                full 8192-token K/V cache (time, GB/s against HBM peak);
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from workload import CONFIGS, allowed_pair_count, make_inputs  # noqa: E402

METRIC = "causal attention fwd+bwd TFLOPS and % bf16 MFMA peak at ctx 512/1024/8192"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 bf16 flop/CU/clk (dense)
PEAK_FP32_TFLOPS = 157.3    # fp32 matrix/vector peak used for fp32 inputs
PEAK_HBM_GBS = 8000.0
HEADLINE = "lm237m_ctx1024"
SEEDS = {"tiny_f32": 1, "lm12m_ctx512": 2, "lm237m_ctx1024": 3, "long_ctx8192": 4, "packed_docs8192": 5,
         "lm237m_ctx1024_gqa4": 6, "lm237m_ctx1024_rope": 7, "lm237m_ctx1024_out16": 8, "long_ctx8192_gqa4": 9}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=HEADLINE, choices=sorted(CONFIGS))
    p.add_argument("--kernel-reps", type=int, default=50, help="repetitions for per-kernel event timing")
    p.add_argument("--no-others", action="store_true", help="skip the other full-size workloads")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time for the oracle sample")
    p.add_argument("--cold-mib", type=int, default=512,
                   help="MiB written before each step of the cold-cache loop (0: no cold loop)")
    p.add_argument("--sclk-seconds", type=float, default=1.0,
                   help="seconds of back-to-back steps while the graphics clock is sampled (0: none)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="also run a plain fp32 elementwise kernel (negation) over MIB MiB, a known number of "
                        "HBM bytes, to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE")
    p.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; csv output) of "
                        "'bench.py --no-others --copy-calibration MIB' into profiles/traffic.json")
    return p.parse_args()


class Workload:
    """Resident device inputs and outputs of one workload."""

    def __init__(self, name):
        import torch
        import causal_attention_amd as ca
        self.ca = ca
        self.name = name
        self.cfg = cfg = CONFIGS[name]
        x = make_inputs(cfg, SEEDS[name])
        self.x = x
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        d = {n: torch.from_numpy(x[n]).to("cuda").to(dt).contiguous() for n in ("q", "k", "v", "do")}
        self.q, self.k, self.v, self.do = d["q"], d["k"], d["v"], d["do"]
        B, H, S, D = x["B"], x["H"], x["S"], x["D"]
        self.grouped = self.k.shape[1] != H
        f32 = dict(dtype=torch.float32, device="cuda")
        out = dict(dtype=dt if cfg.out16 else torch.float32, device="cuda")
        self.o = torch.empty((B, H, S, D), **out)
        self.dq = torch.empty_like(self.o)
        self.dk = torch.empty(tuple(self.k.shape), **out)
        self.dv = torch.empty_like(self.dk)
        self.lse = torch.empty((B, H, S), **f32)
        self.delta = torch.empty((B, H, S), **f32)
        cu = x["cu_seqlens"]
        if cu is not None:
            self.cu = torch.from_numpy(cu).to("cuda")
            self.max_seqlen = int(np.diff(cu).max())
        else:
            self.cu, self.max_seqlen = None, None
        self.pairs = allowed_pair_count(S, B, H, cu)
        self.flops_fwd = 4 * D * self.pairs
        self.flops_bwd = 10 * D * self.pairs
        # a stream of its own (default priority), so the step can be captured
        self.stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        self.sargs = dict(mask_mode=cfg.mask_mode, cu_seqlens=self.cu, max_seqlen=self.max_seqlen,
                          stream=self.stream)
        # grouped heads: the backward's workspace (allocated once, outside the timed steps), where the
        # library splits each group's dK/dV step into parts (None where it does not)
        self.ws = None
        if self.grouped and not cfg.out16 and not cfg.rope:
            n = ca.bwd_workspace_bytes(B, H, self.k.shape[1], S, D, dt, cfg.mask_mode,
                                       0 if cu is None else len(cu) - 1, self.max_seqlen or 0)
            if n > 0:
                self.ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        if cfg.rope:  # RoPE: the table is built once, as a model does; q_rot, k_rot are kept for the backward
            self.tab = ca.rope_table(self.max_seqlen or S, D, 10000.0)
            self.q_rot = torch.empty_like(self.q)
            self.k_rot = torch.empty_like(self.k)

    def fwd(self):
        if self.cfg.out16:
            self.ca.attn_fwd_ex(self.q, self.k, self.v, self.o, self.lse, self.x["scale"], **self.sargs)
        elif self.cfg.rope:
            self.ca.attn_fwd_rope(self.q, self.k, self.v, self.q_rot, self.k_rot, self.o, self.lse, self.tab,
                                  self.x["scale"], **self.sargs)
        else:
            self.ca.attn_fwd(self.q, self.k, self.v, self.o, self.lse, self.x["scale"], **self.sargs)

    def bwd(self):
        if self.cfg.out16:
            self.ca.attn_bwd_ex(self.q, self.k, self.v, self.o, self.do, self.lse, self.dq, self.dk, self.dv,
                                self.delta, self.x["scale"], **self.sargs)
        elif self.cfg.rope:
            self.ca.attn_bwd_rope(self.q_rot, self.k_rot, self.v, self.o, self.do, self.lse, self.dq, self.dk,
                                  self.dv, self.delta, self.tab, self.x["scale"], **self.sargs)
        else:
            self.ca.attn_bwd(self.q, self.k, self.v, self.o, self.do, self.lse, self.dq, self.dk, self.dv,
                             self.delta, self.x["scale"], workspace=self.ws, **self.sargs)

    def pre(self):
        self.ca.attn_bwd_preprocess(self.o, self.do, self.delta, stream=self.stream)

    def dkdv(self):
        self.ca.attn_bwd_dkdv(self.q, self.k, self.v, self.do, self.lse, self.delta, self.dk, self.dv,
                              self.x["scale"], **self.sargs)

    def dqk(self):
        self.ca.attn_bwd_dq(self.q, self.k, self.v, self.do, self.lse, self.delta, self.dq,
                            self.x["scale"], **self.sargs)

    def dq_delta(self):
        self.ca.attn_bwd_dq_delta(self.q, self.k, self.v, self.o, self.do, self.lse, self.dq, self.delta,
                                  self.x["scale"], **self.sargs)

    def step(self):
        self.fwd()
        self.bwd()

    def capture(self):
        """The step captured once as a HIP graph on the workload's stream (its
        launches only: the entry points allocate, copy and clear nothing)."""
        import torch
        self.step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            self.step()
        torch.cuda.synchronize()
        return g

    def host_loop(self, steps, warmup):
        """`warmup` untimed steps, then exactly `steps` steps between two device
        synchronisations with nothing else on the stream: host-clock seconds
        per step (the bench line's value)."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def timed_loop(self, steps, warmup, cold=None):
        """`warmup` untimed steps, then exactly `steps` steps between two device
        synchronisations.  Returns the host-clock seconds per step and, from HIP
        events recorded on the launch stream around each step's forward and
        backward, the per-iteration times (ms) of fwd, bwd and the whole step.
        cold: a device buffer written (on the same stream, outside the events)
        before every step, to evict the last-level cache."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            if cold is not None:
                with torch.cuda.stream(self.stream):
                    cold.fill_(float(i & 1))
            ev[i][0].record(self.stream)
            self.fwd()
            ev[i][1].record(self.stream)
            self.bwd()
            ev[i][2].record(self.stream)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        per = {"fwd": [e[0].elapsed_time(e[1]) for e in ev], "bwd": [e[1].elapsed_time(e[2]) for e in ev],
               "step": [e[0].elapsed_time(e[2]) for e in ev]}
        return sec, per

    def graph_seconds(self, steps, warmup):
        """Host-clock seconds per step of the step captured once and replayed."""
        import torch
        g = self.capture()
        with torch.cuda.stream(self.stream):
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                g.replay()
            torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def stages(self):
        """(name, call) of each kernel this workload's path runs, through the entry
        point that runs it alone: the forward, the two stages of attn_bwd (16-bit
        inputs: dQ with Delta fused, then dK/dV) and the standalone Delta
        preprocess (fp32 inputs run it inside attn_bwd_dq_delta; 16-bit callers
        of the staged API use it).  Workloads whose options have no staged entry
        points (grouped heads, RoPE, 16-bit outputs) time the forward and the
        whole backward only."""
        out = [("fwd", self.fwd), ("bwd", self.bwd)]
        if self.cfg.rope:  # the rotation pass alone (it is part of the forward above)
            out.append(("rope", lambda: self.ca.attn_rope(self.q, self.k, self.q_rot, self.k_rot, self.tab,
                                                          stream=self.stream)))
        elif not self.grouped and not self.cfg.out16:
            out += [("dq_delta", self.dq_delta), ("dkdv", self.dkdv), ("pre", self.pre)]
        return out

    def kernel_times(self, reps):
        """Per-kernel times (ms) from HIP events recorded on the launch stream,
        one pair of events around each stage in each of `reps` repetitions:
        median, p10, p90 and mean."""
        import torch
        stages = self.stages()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(reps)]
        for _ in range(3):
            self.step()
        torch.cuda.synchronize()
        for r in range(reps):
            ev[r][0].record(self.stream)
            for i, (_, fn) in enumerate(stages):
                fn()
                ev[r][i + 1].record(self.stream)
        torch.cuda.synchronize()
        return {name: stats([ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(reps)])
                for i, (name, _) in enumerate(stages)}

    def kernel_work(self):
        """Counted flops and algorithmic HBM bytes of one launch of each kernel:
        every input read once, every output written once (tile re-reads served by
        the caches are not algorithmic).  fwd: q, k, v -> o, lse; dq_delta: q, k,
        v, dO, o, lse -> dq, delta; dkdv: q, k, v, dO, lse, delta -> dk, dv; pre:
        o, dO -> delta."""
        nb = lambda t: t.numel() * t.element_size()  # noqa: E731
        D = self.x["D"]
        qkv = nb(self.q) + nb(self.k) + nb(self.v)
        return {
            "fwd": (4 * D * self.pairs, qkv + nb(self.o) + nb(self.lse)),
            "dq_delta": (2 * D * self.pairs,
                         qkv + nb(self.do) + nb(self.o) + nb(self.lse) + nb(self.delta) + nb(self.dq)),
            "dkdv": (8 * D * self.pairs,
                     qkv + nb(self.do) + nb(self.lse) + nb(self.delta) + nb(self.dk) + nb(self.dv)),
            "pre": (0, nb(self.o) + nb(self.do) + nb(self.delta)),
        }


def stats(ts):
    """median, p10, p90 and mean of a list of times (ms)."""
    a = np.asarray(ts, dtype=np.float64)
    return {"median_ms": float(np.median(a)), "p10_ms": float(np.percentile(a, 10)),
            "p90_ms": float(np.percentile(a, 90)), "mean_ms": float(a.mean()), "n": int(a.size)}


def sources_digest():
    """Digest of the library's sources and build flags (the library's build id)."""
    from causal_attention_amd.build import source_digest
    return source_digest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_digest") != sources_digest():
        return None
    ent = rec.get("kernels", {}).get(workload, {}).get(kernel)
    return None if ent is None else ent.get("bytes_per_launch")


KERNEL_NAMES = {"attn_fwd_kernel": "fwd", "attn_bwd_preprocess_kernel": "pre",
                "attn_bwd_dkdv_kernel": "dkdv", "attn_bwd_dkdv_pair_kernel": "dkdv", "attn_bwd_dq_kernel": "dq",
                "neg_kernel": "copy"}


def kernel_key(name):
    """Short name of a kernel from its (mangled or demangled) name; the dQ kernel
    with Delta fused (last template flag set) is 'dq_delta'."""
    key = next((v for k, v in KERNEL_NAMES.items() if k in name), None)
    if key == "dq" and ("Lb1EEEv" in name or re.search(r"attn_bwd_dq_kernel<[^(]*,\s*true>", name)):
        key = "dq_delta"
    return key


def copy_calibration(mib):
    """A plain elementwise kernel of known HBM traffic: reads and writes mib MiB."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def _counter_rows(directory):
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {directory}")
    for path in files:
        with open(path, newline="") as f:
            yield from csv.DictReader(f)


def _per_dispatch_kib(directory, counter):
    """Mean counter value (KiB) per dispatch, for each kernel this bench launches."""
    acc = {}
    for row in _counter_rows(directory):
        if row["Counter_Name"] != counter:
            continue
        name = kernel_key(row["Kernel_Name"])
        if name is None:
            continue
        d = acc.setdefault(name, {})
        d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in acc.items()}


def write_traffic(fetch_dir, write_dir, workload, mib):
    """HBM bytes per launch of each kernel: FETCH_SIZE + WRITE_SIZE (KiB per dispatch),
    each divided by what the same counter reads for the calibration kernel relative to
    its known traffic (mib MiB read, mib MiB written)."""
    fetch = _per_dispatch_kib(fetch_dir, "FETCH_SIZE")
    write = _per_dispatch_kib(write_dir, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("calibration kernel not found in the counter data")
    known_kib = mib * 1024.0
    f_fetch = fetch["copy"] / known_kib
    f_write = write["copy"] / known_kib
    kernels = {}
    for k in ("fwd", "pre", "dkdv", "dq", "dq_delta"):
        if k in fetch and k in write:
            fb = fetch[k] * 1024 / f_fetch
            wb = write[k] * 1024 / f_write
            kernels[k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb,
                          "raw_fetch_kib": fetch[k], "raw_write_kib": write[k]}
    rec = {"sources_digest": sources_digest(), "calibration": {
        "kernel": "torch.neg over fp32", "mib": mib, "fetch_factor": f_fetch, "write_factor": f_write},
        "kernels": {workload: kernels}}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def kernel_roofline(flops, nbytes, ms, mfma_peak):
    """One kernel against its binding roof: the matrix-core peak, or the HBM peak
    times its arithmetic intensity (flops per algorithmic byte), whichever is
    lower.  `achieved` and `peak` are in the binding roof's unit (TFLOP/s for
    the matrix cores, GB/s for HBM), so frac is the same either way."""
    t = ms * 1e-3
    tflops = flops / t / 1e12
    gbs = nbytes / t / 1e9
    ai = flops / nbytes
    hbm_bound = ai * PEAK_HBM_GBS * 1e9 < mfma_peak * 1e12
    if hbm_bound:
        r = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": tflops, "peak": mfma_peak, "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r.update({"ms": ms, "flops": flops, "bytes": nbytes, "flop_per_byte": ai, "tflops": tflops, "gbs": gbs,
              "frac_of_mfma_peak": tflops / mfma_peak})
    return r


def rooflines(w, times):
    """Every timed kernel of the path against its own binding roof (median times)."""
    peak = PEAK_BF16_TFLOPS if w.cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    work = w.kernel_work()
    return {k: kernel_roofline(*work[k], times[k]["median_ms"], peak) for k in work if k in times}


def roofline(w, times, per_kernel):
    """The top-level entry: the kernel of the path (fwd, dq_delta, dkdv) taking
    the most time per step, with its rocprofv3-measured HBM bytes per launch
    when those were taken on the current sources."""
    on_path = [k for k in ("fwd", "dq_delta", "dkdv") if k in per_kernel]
    if not on_path:
        return None
    dom = max(on_path, key=lambda k: times[k]["median_ms"])
    r = {k: per_kernel[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    r["traffic"] = measured_traffic(dom, w.name)
    r["kernel"] = dom
    r["algorithmic_bytes"] = per_kernel[dom]["bytes"]
    return r


def sample_sclk(w, seconds):
    """Graphics clock (MHz) while the workload's steps run back to back for
    `seconds`: the library's clock probe (one wave on a stream of its own,
    reading the shader-clock and 100 MHz counters) spans the middle 80 % of
    that window; cycles / ticks x 100 MHz is the clock of the chiplet the
    probe ran on."""
    import torch
    import causal_attention_amd as ca
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        w.step()
    t_end = time.perf_counter() + seconds
    n = 0
    launched = False
    while time.perf_counter() < t_end:
        w.step()
        n += 1
        if not launched and n == 8:  # the queue is full of work: start the probe
            ca.clock_probe(out, int(0.8 * seconds * 1e8), stream=side)
            launched = True
        if n % 64 == 0:  # keep the host at most 64 steps ahead
            w.stream.synchronize()
    torch.cuda.synchronize()
    cycles, ticks = (int(x) for x in out.cpu().tolist())
    if ticks <= 0:
        return {"error": "clock probe did not run"}
    return {"mhz": cycles / ticks * 100.0, "steps": n, "probe_ms": ticks / 1e5,
            "method": "s_memtime / s_memrealtime on a side stream during back-to-back steps"}


def cpu_baseline(w, seconds):
    """The fp64 oracle (as it stands) on whole heads of the same workload, until about
    `seconds` of host time are spent; reported in the same unit as the GPU value."""
    from oracle import attention_bwd_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=1)
    except Exception:  # threadpoolctl missing or no BLAS info
        threads = os.cpu_count() or 1
    x = w.x
    B, H, S, D = x["B"], x["H"], x["S"], x["D"]
    args = [x[n].astype(np.float64) for n in ("q", "k", "v", "do")]
    cu = x["cu_seqlens"]
    per_head_pairs = allowed_pair_count(S, 1, 1, cu)
    heads = [(b, h) for b in range(B) for h in range(H)]
    done = 0
    t0 = time.perf_counter()
    # whole heads, cycling through the workload until the time budget is spent
    while time.perf_counter() - t0 < seconds:
        bh = heads[done % len(heads)]
        attention_bwd_ref(*args, x["scale"], x["mask_mode"], cu, heads=[bh])
        done += 1
    dt = time.perf_counter() - t0
    flops = 14 * D * per_head_pairs * done
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"fwd+bwd of {done} heads (of {len(heads)}, cycled) of B{B} H{H} S{S} D{D}, {dt:.1f} s"}


def measure_decode(name, reps):
    """One decode step (attn_decode) on the cache workload: mean time from HIP events
    over `reps` back-to-back calls, and the cache-read rate against HBM peak.
    Algorithmic bytes: K and V rows read (sum of lengths x H_kv x D x 2 tensors),
    q, and the fp32 outputs O and LSE; the chunk partials are not counted."""
    import torch
    import causal_attention_amd as ca
    from workload import DECODE_CONFIGS, make_decode_inputs
    cfg = DECODE_CONFIGS[name]
    x = make_decode_inputs(cfg, 7)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).cuda().to(dt) for n in ("q", "k", "v"))
    lens = torch.from_numpy(x["lens"]).cuda()
    o = torch.empty((cfg.B, cfg.H, cfg.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.B, cfg.H), dtype=torch.float32, device="cuda")
    nbytes = ca.decode_workspace_bytes(cfg.B, cfg.H, cfg.H_kv, cfg.D, int(x["lens"].max()))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        ca.attn_decode(q, k, v, lens, o, lse, ws, x["scale"], int(x["lens"].max()), stream)

    for _ in range(5):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    esz = 2 if cfg.dtype == "bf16" else 4
    kv_bytes = int(x["lens"].sum()) * cfg.H_kv * cfg.D * 2 * esz
    alg = kv_bytes + cfg.B * cfg.H * cfg.D * esz + cfg.B * cfg.H * (cfg.D + 1) * 4
    gbs = alg / t / 1e9
    return {"us_per_step": t * 1e6, "achieved_GBs": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS,
            "bytes_per_step": alg, "config": {"B": cfg.B, "H": cfg.H, "H_kv": cfg.H_kv, "cache": cfg.length,
                                               "D": cfg.D, "dtype": cfg.dtype}}


def measure(name, steps, warmup, reps, cold_mib=0, sclk_seconds=0.0):
    """One workload: the timed loop (host clock + per-iteration events), the
    graph-replayed step, per-kernel event times and rooflines; optionally the
    cold-cache loop and the clock samples."""
    import torch
    w = Workload(name)
    sec = w.host_loop(steps, warmup)
    sec_events, per = w.timed_loop(steps, 3)
    sec_graph = w.graph_seconds(steps, warmup)
    total = w.flops_fwd + w.flops_bwd
    peak = PEAK_BF16_TFLOPS if w.cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    ev = {k: stats(v) for k, v in per.items()}
    times = w.kernel_times(reps)
    per_kernel = rooflines(w, times)
    tflops = total / sec / 1e12
    summary = {
        "tflops": tflops, "pct_peak": 100.0 * tflops / peak, "ms_per_step": sec * 1e3,
        "ms_per_step_graph": sec_graph * 1e3, "ms_per_step_with_events": sec_events * 1e3,
        "events_ms": ev,
        "tflops_events_median": total / (ev["step"]["median_ms"] * 1e-3) / 1e12,
        "fwd_tflops": w.flops_fwd / (ev["fwd"]["median_ms"] * 1e-3) / 1e12,
        "bwd_tflops": w.flops_bwd / (ev["bwd"]["median_ms"] * 1e-3) / 1e12,
        "kernels_ms": {k: round(v["median_ms"], 5) for k, v in times.items()},
        "pairs": w.pairs,
    }
    if per_kernel:
        summary["rooflines"] = {k: {f: v[f] for f in ("bound", "frac", "tflops", "gbs", "ms")}
                                for k, v in per_kernel.items()}
    if "pre" in per_kernel:
        summary["preprocess_GBs"] = per_kernel["pre"]["gbs"]
        summary["preprocess_frac_hbm_peak"] = per_kernel["pre"]["gbs"] / PEAK_HBM_GBS
    if "rope" in times:  # the rotation pass reads q, k and writes q_rot, k_rot once (the table stays in L2)
        nbytes = 2 * (w.q.numel() + w.k.numel()) * w.q.element_size()
        summary["rope_GBs"] = nbytes / (times["rope"]["median_ms"] * 1e-3) / 1e9
    if cold_mib:
        buf = torch.empty(cold_mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
        _, cper = w.timed_loop(max(20, steps // 4), 3, cold=buf)
        cev = {k: stats(v) for k, v in cper.items()}
        summary["cold"] = {"evict_mib": cold_mib, "events_ms": cev,
                           "tflops_events_median": total / (cev["step"]["median_ms"] * 1e-3) / 1e12}
        del buf
    if sclk_seconds:
        summary["sclk_mhz"] = sample_sclk(w, sclk_seconds)
    return w, sec, times, per_kernel, summary


def main():
    a = parse()
    if a.write_traffic:
        rec = write_traffic(*a.write_traffic, a.workload, a.copy_calibration or 256)
        print(json.dumps(rec, indent=1))
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(attention shards by batch and head with no communication: run one process per GPU on its share)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import causal_attention_amd as ca
    ca.load_library()  # refuses a library built from other sources than this tree's

    log(f"[bench] library build {ca.build_id()}; workload {a.workload}: warmup {a.warmup}, steps {a.steps}")
    w, sec, times, per_kernel, summary = measure(a.workload, a.steps, a.warmup, a.kernel_reps,
                                                 cold_mib=a.cold_mib, sclk_seconds=a.sclk_seconds)
    log(f"[bench] {a.workload}: {summary['tflops']:.1f} TFLOPS ({summary['pct_peak']:.1f}% of peak), "
        f"{sec * 1e3:.4f} ms/step, step events median {summary['events_ms']['step']['median_ms']:.4f} ms, "
        f"kernels {summary['kernels_ms']}")
    by_workload = {a.workload: summary}
    if not a.no_others:
        for name in ("lm12m_ctx512", "long_ctx8192", "packed_docs8192", "lm237m_ctx1024_gqa4",
                     "long_ctx8192_gqa4", "lm237m_ctx1024_rope", "lm237m_ctx1024_out16", "lm237m_ctx1024"):
            if name == a.workload:
                continue
            _, _, _, _, s = measure(name, max(50, a.steps // 2), max(10, a.warmup), max(20, a.kernel_reps // 2))
            by_workload[name] = s
            log(f"[bench] {name}: {s['tflops']:.1f} TFLOPS ({s['pct_peak']:.1f}% of peak), "
                f"kernels {s['kernels_ms']}")
        d = measure_decode("decode_ctx8192", max(20, a.kernel_reps))
        by_workload["decode_ctx8192"] = d
        log(f"[bench] decode_ctx8192: {d['us_per_step']:.1f} us/step, {d['achieved_GBs']:.0f} GB/s "
            f"({100 * d['frac_hbm_peak']:.1f}% of HBM peak)")
    rl = roofline(w, times, per_kernel)
    log(f"[bench] roofline: {rl}")
    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host ...")
        cpu = cpu_baseline(w, a.cpu_seconds)
        log(f"[bench] cpu baseline: {cpu}")
    cfg = w.cfg
    line = {
        "metric": METRIC,
        "value": summary["tflops"],
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "S": cfg.S, "D": cfg.D,
                   "mask": "packed_documents" if cfg.mask_mode else "causal",
                   "outputs": cfg.dtype if cfg.out16 else "fp32", "parallelism": "single GPU"},
        "pct_peak": summary["pct_peak"],
        "build_id": ca.build_id(),
        "events_ms": summary["events_ms"],
        "tflops_events_median": summary["tflops_events_median"],
        "ms_per_step_graph": summary["ms_per_step_graph"],
        "ms_per_step_with_events": summary["ms_per_step_with_events"],
        "fwd_tflops": summary["fwd_tflops"],
        "bwd_tflops": summary["bwd_tflops"],
        "cold": summary.get("cold"),
        "sclk_mhz": summary.get("sclk_mhz"),
        "pct_peak_at_sclk": (100.0 * summary["tflops"] / (PEAK_BF16_TFLOPS * summary["sclk_mhz"]["mhz"] / 2400.0)
                             if isinstance(summary.get("sclk_mhz"), dict) and "mhz" in summary["sclk_mhz"]
                             else None),
        "preprocess_GBs": summary.get("preprocess_GBs"),
        "kernels": times,
        "rooflines": per_kernel,
        "roofline": rl,
        "cpu_baseline": cpu,
        "by_workload": by_workload,
    }
    print(json.dumps(line), flush=True)
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)


if __name__ == "__main__":
    main()
