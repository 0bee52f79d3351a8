#!/usr/bin/env python3
"""Throughput of fused causal attention, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path on resident inputs: attn_fwd (forward
with LSE) then attn_bwd (Delta preprocess, dK/dV, dQ), called on a stream of
the workload's own.  (The same step captured as a HIP graph and replayed is
no faster on this stack: ms_per_step_graph.)  Throughput counts the
causal FLOPs actually allowed by the mask: 4*D per allowed (query, key) pair
forward and 10*D backward (the five products of the FlashAttention-2
accounting), divided by the measured time.  One JSON line is printed.

Besides the headline workload the line carries:
  by_workload   the same measurement at the other full-size workloads
                (context 512, 8192, packed documents, grouped-query heads,
                RoPE on q and k, bf16 outputs),
                fewer steps, and one decode step against a full 8192-token
                K/V cache (time, GB/s against HBM peak);
  kernels       per-kernel mean duration from HIP events on the launch stream;
  roofline      the dominant kernel against its roofline;
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
         "lm237m_ctx1024_gqa4": 6, "lm237m_ctx1024_rope": 7, "lm237m_ctx1024_out16": 8}
# algorithmic flops per allowed pair, per kernel (times D)
KERNEL_FLOPS_PER_PAIR = {"fwd": 4, "dkdv": 8, "dq": 2}
KERNEL_SOURCES = ["attn_device.h", "attn_launch.h", "attn_fwd.hip", "attn_bwd.hip"]


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
                             self.delta, self.x["scale"], **self.sargs)

    def pre(self):
        self.ca.attn_bwd_preprocess(self.o, self.do, self.delta, stream=self.stream)

    def dkdv(self):
        self.ca.attn_bwd_dkdv(self.q, self.k, self.v, self.do, self.lse, self.delta, self.dk, self.dv,
                              self.x["scale"], **self.sargs)

    def dqk(self):
        self.ca.attn_bwd_dq(self.q, self.k, self.v, self.do, self.lse, self.delta, self.dq,
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

    def timed_steps(self, steps, warmup, graph=False):
        """Seconds per step over `steps` steps after `warmup`: the entry points
        called in turn, or (graph=True) one replay of the captured step."""
        import torch
        if graph:
            g = self.capture()

            def run():
                with torch.cuda.stream(self.stream):
                    g.replay()
        else:
            run = self.step
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def kernel_times(self, reps):
        """Mean duration (ms) from HIP events recorded on the launch stream: the
        forward, the whole backward call, and the three backward stages run one
        by one through their own entry points (with bf16 inputs attn_bwd runs
        dQ with Delta fused, then dK/dV; the staged dQ reads Delta instead)."""
        import torch
        stages = [("fwd", self.fwd), ("bwd", self.bwd)]
        if self.cfg.rope:  # the rotation pass alone (it is part of the forward above)
            stages.append(("rope", lambda: self.ca.attn_rope(self.q, self.k, self.q_rot, self.k_rot, self.tab,
                                                             stream=self.stream)))
        elif not self.grouped and not self.cfg.out16:  # the staged entry points: fp32 outputs, plain heads
            stages += [("pre", self.pre), ("dkdv", self.dkdv), ("dq", self.dqk)]
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
        out = {}
        for i, (name, _) in enumerate(stages):
            ts = sorted(ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(reps))
            out[name] = {"mean_ms": float(np.mean(ts)), "median_ms": float(np.median(ts))}
        return out

    def preprocess_bytes(self):
        B, H, S, D = self.x["B"], self.x["H"], self.x["S"], self.x["D"]
        in_bytes = 2 if self.cfg.dtype == "bf16" else 4
        return B * H * S * (D * (in_bytes + 4) + 4)


def sources_digest():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "causal_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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


def roofline(w, times):
    """The dominant kernel (most time per step) against its roofline."""
    peak = PEAK_BF16_TFLOPS if w.cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    dom = max((k for k in times if k in KERNEL_FLOPS_PER_PAIR or k == "pre"), key=lambda k: times[k]["mean_ms"])
    t = times[dom]["mean_ms"] * 1e-3
    if dom == "pre":
        achieved = w.preprocess_bytes() / t / 1e9
        r = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        achieved = KERNEL_FLOPS_PER_PAIR[dom] * w.x["D"] * w.pairs / t / 1e12
        r = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["traffic"] = measured_traffic(dom, w.name)
    r["kernel"] = dom
    return r


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


def measure(name, steps, warmup, reps):
    w = Workload(name)
    sec = w.timed_steps(steps, warmup)
    sec_graph = w.timed_steps(steps, warmup, graph=True)
    total = w.flops_fwd + w.flops_bwd
    tflops = total / sec / 1e12
    times = w.kernel_times(reps)
    peak = PEAK_BF16_TFLOPS if w.cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    ms_fwd = times["fwd"]["mean_ms"]
    ms_bwd = times["bwd"]["mean_ms"]
    summary = {
        "tflops": tflops, "pct_peak": 100.0 * tflops / peak, "ms_per_step": sec * 1e3,
        "ms_per_step_graph": sec_graph * 1e3,
        "fwd_tflops": w.flops_fwd / (ms_fwd * 1e-3) / 1e12,
        "bwd_tflops": w.flops_bwd / (ms_bwd * 1e-3) / 1e12,
        "kernels_ms": {k: round(v["mean_ms"], 5) for k, v in times.items()},
        "pairs": w.pairs,
    }
    if "rope" in times:  # the rotation pass reads q, k and writes q_rot, k_rot once (the table stays in L2)
        nbytes = 2 * (w.q.numel() + w.k.numel()) * w.q.element_size()
        summary["rope_GBs"] = nbytes / (times["rope"]["mean_ms"] * 1e-3) / 1e9
    return w, sec, times, summary


def main():
    a = parse()
    if a.write_traffic:
        rec = write_traffic(*a.write_traffic, a.workload, a.copy_calibration or 256)
        print(json.dumps(rec, indent=1))
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(attention shards by batch and head with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import causal_attention_amd as ca
    ca.load_library()

    log(f"[bench] workload {a.workload}: warmup {a.warmup}, steps {a.steps}")
    w, sec, times, summary = measure(a.workload, a.steps, a.warmup, a.kernel_reps)
    log(f"[bench] {a.workload}: {summary['tflops']:.1f} TFLOPS ({summary['pct_peak']:.1f}% of peak), "
        f"{sec * 1e3:.4f} ms/step, kernels {summary['kernels_ms']}")
    by_workload = {a.workload: summary}
    if not a.no_others:
        for name in ("lm12m_ctx512", "long_ctx8192", "packed_docs8192", "lm237m_ctx1024_gqa4",
                     "lm237m_ctx1024_rope", "lm237m_ctx1024_out16", "lm237m_ctx1024"):
            if name == a.workload:
                continue
            _, _, _, s = measure(name, max(10, a.steps // 4), max(3, a.warmup // 2), max(10, a.kernel_reps // 2))
            by_workload[name] = s
            log(f"[bench] {name}: {s['tflops']:.1f} TFLOPS ({s['pct_peak']:.1f}% of peak), "
                f"kernels {s['kernels_ms']}")
        d = measure_decode("decode_ctx8192", max(20, a.kernel_reps))
        by_workload["decode_ctx8192"] = d
        log(f"[bench] decode_ctx8192: {d['us_per_step']:.1f} us/step, {d['achieved_GBs']:.0f} GB/s "
            f"({100 * d['frac_hbm_peak']:.1f}% of HBM peak)")
    rl = roofline(w, times)
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
        "ms_per_step_graph": summary["ms_per_step_graph"],
        "fwd_tflops": summary["fwd_tflops"],
        "bwd_tflops": summary["bwd_tflops"],
        "kernels": {k: v["mean_ms"] for k, v in times.items()},
        "roofline": rl,
        "cpu_baseline": cpu,
        "by_workload": by_workload,
    }
    print(json.dumps(line), flush=True)
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)


if __name__ == "__main__":
    main()
