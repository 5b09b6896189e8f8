#!/usr/bin/env python3
"""Benchmark of the chunked gated-delta-rule prefill forward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: device chunk-index table (built by stage 1 itself
for batches of up to 256 sequences, else by its own kernel) -> intra-chunk
stage -> inter-chunk stage (plus the conv/SiLU/L2 front for workloads that
have one),
launched through the C ABI's whole-forward call on torch's current stream.
W untimed warm-up steps, then exactly K timed steps bracketed by device
synchronisation; value = tokens x K / wall time of the timed region. On
every E-th timed step (default 8) each kernel records a pair of HIP events
at its own start and end (the timed variants of the entry points launch with
hipExtLaunchKernel, so no packet sits between the launches); the other steps
call the plain entry points, because per-dispatch events cost the step they
are on a few microseconds. Each kernel's duration averaged over the sampled
steps is its execution time; the dominant kernel's algorithmic bytes per
launch divided by that duration is the roofline figure.

Workloads 5 and 6 (a draft-verify batch of 64 x 8 tokens, a decode batch of
256 x 1 token) time the token-serial recurrent kernel (gdn_recurrent_fwd)
instead: a step is one call of it, and its roofline is HBM.

Prints ONE JSON line. Default workload: single sequence, T = 4096, H = 16,
Hv = 32, D = 128, bf16 q/k/v (the configuration the metric is quoted on).
The CPU baseline is the fp64 oracle timed on this host's cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunk-prefill tokens/s at 1 GPU; % MFMA peak (intra), % HBM BW (inter)"
METRIC_RECURRENT = "GDN token-serial decode/verify tokens/s at 1 GPU; % HBM BW"
RECURRENT_WORKLOADS = (5, 6)  # run by gdn_recurrent_fwd instead of the chunked forward
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
SOLVE_FLOP = 83328           # 64x64 unit-lower inverse: 41,664 multiply-adds
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def algorithmic_work(wl, nt, qkv_bytes, fused_front=False, u_bytes=4):
    """Bytes and flops each stage must move / perform (counted once; partial
    chunks counted as whole 64-token chunks for flops). w crosses between the
    stages in 2 bytes per value and u in `u_bytes`: 4 (fp32) is the model the
    headline roofline uses; this library stores u in 3 (24-bit floats), which
    gives the smaller, stored-byte figure. With the front fused into stage 1,
    that stage reads the pre-conv bf16 q|k|v channels instead of k and v."""
    T, H, Hv, D = wl.n_tokens, wl.H, wl.Hv, 128
    HG = Hv // H
    n_state = len(wl.cu_seqlens) - 1
    stage1_in = (2 * H + Hv) * D * 2 if fused_front else H * D * qkv_bytes + Hv * D * qkv_bytes
    stage1_bytes = T * (stage1_in + Hv * 4 + Hv * 4 + Hv * D * 2 + Hv * D * u_bytes)
    stage2_bytes = T * (2 * H * D * qkv_bytes + Hv * D * 2 + Hv * D * u_bytes + Hv * 4 +
                        Hv * D * 4)
    stage2_bytes += n_state * Hv * D * D * 4 * (2 if wl.h0 is not None else 1)
    stage1_flop = nt * H * (2 * 64 * 64 * D + HG * (2 * 2 * 64 * 64 * D + SOLVE_FLOP))
    stage2_flop = nt * Hv * (3 * 2 * 64 * D * D + 2 * 2 * 64 * 64 * D)
    front_bytes = 0
    if wl.qkv is not None and not fused_front:
        C = (2 * H + Hv) * D
        front_bytes = T * C * 2 + T * C * 4
    # token-serial kernel: q, k, v, g, beta in, o out per token, the state read
    # (if given) and written once; per token and value head the two sums over
    # the state and its rank-1 update, 6 D^2 flops
    rec_bytes = T * (2 * H * D * qkv_bytes + Hv * D * qkv_bytes + Hv * 8 + Hv * D * 4)
    rec_bytes += n_state * Hv * D * D * 4 * (2 if wl.h0 is not None else 1)
    rec_flop = T * Hv * 6 * D * D
    return dict(intra=(stage1_bytes, stage1_flop), inter=(stage2_bytes, stage2_flop),
                front=(front_bytes, 0), index=(0, 0), recurrent=(rec_bytes, rec_flop))


def kernel_source_digest(name):
    """Digest of a kernel's code (its source and the shared device headers),
    with // comments and blank lines left out, so that counter figures stay
    attached to the code they were measured on and not to its comments."""
    csrc = os.path.join(ROOT, "chunked_gated_delta_rule_amd", "csrc")
    h = hashlib.sha256()
    for f in (name + ".hip", "gdn_common.hpp", "gdn_launch.hpp"):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            code = re.sub(r"//[^\n]*", "", fh.read())
        h.update("\n".join(l.strip() for l in code.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def counter_traffic(kernel, workload_name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current source of that kernel; else None."""
    try:
        with open(COUNTERS) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(kernel, {}).get(workload_name)
    if not ent or ent.get("source_digest") != kernel_source_digest(kernel):
        return None
    return ent.get("traffic_bytes")


class HipEvents:
    """Raw HIP events from the runtime torch has loaded (same soname)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self, n):
        out = []
        for _ in range(n):
            e = self.ct.c_void_p()
            if self.rt.hipEventCreate(self.ct.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        self.made += out
        return out

    def ms(self, a, b):
        t = self.ct.c_float()
        if self.rt.hipEventElapsedTime(self.ct.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def close(self):
        for e in self.made:
            self.rt.hipEventDestroy(e)
        self.made = []


def cpu_baseline(wl, max_seconds=20.0, min_seconds=10.0, one_thread_seconds=4.0):
    """The fp64 oracle on this host's cores, over whole value-head lanes of
    the workload (as many key-head groups as fit the budget), scaled to
    tokens/s. For a workload with a front, the sample is its first sequence:
    the fp64 front over every channel of it (timed on its own, not scaled),
    then the lanes. Short samples are repeated until about min_seconds of CPU
    work (at least 3 runs); the median run is reported. The same is then timed
    on one thread, over fewer lanes."""
    import numpy as np
    from oracle import recurrent

    threads = recurrent.threads()
    HG = wl.Hv // wl.H
    front = wl.qkv is not None
    g, b, h0 = wl.f64("g"), wl.f64("beta"), wl.f64("h0")
    if front:
        tokens = int(wl.cu_seqlens[1])
        cu = np.array([0, tokens], np.int32)
        x, w = wl.f64("qkv")[:tokens], wl.f64("conv_w")
        g, b = g[:tokens], b[:tokens]
        h0 = None if h0 is None else h0[:1]
        q, k, v = recurrent.gdn_front(x, w, cu, wl.H, wl.Hv, 128, 128)
    else:
        tokens = wl.n_tokens
        cu = wl.cu_seqlens
        q, k, v = wl.f64("q"), wl.f64("k"), wl.f64("v")

    def run_front():
        t0 = time.perf_counter()
        recurrent.gdn_front(x, w, cu, wl.H, wl.Hv, 128, 128)
        return time.perf_counter() - t0

    def run_lanes(n_groups):  # the first n_groups key heads and their value heads
        hv_hi = n_groups * HG
        t0 = time.perf_counter()
        recurrent.gdn_recurrent(q[:, :n_groups], k[:, :n_groups], v[:, :hv_hi], g[:, :hv_hi],
                                b[:, :hv_hi], cu, h0=None if h0 is None else h0[:, :hv_hi])
        return time.perf_counter() - t0

    def measure(budget, floor):
        lane_s = run_lanes(1)  # HG lanes side by side (about one lane's time on many threads)
        per_round = max(1, recurrent.threads() // HG)
        fit = int(budget / 3 / max(lane_s, 1e-3)) * per_round
        n_groups = max(1, min(wl.H, fit))
        times = [run_lanes(n_groups) for _ in range(3)]
        while sum(times) < floor and len(times) < 1000:
            times.append(run_lanes(n_groups))
        med = statistics.median(times)
        lanes = n_groups * HG
        full = med * (wl.Hv / lanes)
        what = (f"{'all' if lanes == wl.Hv else lanes} of {wl.Hv} value-head lanes x "
                f"{tokens} tokens, median of {len(times)} runs ({med:.3f} s each, "
                f"{sum(times):.1f} s in all)" + ("" if lanes == wl.Hv else ", scaled to all lanes"))
        if front:
            tf = [run_front() for _ in range(3)]
            full += statistics.median(tf)
            what = (f"sequence 0 of {wl.n_seqs}: the fp64 front over its {tokens} tokens "
                    f"(median of 3 runs, {statistics.median(tf):.3f} s), then " + what)
        return tokens / full, what

    value, sample = measure(max_seconds, min_seconds)
    recurrent.set_threads(1)
    try:
        value1, sample1 = measure(one_thread_seconds, one_thread_seconds / 2)
    finally:
        recurrent.set_threads(threads)
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample,
            "one_thread": {"value": value1, "unit": "tokens/s", "cores": 1, "sample": sample1}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--event-every", type=int, default=8, metavar="E",
                    help="time the kernels of every E-th step with dispatch events (the "
                         "others run the plain entry point: per-dispatch events add a few "
                         "microseconds to the step they are on)")
    ap.add_argument("--workload", type=int, default=1,
                    help="named workload 0..7 (5 and 6 time the token-serial kernel)")
    ap.add_argument("--segments", type=int, default=0, choices=(0, 1, 2, 3, 4),
                    help="stage-2 segments per sequence (default 0: the automatic choice)")
    ap.add_argument("--settle-ms", type=float, default=1000.0, metavar="MS",
                    help="before the W warm-up steps, run untimed steps for this many "
                         "milliseconds of wall time, so that the GPU clocks and the host "
                         "launch path reach steady state even when W is small (reported as "
                         "settle_steps; 0 to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-samples", type=int, default=10, metavar="N",
                    help="after the timed region, time N more steps each preceded by a 1 GiB "
                         "device write that evicts the last-level cache (reported apart from "
                         "the headline value; 0 to skip)")
    ap.add_argument("--front-dtype", choices=("f16", "f32"), default="f16",
                    help="front workload: precision the front's q, k, v enter the chunk "
                         "forward in (fused path: GDN_F16 rounds them to fp16, GDN_F32 keeps "
                         "fp32; the unfused path always hands fp32 to the forward)")
    ap.add_argument("--unfused-front", action="store_true",
                    help="front workload: run the standalone front, then the forward "
                         "(default: the front fused into stage 1)")
    ap.add_argument("--gqa-share", type=int, default=0, choices=(0, 1, 2, 4),
                    help="stage 2 in the GQA-shared shape: one 16-column slice of this many "
                         "value heads of a key head per work-group (default 0: the "
                         "automatic column-tile and segment choice)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import chunked_gated_delta_rule_amd as gdn
    import workloads

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = "cuda:0"
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": args.steps}))
        return
    wl = workloads.make(args.workload)
    if args.gqa_share > 1 and (wl.Hv // wl.H) % args.gqa_share != 0:
        print(f"--gqa-share {args.gqa_share}: workload {args.workload} has {wl.Hv // wl.H} value "
              f"heads per key head, which the share must divide", file=sys.stderr)
        sys.exit(2)
    d = {n: (getattr(wl, n).to(dev).contiguous() if getattr(wl, n) is not None else None)
         for n in ("q", "k", "v", "g", "beta", "h0", "qkv", "conv_w")}
    cu = torch.from_numpy(wl.cu_seqlens).to(dev)
    has_front = wl.qkv is not None
    fused_front = has_front and not args.unfused_front
    serial = args.workload in RECURRENT_WORKLOADS
    qkv_dtype = wl.qkv_dtype
    if has_front:
        qkv_dtype = torch.float16 if fused_front and args.front_dtype == "f16" else torch.float32
    cfg = gdn.make_config(wl.t_max, wl.n_max, wl.H, wl.Hv, qkv_dtype, gqa_share=args.gqa_share,
                          segments=args.segments)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=dev)
    o = torch.empty((wl.t_max, wl.Hv, 128), dtype=torch.float32, device=dev)
    hT = torch.empty((wl.n_max, wl.Hv, 128, 128), dtype=torch.float32, device=dev)
    if has_front and not fused_front:
        q = torch.empty((wl.t_max, wl.H, 128), dtype=torch.float32, device=dev)
        k = torch.empty_like(q)
        v = torch.empty((wl.t_max, wl.Hv, 128), dtype=torch.float32, device=dev)
    else:
        q, k, v = d["q"], d["k"], d["v"]

    # without a caller table, batches of at most GDN_FUSED_INDEX_MAX_SEQS
    # sequences have stage 1 locate its chunks (and fill the table) itself
    table_kernel = wl.n_max > gdn.GDN_FUSED_INDEX_MAX_SEQS
    stages = (["front"] if has_front and not fused_front else []) + \
        (["index"] if table_kernel else []) + ["intra", "inter"]
    if serial:
        stages = ["recurrent"]
    hip = HipEvents()

    def step(evs=None):
        if serial:
            if evs is None:
                gdn.gdn_recurrent_fwd(cfg, q, k, v, d["g"], d["beta"], d["h0"], cu, o, hT)
            else:
                gdn.gdn_recurrent_fwd_timed(cfg, q, k, v, d["g"], d["beta"], d["h0"], cu, o, hT,
                                            evs[0], evs[1])
            return
        if fused_front:
            if evs is None:
                gdn.gdn_chunk_fwd_conv(cfg, d["qkv"], d["conv_w"], wl.d_conv, d["g"], d["beta"],
                                       d["h0"], cu, None, o, hT, ws)
            else:
                gdn.gdn_chunk_fwd_conv_timed(cfg, d["qkv"], d["conv_w"], wl.d_conv, d["g"],
                                             d["beta"], d["h0"], cu, None, o, hT, ws, evs[:6])
            return
        if has_front:
            if evs is None:
                gdn.gdn_front_conv_silu_l2(cfg, d["qkv"], d["conv_w"], wl.d_conv, cu, q, k, v)
            else:
                gdn.gdn_front_conv_silu_l2_timed(cfg, d["qkv"], d["conv_w"], wl.d_conv, cu, q, k,
                                                 v, evs[6], evs[7])
        if evs is None:
            gdn.gdn_chunk_fwd(cfg, q, k, v, d["g"], d["beta"], d["h0"], cu, None, o, hT, ws)
        else:
            gdn.gdn_chunk_fwd_timed(cfg, q, k, v, d["g"], d["beta"], d["h0"], cu, None, o, hT, ws,
                                    evs[:6])

    # Untimed steps run the same launch path as the timed loop: every E-th
    # step carries dispatch events (one reused set), so first-use costs of
    # the event path are paid before timing.
    every = max(1, args.event_every)
    warm_events = hip.create(8 if has_front else 6)

    def untimed(i):
        step(warm_events if i % every == every - 1 else None)

    # settle: untimed steps for a fixed wall time (a fresh process on an idle
    # GPU runs its first steps at lower clocks and with a slower host path)
    settle_steps = 0
    if args.settle_ms > 0:
        t_settle = time.perf_counter()
        while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
            for _ in range(16):
                untimed(settle_steps)
                settle_steps += 1
            torch.cuda.synchronize()
    for i in range(args.warmup):
        untimed(i)
    torch.cuda.synchronize()
    timed = [s_ % every == every - 1 or s_ == args.steps - 1 for s_ in range(args.steps)]
    events = [hip.create(8 if has_front else 6) if t else None for t in timed]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(events[s_])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    events = [ev for ev in events if ev is not None]

    pair = {"index": (0, 1), "intra": (2, 3), "inter": (4, 5), "front": (6, 7),
            "recurrent": (0, 1)}

    def stage_ms(evs):
        return {name: statistics.fmean(hip.ms(ev[pair[name][0]], ev[pair[name][1]]) for ev in evs)
                for name in stages}

    per_stage_ms = stage_ms(events)

    # Cold last-level cache (outside the timed region and the headline value):
    # a 1 GiB device write before each sampled step evicts the 256 MB MALL, so
    # the step's inputs and intermediates come from HBM.
    cold = None
    if args.cold_samples > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold_events = [hip.create(8 if has_front else 6) for _ in range(args.cold_samples)]
        for ev in cold_events:
            flush.fill_(1.0)
            step(ev)
        torch.cuda.synchronize()
        del flush
        cold_ms = stage_ms(cold_events)
        cold = {"samples": args.cold_samples, "flush_bytes": 1 << 30,
                **{f"{name}_us": round(cold_ms[name] * 1e3, 2) for name in stages}}
    hip.close()
    chunks = int(sum(-(-int(x) // 64) for x in np.diff(wl.cu_seqlens)))
    qkv_bytes = 4 if qkv_dtype == torch.float32 else 2
    work = algorithmic_work(wl, chunks, qkv_bytes, fused_front)               # u at 4 bytes
    work_u24 = algorithmic_work(wl, chunks, qkv_bytes, fused_front, u_bytes=3)  # as stored
    ms_per_step = elapsed * 1e3 / args.steps
    tokens = wl.n_tokens
    detail = {}
    for name in stages:
        t_s = per_stage_ms[name] * 1e-3
        b, f = work[name]
        b3 = work_u24[name][0]
        detail[name] = {"us": round(per_stage_ms[name] * 1e3, 2),
                        "alg_bytes": b, "alg_flop": f,
                        "hbm_frac": round(b / t_s / (HBM_PEAK_GBS * 1e9), 4) if b else None,
                        "hbm_frac_u24": round(b3 / t_s / (HBM_PEAK_GBS * 1e9), 4) if b3 else None,
                        "mfma_frac": round(f / t_s / (BF16_PEAK_TFLOPS * 1e12), 4) if f else None}
        if cold:
            detail[name]["cold_us"] = cold[f"{name}_us"]
    dom = "recurrent" if serial else max(("intra", "inter"), key=lambda n: per_stage_ms[n])
    b_dom = work[dom][0]
    t_dom = per_stage_ms[dom] * 1e-3
    ach = b_dom / t_dom / 1e9
    ach3 = work_u24[dom][0] / t_dom / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": counter_traffic(dom, wl.name),
                "alg_bytes": b_dom, "u_bytes": 4,
                "frac_u24": round(ach3 / HBM_PEAK_GBS, 4), "alg_bytes_u24": work_u24[dom][0]}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl)

    line = {
        "metric": METRIC_RECURRENT if serial else METRIC,
        "value": round(args.steps * tokens / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "f16",
                  torch.float32: "f32-split-bf16"}[qkv_dtype],
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": tokens, "sequences": wl.n_seqs, "H": wl.H,
                   "Hv": wl.Hv, "Dk": 128, "Dv": 128, "chunk": 64,
                   "parallelism": "single GPU",
                   **({"stage2": f"GQA-shared, {args.gqa_share} value heads per work-group"}
                      if args.gqa_share > 1 else {}),
                   **({"segments": args.segments} if args.segments else {}),
                   **({"front": "fused into stage 1" if fused_front else "standalone kernel"}
                      if has_front else {})},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages": detail,
        "cold_cache": cold,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
