"""Shared helpers of the GPU parity tests: move a seeded workload to the device,
run the HIP path through the C ABI, and evaluate the CPU oracle on sampled
(sequence, value head) lanes. Imports the product binding and the oracle side
by side; neither of those imports the other."""

from __future__ import annotations

import sys

import numpy as np
import torch

import chunked_gated_delta_rule_amd as gdn
from oracle import recurrent

# Tolerances of the parity bar (max |o - o_ref| / max |o_ref| over the checked
# lanes; relative Frobenius error of the final states).
O_TOL = 2e-3
S_TOL = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(wl, dev="cuda:0"):
    d = {}
    for name in ("q", "k", "v", "qkv", "conv_w"):
        t = getattr(wl, name)
        d[name] = t.to(dev).contiguous() if t is not None else None
    d["g"] = wl.g.to(dev).contiguous()
    d["beta"] = wl.beta.to(dev).contiguous()
    d["h0"] = wl.h0.to(dev).contiguous() if wl.h0 is not None else None
    d["cu"] = torch.from_numpy(wl.cu_seqlens.astype(np.int32)).to(dev)
    return d


def config_of(wl, qkv_dtype=None):
    dt = wl.qkv_dtype if qkv_dtype is None else qkv_dtype
    return gdn.make_config(wl.t_max, wl.n_max, wl.H, wl.Hv, dt)


def run_front(wl, d, dev="cuda:0"):
    cfg = config_of(wl, torch.float32)
    q = torch.zeros((wl.t_max, wl.H, 128), dtype=torch.float32, device=dev)
    k = torch.zeros_like(q)
    v = torch.zeros((wl.t_max, wl.Hv, 128), dtype=torch.float32, device=dev)
    gdn.gdn_front_conv_silu_l2(cfg, d["qkv"], d["conv_w"], wl.d_conv, d["cu"], q, k, v)
    return q, k, v


def run_forward(wl, d=None, dev="cuda:0", h0=None, hT=None, chunk_indices=None):
    """Whole forward through gdn_chunk_fwd (with the front when the workload
    has one). Returns (o, hT, (q, k, v) as fed to the chunk forward)."""
    if d is None:
        d = device_inputs(wl, dev)
    if wl.qkv is not None:
        q, k, v = run_front(wl, d, dev)
    else:
        q, k, v = d["q"], d["k"], d["v"]
    cfg = config_of(wl, q.dtype)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=dev)
    o = torch.full((wl.t_max, wl.Hv, 128), float("nan"), dtype=torch.float32, device=dev)
    if hT is None:
        hT = torch.full((wl.n_max, wl.Hv, 128, 128), float("nan"), dtype=torch.float32, device=dev)
    gdn.gdn_chunk_fwd(cfg, q, k, v, d["g"], d["beta"], d["h0"] if h0 is None else h0, d["cu"],
                      chunk_indices, o, hT, ws)
    torch.cuda.synchronize()
    return o, hT, (q, k, v)


def oracle_inputs_f64(wl):
    """q, k, v in float64 as the oracle sees them (through the fp64 front when
    the workload has one)."""
    if wl.qkv is None:
        return wl.f64("q"), wl.f64("k"), wl.f64("v")
    return recurrent.gdn_front(wl.f64("qkv"), wl.f64("conv_w"), wl.cu_seqlens, wl.H, wl.Hv,
                               128, 128)


def oracle_lanes(wl, lanes, qkv64=None):
    """fp64 recurrence on the given (sequence, value head) lanes only.
    Returns {lane: (o [len, 128], hT [128, 128])}."""
    cu = wl.cu_seqlens
    HG = wl.Hv // wl.H
    out = {}
    g = wl.f64("g")
    b = wl.f64("beta")
    h0 = wl.f64("h0")
    for (s, hv) in lanes:
        a, e = int(cu[s]), int(cu[s + 1])
        h = hv // HG
        if qkv64 is None:
            q = wl.q[a:e, h:h + 1].to(torch.float64).numpy()
            k = wl.k[a:e, h:h + 1].to(torch.float64).numpy()
            v = wl.v[a:e, hv:hv + 1].to(torch.float64).numpy()
        else:
            q, k, v = qkv64[0][a:e, h:h + 1], qkv64[1][a:e, h:h + 1], qkv64[2][a:e, hv:hv + 1]
        s0 = None if h0 is None else h0[s:s + 1, hv:hv + 1]
        o, hT = recurrent.gdn_recurrent(q, k, v, g[a:e, hv:hv + 1], b[a:e, hv:hv + 1],
                                        np.array([0, e - a], np.int32), h0=s0)
        out[(s, hv)] = (o[:, 0], hT[0, 0])
    return out


def lane_errors(wl, o_gpu, hT_gpu, ref):
    """(max |do| / max |o_ref|, relative Frobenius error of the states) over lanes."""
    cu = wl.cu_seqlens
    o_cpu = o_gpu.detach().cpu().to(torch.float64).numpy()
    s_cpu = hT_gpu.detach().cpu().to(torch.float64).numpy()
    num_o = 0.0
    den_o = 0.0
    num_s = 0.0
    den_s = 0.0
    for (s, hv), (o_ref, s_ref) in ref.items():
        a, e = int(cu[s]), int(cu[s + 1])
        og = o_cpu[a:e, hv]
        assert np.all(np.isfinite(og)), f"non-finite o in lane {(s, hv)}"
        if e > a:
            num_o = max(num_o, float(np.max(np.abs(og - o_ref))))
            den_o = max(den_o, float(np.max(np.abs(o_ref))))
        num_s += float(np.sum((s_cpu[s, hv] - s_ref) ** 2))
        den_s += float(np.sum(s_ref ** 2))
    eo = num_o / den_o if den_o > 0 else num_o
    es = np.sqrt(num_s / den_s) if den_s > 0 else np.sqrt(num_s)
    return eo, es
