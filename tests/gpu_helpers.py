"""Shared helpers of the GPU parity tests: move a seeded workload to the device,
run the HIP path through the C ABI, and evaluate the CPU oracle, either on
every (sequence, value head) lane of a batch in one call (the C oracle runs
its lanes in parallel) or on chosen lanes. Imports the product binding and
the oracle side by side; neither of those imports the other."""

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


def run_forward_conv(wl, d=None, dev="cuda:0", chunk_indices=None):
    """Whole forward with the front fused into stage 1 (gdn_chunk_fwd_conv).
    Returns (o, hT)."""
    if d is None:
        d = device_inputs(wl, dev)
    cfg = config_of(wl, torch.float32)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=dev)
    o = torch.full((wl.t_max, wl.Hv, 128), float("nan"), dtype=torch.float32, device=dev)
    hT = torch.full((wl.n_max, wl.Hv, 128, 128), float("nan"), dtype=torch.float32, device=dev)
    gdn.gdn_chunk_fwd_conv(cfg, d["qkv"], d["conv_w"], wl.d_conv, d["g"], d["beta"], d["h0"],
                           d["cu"], chunk_indices, o, hT, ws)
    torch.cuda.synchronize()
    return o, hT


def oracle_inputs_f64(wl):
    """q, k, v in float64 as the oracle sees them (through the fp64 front when
    the workload has one)."""
    if wl.qkv is None:
        return wl.f64("q"), wl.f64("k"), wl.f64("v")
    return recurrent.gdn_front(wl.f64("qkv"), wl.f64("conv_w"), wl.cu_seqlens, wl.H, wl.Hv,
                               128, 128)


def oracle_lanes(wl, lanes, qkv64=None, scale=None):
    """fp64 recurrence on the given (sequence, value head) lanes only (output
    scale 1/sqrt(128) unless given). Returns {lane: (o [len, 128], hT [128, 128])}."""
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
                                        np.array([0, e - a], np.int32), h0=s0, scale=scale)
        out[(s, hv)] = (o[:, 0], hT[0, 0])
    return out


def oracle_full(wl, qkv64=None, scale=None):
    """fp64 recurrence on every lane of the batch in one oracle call (lanes in
    parallel under OpenMP). Returns (o [t_max, Hv, 128], hT [n_max, Hv, 128,
    128]); rows past the batch are zero."""
    if qkv64 is None:
        q, k, v = wl.f64("q"), wl.f64("k"), wl.f64("v")
    else:
        q, k, v = qkv64
    return recurrent.gdn_recurrent(q, k, v, wl.f64("g"), wl.f64("beta"), wl.cu_seqlens,
                                   h0=wl.f64("h0"), scale=scale)


def full_errors(wl, o_gpu, hT_gpu, o_ref, hT_ref):
    """(max |do| / max |o_ref| over every valid (t, hv, d); relative Frobenius
    error over the whole final-state tensor). Non-finite GPU values fail."""
    T = wl.n_tokens
    og = o_gpu[:T].detach().cpu().to(torch.float64).numpy()
    assert np.all(np.isfinite(og)), "non-finite o"
    num_o = float(np.max(np.abs(og - o_ref[:T]))) if T else 0.0
    den_o = float(np.max(np.abs(o_ref[:T]))) if T else 0.0
    del og
    sg = hT_gpu.detach().cpu().to(torch.float64).numpy()
    assert np.all(np.isfinite(sg)), "non-finite final state"
    num_s = float(np.linalg.norm((sg - hT_ref).ravel()))
    den_s = float(np.linalg.norm(hT_ref.ravel()))
    eo = num_o / den_o if den_o > 0 else num_o
    es = num_s / den_s if den_s > 0 else num_s
    return eo, es


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


# --------------------------------------------------------------------------- #
# decoders of the intermediates the intra stage writes (layouts in include/gdn.h)
# --------------------------------------------------------------------------- #

# P pairs: (token block q, output tile R)
PAIRS = [(0, 0), (0, 1), (0, 2), (1, 2), (0, 3), (1, 3)]


def frag_token(q, g, j):
    """Token (within the chunk) of contraction slot j of lane group g in token block q."""
    return 32 * q + (16 if j >= 4 else 0) + 4 * g + (j & 3)


def workspace_views(cfg, ws):
    lay = gdn.gdn_workspace_layout(cfg)
    nt = gdn.gdn_nt_max(cfg.t_max, cfg.n_max)
    nk = 16 if cfg.qkv_dtype == gdn.GDN_BF16 else 32  # K^T terms: hi (+ lo)

    def view(name, dtype, shape):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        return ws[lay[name]:lay[name] + n].view(dtype).view(*shape)

    return dict(
        w16=view("w16", torch.float16, (cfg.hv, nt, 16, 64, 8)),
        q16=view("q16", torch.float16, (cfg.h, nt, 16, 64, 8)),
        kimg=view("kimg", torch.bfloat16, (cfg.h, nt, nk, 64, 8)),
        uimg=view("uimg", torch.int32, (cfg.hv, nt, 8, 4, 64, 3)),
        pimg=view("pimg", torch.float16, (cfg.hv, nt, 5 * 512)),
        gimg=view("gimg", torch.float32, (cfg.hv, nt, 192)),
        nt=nt, nk=nk)


def decode_rowfrag(slot):
    """[16, 64, 8] fp16 fragments (fragment 4 R + p; lane (g, c) holds row
    16 R + c, columns 32 p + 4 g + j and 32 p + 16 + 4 g + j - 4) -> [64, 128]."""
    x = slot.float().numpy().astype(np.float64)
    M = np.zeros((64, 128))
    for f in range(16):
        R, p = f // 4, f % 4
        for lane in range(64):
            g, c = lane // 16, lane % 16
            for j in range(8):
                col = 32 * p + (16 if j >= 4 else 0) + 4 * g + (j & 3)
                M[16 * R + c, col] = x[f, lane, j]
    return M


def decode_kimg(kimg_slot):
    """[nk, 64, 8] fragments -> K [64 tokens, 128] (hi, and lo when nk == 32)."""
    x = kimg_slot.float().numpy()
    out = []
    for term in range(x.shape[0] // 16):
        K = np.zeros((64, 128), np.float64)
        for f in range(16):
            tau, q = f // 2, f % 2
            for lane in range(64):
                g, c = lane // 16, lane % 16
                for j in range(8):
                    K[frag_token(q, g, j), 16 * tau + c] = x[16 * term + f, lane, j]
        out.append(K)
    return out


def unpack_f24(words):
    """[..., 3] little-endian words holding four 24-bit floats (the upper three
    bytes of fp32) -> [..., 4] float64."""
    b = np.ascontiguousarray(words).view(np.uint8).reshape(words.shape[:-1] + (4, 3))
    full = np.zeros(words.shape[:-1] + (4, 4), np.uint8)
    full[..., 1:] = b  # the dropped low byte is zero
    return full.view("<f4").reshape(words.shape[:-1] + (4,)).astype(np.float64)


def decode_uimg(uimg_slot):
    """[8, 4, 64, 3] packed 24-bit words -> u [64 tokens, 128]."""
    x = unpack_f24(uimg_slot.numpy())
    U = np.zeros((64, 128))
    for sl in range(8):
        for R in range(4):
            for lane in range(64):
                g, c = lane // 16, lane % 16
                U[16 * R + 4 * g:16 * R + 4 * g + 4, 16 * sl + c] = x[sl, R, lane]
    return U


P_OFFSET = (0, 512, 1536, 2560, 3072, 4096)  # bytes of each pair's block
P_HALF = (True, False, False, True, False, False)  # 8 bytes per lane


def decode_pimg(pimg_slot):
    """[5 KB of fp16] -> P [64 r, 64 j], zero outside the pairs and in the
    packed-out upper halves of pairs 0 and 3."""
    x = pimg_slot.float().numpy().astype(np.float64)
    P = np.zeros((64, 64))
    for pi, (q, R) in enumerate(PAIRS):
        per = 4 if P_HALF[pi] else 8  # fp16 values per lane
        blk = x[P_OFFSET[pi] // 2:][:64 * per].reshape(64, per)
        for lane in range(64):
            g, c = lane // 16, lane % 16
            for j in range(per):
                P[16 * R + c, frag_token(q, g, j)] = blk[lane, j]
    return P
