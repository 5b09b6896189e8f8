"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar (from the method's tolerance): max |o_gpu - o_ref| / max |o_ref| <= 2e-3
and relative Frobenius error of the final states <= 1e-3 over every checked
lane; the chunk-index table is bit-exact. Small cases are checked on every
lane; the five full-size workloads are run whole on the GPU, in the launch
configuration the benchmark times, and checked on every lane as well, against
one oracle call over the whole batch.
"""

import numpy as np
import pytest
import torch

import chunked_gated_delta_rule_amd as gdn
import workloads
from oracle import chunked, index_table, recurrent

from gpu_helpers import (O_TOL, S_TOL, config_of, decode_kimg, decode_pimg, decode_rowfrag, decode_uimg,
                         device_inputs, full_errors, lane_errors, log, oracle_full,
                         oracle_inputs_f64, oracle_lanes, run_forward, run_forward_conv, run_front,
                         workspace_views)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    gdn.load_library()  # raises if the HIP library is missing


def _all_lanes(wl):
    n = len(wl.cu_seqlens) - 1
    return [(s, hv) for s in range(n) for hv in range(wl.Hv)]


# --------------------------------------------------------------------------- #
# chunk-index table: bit-exact against the oracle's loops
# --------------------------------------------------------------------------- #

def _cu_cases():
    rng = np.random.Generator(np.random.PCG64(3))
    cases = [([256], 256, 1), ([4096], 4096, 1), ([32768], 32768, 1),
             ([1, 63, 64, 65, 0, 128, 129], 600, 9), ([0, 0, 5], 5, 3)]
    w2 = workloads.make(2)
    cases.append((list(np.diff(w2.cu_seqlens)), w2.t_max, w2.n_max))
    lengths = rng.integers(0, 2000, size=700)
    cases.append((list(lengths), int(lengths.sum()) + 77, 1000))
    return cases


@pytest.mark.parametrize("case", range(7))
def test_chunk_index_table_bit_exact(case):
    lengths, t_max, n_max = _cu_cases()[case]
    cu = np.zeros(n_max + 1, np.int32)
    cu[1:len(lengths) + 1] = np.cumsum(lengths)
    cu[len(lengths) + 1:] = cu[len(lengths)]
    cfg = gdn.make_config(t_max, n_max, 1, 1)
    nt = gdn.gdn_nt_max(t_max, n_max)
    log(f"index case {case}: n={len(lengths)} t_max={t_max} n_max={n_max} nt_max={nt}")
    table = torch.full((nt, 2), 12345, dtype=torch.int32, device=DEV)
    gdn.gdn_build_chunk_indices(cfg, torch.from_numpy(cu).to(DEV), table)
    torch.cuda.synchronize()
    ref = np.array(index_table.chunk_index_table(list(cu), nt), dtype=np.int32)
    assert np.array_equal(table.cpu().numpy(), ref)


# --------------------------------------------------------------------------- #
# front: conv + SiLU + L2 norm (fp32) against the fp64 front
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("d_conv", range(1, 9))
def test_front_small_varlen(d_conv):
    """Every tap count the standalone front accepts (one kernel instance
    each), on sequences shorter than the conv window and an empty one."""
    wl = workloads.make_custom([5, 0, 130, 1, 64], 2, 4, seed=11 + d_conv, front=True,
                               d_conv=d_conv, t_max=230, n_max=6)
    log(f"front small varlen, d_conv={d_conv}")
    d = device_inputs(wl)
    q, k, v = run_front(wl, d)
    torch.cuda.synchronize()
    rq, rk, rv = recurrent.gdn_front(wl.f64("qkv"), wl.f64("conv_w"), wl.cu_seqlens, 2, 4, 128, 128)
    T = int(wl.cu_seqlens[-1])
    for got, ref in ((q, rq), (k, rk), (v, rv)):
        g64 = got[:T].cpu().double().numpy()
        assert np.max(np.abs(g64 - ref[:T])) / np.max(np.abs(ref[:T])) < 1e-5


# --------------------------------------------------------------------------- #
# stage 1 alone: every intermediate against the chunked-form oracle
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_intra_stage_intermediates(dtype):
    wl = workloads.make_custom([130, 70, 64, 1], 2, 4, seed=5, dtype=dtype, t_max=300, n_max=5)
    log(f"intra stage {dtype}")
    d = device_inputs(wl)
    cfg = config_of(wl)
    scale = 1.0 / np.sqrt(128.0)
    nt = gdn.gdn_nt_max(wl.t_max, wl.n_max)
    table = torch.empty((nt, 2), dtype=torch.int32, device=DEV)
    gdn.gdn_build_chunk_indices(cfg, d["cu"], table)
    ws = torch.zeros(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    gdn.gdn_chunk_fwd_intra(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], table, ws)
    torch.cuda.synchronize()
    V = {k_: (v_.cpu() if isinstance(v_, torch.Tensor) else v_)
         for k_, v_ in workspace_views(cfg, ws).items()}
    stages = {}
    _, _, W, U = chunked.gdn_chunked(wl.f64("q"), wl.f64("k"), wl.f64("v"), wl.f64("g"),
                                     wl.f64("beta"), wl.cu_seqlens, chunk=64, return_wu=True,
                                     stages=stages)
    T = int(wl.cu_seqlens[-1])
    cu = wl.cu_seqlens
    eu = ep = eg = ew = 0.0
    wmax = np.max(np.abs(W[:, :T]))
    pmax = max(np.max(np.abs(la)) for _, la in stages.values()) * scale
    k64 = wl.f64("k")
    for s_ in range(len(cu) - 1):
        for t0 in range(int(cu[s_]), int(cu[s_ + 1]), 64):
            L = min(64, int(cu[s_ + 1]) - t0)
            slot = (t0 >> 6) + s_
            # K^T fragments: exact copy of k (hi[+lo] for fp32 input), zero past the end
            for h in range(wl.H):
                # q16: q rounded to fp16 (bf16 -> fp16 is exact here, bit for bit; fp32
                # input passes through hi + lo bf16 first: within one fp16 ulp)
                q16 = decode_rowfrag(V["q16"][h, slot])
                qref = np.zeros((64, 128))
                qref[:L] = wl.q[t0:t0 + L, h].double().numpy()
                if dtype != torch.float32:
                    want = torch.from_numpy(qref).float().half().double().numpy()
                    assert np.array_equal(q16, want), "q16 is not q rounded to fp16"
                else:
                    assert np.all(np.abs(q16 - qref) <= np.abs(qref) * 2.0 ** -10 + 2.0 ** -24)
                terms = decode_kimg(V["kimg"][h, slot])
                Kd = sum(terms)
                ref = np.zeros((64, 128))
                ref[:L] = k64[t0:t0 + L, h]
                # bf16 and fp16 inputs are held exactly (fp16 as bf16 hi + lo)
                tol = 2e-5 * np.max(np.abs(k64)) if dtype == torch.float32 else 0.0
                assert np.max(np.abs(Kd - ref)) <= tol
            for hv in range(wl.Hv):
                gamma, la = stages[(hv, t0)]
                wd = -decode_rowfrag(V["w16"][hv, slot])  # stored negated
                assert np.all(wd[L:] == 0.0)
                ew = max(ew, np.max(np.abs(wd[:L] - W[hv, t0:t0 + L])) / wmax)
                Ud = decode_uimg(V["uimg"][hv, slot])
                assert np.all(Ud[L:] == 0.0)
                eu = max(eu, np.max(np.abs(Ud[:L] - U[hv, t0:t0 + L])) / np.max(np.abs(U[hv, :T])))
                Pd = decode_pimg(V["pimg"][hv, slot])
                Pref = np.zeros((64, 64))
                Pref[:L, :L] = scale * la
                ep = max(ep, np.max(np.abs(Pd - Pref)) / pmax)
                gd = V["gimg"][hv, slot].double().numpy()
                gd[64:128] = gd[64:128].reshape(16, 4).T.reshape(64)  # [c][R] -> token order
                gl = gamma[L - 1]
                for got, want in ((gd[:L], np.exp(gl - gamma)), (gd[64:64 + L], scale * np.exp(gamma)),
                                  (gd[128:129], np.exp([gl]))):
                    eg = max(eg, np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-30)))
                assert np.all(gd[L:64] == 0) and np.all(gd[64 + L:128] == 0)
    log(f"  w err {ew:.3e}  u err {eu:.3e}  P err {ep:.3e}  gate err {eg:.3e}")
    assert ew < 1e-3   # fp16 storage of w: half an ulp is 2^-12 of the value
    assert eu < 1e-4
    assert ep < 5e-4   # fp16 storage of P: half an ulp is 2^-12 of the value
    assert eg < 1e-5


# --------------------------------------------------------------------------- #
# whole forward, small cases, every lane
# --------------------------------------------------------------------------- #

SMALL = {
    "dense-256-fp32": dict(lengths=[256], H=2, Hv=2, dtype=torch.float32),
    "ragged-bf16-gqa-h0": dict(lengths=[1, 63, 64, 65, 200, 0, 129], H=2, Hv=4,
                               dtype=torch.bfloat16, h0_sigma=0.02, n_max=8, t_max=600),
    "ragged-fp32-h0": dict(lengths=[70, 3, 190], H=1, Hv=2, dtype=torch.float32, h0_sigma=0.05),
    "strong-decay": dict(lengths=[300], H=1, Hv=1, dtype=torch.bfloat16, g_mu=2.0, h0_sigma=0.02),
    "weak-decay": dict(lengths=[400, 150], H=1, Hv=2, dtype=torch.bfloat16, g_mu=-5.0,
                       h0_sigma=0.02),
    "gqa4": dict(lengths=[100, 60], H=1, Hv=4, dtype=torch.bfloat16),
    "beta-one": dict(lengths=[128], H=2, Hv=2, dtype=torch.bfloat16, beta_mode=1.0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small_every_lane(name):
    p = dict(SMALL[name])
    lengths = p.pop("lengths")
    H, Hv = p.pop("H"), p.pop("Hv")
    wl = workloads.make_custom(lengths, H, Hv, seed=17, name=name, **p)
    log(f"forward small {name}")
    o, hT, _ = run_forward(wl)
    ref = oracle_lanes(wl, _all_lanes(wl))
    eo, es = lane_errors(wl, o, hT, ref)
    log(f"  o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


def test_forward_front_small_every_lane():
    wl = workloads.make_custom([100, 37, 0, 64], 2, 4, seed=23, front=True, n_max=5, t_max=220)
    log("forward front small")
    o, hT, _ = run_forward(wl)
    qkv64 = oracle_inputs_f64(wl)
    ref = oracle_lanes(wl, _all_lanes(wl), qkv64=qkv64)
    eo, es = lane_errors(wl, o, hT, ref)
    log(f"  o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


# --------------------------------------------------------------------------- #
# front fused into stage 1 (gdn_chunk_fwd_conv)
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("d_conv", [1, 2, 3, 4])
def test_fused_front_equals_front_then_forward_bitwise(d_conv):
    """The fused front computes q, k, v with the standalone front's fp32
    arithmetic, so o and the final states are bit for bit those of
    gdn_front_conv_silu_l2 followed by gdn_chunk_fwd (ragged chunks, a
    sequence shorter than the halo, an empty one, h0)."""
    wl = workloads.make_custom([100, 2, 0, 64, 130], 2, 4, seed=71 + d_conv, front=True,
                               d_conv=d_conv, h0_sigma=0.02, n_max=6, t_max=330)
    log(f"fused front vs front + forward, d_conv={d_conv}")
    d = device_inputs(wl)
    o1, s1, _ = run_forward(wl, d)
    o2, s2 = run_forward_conv(wl, d)
    T = wl.n_tokens
    assert torch.equal(o1[:T], o2[:T]) and torch.equal(s1, s2)


def test_fused_front_small_every_lane():
    wl = workloads.make_custom([100, 37, 0, 64, 3], 2, 4, seed=29, front=True, n_max=6, t_max=230)
    log("fused front small, every lane")
    o, hT = run_forward_conv(wl)
    ref = oracle_lanes(wl, _all_lanes(wl), qkv64=oracle_inputs_f64(wl))
    eo, es = lane_errors(wl, o, hT, ref)
    log(f"  o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


def test_fused_front_workload_full_size():
    """The front workload (4 x 8192 tokens) through the fused path, in the
    launch configuration the benchmark times, against the fp64 front +
    recurrence on every lane."""
    wl = workloads.make(4)
    log(f"fused front, workload 4 ({wl.name}) tokens={wl.n_tokens}")
    o, hT = run_forward_conv(wl)
    o_ref, s_ref = oracle_full(wl, qkv64=oracle_inputs_f64(wl))
    eo, es = full_errors(wl, o, hT, o_ref, s_ref)
    log(f"  every lane: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


@pytest.mark.parametrize("d_conv", [1, 2, 3, 4])
def test_fused_front_fp16_equals_front_rounded_then_forward_bitwise(d_conv):
    """With GDN_F16 the fused front rounds its fp32 q, k, v to fp16 (nearest
    even): bit for bit the standalone front, its outputs rounded to fp16 by
    torch, then gdn_chunk_fwd on fp16 inputs (ragged chunks, a sequence
    shorter than the halo, an empty one, h0)."""
    wl = workloads.make_custom([100, 2, 0, 64, 130], 2, 4, seed=171 + d_conv, front=True,
                               d_conv=d_conv, h0_sigma=0.02, n_max=6, t_max=330)
    log(f"fused fp16 front vs front + fp16 forward, d_conv={d_conv}")
    d = device_inputs(wl)
    q, k, v = run_front(wl, d)
    cfg = gdn.make_config(wl.t_max, wl.n_max, wl.H, wl.Hv, torch.float16)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    out = []
    for fused in (False, True):
        o = torch.full((wl.t_max, wl.Hv, 128), float("nan"), dtype=torch.float32, device=DEV)
        hT = torch.full((wl.n_max, wl.Hv, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
        if fused:
            gdn.gdn_chunk_fwd_conv(cfg, d["qkv"], d["conv_w"], wl.d_conv, d["g"], d["beta"], d["h0"],
                                   d["cu"], None, o, hT, ws)
        else:
            gdn.gdn_chunk_fwd(cfg, q.half(), k.half(), v.half(), d["g"], d["beta"], d["h0"], d["cu"],
                              None, o, hT, ws)
        torch.cuda.synchronize()
        out.append((o, hT))
    T = wl.n_tokens
    assert torch.equal(out[0][0][:T], out[1][0][:T]) and torch.equal(out[0][1], out[1][1])


def test_fused_front_fp16_workload_full_size():
    """The front workload (4 x 8192 tokens) through the fused path with fp16
    intermediates (the configuration the benchmark times), against the fp64
    front + recurrence on every lane: the fp16 rounding of q, k, v stays well
    inside the bar."""
    wl = workloads.make(4)
    log(f"fused front, fp16 intermediates, workload 4 ({wl.name})")
    d = device_inputs(wl)
    cfg = gdn.make_config(wl.t_max, wl.n_max, wl.H, wl.Hv, torch.float16)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    o = torch.full((wl.t_max, wl.Hv, 128), float("nan"), dtype=torch.float32, device=DEV)
    hT = torch.full((wl.n_max, wl.Hv, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    gdn.gdn_chunk_fwd_conv(cfg, d["qkv"], d["conv_w"], wl.d_conv, d["g"], d["beta"], d["h0"],
                           d["cu"], None, o, hT, ws)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_full(wl, qkv64=oracle_inputs_f64(wl))
    eo, es = full_errors(wl, o, hT, o_ref, s_ref)
    log(f"  every lane: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


@pytest.mark.parametrize("H,Hv,segments,tiles", [(2, 4, 1, 0), (1, 4, 2, 0), (4, 8, 1, 2),
                                                 (2, 2, 1, 4)])
def test_fp16_inputs_every_lane(H, Hv, segments, tiles):
    """fp16 q, k, v through the chunked forward (stage 1's fp16 path, stage 2
    on the exact bf16 hi + lo K^T image), ragged batches with an empty
    sequence and h0, one and two segments, one, two and four tiles, every lane
    against the oracle on the same fp16 values."""
    lengths = [300, 0, 65, 128, 777]
    wl = workloads.make_custom(lengths, H, Hv, seed=181 + H + Hv, dtype=torch.float16,
                               h0_sigma=0.02, n_max=len(lengths) + 1, t_max=sum(lengths) + 9)
    log(f"fp16 inputs H={H} Hv={Hv} segments={segments} tiles={tiles}")
    d = device_inputs(wl)
    cfg = gdn.make_config(wl.t_max, wl.n_max, H, Hv, torch.float16, segments=segments, tiles=tiles)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    o = torch.full((wl.t_max, Hv, 128), float("nan"), dtype=torch.float32, device=DEV)
    hT = torch.full((wl.n_max, Hv, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], None, o,
                      hT, ws)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_full(wl)
    eo, es = full_errors(wl, o, hT, o_ref, s_ref)
    log(f"  o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL
    assert torch.isnan(o[wl.n_tokens:]).all()


# --------------------------------------------------------------------------- #
# bitwise self-consistency of the HIP path
# --------------------------------------------------------------------------- #

def _wl_props():
    return workloads.make_custom([200, 64, 77], 2, 4, seed=31, h0_sigma=0.02, t_max=400, n_max=4)


def test_replay_is_bitwise_deterministic():
    wl = _wl_props()
    d = device_inputs(wl)
    o1, s1, _ = run_forward(wl, d)
    o2, s2, _ = run_forward(wl, d)
    T = int(wl.cu_seqlens[-1])
    assert torch.equal(o1[:T], o2[:T]) and torch.equal(s1, s2)


def test_packing_invariance_bitwise():
    wl = _wl_props()
    o, hT, _ = run_forward(wl)
    cu = wl.cu_seqlens
    for s in range(3):
        a, e = int(cu[s]), int(cu[s + 1])
        one = workloads.Workload(
            name="alone", cu_seqlens=np.array([0, e - a], np.int32), t_max=e - a, n_max=1,
            H=wl.H, Hv=wl.Hv, qkv_dtype=wl.qkv_dtype, q=wl.q[a:e].clone(), k=wl.k[a:e].clone(),
            v=wl.v[a:e].clone(), g=wl.g[a:e].clone(), beta=wl.beta[a:e].clone(),
            h0=wl.h0[s:s + 1].clone())
        o1, h1, _ = run_forward(one)
        assert torch.equal(o1, o[a:e]) and torch.equal(h1[0], hT[s])


def test_chunk_aligned_continuation_bitwise():
    wl = workloads.make_custom([320], 2, 4, seed=41, h0_sigma=0.02)
    o, hT, _ = run_forward(wl)
    split = 128
    parts = []
    state = wl.h0.clone()
    for a, e in ((0, split), (split, 320)):
        part = workloads.Workload(
            name="part", cu_seqlens=np.array([0, e - a], np.int32), t_max=e - a, n_max=1,
            H=wl.H, Hv=wl.Hv, qkv_dtype=wl.qkv_dtype, q=wl.q[a:e].clone(), k=wl.k[a:e].clone(),
            v=wl.v[a:e].clone(), g=wl.g[a:e].clone(), beta=wl.beta[a:e].clone(), h0=state)
        op, hp, _ = run_forward(part)
        parts.append(op)
        state = hp.cpu()
    assert torch.equal(torch.cat(parts), o) and torch.equal(state.to(DEV), hT)


def test_external_table_and_in_place_state():
    wl = _wl_props()
    d = device_inputs(wl)
    o1, s1, _ = run_forward(wl, d)
    cfg = config_of(wl)
    table = torch.empty((gdn.gdn_nt_max(wl.t_max, wl.n_max), 2), dtype=torch.int32, device=DEV)
    gdn.gdn_build_chunk_indices(cfg, d["cu"], table)
    state = d["h0"].clone()
    o2, s2, _ = run_forward(wl, d, h0=state, hT=state, chunk_indices=table)
    T = wl.n_tokens
    assert torch.equal(o1[:T], o2[:T]) and torch.equal(s1, s2)
    assert s2.data_ptr() == state.data_ptr()


def test_zero_length_sequences_keep_state():
    wl = workloads.make_custom([0, 50, 0], 1, 2, seed=43, h0_sigma=0.1, n_max=5, t_max=64)
    o, hT, _ = run_forward(wl)
    for s in (0, 2, 3, 4):
        assert torch.equal(hT[s].cpu(), wl.h0[s])
    wl.h0 = None
    o, hT, _ = run_forward(wl)
    assert torch.count_nonzero(hT[[0, 2, 3, 4]]) == 0


@pytest.mark.parametrize("n_max", [1, 2, 256, 300])
def test_no_token_capacity_hands_back_every_initial_state(n_max):
    """t_max = 0 (a valid config: nothing to compute): stage 1 does not run,
    and stage 2 must still write hT = h0 for every sequence, including the
    batch sizes for which stage 1 would rank the sequences (2..256)."""
    H, Hv = 1, 2
    cfg = gdn.make_config(0, n_max, H, Hv, torch.bfloat16)
    log(f"t_max = 0, n_max = {n_max}")
    one = lambda *shape, dt=torch.float32: torch.zeros(shape, dtype=dt, device=DEV)
    q, k, v = one(1, H, 128, dt=torch.bfloat16), one(1, H, 128, dt=torch.bfloat16), \
        one(1, Hv, 128, dt=torch.bfloat16)
    g, beta, o = one(1, Hv), one(1, Hv), one(1, Hv, 128)
    cu = torch.zeros(n_max + 1, dtype=torch.int32, device=DEV)
    h0 = torch.full((n_max, Hv, 128, 128), 0.25, dtype=torch.float32, device=DEV)
    h0[-1] = -0.5
    hT = torch.full_like(h0, float("nan"))
    ws = torch.full((max(gdn.gdn_workspace_size(cfg), 256),), 0x7f, dtype=torch.uint8, device=DEV)
    gdn.gdn_chunk_fwd(cfg, q, k, v, g, beta, h0, cu, None, o, hT, ws)
    torch.cuda.synchronize()
    assert torch.equal(hT, h0)
    hT.fill_(float("nan"))
    gdn.gdn_chunk_fwd(cfg, q, k, v, g, beta, None, cu, None, o, hT, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(hT) == 0
    # the split entry points agree
    hT.fill_(float("nan"))
    gdn.gdn_chunk_fwd_inter(cfg, h0, cu, ws, o, hT)
    torch.cuda.synchronize()
    assert torch.equal(hT, h0)


def test_untouched_rows_past_the_batch():
    wl = workloads.make_custom([70, 10], 1, 2, seed=47, t_max=200, n_max=2)
    o, _, _ = run_forward(wl)
    assert torch.isnan(o[80:]).all() and torch.isfinite(o[:80]).all()


def test_no_decay_no_write_keeps_state_bitwise():
    wl = workloads.make_custom([150], 1, 2, seed=53, h0_sigma=0.1)
    wl.g.zero_()
    wl.beta.zero_()
    o, hT, _ = run_forward(wl)
    assert torch.equal(hT.cpu(), wl.h0)


# --------------------------------------------------------------------------- #
# the five named workloads at full size, every lane
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("cfg_id", [0, 1, 2, 3, 4])
def test_named_workload_full_size(cfg_id):
    """Each named workload, whole, in the launch configuration the benchmark
    times (the front workload here through the standalone front kernel), against
    the fp64 oracle on every (t, hv, d) and the whole final-state tensor."""
    wl = workloads.make(cfg_id)
    log(f"workload {cfg_id} ({wl.name}) tokens={wl.n_tokens}")
    o, hT, _ = run_forward(wl)
    o_ref, s_ref = oracle_full(wl, qkv64=oracle_inputs_f64(wl) if wl.qkv is not None else None)
    eo, es = full_errors(wl, o, hT, o_ref, s_ref)
    log(f"  every lane: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


@pytest.mark.parametrize("n", [40, 300])
def test_forward_without_table_builds_it_in_the_workspace(n):
    """gdn_chunk_fwd with no caller table: up to GDN_FUSED_INDEX_MAX_SEQS
    sequences stage 1 locates its chunks and fills the workspace table itself,
    beyond it the table kernel runs first. Either way the workspace table is
    bit-exact and the outputs match the oracle on every lane."""
    rng = np.random.Generator(np.random.PCG64(61 + n))
    lengths = rng.integers(0, 150, size=n)
    lengths[::7] = 0
    wl = workloads.make_custom(lengths, 1, 1, seed=62 + n, h0_sigma=0.02,
                               t_max=int(lengths.sum()) + 77, n_max=n + 3)
    log(f"forward without table: n={n} tokens={wl.n_tokens}")
    d = device_inputs(wl)
    cfg = config_of(wl)
    lay = gdn.gdn_workspace_layout(cfg)
    nt = gdn.gdn_nt_max(wl.t_max, wl.n_max)
    ws = torch.full((gdn.gdn_workspace_size(cfg),), 123, dtype=torch.uint8, device=DEV)
    o = torch.empty((wl.t_max, wl.Hv, 128), dtype=torch.float32, device=DEV)
    hT = torch.empty((wl.n_max, wl.Hv, 128, 128), dtype=torch.float32, device=DEV)
    gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], None, o,
                      hT, ws)
    torch.cuda.synchronize()
    table = ws[lay["table"]:lay["table"] + nt * 8].view(torch.int32).view(nt, 2).cpu().numpy()
    ref = np.array(index_table.chunk_index_table(list(wl.cu_seqlens), nt), dtype=np.int32)
    assert np.array_equal(table, ref)
    eo, es = lane_errors(wl, o, hT, oracle_lanes(wl, _all_lanes(wl)))
    log(f"  o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


@pytest.mark.parametrize("entry,segments", [("chunk", 1), ("chunk", 2), ("chunk", 4),
                                            ("noalloc", 2), ("recurrent", 0)])
def test_graph_capture_replay_with_varying_cu_seqlens(entry, segments):
    """gdn_chunk_fwd (one-piece stage 2, two segments, four segments with their
    chained-state launches), gdn_chunk_fwd_noalloc (the entry point for
    callers that cannot allocate, its workspace the library's own) or
    gdn_recurrent_fwd captured once into a HIP graph at static sizes (t_max, n_max) and static
    addresses, then replayed with different cu_seqlens contents written into
    the same buffer (FLA issue 1155, "Core design": static grids, the
    device-built table, a sentinel for unused slots). Every replay is checked
    bit for bit against an eager call on the same inputs, with eager work and
    synchronisation between the replays."""
    t_max, n_max, H, Hv = 600, 6, 2, 4
    rng = np.random.Generator(np.random.PCG64(81))
    batches = [[600], [1, 63, 64, 65, 200, 0], [100, 0, 0, 37], [300, 300]]
    base = workloads.make_custom([t_max], H, Hv, seed=82, t_max=t_max, n_max=n_max)
    d = device_inputs(base)
    h0 = torch.from_numpy(rng.standard_normal((n_max, Hv, 128, 128)) * 0.02).float().to(DEV)
    cfg = gdn.make_config(base.t_max, base.n_max, base.H, base.Hv, base.qkv_dtype,
                          segments=segments)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    cu = torch.zeros(n_max + 1, dtype=torch.int32, device=DEV)

    def call(o_, h_, ws_):
        if entry == "recurrent":
            gdn.gdn_recurrent_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], h0, cu, o_, h_)
        elif entry == "noalloc":
            gdn.gdn_chunk_fwd_noalloc(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], h0, cu, None,
                                      o_, h_)
        else:
            gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], h0, cu, None, o_, h_,
                              ws_)
    o = torch.zeros((t_max, Hv, 128), dtype=torch.float32, device=DEV)
    hT = torch.zeros((n_max, Hv, 128, 128), dtype=torch.float32, device=DEV)

    def cu_of(lengths):
        c = np.zeros(n_max + 1, np.int32)
        c[1:len(lengths) + 1] = np.cumsum(lengths)
        c[len(lengths) + 1:] = c[len(lengths)]
        return torch.from_numpy(c)

    cu.copy_(cu_of(batches[0]))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):  # warm-up on the capture stream, then capture
        call(o, hT, ws)
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            call(o, hT, ws)
    torch.cuda.synchronize()
    for rep, lengths in enumerate(batches + batches[::-1]):
        log(f"graph replay {rep} ({entry}, segments={segments}): lengths {lengths}")
        cu.copy_(cu_of(lengths))
        o.fill_(float("nan"))
        hT.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        T = int(sum(lengths))
        o_g, s_g = o[:T].clone(), hT.clone()
        # eager reference on the same inputs, fresh outputs and workspace
        ws2 = torch.empty_like(ws)
        o_e = torch.full_like(o, float("nan"))
        s_e = torch.full_like(hT, float("nan"))
        call(o_e, s_e, ws2)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e[:T]) and torch.equal(s_g, s_e)


@pytest.mark.parametrize("H,Hv,dtype", [(2, 8, torch.bfloat16), (1, 8, torch.float32),
                                        (4, 32, torch.bfloat16), (24, 24, torch.bfloat16),
                                        (3, 9, torch.bfloat16), (12, 36, torch.bfloat16),
                                        (12, 24, torch.float32), (5, 15, torch.float32)])
def test_gqa_group_sizes_every_lane(H, Hv, dtype):
    """Other key/value head ratios than the named workloads (groups of 3, 4
    and 8, key-head counts that are not multiples of the 8 XCDs, and many
    heads with a group of 1) through the chunked path (one and two stage-2
    segments; one, two and four column tiles) and the token-serial kernel,
    every lane against the oracle."""
    lengths = [130, 0, 64, 257]
    wl = workloads.make_custom(lengths, H, Hv, seed=31 + H + Hv, dtype=dtype, h0_sigma=0.02,
                               n_max=len(lengths) + 1, t_max=sum(lengths) + 3)
    d = device_inputs(wl)
    ref = oracle_lanes(wl, _all_lanes(wl))
    for tag in ("one segment", "two segments", "two tiles", "four tiles", "token-serial"):
        cfg = gdn.make_config(wl.t_max, wl.n_max, H, Hv, dtype,
                              segments=2 if tag == "two segments" else 1,
                              tiles={"two tiles": 2, "four tiles": 4}.get(tag, 0))
        o = torch.full((wl.t_max, Hv, 128), float("nan"), dtype=torch.float32, device=DEV)
        hT = torch.full((wl.n_max, Hv, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
        if tag == "token-serial":
            gdn.gdn_recurrent_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"],
                                  o, hT)
        else:
            ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
            gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"],
                              None, o, hT, ws)
        torch.cuda.synchronize()
        eo, es = lane_errors(wl, o, hT, ref)
        log(f"  H={H} Hv={Hv} {dtype} {tag}: o err {eo:.3e}  S err {es:.3e}")
        assert eo <= O_TOL and es <= S_TOL


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_caller_output_scale_every_lane(dtype):
    """A caller-set output scale (not 1/sqrt(dk)) multiplies both parts of o,
    the inter-chunk read and the masked intra-chunk attention, and leaves the
    state alone: one and two segments, two column tiles and the token-serial
    kernel, every lane against the oracle at that scale."""
    lengths = [200, 0, 64, 131]
    scale = 0.37
    wl = workloads.make_custom(lengths, 2, 4, seed=41, dtype=dtype, h0_sigma=0.02,
                               n_max=len(lengths) + 1, t_max=sum(lengths) + 5)
    d = device_inputs(wl)
    ref = oracle_lanes(wl, _all_lanes(wl), scale=scale)
    for tag, segments, tiles in (("one segment", 1, 1), ("two segments", 2, 0),
                                 ("two tiles", 1, 2), ("token-serial", 1, 0)):
        cfg = gdn.make_config(wl.t_max, wl.n_max, 2, 4, dtype, scale=scale, segments=segments,
                              tiles=tiles)
        o = torch.full((wl.t_max, 4, 128), float("nan"), dtype=torch.float32, device=DEV)
        hT = torch.full((wl.n_max, 4, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
        log(f"output scale {scale}, {dtype}, {tag}")
        if tag == "token-serial":
            gdn.gdn_recurrent_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"],
                                  o, hT)
        else:
            ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
            gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"],
                              None, o, hT, ws)
        torch.cuda.synchronize()
        eo, es = lane_errors(wl, o, hT, ref)
        log(f"  o err {eo:.3e}  S err {es:.3e}")
        assert eo <= O_TOL and es <= S_TOL


def _nan_bits(dtype):
    """A NaN whose mantissa bits are all ones (the pattern of memory filled with
    0xff), as one element of the given dtype."""
    if dtype == torch.bfloat16:
        return torch.tensor([-1], dtype=torch.int16).view(torch.bfloat16)
    return torch.tensor([-1], dtype=torch.int32).view(torch.float32)


@pytest.mark.parametrize("shape", ["one tile", "two tiles", "token-serial"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_nan_in_v_reaches_exactly_its_column(shape, dtype):
    """A NaN in v[t0, hv, j] must reach column j of that head's outputs for the
    rest of its sequence and column j of its final state, and nothing else:
    value columns are independent and sequences do not mix. The token-serial
    kernel starts exactly at t0. The chunked form may also reach earlier tokens
    of t0's chunk, because its block products multiply the NaN by zeros of the
    triangular T and P (0 * NaN is NaN; which blocks are skipped is the
    kernel's choice), never tokens of earlier chunks. In the chunked form the
    NaN crosses from stage 1 to stage 2 inside u's 24-bit storage, which keeps
    it a NaN."""
    n = 9 if shape == "two tiles" else 3
    lengths = [150, 170, 200, 33, 129, 64, 90, 1, 120][:n]
    wl = workloads.make_custom(lengths, 4, 8, seed=71, dtype=dtype, h0_sigma=0.02)
    d = device_inputs(wl)
    s, hv, j, off = 1, 5, 37, 100  # sequence 1, value head 5, column 37, its 101st token
    bos, e = int(wl.cu_seqlens[s]), int(wl.cu_seqlens[s + 1])
    t0 = bos + off
    first = t0 if shape == "token-serial" else bos + 64 * (off // 64)
    d["v"][t0, hv, j] = _nan_bits(dtype).to(d["v"].device)[0]
    cfg = config_of(wl)
    o = torch.full((wl.t_max, wl.Hv, 128), 0.0, dtype=torch.float32, device=DEV)
    hT = torch.zeros((wl.n_max, wl.Hv, 128, 128), dtype=torch.float32, device=DEV)
    if shape == "token-serial":
        gdn.gdn_recurrent_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], o,
                              hT)
    else:
        ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
        gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], None,
                          o, hT, ws)
    torch.cuda.synchronize()
    must = torch.zeros_like(o, dtype=torch.bool)
    must[t0:e, hv, j] = True
    may = torch.zeros_like(o, dtype=torch.bool)
    may[first:e, hv, j] = True
    nan_o = torch.isnan(o)
    assert bool((must & ~nan_o).any()) is False, "a NaN did not reach a later output"
    assert torch.isfinite(o[~may]).all(), "a NaN or inf reached another column, head or chunk"
    want_h = torch.zeros_like(hT, dtype=torch.bool)
    want_h[s, hv, j, :] = True  # value-major: row j of the state
    assert torch.equal(torch.isnan(hT), want_h)
    assert torch.isfinite(hT[~want_h]).all()
    if shape == "token-serial":
        assert torch.equal(nan_o, must)


@pytest.mark.parametrize("lengths,with_table", [
    ([300, 64, 0, 64, 1000, 65, 1, 128], False),
    ([300, 64, 0, 64, 1000, 65, 1, 128], True),
    ([0, 0, 0], False),
])
def test_walk_order_table_bit_exact(lengths, with_table):
    """Stage 1 ranks the sequences by chunk count, longest first and ties by
    index (capacity slots past the batch count as empty sequences), for stage
    2 to start the longest walks first. Integer work: compared exactly, with
    the workspace filled with 0xff beforehand; also when every sequence is
    empty (no stage-1 work-group has a chunk) and with a caller table."""
    n_max = len(lengths) + 2
    wl = workloads.make_custom(lengths, 2, 4, seed=81, t_max=sum(lengths) + 10, n_max=n_max)
    d = device_inputs(wl)
    cfg = config_of(wl)
    lay = gdn.gdn_workspace_layout(cfg)
    ws = torch.full((gdn.gdn_workspace_size(cfg),), 255, dtype=torch.uint8, device=DEV)
    table = None
    if with_table:
        table = torch.empty((gdn.gdn_nt_max(wl.t_max, n_max), 2), dtype=torch.int32, device=DEV)
        gdn.gdn_build_chunk_indices(cfg, d["cu"], table)
    o = torch.empty((wl.t_max, wl.Hv, 128), dtype=torch.float32, device=DEV)
    hT = torch.empty((n_max, wl.Hv, 128, 128), dtype=torch.float32, device=DEV)
    gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], table, o,
                      hT, ws)
    torch.cuda.synchronize()
    got = ws[lay["order"]:lay["order"] + 4 * n_max].cpu().view(torch.int32).numpy()
    nc = (np.diff(wl.cu_seqlens) + 63) // 64
    want = sorted(range(n_max), key=lambda s: (-int(nc[s]), s))
    assert got.tolist() == want
    # and the forward itself is right (every sequence walked exactly once)
    T = int(wl.cu_seqlens[-1])
    if T:
        ref = oracle_lanes(wl, [(s, hv) for s in range(len(lengths)) for hv in range(wl.Hv)])
        eo, es = lane_errors(wl, o, hT, ref)
        assert eo <= O_TOL and es <= S_TOL


def _with_capacity(wl, t_max, n_max):
    """The same batch in buffers of another capacity (extra rows zero, extra
    sequences empty)."""
    pad = t_max - wl.t_max
    grow = lambda x: torch.cat([x, torch.zeros((pad,) + tuple(x.shape[1:]), dtype=x.dtype)])
    cu = np.concatenate([wl.cu_seqlens[:len(wl.cu_seqlens)],
                         np.full(n_max + 1 - len(wl.cu_seqlens), wl.cu_seqlens[-1], np.int32)])
    h0 = None
    if wl.h0 is not None:
        h0 = torch.cat([wl.h0, torch.zeros((n_max - wl.h0.shape[0],) + tuple(wl.h0.shape[1:]))])
    return workloads.Workload(name="capacity", cu_seqlens=cu.astype(np.int32), t_max=t_max,
                              n_max=n_max, H=wl.H, Hv=wl.Hv, qkv_dtype=wl.qkv_dtype,
                              q=grow(wl.q), k=grow(wl.k), v=grow(wl.v), g=grow(wl.g),
                              beta=grow(wl.beta), h0=h0)


@pytest.mark.parametrize("lengths", [[256], [300, 64, 1, 129, 0, 77]])
@pytest.mark.parametrize("with_table", [False, True])
def test_capacity_invariance_bitwise(lengths, with_table):
    """A batch run at its exact capacity (for one 256-token sequence NT_max is
    exactly its chunk count: no sentinel slot) and at a larger one (sentinel
    slots, empty extra sequences, and possibly another stage-2 shape) gives
    the same bits, with the table built on the fly or passed in."""
    n = len(lengths)
    exact = workloads.make_custom(lengths, 2, 4, seed=101, h0_sigma=0.02)
    big = _with_capacity(exact, exact.t_max + 500, n + 7)
    outs = []
    for wl in (exact, big):
        d = device_inputs(wl)
        table = None
        if with_table:
            table = torch.empty((gdn.gdn_nt_max(wl.t_max, wl.n_max), 2), dtype=torch.int32,
                                device=DEV)
            gdn.gdn_build_chunk_indices(config_of(wl), d["cu"], table)
        o, hT, _ = run_forward(wl, d, chunk_indices=table)
        outs.append((o, hT))
    if lengths == [256]:
        assert gdn.gdn_nt_max(exact.t_max, exact.n_max) == 4
    T = int(exact.cu_seqlens[-1])
    assert torch.equal(outs[0][0][:T], outs[1][0][:T])
    assert torch.equal(outs[0][1], outs[1][1][:n])
    # the extra sequences are empty: their final state is their (zero) initial state
    assert (outs[1][1][n:] == 0).all()


def test_more_chunk_slots_than_a_grid_dimension_bitwise():
    """A batch whose capacity has more chunk slots than a grid's second
    dimension takes (NT_max > 65535; stage 1's one-dimensional grid then has
    over a million work-groups, nearly all sentinels) gives the bits of the
    same batch at exact capacity."""
    exact = workloads.make_custom([100, 200], 1, 1, seed=111, h0_sigma=0.02)
    t_big = 64 * 65536 + 64
    assert gdn.gdn_nt_max(t_big, 2) > 65535
    d = device_inputs(exact)
    o1, h1, _ = run_forward(exact, d)
    big = {}
    for name in ("q", "k", "v", "g", "beta"):
        x = d[name]
        big[name] = torch.zeros((t_big,) + tuple(x.shape[1:]), dtype=x.dtype, device=DEV)
        big[name][:x.shape[0]] = x
    # one-piece stage 2 as at the exact capacity (this capacity would
    # otherwise pick the two-segment walk, which rounds differently)
    cfg = gdn.make_config(t_big, 2, 1, 1, exact.qkv_dtype, segments=1)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    o = torch.empty((t_big, 1, 128), dtype=torch.float32, device=DEV)
    hT = torch.empty((2, 1, 128, 128), dtype=torch.float32, device=DEV)
    gdn.gdn_chunk_fwd(cfg, big["q"], big["k"], big["v"], big["g"], big["beta"], d["h0"], d["cu"],
                      None, o, hT, ws)
    torch.cuda.synchronize()
    assert torch.equal(o[:300], o1[:300]) and torch.equal(hT, h1)
    del big, ws, o
    torch.cuda.empty_cache()


def test_maximum_capacities_with_sequences_at_the_end_of_the_token_range():
    """t_max and n_max at their limits with the checked sequences at the very
    end of the token range, so that token rows, workspace slots and states sit
    at the largest offsets the limits allow (byte offsets far beyond 2^31): a
    zero-input filler sequence takes the first 2^24 - 277 tokens, two ragged
    sequences end at row t_max, and the other 16381 sequences are empty. The
    automatic launch shape and the two-segment walk, each against the oracle on
    every tail lane; the filler's output is zero and every empty sequence keeps
    its initial state bit for bit."""
    t_max, n_max = gdn.GDN_T_MAX_LIMIT, gdn.GDN_N_MAX_LIMIT
    tail = workloads.make_custom([200, 77], 1, 1, seed=131, h0_sigma=0.02)
    T_tail = tail.n_tokens
    F = t_max - T_tail
    log(f"maximum capacities: t_max={t_max} n_max={n_max} filler={F} tail={T_tail}")
    cu = np.full(n_max + 1, t_max, np.int64)
    cu[0], cu[1], cu[2] = 0, F, F + 200
    cu_d = torch.from_numpy(cu.astype(np.int32)).to(DEV)
    d = device_inputs(tail)
    x = {}
    for name in ("q", "k", "v", "g", "beta"):
        src = d[name]
        x[name] = torch.zeros((t_max,) + tuple(src.shape[1:]), dtype=src.dtype, device=DEV)
        x[name][F:] = src
    h0 = torch.zeros((n_max, 1, 128, 128), dtype=torch.float32, device=DEV)
    h0[1:3] = d["h0"]
    h0[3:] = 0.25  # the empty sequences must hand these back unchanged
    ref = oracle_lanes(tail, [(0, 0), (1, 0)])
    o = torch.empty((t_max, 1, 128), dtype=torch.float32, device=DEV)
    hT = torch.empty((n_max, 1, 128, 128), dtype=torch.float32, device=DEV)
    for segments in (0, 2):
        cfg = gdn.make_config(t_max, n_max, 1, 1, tail.qkv_dtype, segments=segments)
        log(f"  segments={segments}: workspace {gdn.gdn_workspace_size(cfg) / 2**30:.1f} GiB")
        ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
        o.fill_(float("nan"))
        hT.fill_(float("nan"))
        gdn.gdn_chunk_fwd(cfg, x["q"], x["k"], x["v"], x["g"], x["beta"], h0, cu_d, None, o, hT,
                          ws)
        torch.cuda.synchronize()
        del ws
        torch.cuda.empty_cache()
        eo, es = lane_errors(tail, o[F:], hT[1:3], ref)
        log(f"    tail: o err {eo:.3e}  S err {es:.3e}")
        assert eo <= O_TOL and es <= S_TOL
        assert (o[:F] == 0).all() and (hT[0] == 0).all()
        assert torch.equal(hT[3:], h0[3:])
    del x, o, hT, h0
    torch.cuda.empty_cache()


def test_front_and_fused_front_at_the_maximum_token_capacity():
    """The standalone front (its token blocks then number 2^18) and the
    forward with the front fused into stage 1 at t_max = 2^24, with the
    checked sequences ending at row t_max after a zero-input filler sequence:
    the tail against the fp64 front and recurrence, the filler's rows zero."""
    t_max = gdn.GDN_T_MAX_LIMIT
    tail = workloads.make_custom([200, 77], 1, 1, seed=137, front=True, d_conv=4, h0_sigma=0.02)
    F = t_max - tail.n_tokens
    n_max = 4
    log(f"front at maximum capacity: t_max={t_max} filler={F}")
    cu = np.full(n_max + 1, t_max, np.int64)
    cu[0], cu[1], cu[2] = 0, F, F + 200
    cu_d = torch.from_numpy(cu.astype(np.int32)).to(DEV)
    d = device_inputs(tail)
    qkv = torch.zeros((t_max, d["qkv"].shape[1]), dtype=d["qkv"].dtype, device=DEV)
    qkv[F:] = d["qkv"]
    cfg = gdn.make_config(t_max, n_max, 1, 1, torch.float32)
    q = torch.full((t_max, 1, 128), float("nan"), dtype=torch.float32, device=DEV)
    k = torch.full_like(q, float("nan"))
    v = torch.full_like(q, float("nan"))
    gdn.gdn_front_conv_silu_l2(cfg, qkv, d["conv_w"], 4, cu_d, q, k, v)
    torch.cuda.synchronize()
    ref = recurrent.gdn_front(tail.f64("qkv"), tail.f64("conv_w"), tail.cu_seqlens, 1, 1, 128, 128)
    for got, want in zip((q, k, v), ref):
        g64 = got[F:].cpu().double().numpy()
        assert np.max(np.abs(g64 - want)) / np.max(np.abs(want)) < 1e-5
        assert (got[:F] == 0).all()
    del q, k, v
    torch.cuda.empty_cache()
    log("  fused front forward")
    x = {}
    for name in ("g", "beta"):
        x[name] = torch.zeros((t_max,) + tuple(d[name].shape[1:]), dtype=d[name].dtype, device=DEV)
        x[name][F:] = d[name]
    h0 = torch.zeros((n_max, 1, 128, 128), dtype=torch.float32, device=DEV)
    h0[1:3] = d["h0"]
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    o = torch.full((t_max, 1, 128), float("nan"), dtype=torch.float32, device=DEV)
    hT = torch.full((n_max, 1, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    gdn.gdn_chunk_fwd_conv(cfg, qkv, d["conv_w"], 4, x["g"], x["beta"], h0, cu_d, None, o, hT, ws)
    torch.cuda.synchronize()
    del ws
    lanes = oracle_lanes(tail, [(0, 0), (1, 0)], qkv64=oracle_inputs_f64(tail))
    eo, es = lane_errors(tail, o[F:], hT[1:3], lanes)
    log(f"    tail: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL
    assert (o[:F] == 0).all() and (hT[0] == 0).all()
    del qkv, x, o, hT, h0
    torch.cuda.empty_cache()
