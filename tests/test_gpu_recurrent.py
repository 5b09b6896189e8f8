"""GPU parity of the token-serial recurrent kernel (gdn_recurrent_fwd: decode
and speculative verify) against the CPU oracle's fp64 token recurrence,
through the C ABI.

Bar: the same tolerance as the chunked path (max |o_gpu - o_ref| / max |o_ref|
<= 2e-3, relative Frobenius error of the final states <= 1e-3), on every lane.
The kernel applies the tokens one at a time in fp32, so it is also held to a
much tighter bound (1e-5), which a reordered (chunked) evaluation would not
meet at these sizes.
"""

import numpy as np
import pytest
import torch

import chunked_gated_delta_rule_amd as gdn
import workloads

from gpu_helpers import O_TOL, S_TOL, config_of, device_inputs, lane_errors, log, oracle_lanes

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SERIAL_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    gdn.load_library()  # raises if the HIP library is missing


def _all_lanes(wl):
    n = len(wl.cu_seqlens) - 1
    return [(s, hv) for s in range(n) for hv in range(wl.Hv)]


def _run(wl, d=None, h0="input", hT=None):
    if d is None:
        d = device_inputs(wl, DEV)
    cfg = config_of(wl)
    o = torch.full((wl.t_max, wl.Hv, 128), float("nan"), dtype=torch.float32, device=DEV)
    if hT is None:
        hT = torch.full((wl.n_max, wl.Hv, 128, 128), float("nan"), dtype=torch.float32,
                        device=DEV)
    gdn.gdn_recurrent_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"],
                          d["h0"] if isinstance(h0, str) else h0, d["cu"], o, hT)
    torch.cuda.synchronize()
    return o, hT


def _check(wl, o, hT, tag):
    ref = oracle_lanes(wl, _all_lanes(wl))
    eo, es = lane_errors(wl, o, hT, ref)
    log(f"  {tag}: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL
    assert eo <= SERIAL_TOL and es <= SERIAL_TOL
    # rows past the last sequence are untouched
    T = int(wl.cu_seqlens[-1])
    assert torch.isnan(o[T:]).all()


@pytest.mark.parametrize("cfg_id", [5, 6])
def test_recurrent_named_workload(cfg_id):
    wl = workloads.make(cfg_id)
    log(f"workload {cfg_id} ({wl.name}) tokens={wl.n_tokens}")
    o, hT = _run(wl)
    _check(wl, o, hT, wl.name)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("with_h0", [True, False])
def test_recurrent_ragged_batch(dtype, with_h0):
    lengths = [0, 1, 2, 5, 16, 17, 3, 0]
    wl = workloads.make_custom(lengths, 2, 4, seed=11, dtype=dtype, t_max=sum(lengths) + 5,
                               n_max=len(lengths) + 2, h0_sigma=0.05 if with_h0 else 0.0)
    log(f"ragged batch {lengths} dtype={dtype} h0={with_h0}")
    o, hT = _run(wl)
    _check(wl, o, hT, "ragged")
    # zero-length (and unused tail) sequences pass the initial state through
    d = device_inputs(wl, DEV)
    for s in range(wl.n_max):
        if wl.cu_seqlens[s + 1] == wl.cu_seqlens[s]:
            want = d["h0"][s] if d["h0"] is not None else torch.zeros_like(hT[s])
            assert torch.equal(hT[s], want)


def test_recurrent_in_place_state():
    wl = workloads.make_custom([3, 9, 1, 16], 4, 8, seed=12, h0_sigma=0.05)
    d = device_inputs(wl, DEV)
    o_ref, hT_ref = _run(wl, d)
    state = d["h0"].clone()
    o, _ = _run(wl, d, h0=state, hT=state)
    assert torch.equal(o[:wl.n_tokens], o_ref[:wl.n_tokens])
    assert torch.equal(state, hT_ref)


def test_recurrent_long_sequences():
    """Beyond verify widths the kernel is still the exact token recurrence."""
    wl = workloads.make_custom([300, 77, 129], 2, 4, seed=13, h0_sigma=0.02)
    log("long sequences [300, 77, 129]")
    o, hT = _run(wl)
    _check(wl, o, hT, "long")


def test_recurrent_matches_chunked_forward_within_tolerance():
    """The serial kernel and the chunked forward compute the same function:
    on a verify-width batch they agree to the parity bar."""
    wl = workloads.make(5)
    d = device_inputs(wl, DEV)
    o_r, h_r = _run(wl, d)
    cfg = config_of(wl)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    o_c = torch.full_like(o_r, float("nan"))
    h_c = torch.full_like(h_r, float("nan"))
    gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], None,
                      o_c, h_c, ws)
    torch.cuda.synchronize()
    T = wl.n_tokens
    eo = float((o_r[:T] - o_c[:T]).abs().max() / o_r[:T].abs().max())
    es = float((h_r - h_c).norm() / h_r.norm())
    log(f"  serial vs chunked: o {eo:.3e}  S {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


def test_recurrent_at_both_capacity_limits_with_sequences_at_the_end():
    """t_max = 2^24 and n_max = 16384 (a grid of n_max * Hv work-groups) with
    the checked sequences as the last two, ending at row t_max: 16382
    zero-input sequences of about 1024 tokens come first. The tail against the
    oracle; the zero-input sequences give zero output and hand back their
    initial states bit for bit."""
    t_max, n_max = gdn.GDN_T_MAX_LIMIT, gdn.GDN_N_MAX_LIMIT
    tail = workloads.make_custom([200, 77], 1, 1, seed=139, h0_sigma=0.02)
    F = t_max - tail.n_tokens
    nf = n_max - 2
    cu = np.empty(n_max + 1, np.int64)
    cu[:nf + 1] = np.arange(nf + 1, dtype=np.int64) * F // nf
    cu[nf + 1], cu[nf + 2] = F + 200, t_max
    log(f"token-serial at the capacity limits: t_max={t_max} n_max={n_max} filler={F}")
    d = device_inputs(tail)
    x = {}
    for name in ("q", "k", "v", "g", "beta"):
        src = d[name]
        x[name] = torch.zeros((t_max,) + tuple(src.shape[1:]), dtype=src.dtype, device=DEV)
        x[name][F:] = src
    h0 = torch.full((n_max, 1, 128, 128), 0.25, dtype=torch.float32, device=DEV)
    h0[nf:] = d["h0"]
    cfg = gdn.make_config(t_max, n_max, 1, 1, tail.qkv_dtype)
    o = torch.full((t_max, 1, 128), float("nan"), dtype=torch.float32, device=DEV)
    hT = torch.full((n_max, 1, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    gdn.gdn_recurrent_fwd(cfg, x["q"], x["k"], x["v"], x["g"], x["beta"], h0,
                          torch.from_numpy(cu.astype(np.int32)).to(DEV), o, hT)
    torch.cuda.synchronize()
    ref = oracle_lanes(tail, [(0, 0), (1, 0)])
    eo, es = lane_errors(tail, o[F:], hT[nf:], ref)
    log(f"  tail: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= SERIAL_TOL and es <= SERIAL_TOL
    assert (o[:F] == 0).all() and torch.equal(hT[:nf], h0[:nf])
    del x, o, hT, h0
    torch.cuda.empty_cache()
