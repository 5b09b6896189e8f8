"""GPU parity of the segmented stage 2 (gdn_config.segments = 2, 3 or 4): each
sequence's segments are walked at once, every segment after the first from
the zero state and from the identity, and fix-up kernels chain the segments'
states and correct their outputs. Checked against the CPU oracle on every
lane of small batches (sequence lengths around the chunk and segment
boundaries, sequences too short to reach the later segments, empty
sequences, fp32 and bf16, with and without initial states), with a weak decay
that makes the corrections large terms, and on the long-context workload in
the launch configuration the benchmark uses (automatic segments) and in four
segments, against the oracle on every lane and against the one-piece walk.
"""

import numpy as np
import pytest
import torch

import chunked_gated_delta_rule_amd as gdn
import workloads

from gpu_helpers import (O_TOL, S_TOL, device_inputs, full_errors, lane_errors, log, oracle_full,
                         oracle_lanes)
from oracle import recurrent

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


def _forward(wl, segments, d=None, with_hT=True):
    if d is None:
        d = device_inputs(wl, DEV)
    cfg = gdn.make_config(wl.t_max, wl.n_max, wl.H, wl.Hv, wl.qkv_dtype, segments=segments)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    o = torch.full((wl.t_max, wl.Hv, 128), float("nan"), dtype=torch.float32, device=DEV)
    hT = torch.full((wl.n_max, wl.Hv, 128, 128), float("nan"), dtype=torch.float32,
                    device=DEV) if with_hT else None
    gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], None, o,
                      hT, ws)
    torch.cuda.synchronize()
    return o, hT


LENGTHS = [0, 1, 64, 65, 127, 128, 129, 300, 1000, 63, 0]


@pytest.mark.parametrize("segments", [2, 3, 4])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("with_h0", [True, False])
def test_segments_every_lane(segments, dtype, with_h0):
    wl = workloads.make_custom(LENGTHS, 2, 4, seed=21, dtype=dtype, t_max=sum(LENGTHS) + 70,
                               n_max=len(LENGTHS) + 1, h0_sigma=0.02 if with_h0 else 0.0)
    log(f"{segments} segments: lengths {LENGTHS} dtype={dtype} h0={with_h0}")
    o, hT = _forward(wl, segments)
    ref = oracle_lanes(wl, _all_lanes(wl))
    eo, es = lane_errors(wl, o, hT, ref)
    log(f"  o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL
    T = int(wl.cu_seqlens[-1])
    assert torch.isnan(o[T:]).all()  # rows past the batch untouched


@pytest.mark.parametrize("segments", [3, 4])
def test_segments_capacity_too_short_for_later_segments(segments):
    """t_max of at most 64 x segments tokens: no sequence reaches a later
    segment (they have no chunks), so segment 0 walks everything and the
    chained states hand its final state through unchanged."""
    lengths = [100, 0, 30, 60]
    wl = workloads.make_custom(lengths, 1, 2, seed=24, t_max=sum(lengths), h0_sigma=0.05)
    assert wl.t_max <= 64 * segments
    log(f"{segments} segments, t_max {wl.t_max}")
    o, hT = _forward(wl, segments)
    eo, es = lane_errors(wl, o, hT, oracle_lanes(wl, _all_lanes(wl)))
    log(f"  o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


@pytest.mark.parametrize("segments", [2, 3, 4])
def test_segments_without_final_state(segments):
    """Without hT the outputs are bitwise those with it (with more than two
    segments the intermediate states are still chained for the outputs, and
    the chain stops before the last state)."""
    wl = workloads.make_custom([700, 5, 190], 2, 4, seed=22, h0_sigma=0.02)
    d = device_inputs(wl, DEV)
    o_ref, _ = _forward(wl, segments, d)
    o, _ = _forward(wl, segments, d, with_hT=False)
    assert torch.equal(o[:wl.n_tokens], o_ref[:wl.n_tokens])


def test_long_context_automatic_segments_vs_one_piece():
    """The long-context workload resolves to two segments on an MI355X; both
    walks meet the bar against the oracle and agree with each other."""
    wl = workloads.make(3)
    cfg = gdn.make_config(wl.t_max, wl.n_max, wl.H, wl.Hv, wl.qkv_dtype)
    lay = gdn.gdn_workspace_layout(cfg)
    assert lay["seg_oh"] < lay["total"], "automatic segments should pick two here"
    d = device_inputs(wl, DEV)
    o2, h2 = _forward(wl, 0, d)
    o1, h1 = _forward(wl, 1, d)
    o_ref, s_ref = oracle_full(wl)
    for tag, (o, h) in (("two segments", (o2, h2)), ("one piece", (o1, h1))):
        eo, es = full_errors(wl, o, h, o_ref, s_ref)
        log(f"  {tag}: o err {eo:.3e}  S err {es:.3e}")
        assert eo <= O_TOL and es <= S_TOL
    T = wl.n_tokens
    eo = float((o2[:T] - o1[:T]).abs().max() / o1[:T].abs().max())
    es = float((h2 - h1).norm() / h1.norm())
    log(f"  two segments vs one piece: o {eo:.3e}  S {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


@pytest.mark.parametrize("segments", [2, 3, 4])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_segments_weak_decay(segments, dtype):
    """With g scaled down the state carries across the whole sequence, so the
    later segments' outputs and the final state depend strongly on the first
    segment: the fix-up's correction is a large term here, not a rounding one."""
    lengths = [2000, 129, 700]
    wl = workloads.make_custom(lengths, 2, 4, seed=23, dtype=dtype, h0_sigma=0.05, g_scale=0.002)
    d = device_inputs(wl, DEV)
    o, hT = _forward(wl, segments, d)
    ref = oracle_lanes(wl, _all_lanes(wl))
    eo, es = lane_errors(wl, o, hT, ref)
    log(f"  weak decay, {segments} segments: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL
    if segments != 2:
        return
    # the first half matters: the second half walked from zero alone (what the
    # fix-up corrects) is far from the true outputs
    s, hv = 0, 1
    a, e = int(wl.cu_seqlens[s]), int(wl.cu_seqlens[s + 1])
    mid = a + 64 * ((((e - a) + 63) // 64 + 1) // 2)
    h = hv // (wl.Hv // wl.H)
    f = lambda name, j: wl.f64(name)[mid:e, j:j + 1]
    o_zero, _ = recurrent.gdn_recurrent(f("q", h), f("k", h), f("v", hv), f("g", hv),
                                        f("beta", hv), np.array([0, e - mid], np.int32))
    o_true = ref[(s, hv)][0][mid - a:]
    gap = np.max(np.abs(o_zero[:, 0] - o_true)) / np.max(np.abs(o_true))
    log(f"  second half from zero vs true: {gap:.3e}")
    assert gap > 50 * O_TOL


def test_long_context_four_segments():
    """The long-context workload walked in four segments (three chained
    states): every lane against the oracle."""
    wl = workloads.make(3)
    log(f"four segments, workload 3 ({wl.name})")
    o, hT = _forward(wl, 4)
    o_ref, s_ref = oracle_full(wl)
    eo, es = full_errors(wl, o, hT, o_ref, s_ref)
    log(f"  every lane: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


def test_long_context_fewer_heads_automatic_segments():
    """The long-context recipe with H = Hv = 8 (a one-piece walk of 64
    work-groups): the automatic choice takes four segments on an MI355X, and
    every lane meets the bar against the oracle."""
    wl = workloads.make(7)
    log(f"automatic segments, workload 7 ({wl.name})")
    cfg = gdn.make_config(wl.t_max, wl.n_max, wl.H, wl.Hv, wl.qkv_dtype)
    lay = gdn.gdn_workspace_layout(cfg)
    state = wl.n_max * wl.Hv * 128 * 128 * 4
    assert lay["seg_phi"] - lay["seg_z"] == 3 * state, "automatic segments should pick four here"
    o, hT = _forward(wl, 0)
    o_ref, s_ref = oracle_full(wl)
    eo, es = full_errors(wl, o, hT, o_ref, s_ref)
    log(f"  every lane: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL
