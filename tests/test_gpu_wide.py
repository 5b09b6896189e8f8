"""GPU parity of the stage-2 shapes with two and four 16-column tiles per
work-group (gdn_config.tiles; automatic for grids larger than the device).
Checked on every lane against the CPU oracle (bf16 and fp32 input, with and
without initial states, lengths around the chunk size and empty sequences),
bitwise across tiles = 1, 2 and 4 on the same batch (every shape does the
same products in the same order per tile), and bitwise against each sequence
run alone, which takes the one-tile shape."""

import numpy as np
import pytest
import torch

import chunked_gated_delta_rule_amd as gdn
import workloads

from gpu_helpers import (O_TOL, S_TOL, device_inputs, lane_errors, log, oracle_lanes,
                         run_forward)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LENGTHS = [0, 1, 64, 65, 127, 200, 333, 63, 129]
H, HV = 4, 8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    gdn.load_library()  # raises if the HIP library is missing


def _batch(dtype, h0_sigma, seed=61):
    return workloads.make_custom(LENGTHS, H, HV, seed=seed, dtype=dtype, t_max=sum(LENGTHS) + 40,
                                 h0_sigma=h0_sigma)


def _one_tile_grid(n, h, hv):
    """Stage-2 one-tile work-groups: (sequence, key head) groups rounded up to
    the 8 XCDs, times 8 column tiles per value head of the group."""
    return -(-n * h // 8) * 8 * (hv // h) * 8


def _forward(wl, tiles, d=None):
    if d is None:
        d = device_inputs(wl, DEV)
    cfg = gdn.make_config(wl.t_max, wl.n_max, wl.H, wl.Hv, wl.qkv_dtype, segments=1, tiles=tiles)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    o = torch.full((wl.t_max, wl.Hv, 128), float("nan"), dtype=torch.float32, device=DEV)
    hT = torch.full((wl.n_max, wl.Hv, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], None, o,
                      hT, ws)
    torch.cuda.synchronize()
    return o, hT


def test_batch_takes_the_two_tile_shape():
    # more one-tile work-groups than an MI355X has CUs, and less capacity
    # than GDN_FOUR_TILE_MIN_TOKENS per sequence: the automatic choice is two
    # tiles; one sequence alone takes one
    assert _one_tile_grid(len(LENGTHS), H, HV) > 256
    assert sum(LENGTHS) + 40 < len(LENGTHS) * gdn.GDN_FOUR_TILE_MIN_TOKENS
    assert _one_tile_grid(1, H, HV) <= 256


@pytest.mark.parametrize("tiles", [2, 4])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("h0_sigma", [0.02, 0.0])
def test_column_tiles_every_lane(tiles, dtype, h0_sigma):
    wl = _batch(dtype, h0_sigma)
    log(f"{tiles} tiles: lengths {LENGTHS} dtype={dtype} h0={h0_sigma}")
    o, hT = _forward(wl, tiles)
    lanes = [(s, hv) for s in range(len(LENGTHS)) for hv in range(HV)]
    ref = oracle_lanes(wl, lanes)
    eo, es = lane_errors(wl, o, hT, ref)
    log(f"  o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL
    T = int(wl.cu_seqlens[-1])
    assert torch.isnan(o[T:]).all()  # rows past the batch untouched


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_tile_shapes_bitwise_equal(dtype):
    wl = _batch(dtype, 0.02, seed=63)
    d = device_inputs(wl, DEV)
    o1, h1 = _forward(wl, 1, d)
    T = int(wl.cu_seqlens[-1])
    for tiles in (2, 4, 0):
        o, h = _forward(wl, tiles, d)
        assert torch.equal(o[:T], o1[:T]), tiles
        assert torch.equal(h, h1), tiles


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_two_tiles_bitwise_equal_to_one_tile(dtype):
    wl = _batch(dtype, 0.02, seed=62)
    o, hT, _ = run_forward(wl)
    cu = wl.cu_seqlens
    for s in range(len(LENGTHS)):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        one = workloads.Workload(
            name="alone", cu_seqlens=np.array([0, e - a], np.int32), t_max=e - a, n_max=1,
            H=wl.H, Hv=wl.Hv, qkv_dtype=wl.qkv_dtype, q=wl.q[a:e].clone(), k=wl.k[a:e].clone(),
            v=wl.v[a:e].clone(), g=wl.g[a:e].clone(), beta=wl.beta[a:e].clone(),
            h0=wl.h0[s:s + 1].clone())
        o1, h1, _ = run_forward(one)
        assert torch.equal(o1, o[a:e]), s
        assert torch.equal(h1[0], hT[s]), s
