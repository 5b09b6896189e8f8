"""GPU parity of the GQA-shared stage 2 (gdn_config.gqa_share = 2 or 4): each
work-group carries one 16-column slice of 2 or 4 value heads of one key head
and loads that key head's K^T and q fragments once for them ("Optimizing GDN
Chunk Prefill on Intel AMX CPU", sections 3 and 5: the inter stage over key
heads, reusing the key head's operands across its value heads).

Every value head's products run in the one-tile order, so the results must
equal the one-tile shape's bit for bit; they are also checked on every lane
against the fp64 oracle (ragged batches with empty sequences and initial
states, bf16, fp16 and fp32 input, groups of 2 to 8 value heads per key head)
and on the T = 4096 single-sequence workload at full size."""

import pytest
import torch

import chunked_gated_delta_rule_amd as gdn
import workloads

from gpu_helpers import (O_TOL, S_TOL, device_inputs, full_errors, lane_errors, log,
                         oracle_full, oracle_lanes)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LENGTHS = [0, 1, 64, 65, 127, 200, 333, 63, 129]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    gdn.load_library()  # raises if the HIP library is missing


def _forward(wl, d, gqa_share, tiles=1):
    cfg = gdn.make_config(wl.t_max, wl.n_max, wl.H, wl.Hv, wl.qkv_dtype, segments=1, tiles=tiles,
                          gqa_share=gqa_share)
    ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    o = torch.full((wl.t_max, wl.Hv, 128), float("nan"), dtype=torch.float32, device=DEV)
    hT = torch.full((wl.n_max, wl.Hv, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], None, o,
                      hT, ws)
    torch.cuda.synchronize()
    return o, hT


@pytest.mark.parametrize("H,Hv,share,dtype", [
    (2, 4, 2, torch.bfloat16),
    (2, 8, 4, torch.bfloat16),
    (1, 8, 2, torch.float32),
    (3, 12, 4, torch.float16),
    (2, 16, 4, torch.float32),   # HG = 8: two work-groups per (key head, slice)
    (5, 30, 2, torch.bfloat16),  # HG = 6, H not a multiple of the XCD count
])
def test_gqa_share_every_lane_and_bitwise_one_tile(H, Hv, share, dtype):
    wl = workloads.make_custom(LENGTHS, H, Hv, seed=301 + 7 * H + Hv, dtype=dtype,
                               t_max=sum(LENGTHS) + 40, h0_sigma=0.02)
    log(f"gqa_share={share} H={H} Hv={Hv} dtype={dtype} lengths {LENGTHS}")
    d = device_inputs(wl, DEV)
    o, hT = _forward(wl, d, share)
    o1, h1 = _forward(wl, d, 1)
    T = int(wl.cu_seqlens[-1])
    assert torch.equal(o[:T], o1[:T])
    assert torch.equal(hT, h1)
    assert torch.isnan(o[T:]).all()  # rows past the batch untouched
    lanes = [(s, hv) for s in range(len(LENGTHS)) for hv in range(Hv)]
    eo, es = lane_errors(wl, o, hT, oracle_lanes(wl, lanes))
    log(f"  every lane: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


def test_gqa_share_single_sequence_full_size():
    """T = 4096, H = 16, Hv = 32, bf16: every lane against the oracle, and
    bitwise equal to the default shape (one tile) on the same inputs."""
    wl = workloads.make(1)
    log(f"gqa_share=2, workload 1 ({wl.name})")
    d = device_inputs(wl, DEV)
    o, hT = _forward(wl, d, 2)
    o1, h1 = _forward(wl, d, 1)
    assert torch.equal(o, o1) and torch.equal(hT, h1)
    o_ref, s_ref = oracle_full(wl)
    eo, es = full_errors(wl, o, hT, o_ref, s_ref)
    log(f"  every lane: o err {eo:.3e}  S err {es:.3e}")
    assert eo <= O_TOL and es <= S_TOL


def test_gqa_share_no_token_capacity():
    """t_max = 0: the walk has no chunk; every final state is the initial one
    (batch sizes with and without the stage-1 sequence ranking)."""
    H, Hv = 2, 8
    for n_max in (1, 3):
        cfg = gdn.make_config(0, n_max, H, Hv, torch.bfloat16, gqa_share=4)
        log(f"gqa_share=4, t_max = 0, n_max = {n_max}")
        one = lambda *shape, dt=torch.float32: torch.zeros(shape, dtype=dt, device=DEV)
        q, k = one(1, H, 128, dt=torch.bfloat16), one(1, H, 128, dt=torch.bfloat16)
        v, g, beta, o = one(1, Hv, 128, dt=torch.bfloat16), one(1, Hv), one(1, Hv), one(1, Hv, 128)
        cu = torch.zeros(n_max + 1, dtype=torch.int32, device=DEV)
        h0 = torch.full((n_max, Hv, 128, 128), 0.25, dtype=torch.float32, device=DEV)
        h0[-1] = -0.5
        hT = torch.full_like(h0, float("nan"))
        ws = torch.empty(max(gdn.gdn_workspace_size(cfg), 256), dtype=torch.uint8, device=DEV)
        gdn.gdn_chunk_fwd(cfg, q, k, v, g, beta, h0, cu, None, o, hT, ws)
        torch.cuda.synchronize()
        assert torch.equal(hT, h0)
