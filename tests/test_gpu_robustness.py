"""Malformed cu_seqlens and chunk tables stay inside the caller's buffers.

cu_seqlens (cu[0] = 0, non-decreasing, cu[n_max] <= t_max) and a caller's
chunk table are documented preconditions that the library never reads on the
host. With invalid ones the results are unspecified, but every kernel clamps
the entries it reads to [0, t_max] and treats table entries that name no
sequence or no chunk as sentinels, so nothing is read or written outside the
buffers the config describes. Here each buffer sits inside a larger
allocation whose guard rows hold a canary; after every call on malformed
input the canaries must be intact.
"""

import numpy as np
import pytest
import torch

import chunked_gated_delta_rule_amd as gdn
import workloads

from gpu_helpers import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PAD = 256          # guard rows / states on each side
CANARY = 1234.5
T_MAX, N_MAX, H, HV = 300, 5, 2, 4
BAD_CU = [
    [0, 100, 50, 400, 250, 9999],   # decreasing, past t_max
    [0, -20, 30, 30, 500, 200],     # negative, past t_max, decreasing
    [7, 7000, 10, 20, 30, 40],      # nonzero start, huge
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    gdn.load_library()  # raises if the HIP library is missing


def _canary(dtype):
    return CANARY if dtype.is_floating_point else 1234


def _guarded(rows, rest, dtype, data=None):
    """(whole allocation, the rows view): guard rows filled with the canary."""
    big = torch.full((PAD + rows + PAD,) + tuple(rest), _canary(dtype), dtype=dtype, device=DEV)
    view = big[PAD:PAD + rows]
    if data is not None:
        view.copy_(data)
    return big, view


def _intact(big, rows):
    c = _canary(big.dtype)
    return bool((big[:PAD] == c).all()) and bool((big[PAD + rows:] == c).all())


def _inputs(dtype=torch.bfloat16):
    wl = workloads.make_custom([60, 60, 60, 60, 60], H, HV, seed=91, dtype=dtype, h0_sigma=0.02,
                               t_max=T_MAX, n_max=N_MAX)
    d = {}
    for name, rest in (("q", (H, 128)), ("k", (H, 128)), ("v", (HV, 128)), ("g", (HV,)),
                       ("beta", (HV,))):
        t = getattr(wl, name)
        d[name] = _guarded(T_MAX, rest, t.dtype, t.to(DEV))
    d["h0"] = _guarded(N_MAX, (HV, 128, 128), torch.float32, wl.h0.to(DEV))
    return d


def _cu(values):
    big = torch.full((N_MAX + 1 + 128,), 1 << 30, dtype=torch.int32, device=DEV)
    big[:N_MAX + 1] = torch.tensor(values, dtype=torch.int32)
    return big[:N_MAX + 1]


def _outputs():
    o = _guarded(T_MAX, (HV, 128), torch.float32)
    hT = _guarded(N_MAX, (HV, 128, 128), torch.float32)
    return o, hT


def _workspace(cfg):
    n = gdn.gdn_workspace_size(cfg)
    big = torch.full((65536 + n + 65536,), 0xA5, dtype=torch.uint8, device=DEV)
    return big, big[65536:65536 + n]


def _ws_intact(big, n):
    return bool((big[:65536] == 0xA5).all()) and bool((big[65536 + n:] == 0xA5).all())


@pytest.mark.parametrize("bad", range(len(BAD_CU)))
@pytest.mark.parametrize("with_table", [False, True])
def test_malformed_cu_seqlens_stays_in_bounds(bad, with_table):
    d = _inputs()
    cu = _cu(BAD_CU[bad])
    cfg = gdn.make_config(T_MAX, N_MAX, H, HV)
    wsb, ws = _workspace(cfg)
    (ob, o), (hb, hT) = _outputs()
    table = None
    if with_table:
        nt = gdn.gdn_nt_max(T_MAX, N_MAX)
        tb, table = _guarded(nt, (2,), torch.int32)
        gdn.gdn_build_chunk_indices(cfg, cu, table)
    log(f"cu {BAD_CU[bad]} table={with_table}")
    gdn.gdn_chunk_fwd(cfg, d["q"][1], d["k"][1], d["v"][1], d["g"][1], d["beta"][1], d["h0"][1],
                      cu, table, o, hT, ws)
    torch.cuda.synchronize()
    assert _intact(ob, T_MAX) and _intact(hb, N_MAX)
    assert _ws_intact(wsb, ws.numel())
    if with_table:
        assert _intact(tb, gdn.gdn_nt_max(T_MAX, N_MAX))
    for name in ("q", "k", "v", "g", "beta", "h0"):  # inputs are read only
        assert _intact(d[name][0], N_MAX if name == "h0" else T_MAX), name


@pytest.mark.parametrize("bad", range(len(BAD_CU)))
def test_malformed_cu_seqlens_token_serial_and_front(bad):
    d = _inputs()
    cu = _cu(BAD_CU[bad])
    cfg = gdn.make_config(T_MAX, N_MAX, H, HV)
    (ob, o), (hb, hT) = _outputs()
    gdn.gdn_recurrent_fwd(cfg, d["q"][1], d["k"][1], d["v"][1], d["g"][1], d["beta"][1],
                          d["h0"][1], cu, o, hT)
    torch.cuda.synchronize()
    assert _intact(ob, T_MAX) and _intact(hb, N_MAX)
    C = (2 * H + HV) * 128
    xb, qkv = _guarded(T_MAX, (C,), torch.bfloat16,
                       torch.randn(T_MAX, C, device=DEV).to(torch.bfloat16))
    w = torch.randn(C, 4, device=DEV).to(torch.bfloat16)
    fcfg = gdn.make_config(T_MAX, N_MAX, H, HV, torch.float32)
    (qb, q), (kb, k), (vb, v) = (_guarded(T_MAX, (H, 128), torch.float32),
                                 _guarded(T_MAX, (H, 128), torch.float32),
                                 _guarded(T_MAX, (HV, 128), torch.float32))
    gdn.gdn_front_conv_silu_l2(fcfg, qkv, w, 4, cu, q, k, v)
    torch.cuda.synchronize()
    assert _intact(qb, T_MAX) and _intact(kb, T_MAX) and _intact(vb, T_MAX)
    assert _intact(xb, T_MAX)


def test_invalid_table_entries_are_sentinels():
    """Entries naming no sequence, a negative chunk or a chunk past its
    sequence's end do no work; the valid entries still compute their chunks,
    bitwise as with the plain table."""
    d = _inputs()
    cu = _cu([0, 60, 120, 180, 240, 300])
    cfg = gdn.make_config(T_MAX, N_MAX, H, HV)
    nt = gdn.gdn_nt_max(T_MAX, N_MAX)
    good = torch.empty((nt, 2), dtype=torch.int32, device=DEV)
    gdn.gdn_build_chunk_indices(cfg, cu, good)
    ws_ref = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    o_ref = torch.empty((T_MAX, HV, 128), dtype=torch.float32, device=DEV)
    h_ref = torch.empty((N_MAX, HV, 128, 128), dtype=torch.float32, device=DEV)
    gdn.gdn_chunk_fwd(cfg, d["q"][1], d["k"][1], d["v"][1], d["g"][1], d["beta"][1], d["h0"][1],
                      cu, good, o_ref, h_ref, ws_ref)
    tb, table = _guarded(nt, (2,), torch.int32, good)
    used = int((good[:, 0] >= 0).sum())
    bad = torch.tensor([[7, 0], [-3, 2], [1, 999999], [0, 3], [N_MAX, 0], [2, -1]],
                       dtype=torch.int32, device=DEV)
    table[used:used + len(bad)] = bad[:nt - used]
    wsb, ws = _workspace(cfg)
    (ob, o), (hb, hT) = _outputs()
    gdn.gdn_chunk_fwd(cfg, d["q"][1], d["k"][1], d["v"][1], d["g"][1], d["beta"][1], d["h0"][1],
                      cu, table, o, hT, ws)
    torch.cuda.synchronize()
    assert _intact(ob, T_MAX) and _intact(hb, N_MAX) and _ws_intact(wsb, ws.numel())
    assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)
