"""gdn_chunk_fwd_noalloc (the forward with its intermediates in the library's
fixed device scratch) against gdn_chunk_fwd with a caller workspace, through
the C ABI: bitwise equal outputs on two calls in a row, the second on a
smaller batch, and a config past the scratch size refused on the host."""

import ctypes

import numpy as np
import pytest
import torch

import chunked_gated_delta_rule_amd as gdn
import workloads

from gpu_helpers import device_inputs, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    gdn.load_library()  # raises if the HIP library is missing


def _both(wl):
    """(o, hT) from gdn_chunk_fwd with a fresh workspace and from
    gdn_chunk_fwd_noalloc, same inputs, outputs pre-filled with NaN."""
    d = device_inputs(wl, DEV)
    cfg = gdn.make_config(wl.t_max, wl.n_max, wl.H, wl.Hv, wl.qkv_dtype)
    out = []
    for noalloc in (False, True):
        o = torch.full((wl.t_max, wl.Hv, 128), float("nan"), dtype=torch.float32, device=DEV)
        hT = torch.full((wl.n_max, wl.Hv, 128, 128), float("nan"), dtype=torch.float32,
                        device=DEV)
        if noalloc:
            gdn.gdn_chunk_fwd_noalloc(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                      d["cu"], None, o, hT)
        else:
            ws = torch.empty(gdn.gdn_workspace_size(cfg), dtype=torch.uint8, device=DEV)
            gdn.gdn_chunk_fwd(cfg, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"],
                              None, o, hT, ws)
        torch.cuda.synchronize()
        out.append((o, hT))
    return out


def test_noalloc_matches_workspace_forward_on_two_calls_in_a_row():
    """The headline workload (T = 4096, H = 16, Hv = 32), then a smaller
    ragged varlen batch with initial states on the same scratch: each call's
    outputs equal the caller-workspace forward's bit for bit, so nothing of the
    first call's intermediates leaks into the second."""
    big = workloads.make(1)
    small = workloads.make_custom([300, 0, 77, 129], 2, 4, seed=151, h0_sigma=0.02,
                                  t_max=600, n_max=6)
    for wl in (big, small):
        cfg = gdn.make_config(wl.t_max, wl.n_max, wl.H, wl.Hv, wl.qkv_dtype)
        log(f"noalloc vs workspace: {wl.name} tokens={wl.n_tokens} "
            f"workspace={gdn.gdn_workspace_size(cfg) / 2**20:.1f} MiB")
        (o1, s1), (o2, s2) = _both(wl)
        T = wl.n_tokens
        assert torch.isfinite(o2[:T]).all()
        assert torch.equal(o1[:T], o2[:T]) and torch.equal(s1, s2)
        assert torch.isnan(o2[T:]).all()  # rows past the batch untouched


def test_noalloc_refuses_configs_past_the_scratch_on_the_host():
    """A config whose workspace exceeds GDN_NOALLOC_SCRATCH_BYTES returns
    GDN_ERR_WORKSPACE before anything is queued; the outputs stay untouched."""
    t_max = 16384
    cfg = gdn.make_config(t_max, 1, 16, 32, torch.bfloat16)
    assert gdn.gdn_workspace_size(cfg) > gdn.GDN_NOALLOC_SCRATCH_BYTES
    lib = gdn.load_library()
    o = torch.full((4, 32, 128), 7.0, dtype=torch.float32, device=DEV)
    x = torch.zeros(16, dtype=torch.float32, device=DEV)  # never read: the call stops first
    p = x.data_ptr()
    st = lib.gdn_chunk_fwd_noalloc(ctypes.byref(cfg), p, p, p, p, p, None, p, None,
                                   o.data_ptr(), None, None)
    torch.cuda.synchronize()
    assert st == 4  # GDN_ERR_WORKSPACE
    assert (o == 7.0).all()
