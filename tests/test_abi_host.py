"""Host-side checks of the C ABI: the library loads, exports every entry point
declared in include/gdn.h, and rejects bad arguments on the host with the
documented status before any HIP call. No test here launches a kernel."""

import ctypes
import os
import re
import subprocess

import pytest

import chunked_gated_delta_rule_amd as gdn
from oracle import index_table

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, INVALID, UNSUPPORTED, CAPACITY, WORKSPACE = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.library_path):
        pytest.fail("libgdn.so is not built (run python -m chunked_gated_delta_rule_amd.build)")
    return gdn.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert set(_declared_functions()) == set(gdn.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in [(0, "GDN_OK"), (1, "GDN_ERR_INVALID_ARG"), (2, "GDN_ERR_UNSUPPORTED"),
                       (3, "GDN_ERR_CAPACITY"), (4, "GDN_ERR_WORKSPACE"), (5, "GDN_ERR_HIP")]:
        assert gdn.gdn_status_str(code) == name
    assert gdn.gdn_status_str(99) == "GDN_ERR_UNKNOWN"


@pytest.mark.parametrize("t_max,n_max", [(0, 1), (1, 1), (64, 1), (65, 1), (4096, 32),
                                         (32768, 32), (32768, 1), (100, 7)])
def test_nt_max_matches_oracle_bound(lib, t_max, n_max):
    assert gdn.gdn_nt_max(t_max, n_max) == index_table.nt_max(t_max, n_max)


def test_nt_max_rejects_bad_arguments(lib):
    assert gdn.gdn_nt_max(-1, 1) == -1
    assert gdn.gdn_nt_max(10, 0) == -1
    assert gdn.gdn_nt_max(10, 1, 0) == -1


@pytest.mark.parametrize("dtype,nk", [(gdn.GDN_BF16, 16), (gdn.GDN_F32, 32)])
def test_workspace_layout(lib, dtype, nk):
    T, N, H, Hv = 4100, 3, 16, 32
    cfg = gdn.make_config(T, N, H, Hv, dtype)
    al = lambda x: (x + 255) // 256 * 256
    nt = index_table.nt_max(T, N)
    sizes = [("w16", Hv * nt * 16 * 1024), ("q16", H * nt * 16 * 1024), ("kimg", H * nt * nk * 1024),
             ("uimg", Hv * nt * 64 * 128 * 3), ("pimg", Hv * nt * 5 * 1024),
             ("gimg", Hv * nt * 192 * 4), ("table", nt * 8), ("order", N * 4)]
    lay = gdn.gdn_workspace_layout(cfg)
    at = 0
    for name, size in sizes:
        assert lay[name] == at, name
        at += al(size)
    assert lay["total"] == at == gdn.gdn_workspace_size(cfg)


@pytest.mark.parametrize("n,ranked", [(1, False), (2, True), (256, True), (257, False)])
def test_workspace_order_region(lib, n, ranked):
    """The sequence ranking for stage 2 takes n_max int32 when stage 1 ranks
    the batch (2 to GDN_FUSED_INDEX_MAX_SEQS sequences), else nothing."""
    assert gdn.GDN_FUSED_INDEX_MAX_SEQS == 256
    lay = gdn.gdn_workspace_layout(gdn.make_config(1000, n, 2, 4))
    al = lambda x: (x + 255) // 256 * 256
    assert lay["order"] == lay["table"] + al(index_table.nt_max(1000, n) * 8)
    assert lay["total"] - lay["order"] == (al(n * 4) if ranked else 0)


def test_workspace_layout_segments(lib):
    """Two segments append the stage-2 scratch (three state arrays and the
    homogeneous output rows); one segment appends nothing."""
    T, N, H, Hv = 5000, 2, 2, 4
    al = lambda x: (x + 255) // 256 * 256
    one = gdn.gdn_workspace_layout(gdn.make_config(T, N, H, Hv, segments=1))
    two = gdn.gdn_workspace_layout(gdn.make_config(T, N, H, Hv, segments=2))
    for name in ("seg_sa", "seg_z", "seg_phi", "seg_oh"):
        assert one[name] == one["total"]
    state = al(N * Hv * 128 * 128 * 4)
    assert two["seg_sa"] == one["total"]
    assert two["seg_z"] == two["seg_sa"] + state
    assert two["seg_phi"] == two["seg_z"] + state
    assert two["seg_oh"] == two["seg_phi"] + state
    assert two["total"] == two["seg_oh"] + al(T * Hv * 128 * 4)
    # automatic: needs the token capacity and a stage-2 grid of at most half
    # the device (one sequence, 16 value heads: 128 work-groups; without a
    # device the library assumes 256 compute units, as on an MI355X)
    lay = gdn.gdn_workspace_layout(gdn.make_config(32768, 1, 16, 16))
    assert lay["seg_oh"] < lay["total"]
    short = gdn.make_config(gdn.GDN_SEGMENT_MIN_TOKENS - 1, 1, 16, 16)
    lay = gdn.gdn_workspace_layout(short)
    assert lay["seg_oh"] == lay["total"]
    wide = gdn.make_config(32768, 1, 16, 32)  # 256 work-groups: one segment
    lay = gdn.gdn_workspace_layout(wide)
    assert lay["seg_oh"] == lay["total"]
    # automatic, fewer heads: the most segments (up to four) whose walks fit
    # the device (H = Hv = 8: 64 work-groups, four segments)
    lay = gdn.gdn_workspace_layout(gdn.make_config(32768, 1, 8, 8))
    four = gdn.gdn_workspace_layout(gdn.make_config(32768, 1, 8, 8, segments=4))
    assert lay == four and lay["seg_phi"] - lay["seg_z"] == 3 * 8 * 128 * 128 * 4
    # P segments: segment 0's state, then P - 1 zero-start and P - 1
    # homogeneous states, then the homogeneous output rows
    for parts in (3, 4):
        lay = gdn.gdn_workspace_layout(gdn.make_config(T, N, H, Hv, segments=parts))
        assert lay["seg_sa"] == one["total"]
        assert lay["seg_z"] == lay["seg_sa"] + state
        assert lay["seg_phi"] == lay["seg_z"] + al((parts - 1) * N * Hv * 128 * 128 * 4)
        assert lay["seg_oh"] == lay["seg_phi"] + al((parts - 1) * N * Hv * 128 * 128 * 4)
        assert lay["total"] == lay["seg_oh"] + al(T * Hv * 128 * 4)


@pytest.mark.parametrize("field,value,status", [
    ("dk", 64, UNSUPPORTED), ("dv", 256, UNSUPPORTED), ("chunk", 32, UNSUPPORTED),
    ("hv", 24, UNSUPPORTED), ("o_dtype", gdn.GDN_BF16, UNSUPPORTED),
    ("t_max", -1, INVALID), ("n_max", 0, INVALID), ("h", 0, INVALID), ("qkv_dtype", 7, INVALID),
    ("qkv_dtype", 2, OK),
    ("scale", float("nan"), INVALID), ("t_max", (1 << 24) + 1, CAPACITY), ("n_max", 16385, CAPACITY),
    ("segments", 5, INVALID), ("segments", -1, INVALID), ("segments", 3, OK), ("segments", 4, OK),
    ("tiles", 3, INVALID),
    ("tiles", -1, INVALID), ("tiles", 8, INVALID), ("tiles", 4, OK), ("tiles", 1, OK),
    ("gqa_share", 3, INVALID), ("gqa_share", -1, INVALID), ("gqa_share", 8, INVALID),
    ("gqa_share", 2, OK), ("gqa_share", 1, OK),
    ("gqa_share", 4, UNSUPPORTED),  # 4 does not divide hv / h = 2
])
def test_config_validation(lib, field, value, status):
    cfg = gdn.make_config(256, 2, 16, 32)
    setattr(cfg, field, value)
    out = ctypes.c_size_t(0)
    assert lib.gdn_workspace_size(ctypes.byref(cfg), ctypes.byref(out)) == status


def test_gqa_share_needs_the_one_piece_one_tile_walk(lib):
    """The GQA-shared stage 2 carries one column slice of 2 or 4 value heads
    per work-group: it needs hv / h divisible by the share, one segment and
    one tile; automatic segments and tiles then resolve to one (no segment
    scratch in the workspace, even where two segments would be chosen)."""
    out = ctypes.c_size_t(0)

    def status(**kw):
        cfg = gdn.make_config(32768, 1, 4, 16, **kw)  # HG = 4
        return lib.gdn_workspace_size(ctypes.byref(cfg), ctypes.byref(out))

    assert status(gqa_share=4) == OK and status(gqa_share=2) == OK
    assert status(gqa_share=2, segments=2) == UNSUPPORTED
    assert status(gqa_share=2, tiles=2) == UNSUPPORTED
    assert status(gqa_share=2, tiles=4) == UNSUPPORTED
    assert status(gqa_share=2, segments=1, tiles=1) == OK
    cfg = gdn.make_config(64, 1, 3, 6, gqa_share=4)  # HG = 2
    assert lib.gdn_workspace_size(ctypes.byref(cfg), ctypes.byref(out)) == UNSUPPORTED
    auto = gdn.gdn_workspace_layout(gdn.make_config(32768, 1, 4, 8))  # 128 work-groups
    shared = gdn.gdn_workspace_layout(gdn.make_config(32768, 1, 4, 8, gqa_share=2))
    assert auto["seg_oh"] < auto["total"]  # automatic: two segments
    assert shared["seg_oh"] == shared["total"]  # shared: one piece, no segment scratch


def test_binding_structs_match_the_header(tmp_path):
    """The ctypes mirrors of gdn_config and gdn_workspace_layout_t have the
    C header's size and field offsets (compiled here with the host C
    compiler, so a field added to one side only fails)."""
    import shutil
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    structs = {"gdn_config": gdn.gdn_config, "gdn_workspace_layout_t": gdn.gdn_workspace_layout_t}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "gdn.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in py._fields_:
            lines.append(f'  printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "offsets.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "offsets"
    subprocess.run([cc, "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out.splitlines()}
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for field, _ in py._fields_:
            assert got[(cname, field)] == getattr(py, field).offset, (cname, field)


def test_null_config_and_output(lib):
    out = ctypes.c_size_t(0)
    assert lib.gdn_workspace_size(None, ctypes.byref(out)) == INVALID
    cfg = gdn.make_config(256, 2, 16, 32)
    assert lib.gdn_workspace_size(ctypes.byref(cfg), None) == INVALID


FAKE = 1 << 20  # 16-byte aligned non-null address; never dereferenced on these paths


def _fwd(lib, cfg, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=FAKE, ci=None, o=FAKE,
                hT=None, ws=FAKE, ws_bytes=1 << 40)
    args.update(over)
    return lib.gdn_chunk_fwd(ctypes.byref(cfg), args["q"], args["k"], args["v"], args["g"],
                             args["beta"], args["h0"], args["cu"], args["ci"], args["o"],
                             args["hT"], args["ws"], args["ws_bytes"], None)


def test_chunk_fwd_host_errors(lib):
    cfg = gdn.make_config(256, 2, 16, 32)
    need = gdn.gdn_workspace_size(cfg)
    assert _fwd(lib, cfg, q=None) == INVALID
    assert _fwd(lib, cfg, o=None) == INVALID
    assert _fwd(lib, cfg, ws=None) == WORKSPACE
    assert _fwd(lib, cfg, ws_bytes=need - 1) == WORKSPACE
    assert _fwd(lib, cfg, ws=FAKE + 16) == WORKSPACE          # not 256-byte aligned
    assert _fwd(lib, cfg, q=FAKE + 2) == INVALID               # not 16-byte aligned
    assert _fwd(lib, cfg, g=FAKE + 2) == INVALID
    bad = gdn.make_config(256, 2, 16, 24)
    assert _fwd(lib, bad) == UNSUPPORTED


def test_stage_entry_points_host_errors(lib):
    cfg = gdn.make_config(256, 2, 16, 32)
    c = ctypes.byref(cfg)
    F = FAKE
    need = gdn.gdn_workspace_size(cfg)
    # intra: (cfg, q, k, v, g, beta, cu, table, workspace, ws_bytes, stream)
    assert lib.gdn_chunk_fwd_intra(c, F, F, F, F, F, F, None, F, need, None) == INVALID
    assert lib.gdn_chunk_fwd_intra(c, None, F, F, F, F, F, F, F, need, None) == INVALID
    assert lib.gdn_chunk_fwd_intra(c, F, F, F, F, F, F, F + 8, F, need, None) == INVALID
    assert lib.gdn_chunk_fwd_intra(c, F, F, F, F, F, F, F, None, need, None) == WORKSPACE
    assert lib.gdn_chunk_fwd_intra(c, F, F, F, F, F, F, F, F, need - 1, None) == WORKSPACE
    assert lib.gdn_chunk_fwd_intra(c, F, F, F, F, F, F, F, F + 16, need, None) == WORKSPACE
    # inter: (cfg, h0, cu, workspace, ws_bytes, o, hT, stream)
    assert lib.gdn_chunk_fwd_inter(c, None, F, F, need, None, None, None) == INVALID
    assert lib.gdn_chunk_fwd_inter(c, None, None, F, need, F, None, None) == INVALID
    assert lib.gdn_chunk_fwd_inter(c, F + 4, F, F, need, F, None, None) == INVALID
    assert lib.gdn_chunk_fwd_inter(c, None, F, None, need, F, None, None) == WORKSPACE
    assert lib.gdn_chunk_fwd_inter(c, None, F, F, need - 1, F, None, None) == WORKSPACE
    assert lib.gdn_build_chunk_indices(c, F, None, None) == INVALID
    assert lib.gdn_front_conv_silu_l2(c, F, F, 9, F, F, F, F, None) == UNSUPPORTED
    assert lib.gdn_front_conv_silu_l2(c, F, F, 0, F, F, F, F, None) == UNSUPPORTED
    assert lib.gdn_front_conv_silu_l2(c, None, F, 4, F, F, F, F, None) == INVALID


def test_timed_entry_points_host_errors(lib):
    """The timed variants reject a missing event, and otherwise validate like
    the entry points they extend, all before any launch."""
    cfg = gdn.make_config(256, 2, 16, 32)
    c = ctypes.byref(cfg)
    F = FAKE
    need = gdn.gdn_workspace_size(cfg)
    vp6 = ctypes.c_void_p * 6

    def timed(events, **over):
        a = dict(q=F, o=F, ws=F, ws_bytes=need)
        a.update(over)
        return lib.gdn_chunk_fwd_timed(c, a["q"], F, F, F, F, None, F, None, a["o"], None, a["ws"],
                                       a["ws_bytes"], None, events)

    assert timed(None) == INVALID
    assert timed(vp6(1, 2, 3, 4, 5, None)) == INVALID
    assert timed(vp6(1, 2, 3, 4, 5, 6), q=None) == INVALID
    assert timed(vp6(1, 2, 3, 4, 5, 6), ws_bytes=need - 1) == WORKSPACE
    assert lib.gdn_front_conv_silu_l2_timed(c, F, F, 4, F, F, F, F, None, None, 8) == INVALID
    assert lib.gdn_front_conv_silu_l2_timed(c, F, F, 9, F, F, F, F, None, 8, 8) == UNSUPPORTED


def test_header_constants_match_binding():
    text = open(HEADER).read()
    m = re.search(r"#define GDN_FUSED_INDEX_MAX_SEQS (\d+)", text)
    assert m and int(m.group(1)) == gdn.GDN_FUSED_INDEX_MAX_SEQS
    m = re.search(r"#define GDN_SEGMENT_MIN_TOKENS (\d+)", text)
    assert m and int(m.group(1)) == gdn.GDN_SEGMENT_MIN_TOKENS
    m = re.search(r"#define GDN_FOUR_TILE_MIN_TOKENS (\d+)", text)
    assert m and int(m.group(1)) == gdn.GDN_FOUR_TILE_MIN_TOKENS
    m = re.search(r"#define GDN_T_MAX_LIMIT \(1 << (\d+)\)", text)
    assert m and 1 << int(m.group(1)) == gdn.GDN_T_MAX_LIMIT
    m = re.search(r"#define GDN_N_MAX_LIMIT (\d+)", text)
    assert m and int(m.group(1)) == gdn.GDN_N_MAX_LIMIT


def test_fused_front_entry_point_host_errors(lib):
    cfg = gdn.make_config(256, 2, 16, 32, gdn.GDN_F32)
    c = ctypes.byref(cfg)
    F = FAKE
    need = gdn.gdn_workspace_size(cfg)
    # (cfg, qkv, conv_w, d_conv, g, beta, h0, cu, ci, o, hT, ws, ws_bytes, stream)
    assert lib.gdn_chunk_fwd_conv(c, None, F, 4, F, F, None, F, None, F, None, F, need, None) == INVALID
    assert lib.gdn_chunk_fwd_conv(c, F, None, 4, F, F, None, F, None, F, None, F, need, None) == INVALID
    assert lib.gdn_chunk_fwd_conv(c, F, F, 5, F, F, None, F, None, F, None, F, need, None) == UNSUPPORTED
    assert lib.gdn_chunk_fwd_conv(c, F, F, 0, F, F, None, F, None, F, None, F, need, None) == UNSUPPORTED
    assert lib.gdn_chunk_fwd_conv(c, F + 2, F, 4, F, F, None, F, None, F, None, F, need,
                                  None) == INVALID
    assert lib.gdn_chunk_fwd_conv(c, F, F, 4, F, F, None, F, None, F, None, F, need - 1,
                                  None) == WORKSPACE
    bf = gdn.make_config(256, 2, 16, 32, gdn.GDN_BF16)
    assert lib.gdn_chunk_fwd_conv(ctypes.byref(bf), F, F, 4, F, F, None, F, None, F, None, F,
                                  1 << 40, None) == UNSUPPORTED
    vp6 = ctypes.c_void_p * 6
    assert lib.gdn_chunk_fwd_conv_timed(c, F, F, 4, F, F, None, F, None, F, None, F, need, None,
                                        None) == INVALID
    assert lib.gdn_chunk_fwd_conv_timed(c, F, F, 4, F, F, None, F, None, F, None, F, need, None,
                                        vp6(1, 2, 3, 4, None, 6)) == INVALID


def test_recurrent_entry_points_host_errors(lib):
    """gdn_recurrent_fwd validates like the chunk forward (no workspace); its
    timed variant also rejects a missing event; nothing is launched."""
    c = ctypes.byref(gdn.make_config(256, 2, 16, 32))
    F = FAKE
    # (cfg, q, k, v, g, beta, h0, cu, o, hT, stream)
    assert lib.gdn_recurrent_fwd(None, F, F, F, F, F, None, F, F, None, None) == INVALID
    for i in range(8):
        args = [F] * 8
        args[i] = None
        q, k, v, g, b, cu, o = args[:5] + args[6:8]
        if i == 5:
            continue  # that slot is h0 below, which may be null
        assert lib.gdn_recurrent_fwd(c, q, k, v, g, b, None, cu, o, None, None) == INVALID, i
    assert lib.gdn_recurrent_fwd(c, F + 8, F, F, F, F, None, F, F, None, None) == INVALID
    assert lib.gdn_recurrent_fwd(c, F, F, F, F + 2, F, None, F, F, None, None) == INVALID
    assert lib.gdn_recurrent_fwd(c, F, F, F, F, F, F + 4, F, F, None, None) == INVALID
    assert lib.gdn_recurrent_fwd(c, F, F, F, F, F, None, F, F, F + 4, None) == INVALID
    bad = gdn.make_config(256, 2, 16, 24)
    assert lib.gdn_recurrent_fwd(ctypes.byref(bad), F, F, F, F, F, None, F, F, None,
                                 None) == UNSUPPORTED
    f16 = gdn.make_config(256, 2, 16, 32, gdn.GDN_F16)  # fp16 input: chunked forward only
    assert lib.gdn_recurrent_fwd(ctypes.byref(f16), F, F, F, F, F, None, F, F, None,
                                 None) == UNSUPPORTED
    assert lib.gdn_recurrent_fwd_timed(c, F, F, F, F, F, None, F, F, None, None, None, 8) == INVALID
    assert lib.gdn_recurrent_fwd_timed(c, F, F, F, F, F, None, F, F, None, None, 8, None) == INVALID
    assert lib.gdn_recurrent_fwd_timed(c, None, F, F, F, F, None, F, F, None, None, 8, 8) == INVALID


def test_two_segment_fixup_past_the_launch_limit_is_refused_on_the_host(lib):
    """Both capacities at their limits with two segments forced and three
    value heads: segment B holds 2/5 of the 2^18 chunks, so the fix-up would
    need 16384 * 3 * (52429 + 1) > 2^31 - 1 work-groups, and the forward (and
    the inter stage alone) returns GDN_ERR_CAPACITY from the host checks,
    before anything is queued (no device exists here)."""
    cfg = gdn.make_config(gdn.GDN_T_MAX_LIMIT, gdn.GDN_N_MAX_LIMIT, 1, 3, segments=2)
    need = gdn.gdn_workspace_size(cfg)
    assert _fwd(lib, cfg, ws_bytes=need) == CAPACITY
    assert lib.gdn_chunk_fwd_inter(ctypes.byref(cfg), None, FAKE, FAKE, need, FAKE, None,
                                   None) == CAPACITY
    one = gdn.make_config(gdn.GDN_T_MAX_LIMIT, gdn.GDN_N_MAX_LIMIT, 1, 2, segments=2)
    assert lib.gdn_workspace_size(ctypes.byref(one), ctypes.byref(ctypes.c_size_t())) == OK


def test_binding_rejects_wrong_dtypes_and_sizes():
    """The Python binding checks tensor dtypes and sizes against the config
    before any pointer reaches the library (CPU tensors suffice: the checks run
    first)."""
    import torch
    with pytest.raises(ValueError, match="dtype"):
        gdn.make_config(64, 1, 1, 1, torch.float64)
    assert gdn.make_config(64, 1, 1, 1, torch.float16).qkv_dtype == gdn.GDN_F16
    T, n, H, Hv = 64, 1, 1, 2
    cfg = gdn.make_config(T, n, H, Hv, torch.bfloat16)
    ok = dict(q=torch.zeros(T, H, 128, dtype=torch.bfloat16),
              k=torch.zeros(T, H, 128, dtype=torch.bfloat16),
              v=torch.zeros(T, Hv, 128, dtype=torch.bfloat16),
              g=torch.zeros(T, Hv), beta=torch.zeros(T, Hv),
              h0=torch.zeros(n, Hv, 128, 128), cu=torch.tensor([0, T], dtype=torch.int32),
              o=torch.zeros(T, Hv, 128), hT=torch.zeros(n, Hv, 128, 128))
    bad_cases = [
        ("q", torch.zeros(T, H, 128, dtype=torch.float16), "dtype"),  # fp16 in a bf16 config
        ("k", torch.zeros(T, H, 128), "dtype"),                       # fp32 in a bf16 config
        ("v", torch.zeros(T, Hv, 64, dtype=torch.bfloat16), "elements"),
        ("q", torch.zeros(2 * T, H, 64, dtype=torch.bfloat16), "last dimension"),
        ("g", torch.zeros(T, Hv, dtype=torch.bfloat16), "dtype"),
        ("beta", torch.zeros(T, 1), "elements"),
        ("h0", torch.zeros(n, Hv, 128, 64), "elements"),
        ("cu", torch.tensor([0, T]), "dtype"),                         # int64
        ("o", torch.zeros(T, Hv, 128, dtype=torch.bfloat16), "dtype"),
        ("hT", torch.zeros(n, 1, 128, 128), "elements"),
    ]
    for name, t, what in bad_cases:
        a = dict(ok, **{name: t})
        with pytest.raises(ValueError, match=what):
            gdn.gdn_chunk_fwd(cfg, a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"],
                              None, a["o"], a["hT"], torch.zeros(16, dtype=torch.uint8),
                              ws_bytes=16)
        with pytest.raises(ValueError, match=what):
            gdn.gdn_recurrent_fwd(cfg, a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"],
                                  a["cu"], a["o"], a["hT"])
    with pytest.raises(ValueError, match="one dtype"):
        gdn.chunk_gated_delta_rule(ok["q"], ok["k"].float(), ok["v"], ok["g"], ok["beta"],
                                   ok["cu"])
    with pytest.raises(ValueError, match="workspace"):
        gdn.gdn_chunk_fwd(cfg, ok["q"], ok["k"], ok["v"], ok["g"], ok["beta"], None, ok["cu"],
                          None, ok["o"], None, torch.zeros(16, dtype=torch.uint8), ws_bytes=4096)
    # every check passed: the CPU tensors are then refused as non-device memory
    with pytest.raises(ValueError, match="device tensor"):
        gdn.gdn_chunk_fwd(cfg, ok["q"], ok["k"], ok["v"], ok["g"], ok["beta"], ok["h0"],
                          ok["cu"], None, ok["o"], ok["hT"], torch.zeros(16, dtype=torch.uint8),
                          ws_bytes=16)
