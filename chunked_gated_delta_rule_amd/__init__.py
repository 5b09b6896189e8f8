"""Python binding of libgdn.so, the MI355X (gfx950) chunked gated-delta-rule
prefill forward.

The functions below carry the names of the C ABI in ``include/gdn.h`` and
only marshal arguments: torch tensors become device pointers, the current
torch stream becomes the hipStream_t, and a non-OK status becomes a
``GDNError``. Every step of the computation runs in the library's HIP
kernels; there is no fallback of any kind. If the library has not been built
(``python -m chunked_gated_delta_rule_amd.build``), importing the binding
still works but the first call raises.

Layouts (packed varlen, batch 1): q, k [t_max, h, 128]; v, o [t_max, hv, 128];
g, beta [t_max, hv] fp32; states [n_max, hv, 128 (v), 128 (k)] fp32;
cu_seqlens int32 [n_max + 1].
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "GDNError", "gdn_config", "GDN_BF16", "GDN_F32", "GDN_F16", "load_library", "library_path",
    "gdn_nt_max", "gdn_workspace_size", "gdn_build_chunk_indices", "gdn_front_conv_silu_l2",
    "gdn_chunk_fwd_intra", "gdn_chunk_fwd_inter", "gdn_chunk_fwd", "gdn_status_str",
    "gdn_workspace_layout", "make_config", "chunk_gated_delta_rule", "EXPORTED_SYMBOLS",
    "gdn_chunk_fwd_timed", "gdn_front_conv_silu_l2_timed", "GDN_FUSED_INDEX_MAX_SEQS",
    "gdn_chunk_fwd_conv", "gdn_chunk_fwd_conv_timed", "gdn_recurrent_fwd",
    "gdn_recurrent_fwd_timed", "recurrent_gated_delta_rule", "GDN_SEGMENT_MIN_TOKENS", "GDN_FOUR_TILE_MIN_TOKENS",
    "GDN_T_MAX_LIMIT", "GDN_N_MAX_LIMIT", "gdn_chunk_fwd_noalloc", "GDN_NOALLOC_SCRATCH_BYTES",
]

GDN_BF16 = 0
GDN_F32 = 1
GDN_F16 = 2
GDN_FUSED_INDEX_MAX_SEQS = 256  # include/gdn.h
GDN_SEGMENT_MIN_TOKENS = 2048  # include/gdn.h
GDN_FOUR_TILE_MIN_TOKENS = 384  # include/gdn.h
GDN_T_MAX_LIMIT = 1 << 24  # include/gdn.h
GDN_N_MAX_LIMIT = 16384  # include/gdn.h
GDN_NOALLOC_SCRATCH_BYTES = 256 << 20  # include/gdn.h
_STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARG", 2: "GDN_ERR_UNSUPPORTED",
           3: "GDN_ERR_CAPACITY", 4: "GDN_ERR_WORKSPACE", 5: "GDN_ERR_HIP"}
EXPORTED_SYMBOLS = ("gdn_nt_max", "gdn_workspace_layout", "gdn_workspace_size",
                    "gdn_build_chunk_indices", "gdn_front_conv_silu_l2", "gdn_chunk_fwd_intra",
                    "gdn_chunk_fwd_inter", "gdn_chunk_fwd", "gdn_status_str",
                    "gdn_chunk_fwd_timed", "gdn_front_conv_silu_l2_timed", "gdn_chunk_fwd_conv",
                    "gdn_chunk_fwd_conv_timed", "gdn_recurrent_fwd", "gdn_recurrent_fwd_timed",
                    "gdn_chunk_fwd_noalloc")

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libgdn.so")


class gdn_config(ctypes.Structure):
    _fields_ = [("t_max", ctypes.c_int32), ("n_max", ctypes.c_int32), ("h", ctypes.c_int32),
                ("hv", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("qkv_dtype", ctypes.c_int), ("o_dtype", ctypes.c_int),
                ("scale", ctypes.c_float), ("segments", ctypes.c_int32),
                ("tiles", ctypes.c_int32), ("gqa_share", ctypes.c_int32)]


class gdn_workspace_layout_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("w16", "q16", "kimg", "uimg", "pimg", "gimg", "table", "order", "seg_sa", "seg_z",
                 "seg_phi", "seg_oh", "total")]


class GDNError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)}")


_lib = None


def load_library():
    """Load libgdn.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is missing: build it with "
                           "`python -m chunked_gated_delta_rule_amd.build`")
    lib = ctypes.CDLL(library_path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(gdn_config)
    lib.gdn_nt_max.argtypes = [i32, i32, i32]
    lib.gdn_nt_max.restype = ctypes.c_int64
    lib.gdn_workspace_size.argtypes = [cfgp, ctypes.POINTER(sz)]
    lib.gdn_workspace_layout.argtypes = [cfgp, ctypes.POINTER(gdn_workspace_layout_t)]
    lib.gdn_build_chunk_indices.argtypes = [cfgp, vp, vp, vp]
    lib.gdn_front_conv_silu_l2.argtypes = [cfgp, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.gdn_chunk_fwd_intra.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_chunk_fwd_inter.argtypes = [cfgp, vp, vp, vp, sz, vp, vp, vp]
    lib.gdn_chunk_fwd.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_chunk_fwd_timed.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                        ctypes.POINTER(vp)]
    lib.gdn_front_conv_silu_l2_timed.argtypes = [cfgp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_chunk_fwd_conv.argtypes = [cfgp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_chunk_fwd_conv_timed.argtypes = [cfgp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                             vp, ctypes.POINTER(vp)]
    lib.gdn_recurrent_fwd.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_chunk_fwd_noalloc.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_recurrent_fwd_timed.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    for name in ("gdn_workspace_size", "gdn_workspace_layout", "gdn_build_chunk_indices", "gdn_front_conv_silu_l2",
                 "gdn_chunk_fwd_intra", "gdn_chunk_fwd_inter", "gdn_chunk_fwd",
                 "gdn_chunk_fwd_timed", "gdn_front_conv_silu_l2_timed", "gdn_chunk_fwd_conv",
                 "gdn_chunk_fwd_conv_timed", "gdn_recurrent_fwd", "gdn_recurrent_fwd_timed",
                 "gdn_chunk_fwd_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    lib.gdn_status_str.argtypes = [ctypes.c_int]
    lib.gdn_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


_TORCH_DTYPE = {torch.bfloat16: GDN_BF16, torch.float32: GDN_F32, torch.float16: GDN_F16}
_GDN_DTYPE = {GDN_BF16: torch.bfloat16, GDN_F32: torch.float32, GDN_F16: torch.float16}


def make_config(t_max, n_max, h, hv, qkv_dtype=GDN_BF16, scale=0.0, o_dtype=GDN_F32,
                dk=128, dv=128, chunk=64, segments=0, tiles=0, gqa_share=0) -> gdn_config:
    """A gdn_config; qkv_dtype is GDN_BF16 / GDN_F32 / GDN_F16 or the torch
    dtype (bfloat16, float32, float16; any other raises ValueError)."""
    if isinstance(qkv_dtype, torch.dtype):
        if qkv_dtype not in _TORCH_DTYPE:
            raise ValueError(f"q/k/v dtype {qkv_dtype}: bfloat16, float32 or float16 expected")
        qkv_dtype = _TORCH_DTYPE[qkv_dtype]
    return gdn_config(int(t_max), int(n_max), int(h), int(hv), int(dk), int(dv), int(chunk),
                      int(qkv_dtype), int(o_dtype), float(scale), int(segments), int(tiles),
                      int(gqa_share))


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        if not x.is_cuda:
            raise ValueError("device tensor expected")
        if not x.is_contiguous():
            raise ValueError("contiguous tensor expected")
        return x.data_ptr()
    raise TypeError(type(x))


def _need(x, name, elems, dtype, last=None):
    """A tensor argument must have `dtype`, hold at least `elems` elements (the
    kernels index that many from its start) and, when `last` is given and the
    tensor has more than one dimension, end in a dimension of that size. Raw
    pointers (ints) and None are passed through unchecked."""
    if not isinstance(x, torch.Tensor):
        return
    if x.dtype != dtype:
        raise ValueError(f"{name}: dtype {x.dtype}, {dtype} expected")
    if x.numel() < elems:
        raise ValueError(f"{name}: {x.numel()} elements, at least {elems} expected")
    if last is not None and x.dim() > 1 and x.shape[-1] != last:
        raise ValueError(f"{name}: last dimension {x.shape[-1]}, {last} expected")


def _check_tensors(cfg, q=None, k=None, v=None, g=None, beta=None, h0=None, cu=None,
                   table=None, o=None, hT=None):
    """Dtypes and sizes of the tensor arguments against `cfg` (include/gdn.h layouts)."""
    T, n, h, hv, dk, dv = cfg.t_max, cfg.n_max, cfg.h, cfg.hv, cfg.dk, cfg.dv
    qdt = _GDN_DTYPE.get(cfg.qkv_dtype, torch.bfloat16)
    _need(q, "q", T * h * dk, qdt, dk)
    _need(k, "k", T * h * dk, qdt, dk)
    _need(v, "v", T * hv * dv, qdt, dv)
    _need(g, "g", T * hv, torch.float32)
    _need(beta, "beta", T * hv, torch.float32)
    _need(h0, "h0", n * hv * dv * dk, torch.float32, dk)
    _need(hT, "hT", n * hv * dv * dk, torch.float32, dk)
    _need(cu, "cu_seqlens", n + 1, torch.int32)
    if table is not None:
        _need(table, "chunk_indices", 2 * max(gdn_nt_max(T, n, cfg.chunk), 0), torch.int32)
    _need(o, "o", T * hv * dv, torch.float32, dv)


def _check_front(cfg, qkv, conv_w, d_conv):
    C = (2 * cfg.h * cfg.dk + cfg.hv * cfg.dv)
    _need(qkv, "qkv", cfg.t_max * C, torch.bfloat16, C)
    _need(conv_w, "conv_w", C * int(d_conv), torch.bfloat16)


def _check_ws(workspace, ws_bytes):
    if isinstance(workspace, torch.Tensor) and \
            workspace.numel() * workspace.element_size() < int(ws_bytes):
        raise ValueError(f"workspace: {workspace.numel() * workspace.element_size()} bytes, "
                         f"ws_bytes = {int(ws_bytes)}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st: int, where: str):
    if st != 0:
        raise GDNError(st, where)


def gdn_status_str(status: int) -> str:
    return load_library().gdn_status_str(int(status)).decode()


def gdn_nt_max(t_max: int, n_max: int, chunk: int = 64) -> int:
    return int(load_library().gdn_nt_max(int(t_max), int(n_max), int(chunk)))


def gdn_workspace_size(cfg: gdn_config) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().gdn_workspace_size(ctypes.byref(cfg), ctypes.byref(out)),
           "gdn_workspace_size")
    return int(out.value)


def gdn_build_chunk_indices(cfg, cu_seqlens, chunk_indices, stream=None):
    _check_tensors(cfg, cu=cu_seqlens, table=chunk_indices)
    _check(load_library().gdn_build_chunk_indices(ctypes.byref(cfg), _ptr(cu_seqlens),
                                                  _ptr(chunk_indices), _stream(stream)),
           "gdn_build_chunk_indices")


def gdn_front_conv_silu_l2(cfg, qkv, conv_w, d_conv, cu_seqlens, q, k, v, stream=None):
    _check_front(cfg, qkv, conv_w, d_conv)
    _check_tensors(make_config(cfg.t_max, cfg.n_max, cfg.h, cfg.hv, GDN_F32), q=q, k=k, v=v,
                   cu=cu_seqlens)
    _check(load_library().gdn_front_conv_silu_l2(ctypes.byref(cfg), _ptr(qkv), _ptr(conv_w),
                                                 int(d_conv), _ptr(cu_seqlens), _ptr(q), _ptr(k),
                                                 _ptr(v), _stream(stream)),
           "gdn_front_conv_silu_l2")


def gdn_workspace_layout(cfg: gdn_config) -> dict:
    """Byte offsets of the intermediates inside a workspace (and its total size)."""
    out = gdn_workspace_layout_t()
    _check(load_library().gdn_workspace_layout(ctypes.byref(cfg), ctypes.byref(out)),
           "gdn_workspace_layout")
    return {name: int(getattr(out, name)) for name, _ in gdn_workspace_layout_t._fields_}


def _ws_bytes(workspace, ws_bytes):
    if ws_bytes is not None:
        return int(ws_bytes)
    return workspace.numel() * workspace.element_size()


def gdn_chunk_fwd_intra(cfg, q, k, v, g, beta, cu_seqlens, chunk_indices, workspace,
                        ws_bytes=None, stream=None):
    _check_tensors(cfg, q=q, k=k, v=v, g=g, beta=beta, cu=cu_seqlens, table=chunk_indices)
    _check_ws(workspace, _ws_bytes(workspace, ws_bytes))
    _check(load_library().gdn_chunk_fwd_intra(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                              _ptr(chunk_indices), _ptr(workspace),
                                              _ws_bytes(workspace, ws_bytes), _stream(stream)),
           "gdn_chunk_fwd_intra")


def gdn_chunk_fwd_inter(cfg, h0, cu_seqlens, workspace, o, hT, ws_bytes=None, stream=None):
    _check_tensors(cfg, h0=h0, cu=cu_seqlens, o=o, hT=hT)
    _check_ws(workspace, _ws_bytes(workspace, ws_bytes))
    _check(load_library().gdn_chunk_fwd_inter(ctypes.byref(cfg), _ptr(h0), _ptr(cu_seqlens),
                                              _ptr(workspace), _ws_bytes(workspace, ws_bytes),
                                              _ptr(o), _ptr(hT), _stream(stream)),
           "gdn_chunk_fwd_inter")


def gdn_chunk_fwd(cfg, q, k, v, g, beta, h0, cu_seqlens, chunk_indices, o, hT, workspace,
                  ws_bytes=None, stream=None):
    ws_bytes = _ws_bytes(workspace, ws_bytes)
    _check_tensors(cfg, q, k, v, g, beta, h0, cu_seqlens, chunk_indices, o, hT)
    _check_ws(workspace, ws_bytes)
    _check(load_library().gdn_chunk_fwd(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                        _ptr(beta), _ptr(h0), _ptr(cu_seqlens),
                                        _ptr(chunk_indices), _ptr(o), _ptr(hT), _ptr(workspace),
                                        int(ws_bytes), _stream(stream)),
           "gdn_chunk_fwd")


def gdn_chunk_fwd_noalloc(cfg, q, k, v, g, beta, h0, cu_seqlens, chunk_indices, o, hT,
                          stream=None):
    """gdn_chunk_fwd with the intermediates in the library's fixed device
    scratch (no workspace argument; nothing is allocated)."""
    _check_tensors(cfg, q, k, v, g, beta, h0, cu_seqlens, chunk_indices, o, hT)
    _check(load_library().gdn_chunk_fwd_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v),
                                                _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu_seqlens),
                                                _ptr(chunk_indices), _ptr(o), _ptr(hT),
                                                _stream(stream)),
           "gdn_chunk_fwd_noalloc")


def gdn_chunk_fwd_timed(cfg, q, k, v, g, beta, h0, cu_seqlens, chunk_indices, o, hT, workspace,
                        events, ws_bytes=None, stream=None):
    """gdn_chunk_fwd whose kernels record `events` (six raw hipEvent_t handles,
    ints) at their own start and end: table, intra, inter."""
    ws_bytes = _ws_bytes(workspace, ws_bytes)
    _check_tensors(cfg, q, k, v, g, beta, h0, cu_seqlens, chunk_indices, o, hT)
    _check_ws(workspace, ws_bytes)
    if len(events) != 6:
        raise ValueError("six events expected")
    arr = (ctypes.c_void_p * 6)(*[int(e) for e in events])
    _check(load_library().gdn_chunk_fwd_timed(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu_seqlens),
                                              _ptr(chunk_indices), _ptr(o), _ptr(hT),
                                              _ptr(workspace), int(ws_bytes), _stream(stream),
                                              arr),
           "gdn_chunk_fwd_timed")


def gdn_front_conv_silu_l2_timed(cfg, qkv, conv_w, d_conv, cu_seqlens, q, k, v, ev_start, ev_stop,
                                 stream=None):
    _check_front(cfg, qkv, conv_w, d_conv)
    _check_tensors(make_config(cfg.t_max, cfg.n_max, cfg.h, cfg.hv, GDN_F32), q=q, k=k, v=v,
                   cu=cu_seqlens)
    _check(load_library().gdn_front_conv_silu_l2_timed(
        ctypes.byref(cfg), _ptr(qkv), _ptr(conv_w), int(d_conv), _ptr(cu_seqlens), _ptr(q),
        _ptr(k), _ptr(v), _stream(stream), int(ev_start), int(ev_stop)),
        "gdn_front_conv_silu_l2_timed")


def gdn_chunk_fwd_conv(cfg, qkv, conv_w, d_conv, g, beta, h0, cu_seqlens, chunk_indices, o, hT,
                       workspace, ws_bytes=None, stream=None):
    ws_bytes = _ws_bytes(workspace, ws_bytes)
    _check_front(cfg, qkv, conv_w, d_conv)
    _check_tensors(cfg, g=g, beta=beta, h0=h0, cu=cu_seqlens, table=chunk_indices, o=o, hT=hT)
    _check_ws(workspace, ws_bytes)
    _check(load_library().gdn_chunk_fwd_conv(ctypes.byref(cfg), _ptr(qkv), _ptr(conv_w),
                                             int(d_conv), _ptr(g), _ptr(beta), _ptr(h0),
                                             _ptr(cu_seqlens), _ptr(chunk_indices), _ptr(o),
                                             _ptr(hT), _ptr(workspace), int(ws_bytes),
                                             _stream(stream)),
           "gdn_chunk_fwd_conv")


def gdn_chunk_fwd_conv_timed(cfg, qkv, conv_w, d_conv, g, beta, h0, cu_seqlens, chunk_indices, o,
                             hT, workspace, events, ws_bytes=None, stream=None):
    """gdn_chunk_fwd_conv whose kernels record `events` (six raw hipEvent_t
    handles): table, intra (with the fused front), inter."""
    ws_bytes = _ws_bytes(workspace, ws_bytes)
    _check_front(cfg, qkv, conv_w, d_conv)
    _check_tensors(cfg, g=g, beta=beta, h0=h0, cu=cu_seqlens, table=chunk_indices, o=o, hT=hT)
    _check_ws(workspace, ws_bytes)
    if len(events) != 6:
        raise ValueError("six events expected")
    arr = (ctypes.c_void_p * 6)(*[int(e) for e in events])
    _check(load_library().gdn_chunk_fwd_conv_timed(ctypes.byref(cfg), _ptr(qkv), _ptr(conv_w),
                                                   int(d_conv), _ptr(g), _ptr(beta), _ptr(h0),
                                                   _ptr(cu_seqlens), _ptr(chunk_indices), _ptr(o),
                                                   _ptr(hT), _ptr(workspace), int(ws_bytes),
                                                   _stream(stream), arr),
           "gdn_chunk_fwd_conv_timed")


def gdn_recurrent_fwd(cfg, q, k, v, g, beta, h0, cu_seqlens, o, hT, stream=None):
    _check_tensors(cfg, q, k, v, g, beta, h0, cu_seqlens, None, o, hT)
    _check(load_library().gdn_recurrent_fwd(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                            _ptr(beta), _ptr(h0), _ptr(cu_seqlens), _ptr(o),
                                            _ptr(hT), _stream(stream)),
           "gdn_recurrent_fwd")


def gdn_recurrent_fwd_timed(cfg, q, k, v, g, beta, h0, cu_seqlens, o, hT, ev_start, ev_stop,
                            stream=None):
    """gdn_recurrent_fwd whose kernel records raw hipEvent_t handles at its start and end."""
    _check_tensors(cfg, q, k, v, g, beta, h0, cu_seqlens, None, o, hT)
    _check(load_library().gdn_recurrent_fwd_timed(
        ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
        _ptr(cu_seqlens), _ptr(o), _ptr(hT), _stream(stream), int(ev_start), int(ev_stop)),
        "gdn_recurrent_fwd_timed")


def _same_qkv_dtype(q, k, v):
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _TORCH_DTYPE:
        raise ValueError(f"q, k, v must share one dtype in (bfloat16, float32, float16): "
                         f"{q.dtype}, {k.dtype}, {v.dtype}")
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[0] != q.shape[0]:
        raise ValueError(f"q, k [T, H, 128] and v [T, Hv, 128] expected: {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")


def recurrent_gated_delta_rule(q, k, v, g, beta, cu_seqlens, initial_state=None,
                               output_final_state=True, scale=None, n_max=None):
    """Allocate outputs with torch and run gdn_recurrent_fwd (token-serial decode /
    verify) on the current stream. Arguments as chunk_gated_delta_rule, with
    q, k, v in bf16 or fp32 (the token-serial kernel takes no fp16)."""
    _same_qkv_dtype(q, k, v)
    T, H, _ = q.shape
    Hv = v.shape[1]
    n = cu_seqlens.numel() - 1 if n_max is None else n_max
    cfg = make_config(T, n, H, Hv, q.dtype, scale or 0.0)
    o = torch.empty((T, Hv, 128), dtype=torch.float32, device=q.device)
    hT = torch.empty((n, Hv, 128, 128), dtype=torch.float32, device=q.device) \
        if output_final_state else None
    gdn_recurrent_fwd(cfg, q, k, v, g, beta, initial_state, cu_seqlens, o, hT)
    return o, hT


def chunk_gated_delta_rule(q, k, v, g, beta, cu_seqlens, initial_state=None,
                           output_final_state=True, scale=None, chunk_indices=None,
                           workspace=None, n_max=None):
    """Allocate outputs with torch and run gdn_chunk_fwd on the current stream.

    q, k [T, H, 128] and v [T, Hv, 128] (bf16, fp16 or fp32, one dtype); g, beta
    [T, Hv] fp32; cu_seqlens int32 [N + 1] on the device; initial_state
    [N, Hv, 128, 128] fp32 or None. Returns (o [T, Hv, 128] fp32, final state
    or None).
    """
    _same_qkv_dtype(q, k, v)
    T, H, _ = q.shape
    Hv = v.shape[1]
    n = cu_seqlens.numel() - 1 if n_max is None else n_max
    cfg = make_config(T, n, H, Hv, q.dtype, scale or 0.0)
    if workspace is None:
        workspace = torch.empty(gdn_workspace_size(cfg), dtype=torch.uint8, device=q.device)
    o = torch.empty((T, Hv, 128), dtype=torch.float32, device=q.device)
    hT = torch.empty((n, Hv, 128, 128), dtype=torch.float32, device=q.device) \
        if output_final_state else None
    gdn_chunk_fwd(cfg, q, k, v, g, beta, initial_state, cu_seqlens, chunk_indices, o, hT,
                  workspace)
    return o, hT
