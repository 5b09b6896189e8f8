"""ctypes front end of the plain-C fp64 oracle (``gdn_oracle.c``).

Test infrastructure: see the package docstring. The shared library is built
with gcc by ``build()``; loading builds it once if it is missing.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build() -> str:
    """Compile gdn_oracle.c with gcc (-O3, OpenMP, no fast-math)."""
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    i32 = ctypes.c_int32
    lib.gdn_oracle_recurrent.argtypes = [dp, dp, dp, dp, dp, dp, ip, i32, i32, i32, i32,
                                         i32, ctypes.c_double, dp, dp]
    lib.gdn_oracle_recurrent.restype = None
    lib.gdn_oracle_front.argtypes = [dp, dp, i32, ip, i32, i32, i32, i32, i32,
                                     ctypes.c_double, dp]
    lib.gdn_oracle_front.restype = None
    lib.gdn_oracle_threads.argtypes = []
    lib.gdn_oracle_threads.restype = ctypes.c_int
    lib.gdn_oracle_set_threads.argtypes = [ctypes.c_int]
    lib.gdn_oracle_set_threads.restype = None
    _lib = lib
    return lib


def threads() -> int:
    """OpenMP threads the oracle's lane loop runs on."""
    return int(_load().gdn_oracle_threads())


def set_threads(n: int) -> None:
    """Run later oracle calls on n OpenMP threads."""
    _load().gdn_oracle_set_threads(int(n))


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if a is not None else None


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def gdn_recurrent(q, k, v, g, beta, cu_seqlens, h0=None, scale=None):
    """fp64 token recurrence (decay, correct, write, read), every lane.

    Source: Alloy page ("Chunking Qwen3.5's gated DeltaNet ..."), section
    "What is the gated delta rule in Qwen3.5?"; state layout of the AMX page,
    section 9 (value-major final state). Arrays:
      q, k [T, H, Dk]; v [T, Hv, Dv]; g, beta [T, Hv];
      h0 [N, Hv, Dv, Dk] or None; cu_seqlens [N + 1].
    Returns (o [T, Hv, Dv], hT [N, Hv, Dv, Dk]) in float64.
    """
    lib = _load()
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    T, H, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    assert k.shape == q.shape and v.shape[0] == T and g.shape == (T, Hv) == beta.shape
    assert Hv % H == 0
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    n = cu.shape[0] - 1
    assert cu[0] == 0 and np.all(np.diff(cu) >= 0) and cu[-1] <= T
    if scale is None:
        scale = 1.0 / np.sqrt(Dk)
    h0a = _f64(h0) if h0 is not None else None
    if h0a is not None:
        assert h0a.shape == (n, Hv, Dv, Dk)
    o = np.zeros((T, Hv, Dv), np.float64)
    hT = np.zeros((n, Hv, Dv, Dk), np.float64)
    lib.gdn_oracle_recurrent(_dptr(q), _dptr(k), _dptr(v), _dptr(g), _dptr(beta), _dptr(h0a),
                             cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n, H, Hv, Dk,
                             Dv, float(scale), _dptr(o), _dptr(hT))
    return o, hT


def gdn_front(x, conv_w, cu_seqlens, H, Hv, Dk, Dv, eps=1e-6):
    """fp64 causal depthwise conv + SiLU + per-head L2 norm of q and k.

    Source: llama.cpp PR 399 page, section "How (exactness)" (conv sum with the
    current token as the last tap, no bias) and the AMX page, section 7 (norm
    as x / sqrt(sum x^2 + eps)). x [T, 2*H*Dk + Hv*Dv]; conv_w [C, d_conv].
    Returns (q [T, H, Dk], k [T, H, Dk], v [T, Hv, Dv]) in float64.
    """
    lib = _load()
    x = _f64(x)
    w = _f64(conv_w)
    T, C = x.shape
    assert C == 2 * H * Dk + Hv * Dv and w.shape[0] == C
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    n = cu.shape[0] - 1
    y = np.zeros_like(x)
    lib.gdn_oracle_front(_dptr(x), _dptr(w), int(w.shape[1]),
                         cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n, H, Hv, Dk, Dv,
                         float(eps), _dptr(y))
    q = y[:, : H * Dk].reshape(T, H, Dk)
    k = y[:, H * Dk: 2 * H * Dk].reshape(T, H, Dk)
    vv = y[:, 2 * H * Dk:].reshape(T, Hv, Dv)
    return q, k, vv
