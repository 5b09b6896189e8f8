"""Seeded synthetic inputs for the GDN chunk-prefill forward.

This module only draws random numbers and rounds them to the input dtype; it
holds none of the method's arithmetic. Both the HIP path (through the tests
and the benchmark) and the CPU oracle consume the same arrays from here.

Recipe (fixed draw order, NumPy PCG64, seed = workload number unless given):
lengths -> q -> k -> v -> beta-normal -> g-normal -> h0 -> conv weights.
Values are drawn in float64, shaped as stated, then rounded to nearest-even
into the input dtype (bf16 or fp32); g and beta are fp32; the oracle reads
the rounded values exactly.

  q, k      N(0, 1) per element, then each head vector divided by its 2-norm
  v         N(0, 1)
  beta      sigmoid(N(0, 1))
  g         -softplus(N(mu_g, 1)), mu_g = 0 (2 for the long-context workload)
  h0        N(0, sigma_h0) fp32, value-major [N_max, Hv, Dv, Dk], or none
  front     pre-conv q|k|v channels N(0, 1) bf16, conv weights N(0, 0.5) bf16

The named workloads are the ones the benchmark and the parity tests use (0-4
for the chunked prefill; 5 and 6 for the token-serial decode / verify kernel):
  0 tiny dense     N=1,  T=256,  H=Hv=2,            fp32 q/k/v
  1 single seq     N=1,  T=4096, H=16, Hv=32,       bf16
  2 varlen batch   N=32, lengths U{1..1024}, H=16, Hv=32, bf16, h0 ~ N(0, 0.02),
                   T_max=32768, N_max=32
  3 long context   N=1,  T=32768, H=Hv=16, bf16, g mean 2, h0 ~ N(0, 0.02)
  4 front + GDN    N=4 x 8192, H=16, Hv=32, d_conv=4; q/k/v come out of the
                   conv/SiLU/L2 front as fp32
  5 verify         N=64 sequences x 8 tokens (a draft-verify width), H=16, Hv=32,
                   bf16, h0 ~ N(0, 0.02)
  6 decode         N=256 sequences x 1 token, H=16, Hv=32, bf16, h0 ~ N(0, 0.02)
  7 long, 8 heads  N=1,  T=32768, H=Hv=8, bf16, g mean 2, h0 ~ N(0, 0.02): the
                   long-context recipe with fewer heads, whose stage-2 walk
                   fills a quarter of the device (the segmented walk's case)
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

D = 128
CHUNK = 64


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _unit_heads(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _round(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Round float64 -> dtype to nearest-even (via fp32 for bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t


@dataclass
class Workload:
    name: str
    cu_seqlens: np.ndarray          # int32 [n_max + 1], zero-length tail padding
    t_max: int
    n_max: int
    H: int
    Hv: int
    qkv_dtype: torch.dtype           # dtype of q/k/v as handed to the chunk forward
    q: Optional[torch.Tensor]        # [t_max, H, D]   (None when a front produces them)
    k: Optional[torch.Tensor]
    v: Optional[torch.Tensor]        # [t_max, Hv, D]
    g: torch.Tensor                  # [t_max, Hv] fp32
    beta: torch.Tensor               # [t_max, Hv] fp32
    h0: Optional[torch.Tensor]       # [n_max, Hv, D, D] fp32 or None
    qkv: Optional[torch.Tensor] = None     # [t_max, 2*H*D + Hv*D] bf16 (front input)
    conv_w: Optional[torch.Tensor] = None  # [2*H*D + Hv*D, d_conv] bf16
    d_conv: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_seqs(self) -> int:
        return int(np.count_nonzero(np.diff(self.cu_seqlens) > 0))

    def f64(self, name: str) -> Optional[np.ndarray]:
        t = getattr(self, name)
        return None if t is None else t.to(torch.float64).numpy()


def make_custom(lengths, H, Hv, *, seed=0, dtype=torch.bfloat16, t_max=None, n_max=None,
                g_mu=0.0, h0_sigma=0.0, front=False, d_conv=4, name="custom",
                g_scale=1.0, beta_mode="sigmoid") -> Workload:
    """General generator. lengths: per-sequence token counts (zeros allowed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(lengths, dtype=np.int64)
    n = len(lengths)
    n_max = n if n_max is None else n_max
    assert n_max >= n
    total = int(lengths.sum())
    t_max = total if t_max is None else t_max
    assert t_max >= total
    cu = np.zeros(n_max + 1, np.int32)
    cu[1: n + 1] = np.cumsum(lengths)
    cu[n + 1:] = total
    T = t_max

    def pad(a, rows):
        out = np.zeros((rows,) + a.shape[1:])
        out[: a.shape[0]] = a
        return out

    q = k = v = qkv = conv_w = None
    if not front:
        q = _round(pad(_unit_heads(rng.standard_normal((total, H, D))), T), dtype)
        k = _round(pad(_unit_heads(rng.standard_normal((total, H, D))), T), dtype)
        v = _round(pad(rng.standard_normal((total, Hv, D)), T), dtype)
    else:
        C = 2 * H * D + Hv * D
        qkv = _round(pad(rng.standard_normal((total, C)), T), torch.bfloat16)
    if beta_mode == "sigmoid":
        beta = _sigmoid(rng.standard_normal((total, Hv)))
    else:
        beta = np.full((total, Hv), float(beta_mode))
        rng.standard_normal((total, Hv))
    g = -_softplus(rng.standard_normal((total, Hv)) + g_mu) * g_scale
    beta_t = _round(pad(beta, T), torch.float32)
    g_t = _round(pad(g, T), torch.float32)
    h0 = None
    if h0_sigma > 0:
        h0 = _round(rng.standard_normal((n_max, Hv, D, D)) * h0_sigma, torch.float32)
        h0[n:] = 0.0
    if front:
        C = 2 * H * D + Hv * D
        conv_w = _round(rng.standard_normal((C, d_conv)) * 0.5, torch.bfloat16)
        dtype = torch.float32
    return Workload(name=name, cu_seqlens=cu, t_max=t_max, n_max=n_max, H=H, Hv=Hv,
                    qkv_dtype=dtype, q=q, k=k, v=v, g=g_t, beta=beta_t, h0=h0, qkv=qkv,
                    conv_w=conv_w, d_conv=d_conv if front else 0)


NAMES = {
    0: "tiny-dense-T256-H2-Hv2-fp32",
    1: "single-seq-T4096-H16-Hv32-bf16",
    2: "varlen-32seq-U1..1024-H16-Hv32-bf16-h0",
    3: "long-T32768-H16-Hv16-bf16-strong-decay-h0",
    4: "front-4x8192-H16-Hv32-dconv4",
    5: "verify-64x8-H16-Hv32-bf16-h0",
    6: "decode-256x1-H16-Hv32-bf16-h0",
    7: "long-T32768-H8-Hv8-bf16-strong-decay-h0",
}


def make(cfg: int, seed: Optional[int] = None) -> Workload:
    """The named workloads (see the module docstring)."""
    s = cfg if seed is None else seed
    if cfg == 0:
        return make_custom([256], 2, 2, seed=s, dtype=torch.float32, name=NAMES[0])
    if cfg == 1:
        return make_custom([4096], 16, 32, seed=s, name=NAMES[1])
    if cfg == 2:
        rng = np.random.Generator(np.random.PCG64(s))
        lengths = rng.integers(1, 1024, size=32, endpoint=True)
        # the lengths draw comes first in the recipe; continue from a derived seed
        w = make_custom(lengths, 16, 32, seed=s + 1000, t_max=32768, n_max=32,
                        h0_sigma=0.02, name=NAMES[2])
        return w
    if cfg == 3:
        return make_custom([32768], 16, 16, seed=s, g_mu=2.0, h0_sigma=0.02, name=NAMES[3])
    if cfg == 4:
        return make_custom([8192] * 4, 16, 32, seed=s, front=True, d_conv=4, name=NAMES[4])
    if cfg == 5:
        return make_custom([8] * 64, 16, 32, seed=s, h0_sigma=0.02, name=NAMES[5])
    if cfg == 6:
        return make_custom([1] * 256, 16, 32, seed=s, h0_sigma=0.02, name=NAMES[6])
    if cfg == 7:
        return make_custom([32768], 8, 8, seed=s, g_mu=2.0, h0_sigma=0.02, name=NAMES[7])
    raise ValueError(cfg)
