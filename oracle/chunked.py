"""fp64 NumPy evaluation of the chunked (intra-chunk / inter-chunk) form.

Test infrastructure: see the package docstring. This is a second, independent
route to the same result as the token recurrence; the tests require the two to
agree for every chunk size C, which pins both.

Source: "Optimizing GDN Chunk Prefill on Intel AMX CPU".
  * Section 4 (intra stage, per chunk and key head): attn = K K^T once, then per
    value head of the GQA group a beta- and decay-masked copy, a triangular
    solve, and w = solve @ (K * beta * exp(g)), u = solve @ (V * beta).
  * Section 5 (inter stage, per sequence and value head, chunks in order):
    v' = u - w @ S; inter = (q * exp(g)) @ S; o = local_attn @ v' + inter;
    S = S * exp(g_last) + (k * exp(g_last - g))^T @ v'.
  * g is the chunk-local cumulative sum of the log decay (the wrapper's
    chunk_local_cumsum, section 3).
Readings where the page text is garbled (its equations were stripped):
  * A = strict_lower(diag(beta) (K K^T * Gamma)), T = (I + A)^-1, with
    Gamma[r, i] = exp(gamma_r - gamma_i) for i <= r and 0 above the diagonal;
    beta scales rows. This is the only sign and side that reproduces the token
    recurrence.
  * local_attn = tril(Q K^T * Gamma) with the diagonal included (the output is
    read after the token's own write), scaled by `scale` together with the
    inter term.
  * Gamma is formed from a masked difference, so no exp of a large positive
    number is ever taken.
The triangular solve is plain forward substitution (one row after another).
"""

from __future__ import annotations

import numpy as np


def chunk_local_cumsum(g_chunk: np.ndarray) -> np.ndarray:
    """Cumulative sum of the log decay inside one chunk (AMX page, section 3)."""
    return np.cumsum(g_chunk, axis=0)


def decay_mask(gamma: np.ndarray) -> np.ndarray:
    """Gamma[r, i] = exp(gamma_r - gamma_i) for i <= r, else 0 (AMX page, s.4 and s.8)."""
    c = gamma.shape[0]
    diff = gamma[:, None] - gamma[None, :]
    lower = np.tril(np.ones((c, c), dtype=bool))
    out = np.zeros((c, c))
    out[lower] = np.exp(diff[lower])
    return out


def solve_unit_lower(A: np.ndarray) -> np.ndarray:
    """T = (I + A)^-1 for strictly lower triangular A, by forward substitution.

    Row r of T: T[r] = e_r - sum_{i<r} A[r, i] T[i]  (AMX page, section 4,
    the solve_tril step).
    """
    c = A.shape[0]
    T = np.zeros((c, c))
    for r in range(c):
        T[r, r] = 1.0
        for i in range(r):
            T[r] -= A[r, i] * T[i]
    return T


def intra_chunk(Kc, Vc, gc, bc):
    """Intra stage for one chunk and one value head (AMX page, section 4).

    Kc [C, Dk], Vc [C, Dv], gc, bc [C] (log decay and beta of the tokens).
    Returns (w [C, Dk], u [C, Dv], gamma [C], Gamma [C, C]).
    """
    gamma = chunk_local_cumsum(gc)
    Gam = decay_mask(gamma)
    attn = Kc @ Kc.T
    A = np.tril(bc[:, None] * attn * Gam, k=-1)
    T = solve_unit_lower(A)
    w = T @ (Kc * (bc * np.exp(gamma))[:, None])
    u = T @ (Vc * bc[:, None])
    return w, u, gamma, Gam


def local_attention(Qc, Kc, Gam):
    """tril(Q K^T * Gamma), diagonal kept: the intra-chunk attention of the
    output (AMX page, section 5), before the output scale."""
    return np.tril(Qc @ Kc.T * Gam)


def inter_chunk(Qc, Kc, w, u, gamma, Gam, S, scale):
    """Inter stage step for one chunk (AMX page, section 5). S is [Dk, Dv]."""
    v_prime = u - w @ S
    attn_inter = (Qc * np.exp(gamma)[:, None]) @ S
    local_attn = local_attention(Qc, Kc, Gam)
    o = scale * (local_attn @ v_prime + attn_inter)
    g_last = gamma[-1]
    S_new = S * np.exp(g_last) + (Kc * np.exp(g_last - gamma)[:, None]).T @ v_prime
    return o, S_new


def gdn_chunked(q, k, v, g, beta, cu_seqlens, h0=None, scale=None, chunk=64,
                return_wu=False, stages=None):
    """Chunked-form forward over a packed varlen batch, every (seq, value head).

    Same array conventions as ``oracle.recurrent.gdn_recurrent``. A sequence's
    last chunk may be partial; it is evaluated at its real length (which is
    what zero-padding g and beta past the end would also give).
    With return_wu, also returns w, u as [Hv, T, D] arrays (the intra stage's
    outputs, indexed by token). A dict passed as `stages` receives, per
    (value head, chunk start token), the chunk's gamma and local attention.
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, H, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    HG = Hv // H
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = cu.shape[0] - 1
    if scale is None:
        scale = 1.0 / np.sqrt(Dk)
    o = np.zeros((T, Hv, Dv))
    hT = np.zeros((n, Hv, Dv, Dk))
    W = np.zeros((Hv, T, Dk)) if return_wu else None
    U = np.zeros((Hv, T, Dv)) if return_wu else None
    for s in range(n):
        bos, eos = int(cu[s]), int(cu[s + 1])
        for hv in range(Hv):
            h = hv // HG
            S = np.zeros((Dk, Dv)) if h0 is None else np.array(h0[s, hv], dtype=np.float64).T
            for t0 in range(bos, eos, chunk):
                t1 = min(t0 + chunk, eos)
                Kc, Qc = k[t0:t1, h], q[t0:t1, h]
                w, u, gamma, Gam = intra_chunk(Kc, v[t0:t1, hv], g[t0:t1, hv], beta[t0:t1, hv])
                if return_wu:
                    W[hv, t0:t1] = w
                    U[hv, t0:t1] = u
                if stages is not None:
                    stages[(hv, t0)] = (gamma, local_attention(Qc, Kc, Gam))
                o[t0:t1, hv], S = inter_chunk(Qc, Kc, w, u, gamma, Gam, S, scale)
            hT[s, hv] = S.T
    if return_wu:
        return o, hT, W, U
    return o, hT


def series_inverse(A: np.ndarray) -> np.ndarray:
    """(I + A)^-1 for strictly lower A via the finite series, evaluated by
    repeated squaring: prod_j (I + (-A)^(2^j)) over ceil(log2 C) rounds.

    Source: Alloy page, section "How do you parallelize a recurrence for
    prefill?": a strictly triangular in-chunk matrix is nilpotent (A^C = 0), so
    the inverse is a finite series evaluated in log2(C) rounds.
    """
    c = A.shape[0]
    P = -A
    T = np.eye(c)
    span = 1
    while span < c:
        T = T @ (np.eye(c) + P)
        P = P @ P
        span *= 2
    return T
