"""Exact rational brute force of the gated delta rule on tiny inputs.

Test infrastructure: see the package docstring.

It uses the per-token *transition* form, derived once by hand from the four
steps of the Alloy page ("What is the gated delta rule in Qwen3.5?"):
decay by alpha_t = exp(g_t), correction d = beta_t (v_t - (alpha_t S)^T k_t),
write S + k_t d^T. Collecting terms gives

    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
    o_t = scale * S_t^T q_t,

an affine map per token (a product of transition matrices plus a rank-one
input), which is a different arithmetic route from the oracle's step-by-step
update. Everything is a ``fractions.Fraction``; alpha_t is supplied directly
as a rational in [0, 1] (alpha_t = 0 is the g = -inf limit), so no
transcendental function is involved and the result is exact.

Matrices are lists of lists; S is [Dk][Dv] (key rows, value columns).
"""

from __future__ import annotations

from fractions import Fraction


def _zeros(r, c):
    return [[Fraction(0)] * c for _ in range(r)]


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def gdn_bruteforce(q, k, v, alpha, beta, S0=None, scale=Fraction(1)):
    """One lane: q, k [T][Dk], v [T][Dv], alpha, beta [T], S0 [Dk][Dv] or None.

    Returns (o [T][Dv], S_T [Dk][Dv]) as Fractions.
    """
    T = len(q)
    Dk = len(k[0]) if T else (len(S0) if S0 else 0)
    Dv = len(v[0]) if T else (len(S0[0]) if S0 else 0)
    S = [row[:] for row in S0] if S0 is not None else _zeros(Dk, Dv)
    outs = []
    for t in range(T):
        kt, vt, qt = k[t], v[t], q[t]
        a, b = Fraction(alpha[t]), Fraction(beta[t])
        # M = alpha (I - beta k k^T)
        M = [[a * ((1 if i == j else 0) - b * kt[i] * kt[j]) for j in range(Dk)] for i in range(Dk)]
        S = _matmul(M, S)
        for i in range(Dk):
            for j in range(Dv):
                S[i][j] += b * kt[i] * vt[j]
        outs.append([scale * sum((S[i][j] * qt[i] for i in range(Dk)), Fraction(0))
                     for j in range(Dv)])
    return outs, S
