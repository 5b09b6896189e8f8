"""Pins for the CPU oracle: it is checked against exact arithmetic, closed forms
and an independent chunked evaluation, never against the HIP path.

Sources are the four pages on the chunked gated delta rule:
  * Alloy, "Chunking Qwen3.5's gated DeltaNet ..." -- the per-token rule
    ("What is the gated delta rule in Qwen3.5?") and the finite-series inverse
    ("How do you parallelize a recurrence for prefill?").
  * "Optimizing GDN Chunk Prefill on Intel AMX CPU" -- chunked formulas
    (sections 4 and 5), GQA grouping (section 4), state layout (section 9).
  * llama.cpp PR 399 -- conv sum and L2 norm ("How (exactness)").
  * FLA issue 1155 -- NT_max bound and chunk-index table ("Core design").
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import bruteforce, chunked, index_table, recurrent

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _relmax(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def _rand_inputs(rng, lengths, H, Hv, Dk, Dv, h0_sigma=0.0, g_mu=0.0):
    T = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q = rng.standard_normal((T, H, Dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, H, Dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Hv, Dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Hv))))
    g = -np.logaddexp(0, rng.standard_normal((T, Hv)) + g_mu)
    h0 = rng.standard_normal((len(lengths), Hv, Dv, Dk)) * h0_sigma if h0_sigma else None
    return q, k, v, g, beta, cu, h0


# --------------------------------------------------------------------------- #
# 1. Exact rational brute force (transition form) vs the fp64 recurrence.
# --------------------------------------------------------------------------- #

def test_bruteforce_hand_worked_scalar_case():
    # Dk = Dv = 1, two tokens, worked by hand from the four steps:
    # t=1: decay 0 -> 0; d = 1*(2 - 0) = 2; S = 0 + 1*2 = 2; o = 2.
    # t=2: decay 1*2 = 2; d = 1/2*(4 - 2*1) = 1; S = 2 + 1*1 = 3; o = 3.
    o, S = bruteforce.gdn_bruteforce(q=[[1], [1]], k=[[1], [1]], v=[[2], [4]],
                                     alpha=[Fraction(1, 2), 1], beta=[1, Fraction(1, 2)])
    assert o == [[2], [3]] and S == [[3]]


def _rational_lane(rng, T, D):
    vals = lambda n: [Fraction(int(x), 8) for x in rng.integers(-8, 9, size=n)]
    q = [vals(D) for _ in range(T)]
    k = [vals(D) for _ in range(T)]
    v = [vals(D) for _ in range(T)]
    alpha = [Fraction(int(x), 16) for x in rng.integers(1, 17, size=T)]
    beta = [Fraction(int(x), 16) for x in rng.integers(0, 17, size=T)]
    S0 = [vals(D) for _ in range(D)]
    return q, k, v, alpha, beta, S0


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_matches_recurrent(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    D = 4
    lengths = [int(x) for x in rng.integers(0, 9, size=3)]
    H, Hv = 1, 2
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q = np.zeros((T, H, D)); k = np.zeros((T, H, D)); v = np.zeros((T, Hv, D))
    g = np.zeros((T, Hv)); b = np.zeros((T, Hv)); h0 = np.zeros((3, Hv, D, D))
    exact_o = np.zeros((T, Hv, D)); exact_S = np.zeros((3, Hv, D, D))
    lanes = {}
    for s in range(3):
        for hv in range(Hv):
            lanes[s, hv] = _rational_lane(rng, lengths[s], D)
    for s in range(3):
        bos = cu[s]
        for hv in range(Hv):
            ql, kl, vl, al, bl, S0 = lanes[s, hv]
            if hv == 0:  # both value heads share key head 0 (H=1): use lane 0's q/k
                qk = (ql, kl)
            ql, kl = qk
            for t in range(lengths[s]):
                q[bos + t, 0] = [float(x) for x in ql[t]]
                k[bos + t, 0] = [float(x) for x in kl[t]]
                v[bos + t, hv] = [float(x) for x in vl[t]]
                g[bos + t, hv] = math.log(al[t])
                b[bos + t, hv] = float(bl[t])
            h0[s, hv] = np.array([[float(S0[i][j]) for i in range(D)] for j in range(D)])
            o_ex, S_ex = bruteforce.gdn_bruteforce(ql, kl, vl, al, bl, S0, scale=Fraction(1, 2))
            for t in range(lengths[s]):
                exact_o[bos + t, hv] = [float(x) for x in o_ex[t]]
            exact_S[s, hv] = np.array([[float(S_ex[i][j]) for i in range(D)] for j in range(D)])
    o, hT = recurrent.gdn_recurrent(q, k, v, g, b, cu, h0=h0, scale=0.5)
    assert np.allclose(o, exact_o, rtol=0, atol=1e-13 * max(1, np.abs(exact_o).max()))
    assert np.allclose(hT, exact_S, rtol=0, atol=1e-13 * max(1, np.abs(exact_S).max()))


def test_bruteforce_rejects_planted_mistakes():
    """Mistakes planted in a NumPy copy of the step form are caught by the
    exact brute force: correction before decay, reading before writing, a
    flipped sign in the correction, and the state read transposed."""
    rng = np.random.Generator(np.random.PCG64(7))
    T, D = 6, 4
    ql, kl, vl, al, bl, S0 = _rational_lane(rng, T, D)
    o_ex, _ = bruteforce.gdn_bruteforce(ql, kl, vl, al, bl, S0)
    f = lambda M: np.array([[float(x) for x in r] for r in M])
    q, k, v, S_init = f(ql), f(kl), f(vl), f(S0)

    def step_form(order):
        S = S_init.copy(); outs = []
        for t in range(T):
            a, b = float(al[t]), float(bl[t])
            if order == "correct_then_decay":
                d = b * (v[t] - S.T @ k[t]); S = a * S + np.outer(k[t], d)
                outs.append(S.T @ q[t])
            elif order == "read_before_write":
                S = a * S; outs.append(S.T @ q[t])
                d = b * (v[t] - S.T @ k[t]); S = S + np.outer(k[t], d)
            elif order == "flipped_sign":
                S = a * S; d = b * (v[t] + S.T @ k[t]); S = S + np.outer(k[t], d)
                outs.append(S.T @ q[t])
            elif order == "transposed_read":
                S = a * S; d = b * (v[t] - S.T @ k[t]); S = S + np.outer(k[t], d)
                outs.append(S @ q[t])
            else:
                S = a * S; d = b * (v[t] - S.T @ k[t]); S = S + np.outer(k[t], d)
                outs.append(S.T @ q[t])
        return np.array(outs)

    exact = f(o_ex)
    assert _relmax(step_form("right"), exact) < 1e-13
    assert _relmax(step_form("correct_then_decay"), exact) > 1e-3
    assert _relmax(step_form("read_before_write"), exact) > 1e-3
    assert _relmax(step_form("flipped_sign"), exact) > 1e-3
    assert _relmax(step_form("transposed_read"), exact) > 1e-3


# --------------------------------------------------------------------------- #
# 2. Closed forms on the full-size recurrence (Dk = Dv = 128).
# --------------------------------------------------------------------------- #

def test_no_decay_no_write_keeps_state(rng):
    q, k, v, g, b, cu, h0 = _rand_inputs(rng, [37, 5], 1, 2, 128, 128, h0_sigma=0.1)
    g[:] = 0.0; b[:] = 0.0
    o, hT = recurrent.gdn_recurrent(q, k, v, g, b, cu, h0=h0)
    assert np.array_equal(hT, h0)
    for s in range(2):
        for t in range(cu[s], cu[s + 1]):
            for hv in range(2):
                ref = h0[s, hv] @ q[t, 0] / np.sqrt(128)
                assert _relmax(o[t, hv], ref) < 1e-13


def test_single_token_from_zero_state(rng):
    q, k, v, g, b, cu, _ = _rand_inputs(rng, [1, 1, 1], 2, 4, 128, 128)
    o, hT = recurrent.gdn_recurrent(q, k, v, g, b, cu)
    for t in range(3):
        for hv in range(4):
            h = hv // 2
            assert _relmax(hT[t, hv], b[t, hv] * np.outer(v[t, hv], k[t, h])) < 1e-14
            ref = b[t, hv] * (q[t, h] @ k[t, h]) * v[t, hv] / np.sqrt(128)
            assert _relmax(o[t, hv], ref) < 1e-13


def test_unit_write_with_onehot_key_returns_value(rng):
    q, k, v, g, b, cu, h0 = _rand_inputs(rng, [50], 1, 1, 128, 128, h0_sigma=0.3)
    idx = rng.integers(0, 128, size=50)
    k[:] = 0.0; k[np.arange(50), 0, idx] = 1.0
    q[:] = k
    b[:] = 1.0
    o, _ = recurrent.gdn_recurrent(q, k, v, g, b, cu, h0=h0, scale=0.25)
    assert _relmax(o, 0.25 * v) < 1e-14


def test_full_forgetting_limit(rng):
    q, k, v, g, b, cu, h0 = _rand_inputs(rng, [9], 1, 1, 128, 128, h0_sigma=0.3)
    g[:] = -np.inf
    o, hT = recurrent.gdn_recurrent(q, k, v, g, b, cu, h0=h0)
    ref = b[:, 0, None] * np.einsum("td,td->t", q[:, 0], k[:, 0])[:, None] * v[:, 0] / np.sqrt(128)
    assert _relmax(o[:, 0], ref) < 1e-13
    assert _relmax(hT[0, 0], b[-1, 0] * np.outer(v[-1, 0], k[-1, 0])) < 1e-14


def test_linear_in_values_and_initial_state(rng):
    q, k, v1, g, b, cu, h1 = _rand_inputs(rng, [40, 24], 1, 2, 128, 128, h0_sigma=0.2)
    v2 = rng.standard_normal(v1.shape); h2 = rng.standard_normal(h1.shape) * 0.2
    o1, s1 = recurrent.gdn_recurrent(q, k, v1, g, b, cu, h0=h1)
    o2, s2 = recurrent.gdn_recurrent(q, k, v2, g, b, cu, h0=h2)
    o3, s3 = recurrent.gdn_recurrent(q, k, 2 * v1 - 3 * v2, g, b, cu, h0=2 * h1 - 3 * h2)
    assert _relmax(o3, 2 * o1 - 3 * o2) < 1e-12
    assert _relmax(s3, 2 * s1 - 3 * s2) < 1e-12


def test_value_column_permutation(rng):
    q, k, v, g, b, cu, h0 = _rand_inputs(rng, [33], 1, 1, 128, 128, h0_sigma=0.2)
    perm = rng.permutation(128)
    o, hT = recurrent.gdn_recurrent(q, k, v, g, b, cu, h0=h0)
    op, hTp = recurrent.gdn_recurrent(q, k, v[:, :, perm], g, b, cu, h0=h0[:, :, perm, :])
    assert np.array_equal(op, o[:, :, perm])
    assert np.array_equal(hTp, hT[:, :, perm, :])


def test_gqa_pairs_value_head_with_key_head_hv_div_group(rng):
    """AMX page s.4: value head hv uses key head hv // (Hv/H) (not hv mod H)."""
    q, k, v, g, b, cu, h0 = _rand_inputs(rng, [30], 2, 4, 128, 128, h0_sigma=0.1)
    o, hT = recurrent.gdn_recurrent(q, k, v, g, b, cu, h0=h0)
    qr, kr = np.repeat(q, 2, axis=1), np.repeat(k, 2, axis=1)  # [h0 h0 h1 h1]
    o2, hT2 = recurrent.gdn_recurrent(qr, kr, v, g, b, cu, h0=h0)
    assert np.array_equal(o, o2) and np.array_equal(hT, hT2)
    qt, kt = np.tile(q, (1, 2, 1)), np.tile(k, (1, 2, 1))      # [h0 h1 h0 h1]
    o3, _ = recurrent.gdn_recurrent(qt, kt, v, g, b, cu, h0=h0)
    assert not np.allclose(o, o3)


def test_sequences_in_a_pack_are_independent(rng):
    q, k, v, g, b, cu, h0 = _rand_inputs(rng, [20, 0, 45, 7], 1, 2, 128, 128, h0_sigma=0.1)
    o, hT = recurrent.gdn_recurrent(q, k, v, g, b, cu, h0=h0)
    for s in range(4):
        a, e = cu[s], cu[s + 1]
        oa, ha = recurrent.gdn_recurrent(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e],
                                         np.array([0, e - a], np.int32), h0=h0[s:s + 1])
        assert np.array_equal(oa, o[a:e]) and np.array_equal(ha[0], hT[s])
    assert np.array_equal(hT[1], h0[1])  # empty sequence keeps its state


# --------------------------------------------------------------------------- #
# 3. Chunked form (AMX page s.4-5) vs the token recurrence, for every chunk size.
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("C", [1, 2, 4, 8, 16, 32, 64, 128])
def test_chunked_form_is_invariant_to_chunk_size(rng, C):
    q, k, v, g, b, cu, h0 = _rand_inputs(rng, [150, 1, 64, 0, 77], 2, 4, 16, 12, h0_sigma=0.3)
    o_r, s_r = recurrent.gdn_recurrent(q, k, v, g, b, cu, h0=h0)
    o_c, s_c = chunked.gdn_chunked(q, k, v, g, b, cu, h0=h0, chunk=C)
    assert _relmax(o_c, o_r) < 1e-12
    assert _relmax(s_c, s_r) < 1e-12


def test_chunked_form_full_width_strong_decay(rng):
    q, k, v, g, b, cu, h0 = _rand_inputs(rng, [130, 64], 1, 2, 128, 128, h0_sigma=0.02, g_mu=2.0)
    o_r, s_r = recurrent.gdn_recurrent(q, k, v, g, b, cu, h0=h0)
    o_c, s_c = chunked.gdn_chunked(q, k, v, g, b, cu, h0=h0, chunk=64)
    assert _relmax(o_c, o_r) < 1e-12 and _relmax(s_c, s_r) < 1e-12


def test_chunked_form_weak_decay(rng):
    q, k, v, g, b, cu, h0 = _rand_inputs(rng, [300], 1, 1, 32, 32, h0_sigma=0.5, g_mu=-6.0)
    o_r, s_r = recurrent.gdn_recurrent(q, k, v, g, b, cu, h0=h0)
    o_c, s_c = chunked.gdn_chunked(q, k, v, g, b, cu, h0=h0, chunk=64)
    assert _relmax(o_c, o_r) < 1e-11 and _relmax(s_c, s_r) < 1e-11


@pytest.mark.parametrize("mutation", ["no_diagonal", "exclusive_cumsum", "first_order_solve",
                                      "flipped_solve_sign", "transposed_decay_mask"])
def test_chunked_pins_reject_planted_mistakes(rng, monkeypatch, mutation):
    q, k, v, g, b, cu, h0 = _rand_inputs(rng, [100], 1, 1, 16, 16, h0_sigma=0.3)
    o_r, _ = recurrent.gdn_recurrent(q, k, v, g, b, cu, h0=h0)
    if mutation == "no_diagonal":
        orig = chunked.decay_mask
        monkeypatch.setattr(chunked, "decay_mask",
                            lambda gm: orig(gm) - np.diag(np.diag(orig(gm))))
    elif mutation == "exclusive_cumsum":
        monkeypatch.setattr(chunked, "chunk_local_cumsum",
                            lambda gc: np.concatenate([[0.0], np.cumsum(gc)[:-1]]))
    elif mutation == "first_order_solve":
        monkeypatch.setattr(chunked, "solve_unit_lower", lambda A: np.eye(A.shape[0]) - A)
    elif mutation == "flipped_solve_sign":  # (I - A)^-1 instead of (I + A)^-1
        orig = chunked.solve_unit_lower
        monkeypatch.setattr(chunked, "solve_unit_lower", lambda A: orig(-A))
    else:
        orig = chunked.decay_mask
        monkeypatch.setattr(chunked, "decay_mask", lambda gm: orig(gm).T)
    o_c, _ = chunked.gdn_chunked(q, k, v, g, b, cu, h0=h0, chunk=16)
    assert _relmax(o_c, o_r) > 1e-4


def test_series_inverse_matches_forward_substitution(rng):
    q, k, v, g, b, cu, _ = _rand_inputs(rng, [64], 1, 1, 128, 128)
    gamma = chunked.chunk_local_cumsum(g[:, 0])
    A = np.tril(b[:, 0, None] * (k[:, 0] @ k[:, 0].T) * chunked.decay_mask(gamma), k=-1)
    T1 = chunked.solve_unit_lower(A)
    T2 = chunked.series_inverse(A)
    assert np.max(np.abs(T1 - T2)) < 1e-13
    assert np.max(np.abs((np.eye(64) + A) @ T1 - np.eye(64))) < 1e-14
    assert np.array_equal(np.triu(T1, 1), np.zeros((64, 64)))
    assert np.array_equal(np.diag(T1), np.ones(64))


def test_decay_mask_never_overflows_under_strong_decay():
    gamma = np.cumsum(np.full(64, -40.0))  # gamma reaches -2560
    G = chunked.decay_mask(gamma)
    assert np.all(np.isfinite(G)) and np.array_equal(np.diag(G), np.ones(64))
    assert np.array_equal(np.triu(G, 1), np.zeros((64, 64)))


# --------------------------------------------------------------------------- #
# 4. Front: causal depthwise conv + SiLU + L2 norm (llama.cpp PR 399; AMX s.7).
# --------------------------------------------------------------------------- #

def _front_inputs(rng, lengths, H=1, Hv=1, D=8, d_conv=4):
    C = 2 * H * D + Hv * D
    T = sum(lengths)
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, d_conv)) * 0.5
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return x, w, cu, C


def _silu(x):
    return x / (1 + np.exp(-x))


def test_front_matches_numpy_convolve(rng):
    H, Hv, D = 1, 2, 8
    x, w, cu, C = _front_inputs(rng, [11, 3, 20], H, Hv, D)
    q, k, v = recurrent.gdn_front(x, w, cu, H, Hv, D, D)
    y = np.zeros_like(x)
    for s in range(3):
        a, e = cu[s], cu[s + 1]
        for c in range(C):
            y[a:e, c] = _silu(np.convolve(x[a:e, c], w[c, ::-1])[: e - a])
    qr = y[:, :H * D].reshape(-1, H, D); kr = y[:, H * D:2 * H * D].reshape(-1, H, D)
    qr = qr / np.sqrt((qr ** 2).sum(-1, keepdims=True) + 1e-6)
    kr = kr / np.sqrt((kr ** 2).sum(-1, keepdims=True) + 1e-6)
    assert _relmax(q, qr) < 1e-14 and _relmax(k, kr) < 1e-14
    assert _relmax(v, y[:, 2 * H * D:].reshape(-1, Hv, D)) < 1e-14


def test_front_identity_and_delay_taps(rng):
    H, Hv, D = 1, 1, 8
    x, _, cu, C = _front_inputs(rng, [10], H, Hv, D)
    w_id = np.zeros((C, 4)); w_id[:, 3] = 1.0
    _, _, v = recurrent.gdn_front(x, w_id, cu, H, Hv, D, D)
    assert _relmax(v[:, 0], _silu(x[:, 2 * D:])) < 1e-15
    w_del = np.zeros((C, 4)); w_del[:, 0] = 1.0
    _, _, v = recurrent.gdn_front(x, w_del, cu, H, Hv, D, D)
    assert np.array_equal(v[:3, 0], np.zeros((3, D)))
    assert _relmax(v[3:, 0], _silu(x[:-3, 2 * D:])) < 1e-15


def test_front_silu_closed_forms(rng):
    """SiLU inside the front, pinned without restating it: with the identity
    tap the v channels are SiLU(x) exactly, so SiLU(0) = 0, SiLU(x) - SiLU(-x)
    = x, SiLU(x) + SiLU(-x) = x tanh(x / 2), SiLU(1) = sigmoid(1) and
    SiLU(-1) = -sigmoid(-1) (textbook values), and SiLU(x) -> x, SiLU(-x) -> 0
    for large x."""
    H, Hv, D = 1, 1, 8
    C = 2 * H * D + Hv * D
    w_id = np.zeros((C, 4)); w_id[:, 3] = 1.0

    def silu_of(vals):  # the oracle front's v channels for inputs `vals`
        x = np.zeros((len(vals), C))
        x[:, 2 * D:] = np.asarray(vals, np.float64)[:, None]
        cu = np.arange(len(vals) + 1, dtype=np.int32)  # one token per sequence
        _, _, v = recurrent.gdn_front(x, w_id, cu, H, Hv, D, D)
        return v[:, 0, 0]

    xs = rng.standard_normal(64) * 3
    pos, neg = silu_of(xs), silu_of(-xs)
    assert silu_of([0.0])[0] == 0.0
    assert np.max(np.abs((pos - neg) - xs)) < 4e-15 * np.max(np.abs(xs))
    assert np.max(np.abs((pos + neg) - xs * np.tanh(xs / 2))) < 4e-15 * np.max(np.abs(xs))
    one = silu_of([1.0, -1.0])
    assert abs(one[0] - 0.7310585786300049) < 1e-15  # 1 / (1 + e^-1)
    assert abs(one[1] + 0.2689414213699951) < 1e-15  # -1 / (1 + e)
    big = silu_of([40.0, -40.0])
    assert big[0] == 40.0 and 0.0 > big[1] > -1e-15


def test_front_unit_norm_heads(rng):
    x, w, cu, C = _front_inputs(rng, [40], 2, 2, 128)
    q, k, _ = recurrent.gdn_front(x, w, cu, 2, 2, 128, 128)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1, atol=1e-5)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1, atol=1e-5)


# --------------------------------------------------------------------------- #
# 5. Chunk-index table and static bound (FLA issue 1155, "Core design").
# --------------------------------------------------------------------------- #

def test_static_bound_reproduces_page_memory_estimate():
    with open(os.path.join(GOLDEN, "p4_static_bound.json")) as f:
        fx = json.load(f)
    nt = index_table.nt_max(fx["t_max"], fx["n_max"], fx["chunk"])
    per_chunk = fx["k"] * fx["v"] * 4
    assert per_chunk == 64 * 1024  # "64 KB per head per chunk"
    resident = nt * fx["heads"] * per_chunk
    assert abs(resident / 2 ** 20 - fx["resident_page_mb"]) < 0.5  # "~190 MB"


def _table_by_searchsorted(cu, nt_cap, chunk=64):
    """Second algorithm: slot j -> sequence by searchsorted over chunk offsets."""
    cu = np.asarray(cu, np.int64)
    nc = -(-(cu[1:] - cu[:-1]) // chunk)
    co = np.concatenate([[0], np.cumsum(nc)])
    out = np.full((nt_cap, 2), -1, np.int64)
    j = np.arange(co[-1])
    s = np.searchsorted(co, j, side="right") - 1
    out[: co[-1], 0] = s
    out[: co[-1], 1] = j - co[s]
    return out


@pytest.mark.parametrize("seed", range(20))
def test_index_table_two_algorithms_and_bound(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    n_max = int(rng.integers(1, 40))
    n = int(rng.integers(0, n_max + 1))
    lengths = rng.integers(0, 300, size=n)
    lengths[rng.random(n) < 0.2] = 0
    edge = np.array([1, 63, 64, 65, 128, 129])
    lengths = np.where(rng.random(n) < 0.3, edge[rng.integers(0, 6, size=n)], lengths)
    cu = [0] + list(np.cumsum(lengths)) + [int(lengths.sum())] * (n_max - n)
    t_max = int(lengths.sum()) + int(rng.integers(0, 100))
    cap = index_table.nt_max(t_max, n_max)
    assert index_table.chunk_count(cu) <= cap
    tab = np.array(index_table.chunk_index_table(cu, cap))
    assert np.array_equal(tab, _table_by_searchsorted(cu, cap))


def test_static_bound_is_tight():
    # every sequence one token past a chunk boundary: T = 64a + N gives a + N chunks
    n_max = 5
    t_max = 64 * 10 + n_max
    lengths = [1] + [64 + 1] * (n_max - 1)
    lengths[-1] += t_max - sum(lengths)
    cu = [0] + list(np.cumsum(lengths))
    assert sum(lengths) == t_max
    assert index_table.chunk_count(cu) == index_table.nt_max(t_max, n_max)
