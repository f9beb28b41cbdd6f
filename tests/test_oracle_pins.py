"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test ties the oracle to a hand-worked example, exact rational arithmetic of a
different algebraic form, a closed form, or an invariant of the method, chosen so
that a plausible slip (a dropped term, a wrong sign, index or transpose) fails at
least one of them.  ``test_planted_mistakes_are_caught`` plants such slips in the
oracle and checks exactly that.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import gdn_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng(1234)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(rng, T, Hq, Hv, dk, dv, s0_std=0.3):
    q = _unit(rng.standard_normal((T, Hq, dk)))
    k = _unit(rng.standard_normal((T, Hq, dk)))
    v = rng.standard_normal((T, Hv, dv))
    g = -np.logaddexp(0, rng.standard_normal((T, Hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Hv))))
    return q, k, v, g, beta


def _load_fixture(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = np.array([float(x) for x in rest])
    return vals


# --------------------------------------------------------------------------- #
# 1. hand-worked example (tests/golden/hand_worked_two_tokens.txt)
# --------------------------------------------------------------------------- #
def check_hand_worked():
    fx = _load_fixture("hand_worked_two_tokens.txt")
    dk, dv = int(fx["dk"][0]), int(fx["dv"][0])
    k = fx["k"].reshape(2, 1, dk)
    v = fx["v"].reshape(2, 1, dv)
    q = fx["q"].reshape(2, 1, dk)
    g = np.log(fx["alpha"]).reshape(2, 1)
    beta = fx["beta"].reshape(2, 1)
    r = oracle.recurrent(q, k, v, g, beta, float(fx["scale"][0]), 1, 1)
    np.testing.assert_allclose(r["o"].reshape(-1), fx["o"], atol=1e-12)
    np.testing.assert_allclose(r["delta"].reshape(-1), fx["delta"], atol=1e-12)
    np.testing.assert_allclose(r["final"].reshape(-1), fx["final"], atol=1e-12)


def test_hand_worked_example():
    check_hand_worked()


# --------------------------------------------------------------------------- #
# 2. exact rational arithmetic of the product form (a different algebraic form):
#    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
# --------------------------------------------------------------------------- #
def _frac_matmul(A, B):
    return [[sum((A[i][l] * B[l][j] for l in range(len(B))), Fraction(0))
             for j in range(len(B[0]))] for i in range(len(A))]


def check_exact_product_form():
    rng = np.random.default_rng(7)
    T, Hq, Hv, dk, dv = 6, 1, 2, 3, 3
    F = lambda a, b: Fraction(int(a), int(b))
    k = [[[F(rng.integers(-5, 6), 4) for _ in range(dk)]] for _ in range(T)]        # unnormalised
    q = [[[F(rng.integers(-5, 6), 3) for _ in range(dk)]] for _ in range(T)]
    v = [[[F(rng.integers(-7, 8), 2) for _ in range(dv)] for _ in range(Hv)] for _ in range(T)]
    alpha = [[F(rng.integers(1, 9), 8) for _ in range(Hv)] for _ in range(T)]
    beta = [[F(rng.integers(0, 5), 4) for _ in range(Hv)] for _ in range(T)]
    S0 = [[[F(rng.integers(-3, 4), 5) for _ in range(dv)] for _ in range(dk)] for _ in range(Hv)]
    scale = Fraction(1, 2)
    o_exact = np.zeros((T, Hv, dv))
    S = [[row[:] for row in S0[h]] for h in range(Hv)]
    for t in range(T):
        for h in range(Hv):
            kk = k[t][0]
            a, b = alpha[t][h], beta[t][h]
            P = [[a * ((1 if i == j else 0) - b * kk[i] * kk[j]) for j in range(dk)] for i in range(dk)]
            S[h] = _frac_matmul(P, S[h])
            for i in range(dk):
                for j in range(dv):
                    S[h][i][j] += b * kk[i] * v[t][h][j]
            for j in range(dv):
                o_exact[t, h, j] = float(scale * sum(S[h][i][j] * q[t][0][i] for i in range(dk)))
    fin_exact = np.array([[[float(x) for x in row] for row in S[h]] for h in range(Hv)])
    tof = lambda x: np.array(x, dtype=object).astype(float)
    r = oracle.recurrent(tof(q), tof(k), tof(v), np.log(tof(alpha)), tof(beta), float(scale),
                         Hq, Hv, initial_state=tof(S0)[None])
    np.testing.assert_allclose(r["o"], o_exact, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["final"][0], fin_exact, rtol=1e-12, atol=1e-12)


def test_exact_rational_product_form():
    check_exact_product_form()


# --------------------------------------------------------------------------- #
# 3. closed forms
# --------------------------------------------------------------------------- #
def check_closed_forms():
    rng = np.random.default_rng(11)
    T, Hq, Hv, dk, dv = 9, 1, 2, 5, 4
    q, k, v, g, beta = _case(rng, T, Hq, Hv, dk, dv)
    S0 = rng.standard_normal((1, Hv, dk, dv))
    sc = 0.7
    # (a) beta = 0, alpha = 1: nothing is written, nothing decays.
    r = oracle.recurrent(q, k, v, np.zeros_like(g), np.zeros_like(beta), sc, Hq, Hv, initial_state=S0)
    np.testing.assert_allclose(r["final"], S0, atol=1e-14)
    np.testing.assert_allclose(r["o"], sc * np.einsum("hij,ti->thj", S0[0], q[:, 0]), atol=1e-13)
    # (b) beta = 0: pure decay, S_T = exp(sum g) S0.
    r = oracle.recurrent(q, k, v, g, np.zeros_like(beta), sc, Hq, Hv, initial_state=S0)
    np.testing.assert_allclose(r["final"][0], np.exp(g.sum(0))[:, None, None] * S0[0], rtol=1e-12)
    # (c) zero state, one token: S = beta k v^T, o = scale beta (q.k) v.
    r = oracle.recurrent(q[:1], k[:1], v[:1], g[:1], beta[:1], sc, Hq, Hv)
    for h in range(Hv):
        np.testing.assert_allclose(r["final"][0, h], beta[0, h] * np.outer(k[0, 0], v[0, h]), atol=1e-14)
        np.testing.assert_allclose(r["o"][0, h], sc * beta[0, h] * (q[0, 0] @ k[0, 0]) * v[0, h], atol=1e-14)
    # (d) beta = 1 and a unit key: the state then reads back exactly v_t at k_t
    #     (query = key, post-update state), whatever alpha and S_{t-1} were.
    r = oracle.recurrent(k, k, v, g, np.ones_like(beta), sc, Hq, Hv, initial_state=S0)
    np.testing.assert_allclose(r["o"], sc * v, atol=1e-12)
    # (e) alpha = beta = 1 with basis-vector keys is a key-value store: row i holds
    #     the value last written under key e_i (or the initial row).
    dk2 = 4
    idx = rng.integers(0, dk2, size=T)
    kb = np.eye(dk2)[idx][:, None, :]
    S0b = rng.standard_normal((1, Hv, dk2, dv))
    r = oracle.recurrent(kb, kb, v, np.zeros_like(g), np.ones_like(beta), 1.0, Hq, Hv, initial_state=S0b)
    expect = S0b[0].copy()
    for t in range(T):
        expect[:, idx[t], :] = v[t]
    np.testing.assert_allclose(r["final"][0], expect, atol=1e-13)


def test_closed_forms():
    check_closed_forms()


# --------------------------------------------------------------------------- #
# 4. invariants
# --------------------------------------------------------------------------- #
def test_linearity_in_state_and_values():
    rng = np.random.default_rng(5)
    T, Hq, Hv, dk, dv = 12, 2, 4, 6, 5
    q, k, v1, g, beta = _case(rng, T, Hq, Hv, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    s1 = rng.standard_normal((1, Hv, dk, dv))
    s2 = rng.standard_normal((1, Hv, dk, dv))
    a, b = 0.37, -1.9
    r1 = oracle.recurrent(q, k, v1, g, beta, 0.4, Hq, Hv, initial_state=s1)
    r2 = oracle.recurrent(q, k, v2, g, beta, 0.4, Hq, Hv, initial_state=s2)
    r = oracle.recurrent(q, k, a * v1 + b * v2, g, beta, 0.4, Hq, Hv, initial_state=a * s1 + b * s2)
    for key in ("o", "final"):
        np.testing.assert_allclose(r[key], a * r1[key] + b * r2[key], atol=1e-12)


def check_chunked_equals_recurrent(chunk):
    rng = np.random.default_rng(100 + chunk)
    lengths = [64, 37, 1, 0, 100]
    T = sum(lengths)
    Hq, Hv, dk, dv = 2, 4, 16, 12
    q, k, v, g, beta = _case(rng, T, Hq, Hv, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    S0 = rng.standard_normal((len(lengths), Hv, dk, dv)) * 0.1
    r = oracle.recurrent(q, k, v, g, beta, 0.25, Hq, Hv, cu_seqlens=cu, initial_state=S0)
    c = oracle.chunked(q, k, v, g, beta, 0.25, Hq, Hv, chunk, cu_seqlens=cu, initial_state=S0)
    np.testing.assert_allclose(c["o"], r["o"], atol=1e-12)
    np.testing.assert_allclose(c["final"], r["final"], atol=1e-12)


@pytest.mark.parametrize("chunk", [7, 16, 64])
def test_chunked_form_equals_recurrence(chunk):
    check_chunked_equals_recurrent(chunk)


def test_state_carry_split_equals_whole():
    rng = np.random.default_rng(21)
    T, Hq, Hv, dk, dv = 40, 1, 3, 8, 8
    q, k, v, g, beta = _case(rng, T, Hq, Hv, dk, dv)
    S0 = rng.standard_normal((1, Hv, dk, dv))
    whole = oracle.recurrent(q, k, v, g, beta, 0.3, Hq, Hv, initial_state=S0)
    m = 17
    a = oracle.recurrent(q[:m], k[:m], v[:m], g[:m], beta[:m], 0.3, Hq, Hv, initial_state=S0)
    b = oracle.recurrent(q[m:], k[m:], v[m:], g[m:], beta[m:], 0.3, Hq, Hv, initial_state=a["final"])
    np.testing.assert_allclose(b["final"], whole["final"], atol=1e-13)
    np.testing.assert_allclose(np.concatenate([a["o"], b["o"]]), whole["o"], atol=1e-13)


def test_varlen_equals_independent_runs_and_empty_sequence():
    rng = np.random.default_rng(22)
    lengths = [5, 0, 9]
    T = sum(lengths)
    Hq, Hv, dk, dv = 1, 2, 4, 3
    q, k, v, g, beta = _case(rng, T, Hq, Hv, dk, dv)
    S0 = rng.standard_normal((3, Hv, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    r = oracle.recurrent(q, k, v, g, beta, 1.0, Hq, Hv, cu_seqlens=cu, initial_state=S0)
    np.testing.assert_array_equal(r["final"][1], S0[1])          # empty: final = initial
    for s in (0, 2):
        sl = slice(cu[s], cu[s + 1])
        rs = oracle.recurrent(q[sl], k[sl], v[sl], g[sl], beta[sl], 1.0, Hq, Hv,
                              initial_state=S0[s:s + 1])
        np.testing.assert_allclose(r["final"][s], rs["final"][0], atol=1e-14)
        np.testing.assert_allclose(r["o"][sl], rs["o"], atol=1e-14)
    # broadcast of one initial state over rows equals explicit repetition
    rb = oracle.recurrent(q, k, v, g, beta, 1.0, Hq, Hv, cu_seqlens=cu, initial_state=S0[:1],
                          initial_state_broadcast=True)
    re = oracle.recurrent(q, k, v, g, beta, 1.0, Hq, Hv, cu_seqlens=cu,
                          initial_state=np.repeat(S0[:1], 3, axis=0))
    np.testing.assert_array_equal(rb["final"], re["final"])


def test_chunk_boundary_states():
    """The recorded boundary states are the states of the prefixes that end on
    chunk boundaries: with beta = 0 the state after m tokens is the closed form
    exp(sum_{t<m} g_t) S0 (an off-by-one in the recording position changes the
    exponent); for generic inputs the entries equal the chunk-end states of the
    chunked form (a different algorithm), each sequence's last entry equals its
    final state, and an entry equals a separate run over that prefix."""
    rng = np.random.default_rng(24)
    lengths = [10, 0, 4, 1, 8]
    C = 4
    T = sum(lengths)
    Hq, Hv, dk, dv = 1, 2, 3, 2
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k, v, g, _ = _case(rng, T, Hq, Hv, dk, dv)
    S0 = rng.standard_normal((len(lengths), Hv, dk, dv))
    r = oracle.recurrent(q, k, v, g, np.zeros((T, Hv)), 0.5, Hq, Hv, cu_seqlens=cu, initial_state=S0,
                         boundary_every=C)
    counts = [-(-L // C) for L in lengths]
    assert r["boundary"].shape == (sum(counts), Hv, dk, dv)
    i = 0
    for s, L in enumerate(lengths):
        for j in range(counts[s]):
            m = min((j + 1) * C, L)
            decay = np.exp(g[cu[s]:cu[s] + m].sum(axis=0))              # [Hv]
            np.testing.assert_allclose(r["boundary"][i], decay[:, None, None] * S0[s], rtol=1e-13)
            i += 1
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Hv))))
    r = oracle.recurrent(q, k, v, g, beta, 0.5, Hq, Hv, cu_seqlens=cu, initial_state=S0, boundary_every=C)
    c = oracle.chunked(q, k, v, g, beta, 0.5, Hq, Hv, C, cu_seqlens=cu, initial_state=S0)
    np.testing.assert_allclose(r["boundary"], c["boundary"], atol=1e-12)
    last = np.cumsum(counts) - 1
    for s, L in enumerate(lengths):
        if L:
            np.testing.assert_array_equal(r["boundary"][last[s]], r["final"][s])
    # entry 1 of sequence 0 = the state after its first 8 tokens
    p = oracle.recurrent(q[:8], k[:8], v[:8], g[:8], beta[:8], 0.5, Hq, Hv, initial_state=S0[:1])
    np.testing.assert_allclose(r["boundary"][1], p["final"][0], atol=1e-14)


def test_prologue_closed_forms():
    """Input prologue pins: a 3-4-5 key normalises to (0.6, 0.8); sigmoid(0) =
    1/2 and sigmoid(ln 3) = 3/4; with A_log = 0 the gate's decay is
    exp(-softplus(x)) = 1 / (1 + e^x), and with A_log = ln 2 its square; the
    identity prologue returns its inputs."""
    q = np.array([[[0.0, 2.0]]])
    k = np.array([[[3.0, 4.0]]])
    a = np.array([[0.3, -1.2, 2.5]])
    b = np.array([[0.0, np.log(3.0), -np.log(3.0)]])
    qn, kn, g, beta = oracle.prologue(q, k, a, b, qk_l2norm=True, eps=0.0, beta_is_logit=True,
                                      A_log=np.zeros(3), dt_bias=np.array([0.1, 0.0, -0.5]))
    np.testing.assert_allclose(kn[0, 0], [0.6, 0.8], rtol=1e-15)
    np.testing.assert_allclose(qn[0, 0], [0.0, 1.0], rtol=1e-15)
    np.testing.assert_allclose(beta[0], [0.5, 0.75, 0.25], rtol=1e-15)
    x = a[0] + np.array([0.1, 0.0, -0.5])
    np.testing.assert_allclose(np.exp(g[0]), 1.0 / (1.0 + np.exp(x)), rtol=1e-14)
    _, _, g2, _ = oracle.prologue(q, k, a, b, A_log=np.full(3, np.log(2.0)))
    np.testing.assert_allclose(np.exp(g2[0]), (1.0 + np.exp(a[0])) ** -2, rtol=1e-14)
    # eps enters under the root
    _, ke, _, _ = oracle.prologue(q, k, a, b, qk_l2norm=True, eps=11.0)
    np.testing.assert_allclose(ke[0, 0], [0.5, 4.0 / 6.0], rtol=1e-15)
    for x0, x1 in zip((q, k, a, b), oracle.prologue(q, k, a, b)):
        np.testing.assert_array_equal(x0, x1)


def test_prologue_l2norm_scale_invariance():
    """With the l2norm prologue (eps = 0) the layer output does not change when
    each q_t and k_t is scaled by its own positive factor, and equals the plain
    recurrence on unit-norm inputs."""
    rng = np.random.default_rng(25)
    T, Hq, Hv, dk, dv = 9, 2, 4, 5, 3
    q, k, v, g, beta = _case(rng, T, Hq, Hv, dk, dv)
    cq = rng.uniform(0.2, 5.0, (T, Hq, 1))
    ck = rng.uniform(0.2, 5.0, (T, Hq, 1))
    p1 = oracle.prologue(q * cq, k * ck, g, beta, qk_l2norm=True, eps=0.0)
    r1 = oracle.recurrent(p1[0], p1[1], v, p1[2], p1[3], 0.7, Hq, Hv)
    r0 = oracle.recurrent(q, k, v, g, beta, 0.7, Hq, Hv)          # _case draws unit-norm q, k
    np.testing.assert_allclose(r1["o"], r0["o"], atol=1e-13)
    np.testing.assert_allclose(r1["final"], r0["final"], atol=1e-13)


def test_shared_key_heads_equal_single_head_runs():
    rng = np.random.default_rng(23)
    T, Hq, Hv, dk, dv = 11, 2, 6, 5, 4
    q, k, v, g, beta = _case(rng, T, Hq, Hv, dk, dv)
    S0 = rng.standard_normal((1, Hv, dk, dv))
    r = oracle.recurrent(q, k, v, g, beta, 0.5, Hq, Hv, initial_state=S0)
    for h in range(Hv):
        hk = h // (Hv // Hq)
        rs = oracle.recurrent(q[:, hk:hk + 1], k[:, hk:hk + 1], v[:, h:h + 1], g[:, h:h + 1],
                              beta[:, h:h + 1], 0.5, 1, 1, initial_state=S0[:, h:h + 1])
        np.testing.assert_allclose(r["o"][:, h], rs["o"][:, 0], atol=1e-14)
        np.testing.assert_allclose(r["final"][0, h], rs["final"][0, 0], atol=1e-14)
    # the subset-of-heads mode gives the same numbers as the full run
    rsub = oracle.recurrent(q, k, v, g, beta, 0.5, Hq, Hv, initial_state=S0, heads=[1, 4])
    np.testing.assert_array_equal(rsub["final"][0, [1, 4]], r["final"][0, [1, 4]])


# --------------------------------------------------------------------------- #
# 5. capture / replay / snapshot
# --------------------------------------------------------------------------- #
def check_capture_replay():
    rng = np.random.default_rng(31)
    lengths = [3, 7, 1, 5]
    T = sum(lengths)
    Hq, Hv, dk, dv, cap = 2, 4, 6, 5, 7
    q, k, v, g, beta = _case(rng, T, Hq, Hv, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    S0 = rng.standard_normal((4, Hv, dk, dv))
    r = oracle.recurrent(q, k, v, g, beta, 0.5, Hq, Hv, cu_seqlens=cu, initial_state=S0)
    counts = np.array([-2, 7, 9, 3])                      # negative, full, over cap, partial
    buf, mask = oracle.capture(k, r["alpha"], r["delta"], Hq, Hv, cap, counts, 1, cu_seqlens=cu)
    n = [min(max(c, 0), cap, L) for c, L in zip(counts, lengths)]
    assert n == [0, 7, 1, 3]
    R = oracle.record_width(Hq, Hv, dk, dv)
    for b in range(4):
        assert mask[b, :n[b]].all() and not mask[b, n[b]:].any()
        for c in range(n[b]):
            t = cu[b] + c
            np.testing.assert_array_equal(buf[b, c, Hv:Hv + Hq * dk], k[t].reshape(-1))
            np.testing.assert_allclose(buf[b, c, :Hv], np.exp(g[t]), rtol=1e-15)
    # full replay reproduces the final state; partial replay the prefix run's state
    full = oracle.replay(S0, buf, n, Hq, Hv, dk, dv, cap)
    for b in (1, 2):
        np.testing.assert_allclose(full[b], r["final"][b], atol=1e-13)
    m = 2
    part = oracle.replay(S0, buf, [0, m, 0, m], Hq, Hv, dk, dv, cap)
    sl = slice(cu[1], cu[1] + m)
    rp = oracle.recurrent(q[sl], k[sl], v[sl], g[sl], beta[sl], 0.5, Hq, Hv, initial_state=S0[1:2])
    np.testing.assert_allclose(part[1], rp["final"][0], atol=1e-13)
    np.testing.assert_array_equal(part[0], S0[0])
    # inactive: all zero and all specified
    z, zm = oracle.capture(k, r["alpha"], r["delta"], Hq, Hv, cap, counts, 0, cu_seqlens=cu)
    assert z.shape == (4, cap, R) and not z.any() and zm.all()


def test_capture_then_replay_reproduces_state():
    check_capture_replay()


def test_snapshot_is_an_independent_copy():
    src = rng0.standard_normal((2, 3, 4, 4))
    dst = oracle.snapshot(src)
    np.testing.assert_array_equal(dst, src)
    dst[0, 0, 0, 0] += 1
    assert src[0, 0, 0, 0] != dst[0, 0, 0, 0]


# --------------------------------------------------------------------------- #
# 6. planted mistakes must be caught by the pins above
# --------------------------------------------------------------------------- #
def _mut_o_from_old_state(S, a, kt, vt, b, qt, scale):
    u = np.einsum("hij,hi->hj", a[:, None, None] * S, kt)
    delta = b[:, None] * (vt - u)
    o = scale * np.einsum("hij,hi->hj", S, qt)
    return a[:, None, None] * S + kt[:, :, None] * delta[:, None, :], o, delta


def _mut_no_alpha_in_delta(S, a, kt, vt, b, qt, scale):
    u = np.einsum("hij,hi->hj", S, kt)
    delta = b[:, None] * (vt - u)
    S_new = a[:, None, None] * S + kt[:, :, None] * delta[:, None, :]
    return S_new, scale * np.einsum("hij,hi->hj", S_new, qt), delta


def _mut_sign(S, a, kt, vt, b, qt, scale):
    u = np.einsum("hij,hi->hj", a[:, None, None] * S, kt)
    delta = b[:, None] * (vt + u)
    S_new = a[:, None, None] * S + kt[:, :, None] * delta[:, None, :]
    return S_new, scale * np.einsum("hij,hi->hj", S_new, qt), delta


def _mut_transposed_read(S, a, kt, vt, b, qt, scale):
    u = np.einsum("hji,hi->hj", a[:, None, None] * S, kt)       # S k instead of S^T k
    delta = b[:, None] * (vt - u)
    S_new = a[:, None, None] * S + kt[:, :, None] * delta[:, None, :]
    return S_new, scale * np.einsum("hij,hi->hj", S_new, qt), delta


def _mut_no_beta(S, a, kt, vt, b, qt, scale):
    u = np.einsum("hij,hi->hj", a[:, None, None] * S, kt)
    delta = vt - u
    S_new = a[:, None, None] * S + kt[:, :, None] * delta[:, None, :]
    return S_new, scale * np.einsum("hij,hi->hj", S_new, qt), delta


def _mut_no_decay_of_state(S, a, kt, vt, b, qt, scale):
    u = np.einsum("hij,hi->hj", a[:, None, None] * S, kt)
    delta = b[:, None] * (vt - u)
    S_new = S + kt[:, :, None] * delta[:, None, :]
    return S_new, scale * np.einsum("hij,hi->hj", S_new, qt), delta


@pytest.mark.parametrize("mutant", [_mut_o_from_old_state, _mut_no_alpha_in_delta, _mut_sign,
                                    _mut_transposed_read, _mut_no_beta, _mut_no_decay_of_state])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(gdn_oracle, "_token_update", mutant)
    caught = 0
    for check in (check_hand_worked, check_exact_product_form, check_closed_forms):
        try:
            check()
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1, f"{mutant.__name__} slipped through every pin"
