"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each ``check_*`` takes an oracle object (``alpha``, ``fwd``, ``step``) so that the same pins
can be run against deliberately broken copies of the oracle source (see ``test_pins_catch_mutants``).

Sources of the pins:
  * the worked example printed in "Error-Free Linear Attention is a Free Lunch" (howistudyai.com),
    Steps 1-3 (tests/golden/page4_worked_example.json);
  * the closed-form matrix exponential of the rank-1 dynamics, "Exact Flow Linear Attention"
    (gist.science), Metodologia item 2 -- checked against scipy's Pade/scaling-and-squaring expm;
  * the zero-order-hold ODE dS/dt = -k k^T S + k v^T of Metodologia item 1 -- checked by the
    augmented-matrix exponential (Van Loan) and by brute-force fine-step RK4 integration;
  * the directional decay e^{-beta lambda} along k and the untouched orthogonal complement
    (Contributi Chiave, "Stabilita Teorica"; howistudyai.com Step 5);
  * the Euler / delta-rule limit for small beta*lambda (howistudyai.com Step 5, "Delta Rule");
  * the chunkwise WY/UT rewriting (Metodologia item 3; howistudyai.com Step 4), checked with an
    independent fp64 numpy model of the chunked form;
  * state passing between chunks (howistudyai.com Step 4) and prefill followed by decode;
  * the integrator family the exact flow closes ("Error-Free Linear Attention guida completa"
    (mauroscia.it), section on RK-infinity; howistudyai.com building blocks "Delta Rule" and
    "Runge-Kutta Methods"): a gate of order p must be one step of a textbook p-th order Runge-Kutta
    method applied to the ODE itself, order 1 the delta rule, and high orders the exact flow;
  * the gradients (the pages train their models but print no backward pass): central finite differences
    of the pinned forward, a one-token closed form with the gate's derivatives d alpha / d beta = e^{-x},
    d alpha / d lambda = -(alpha - beta e^{-x}) / lambda, linearity in the incoming gradients, and
    chaining through the state gradient of a split sequence.
"""
import json
import os
import re
import shutil
import tempfile

import mpmath
import numpy as np
import pytest
import scipy.linalg

import oracle
from exact_flow_delta_amd import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "page4_worked_example.json")) as f:
    GOLD = json.load(f)


def _one_token(orc, k, v, beta, S0, q=None):
    d_k, d_v = len(k), len(v)
    q = np.zeros(d_k) if q is None else np.asarray(q, float)
    o, S, _ = orc.fwd(q.reshape(1, 1, 1, d_k), np.asarray(k, float).reshape(1, 1, 1, d_k),
                      np.asarray(v, float).reshape(1, 1, 1, d_v), np.array([[[beta]]]),
                      np.asarray(S0, float).reshape(1, 1, d_k, d_v))
    return o[0, 0, 0], S[0, 0]


def _one_token_gate(orc, k, v, beta, S0, q, gate):
    d_k, d_v = len(k), len(v)
    o, S, _ = orc.fwd(np.asarray(q, float).reshape(1, 1, 1, d_k), np.asarray(k, float).reshape(1, 1, 1, d_k),
                      np.asarray(v, float).reshape(1, 1, 1, d_v), np.array([[[beta]]]),
                      np.asarray(S0, float).reshape(1, 1, d_k, d_v), gate=gate)
    return o[0, 0, 0], S[0, 0]


def _mixed_keys(rng, L, d_k, lo=1e-2, hi=3.0):
    g = rng.standard_normal((L, d_k))
    u = g / np.linalg.norm(g, axis=-1, keepdims=True)
    s = np.exp(rng.uniform(np.log(lo), np.log(hi), (L, 1)))
    return u * s


# ----------------------------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------------------------

def check_worked_example(orc):
    """Printed numbers of the worked example (d = 2)."""
    p = GOLD["printed"]
    tol = 0.5 * 10.0 ** -p["printed_decimals"]
    k = np.array(GOLD["k"])
    v = np.array(GOLD["v"])
    q = np.array(GOLD["q"])
    beta = GOLD["beta"]
    a = orc.alpha(k[None], np.array([beta]))[0]
    assert abs(a - p["alpha"]) <= tol, a
    # 1 - alpha*lambda is the decay factor e^{-beta lambda} printed as 0.3679, and 1 - e^{-1} as 0.6321
    assert abs((1.0 - a * p["lambda"]) - p["exp_minus_beta_lambda"]) <= tol
    assert abs(a * p["lambda"] - p["one_minus_exp"]) <= tol
    # from an empty memory the update writes alpha * k v^T; the page prints k v^T
    o, S = _one_token(orc, k, v, beta, np.zeros((2, 2)), q)
    np.testing.assert_allclose(S / a, np.array(p["k_vT"]), rtol=0, atol=1e-12)
    # readout o = S^T q with the printed q, from the printed alpha and k v^T
    want = p["alpha"] * (np.array(p["k_vT"]).T @ q)
    assert np.max(np.abs(o - want)) <= 2 * tol, (o, want)


def check_expm_erase(orc):
    """v = 0: one token maps S0 to expm(-beta k k^T) S0 (closed form of the rank-1 exponential)."""
    rng = np.random.default_rng(11)
    cases = [(2, 3, 1.0, 0.2), (3, 2, 3.0, 0.7), (4, 4, 0.01, 0.5), (4, 1, 10.0, 0.9), (3, 3, 1e-5, 0.3),
             (2, 2, 30.0, 0.05)]
    for d_k, d_v, scale, beta in cases:
        k = rng.standard_normal(d_k) * scale
        S0 = rng.standard_normal((d_k, d_v))
        E = scipy.linalg.expm(-beta * np.outer(k, k))
        _, S1 = _one_token(orc, k, np.zeros(d_v), beta, S0)
        np.testing.assert_allclose(S1, E @ S0, rtol=0, atol=1e-12 * max(1.0, np.abs(S0).max()))


def check_van_loan(orc):
    """Full ZOH step: expm(beta [[-A, k v^T], [0, 0]]) gives e^{-beta A} and the input integral."""
    rng = np.random.default_rng(12)
    cases = [(2, 2, 1.0, 0.2), (3, 4, 2.0, 0.8), (4, 3, 0.05, 0.6), (3, 3, 6.0, 0.9), (4, 2, 1e-4, 0.4)]
    for d_k, d_v, scale, beta in cases:
        k = rng.standard_normal(d_k) * scale
        v = rng.standard_normal(d_v)
        S0 = rng.standard_normal((d_k, d_v))
        M = np.zeros((d_k + d_v, d_k + d_v))
        M[:d_k, :d_k] = -np.outer(k, k)
        M[:d_k, d_k:] = np.outer(k, v)
        E = scipy.linalg.expm(beta * M)
        want = E[:d_k, :d_k] @ S0 + E[:d_k, d_k:]
        _, S1 = _one_token(orc, k, v, beta, S0)
        np.testing.assert_allclose(S1, want, rtol=0, atol=1e-12 * max(1.0, np.abs(want).max()))
        # the decode step is the same token update
        q = rng.standard_normal(d_k)
        o, S2, _ = orc.step(q[None], k[None], v[None], np.array([beta]), S0[None])
        np.testing.assert_allclose(S2[0], want, rtol=0, atol=1e-12 * max(1.0, np.abs(want).max()))
        np.testing.assert_allclose(o[0], want.T @ q, rtol=0, atol=1e-12 * max(1.0, np.abs(want).max()))


def _rk4_token(S, k, v, beta, nsub):
    A = np.outer(k, k)
    Bm = np.outer(k, v)
    h = beta / nsub

    def f(X):
        return -A @ X + Bm

    for _ in range(nsub):
        k1 = f(S)
        k2 = f(S + 0.5 * h * k1)
        k3 = f(S + 0.5 * h * k2)
        k4 = f(S + h * k3)
        S = S + (h / 6.0) * (k1 + 2 * k2 + 2 * k3 + k4)
    return S


def check_rk4_sequence(orc):
    """A sequence of tokens: integrate the ODE over each hold interval [0, beta_t] with fine RK4,
    read o_t = S_t^T q_t after each interval, and compare with the closed-form recurrence."""
    rng = np.random.default_rng(13)
    L, d_k, d_v = 10, 3, 2
    k = _mixed_keys(rng, L, d_k, 0.1, 2.0)
    v = rng.standard_normal((L, d_v))
    q = rng.standard_normal((L, d_k))
    beta = rng.uniform(0.05, 1.0, L)
    S = rng.standard_normal((d_k, d_v)) * 0.3
    S0 = S.copy()
    o_ref = np.zeros((L, d_v))
    for t in range(L):
        S = _rk4_token(S, k[t], v[t], beta[t], 2000)
        o_ref[t] = S.T @ q[t]
    o, Sf, _ = orc.fwd(q[None, None], k[None, None], v[None, None], beta[None, None], S0[None, None])
    np.testing.assert_allclose(o[0, 0], o_ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(Sf[0, 0], S, rtol=0, atol=1e-10)


def check_alpha_extremes(orc):
    """alpha against a 50-digit evaluation of (1 - e^{-beta lambda}) / lambda, and lambda = 0 -> beta."""
    mpmath.mp.dps = 50
    for kk in [1e-150, 1e-8, 1e-4, 0.03, 1.0, 2.2360679, 31.6, 1e3, 1e5]:
        for beta in [1e-7, 0.2, 0.5, 0.97]:
            a = orc.alpha(np.array([[kk]]), np.array([beta]))[0]
            lam = mpmath.mpf(kk) ** 2
            x = mpmath.mpf(beta) * lam
            ref = beta if lam == 0 else -mpmath.expm1(-x) / lam
            assert abs(a - float(ref)) <= 4e-16 * abs(float(ref)), (kk, beta, a, ref)
    for beta in [0.0, 0.3, 1.0]:
        assert orc.alpha(np.zeros((1, 4)), np.array([beta]))[0] == beta
    assert orc.alpha(np.ones((1, 4)), np.array([0.0]))[0] == 0.0


def check_euler_limit(orc):
    """beta*lambda -> 0: alpha -> beta (one explicit Euler step = delta rule) with |alpha - beta| <= beta^2 lambda / 2."""
    rng = np.random.default_rng(14)
    for _ in range(40):
        d_k = 4
        k = rng.standard_normal(d_k) * 10.0 ** rng.uniform(-4, 0)
        beta = rng.uniform(0.01, 1.0)
        lam = float(k @ k)
        a = orc.alpha(k[None], np.array([beta]))[0]
        slack = 8e-16 * beta  # rounding of the difference beta - alpha
        assert -slack <= beta - a <= 0.5 * beta * beta * lam + slack
        # and from the other side: the second-order term is not dropped
        assert beta - a >= 0.5 * beta * beta * lam * (1 - beta * lam / 3.0) - slack


def check_directional_decay(orc):
    """Memory along k relaxes by e^{-beta lambda} towards v; the part orthogonal to k is untouched."""
    rng = np.random.default_rng(15)
    for scale in [0.01, 0.5, 1.0, 4.0, 20.0]:
        d_k, d_v = 5, 3
        k = rng.standard_normal(d_k) * scale
        v = rng.standard_normal(d_v)
        beta = rng.uniform(0.1, 1.0)
        S0 = rng.standard_normal((d_k, d_v))
        _, S1 = _one_token(orc, k, v, beta, S0)
        lam = float(k @ k)
        decay = np.exp(-beta * lam)
        np.testing.assert_allclose(k @ S1, decay * (k @ S0) + (1 - decay) * v,
                                   rtol=0, atol=1e-12 * max(1.0, lam) * max(1.0, np.abs(S0).max()))
        u = rng.standard_normal(d_k)
        u -= (u @ k) / lam * k
        np.testing.assert_allclose(u @ S1, u @ S0, rtol=0, atol=1e-12 * max(1.0, scale))


def check_stiff_overwrite(orc):
    """beta*lambda >> 1: the memory along k is overwritten, k^T S_t = v_t^T."""
    rng = np.random.default_rng(16)
    for scale in [8.0, 30.0, 300.0]:
        d_k, d_v = 4, 3
        k = rng.standard_normal(d_k) * scale
        v = rng.standard_normal(d_v)
        _, S1 = _one_token(orc, k, v, 0.9, rng.standard_normal((d_k, d_v)))
        np.testing.assert_allclose(k @ S1, v, rtol=0, atol=1e-9)


def check_contractive(orc):
    """v = 0: ||S_t||_F never grows (eigenvalues of e^{-beta k k^T} are e^{-beta lambda} and 1)."""
    rng = np.random.default_rng(17)
    L, d_k, d_v = 40, 4, 3
    k = _mixed_keys(rng, L, d_k, 0.01, 10.0)
    beta = rng.uniform(0.0, 1.0, L)
    S = rng.standard_normal((d_k, d_v))
    prev = np.linalg.norm(S)
    for t in range(L):
        _, S = _one_token(orc, k[t], np.zeros(d_v), beta[t], S)
        cur = np.linalg.norm(S)
        assert cur <= prev * (1 + 1e-14)
        prev = cur


def check_linearity(orc):
    """For fixed q, k, beta the outputs and state are jointly linear in (S0, V)."""
    rng = np.random.default_rng(18)
    B, H, L, d_k, d_v = 1, 2, 17, 4, 3
    q = rng.standard_normal((B, H, L, d_k))
    k = rng.standard_normal((B, H, L, d_k))
    beta = rng.uniform(0, 1, (B, H, L))
    va, vb = rng.standard_normal((2, B, H, L, d_v))
    sa, sb = rng.standard_normal((2, B, H, d_k, d_v))
    c = -1.7
    oa, Sa, _ = orc.fwd(q, k, va, beta, sa)
    ob, Sb, _ = orc.fwd(q, k, vb, beta, sb)
    oc, Sc, _ = orc.fwd(q, k, va + c * vb, beta, sa + c * sb)
    np.testing.assert_allclose(oc, oa + c * ob, rtol=0, atol=1e-11)
    np.testing.assert_allclose(Sc, Sa + c * Sb, rtol=0, atol=1e-11)


def _chunked_model(q, k, v, beta, S0, C, alpha=None):
    """Independent fp64 model of the chunkwise WY/UT form (one head):
    A = strict_tril(diag(alpha) K K^T), T = (I + A)^{-1}, W = T diag(alpha) K, U = T diag(alpha) V,
    Delta = U - W S, O = Q S + tril(Q K^T) Delta, S <- S + K^T Delta.  alpha: the exact gate unless given."""
    L = k.shape[0]
    if alpha is None:
        lam = np.sum(k * k, axis=-1)
        x = beta * lam
        alpha = np.where(x == 0, beta, -np.expm1(-x) / np.where(lam == 0, 1.0, lam))
    S = S0.copy()
    o = np.zeros((L, v.shape[1]))
    for t0 in range(0, L, C):
        sl = slice(t0, min(L, t0 + C))
        K, Q, V, a = k[sl], q[sl], v[sl], alpha[sl]
        n = K.shape[0]
        A = np.tril(a[:, None] * (K @ K.T), -1)
        T = np.linalg.inv(np.eye(n) + A)
        Wm = T @ (a[:, None] * K)
        U = T @ (a[:, None] * V)
        D = U - Wm @ S
        o[sl] = Q @ S + np.tril(Q @ K.T) @ D
        S = S + K.T @ D
    return o, S


def check_chunk_identity(orc):
    """The chunkwise-parallel form reaches the recurrence's result for every chunk size."""
    rng = np.random.default_rng(19)
    L, d_k, d_v = 100, 8, 6
    k = _mixed_keys(rng, L, d_k, 1e-3, 6.0)
    q = rng.standard_normal((L, d_k))
    v = rng.standard_normal((L, d_v))
    beta = rng.uniform(0, 1, L)
    S0 = rng.standard_normal((d_k, d_v)) * 0.1
    o, Sf, _ = orc.fwd(q[None, None], k[None, None], v[None, None], beta[None, None], S0[None, None])
    for C in [1, 2, 4, 16, 64, L]:
        oc, Sc = _chunked_model(q, k, v, beta, S0, C)
        np.testing.assert_allclose(o[0, 0], oc, rtol=0, atol=1e-11)
        np.testing.assert_allclose(Sf[0, 0], Sc, rtol=0, atol=1e-11)


def check_state_chaining(orc):
    """fwd over [0, L) equals fwd over [0, L1) then [L1, L) from its final state; prefill then decode steps."""
    rng = np.random.default_rng(20)
    B, H, L, d_k, d_v = 2, 2, 33, 5, 4
    q = rng.standard_normal((B, H, L, d_k))
    k = rng.standard_normal((B, H, L, d_k))
    v = rng.standard_normal((B, H, L, d_v))
    beta = rng.uniform(0, 1, (B, H, L))
    S0 = rng.standard_normal((B, H, d_k, d_v))
    o, Sf, _ = orc.fwd(q, k, v, beta, S0)
    L1 = 20
    o1, S1, _ = orc.fwd(q[:, :, :L1], k[:, :, :L1], v[:, :, :L1], beta[:, :, :L1], S0)
    o2, S2, _ = orc.fwd(q[:, :, L1:], k[:, :, L1:], v[:, :, L1:], beta[:, :, L1:], S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S2, Sf, rtol=0, atol=1e-12)
    S = S1.reshape(B * H, d_k, d_v)
    for t in range(L1, L):
        ot, S, _ = orc.step(q[:, :, t].reshape(B * H, d_k), k[:, :, t].reshape(B * H, d_k),
                            v[:, :, t].reshape(B * H, d_v), beta[:, :, t].reshape(B * H), S)
        np.testing.assert_allclose(ot.reshape(B, H, d_v), o[:, :, t], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S.reshape(B, H, d_k, d_v), Sf, rtol=0, atol=1e-12)


def check_zero_initial_state(orc):
    """An absent initial state is the zero matrix."""
    rng = np.random.default_rng(21)
    q, k = rng.standard_normal((2, 1, 2, 9, 4))
    v = rng.standard_normal((1, 2, 9, 3))
    beta = rng.uniform(0, 1, (1, 2, 9))
    o1, S1, _ = orc.fwd(q, k, v, beta, None)
    o2, S2, _ = orc.fwd(q, k, v, beta, np.zeros((1, 2, 4, 3)))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def check_ut_chunk_identity(orc):
    """The oracle's UT output, used in the chunked form, reproduces the token recurrence.

    With T diag(alpha) from ``orc.ut`` for each chunk and S the recurrence's own state entering it,
    Delta = T diag(alpha) (V - K S) must give the recurrence's state after the chunk as S + K^T Delta and
    its outputs as Q S + lower_incl(Q K^T) Delta ("Error-Free Linear Attention is a Free Lunch", Step 4;
    "Exact Flow Linear Attention", Metodologia item 3).  Ragged last chunk; padding must be zero.
    """
    rng = np.random.default_rng(31)
    B, H, C, d_k, d_v = 1, 2, 8, 6, 5
    L = 2 * C + 5
    k = np.stack([_mixed_keys(rng, L, d_k, 0.05, 2.5) for _ in range(B * H)]).reshape(B, H, L, d_k)
    q = rng.standard_normal((B, H, L, d_k))
    v = rng.standard_normal((B, H, L, d_v))
    beta = rng.uniform(0.05, 1.0, (B, H, L))
    S0 = 0.3 * rng.standard_normal((B, H, d_k, d_v))
    T = orc.ut(k, beta, C)
    nc = (L + C - 1) // C
    assert T.shape == (B, H, nc, C, C)
    o_ref, _, _ = orc.fwd(q, k, v, beta, S0)
    for c in range(nc):
        t0, t1 = c * C, min(L, (c + 1) * C)
        n = t1 - t0
        assert np.all(T[:, :, c, n:, :] == 0) and np.all(T[:, :, c, :, n:] == 0)
        if c == 0:
            S_in = S0
        else:
            _, S_in, _ = orc.fwd(q[:, :, :t0], k[:, :, :t0], v[:, :, :t0], beta[:, :, :t0], S0)
        _, S_out, _ = orc.fwd(q[:, :, :t1], k[:, :, :t1], v[:, :, :t1], beta[:, :, :t1], S0)
        for b in range(B):
            for h in range(H):
                Kc, Qc, Vc = k[b, h, t0:t1], q[b, h, t0:t1], v[b, h, t0:t1]
                Tc = T[b, h, c, :n, :n]
                assert np.all(np.triu(Tc, 1) == 0)
                D = Tc @ (Vc - Kc @ S_in[b, h])
                S_new = S_in[b, h] + Kc.T @ D
                O = Qc @ S_in[b, h] + np.tril(Qc @ Kc.T) @ D
                assert np.max(np.abs(S_new - S_out[b, h])) <= 1e-12 * max(1.0, np.max(np.abs(S_out[b, h])))
                assert np.max(np.abs(O - o_ref[b, h, t0:t1])) <= 1e-12 * max(1.0, np.max(np.abs(o_ref[b, h, t0:t1])))


def check_ut_orthogonal_keys(orc):
    """Mutually orthogonal keys make A = 0, so T diag(alpha) = diag(alpha) with alpha the exact gate."""
    rng = np.random.default_rng(32)
    C, d_k = 16, 16
    Qm, _ = np.linalg.qr(rng.standard_normal((d_k, d_k)))
    k = (Qm.T * np.exp(rng.uniform(-2, 2, (C, 1))))[None, None]
    beta = rng.uniform(0.1, 2.0, (1, 1, C))
    T = orc.ut(k, beta, C)[0, 0, 0]
    lam = np.sum(k[0, 0] ** 2, axis=-1)
    a = -np.expm1(-beta[0, 0] * lam) / lam
    assert np.max(np.abs(T - np.diag(a))) <= 1e-13


# explicit Runge-Kutta methods of order p (Butcher tableaux: stage coefficients a, weights b)
RK_TABLEAUS = {
    1: ([[]], [1.0]),                                                          # explicit Euler
    2: ([[], [1.0]], [0.5, 0.5]),                                              # Heun
    3: ([[], [0.5], [-1.0, 2.0]], [1 / 6, 2 / 3, 1 / 6]),                      # Kutta's third-order method
    4: ([[], [0.5], [0.0, 0.5], [0.0, 0.0, 1.0]], [1 / 6, 1 / 3, 1 / 3, 1 / 6]),  # classical RK4
}


def _rk_step(S, k, v, beta, tableau):
    """One step of size beta of an explicit Runge-Kutta method for dS/dt = -k (k^T S) + k v^T."""
    a, b = tableau
    f = lambda X: -np.outer(k, k @ X) + np.outer(k, v)
    stages = []
    for i in range(len(b)):
        X = S.copy()
        for j, aij in enumerate(a[i]):
            X = X + beta * aij * stages[j]
        stages.append(f(X))
    out = S.copy()
    for bi, Ki in zip(b, stages):
        out = out + beta * bi * Ki
    return out


def check_gate_rk_tableaus(orc):
    """Gate p <= 4 is one step of a textbook p-th order Runge-Kutta method of the ODE itself (the stages
    integrate the full matrix dynamics; nothing here uses the rank-1 closed form)."""
    rng = np.random.default_rng(41)
    d_k, d_v = 5, 4
    for p, tab in RK_TABLEAUS.items():
        for _ in range(4):
            k = rng.standard_normal(d_k) * rng.uniform(0.3, 1.5)
            v, q = rng.standard_normal(d_v), rng.standard_normal(d_k)
            S0 = rng.standard_normal((d_k, d_v))
            beta = rng.uniform(0.05, 0.9)
            o, S = _one_token_gate(orc, k, v, beta, S0, q, p)
            S_ref = _rk_step(S0, k, v, beta, tab)
            scale = max(1.0, np.max(np.abs(S_ref)))
            assert np.max(np.abs(S - S_ref)) <= 1e-12 * scale, p
            assert np.max(np.abs(o - S_ref.T @ q)) <= 1e-12 * scale * max(1.0, np.abs(q).sum()), p
            o1, S1, _ = orc.step(q[None], k[None], v[None], np.array([beta]), S0[None], gate=p)
            assert np.max(np.abs(S1[0] - S_ref)) <= 1e-12 * scale, p


def check_gate_limits(orc):
    """Order 1 is the delta rule's alpha = beta for every key (zero keys included); high orders reach
    the exact flow where the series converges fast."""
    rng = np.random.default_rng(42)
    k = rng.standard_normal((64, 7)) * np.exp(rng.uniform(-3, 1.5, (64, 1)))
    k[5] = 0.0
    beta = rng.uniform(0.0, 1.0, 64)
    np.testing.assert_array_equal(orc.alpha(k, beta, gate=1), beta)
    small = np.sum(k * k, axis=-1) * beta <= 1.0
    a16 = orc.alpha(k[small], beta[small], gate=16)
    a = orc.alpha(k[small], beta[small])
    assert np.max(np.abs(a16 - a) / np.maximum(a, 1e-300)) <= 1e-13


def check_gate_chunk_identity(orc):
    """With a Runge-Kutta gate the recurrence, the decode step, the chunked form and the UT transform all use
    the same coefficient: the chunk algebra reproduces the gated recurrence for any chunk size, and the UT
    output satisfies the chunk identity of the gated recurrence."""
    rng = np.random.default_rng(43)
    L, d_k, d_v, gate, C = 40, 6, 5, 3, 8
    k = _mixed_keys(rng, L, d_k, 0.05, 1.5)
    q = rng.standard_normal((L, d_k))
    v = rng.standard_normal((L, d_v))
    beta = rng.uniform(0.05, 0.8, L)
    S0 = 0.2 * rng.standard_normal((d_k, d_v))
    o, Sf, _ = orc.fwd(q[None, None], k[None, None], v[None, None], beta[None, None], S0[None, None], gate=gate)
    ap = orc.alpha(k, beta, gate=gate)
    for c in [1, 4, 16, L]:
        oc, Sc = _chunked_model(q, k, v, beta, S0, c, alpha=ap)
        np.testing.assert_allclose(o[0, 0], oc, rtol=0, atol=1e-11)
        np.testing.assert_allclose(Sf[0, 0], Sc, rtol=0, atol=1e-11)
    T = orc.ut(k[None, None], beta[None, None], C, gate=gate)[0, 0]
    S = S0.copy()
    for c in range(L // C):
        sl = slice(c * C, (c + 1) * C)
        D = T[c] @ (v[sl] - k[sl] @ S)
        oc = q[sl] @ S + np.tril(q[sl] @ k[sl].T) @ D
        S = S + k[sl].T @ D
        np.testing.assert_allclose(oc, o[0, 0, sl], rtol=0, atol=1e-11)
    np.testing.assert_allclose(S, Sf[0, 0], rtol=0, atol=1e-11)


def _bwd_problem(rng, L=7, d_k=3, d_v=2, H=2):
    """Tiny inputs with a zero key, small and large beta lambda, and a random initial state."""
    k = np.stack([_mixed_keys(rng, L, d_k, 0.05, 3.0) for _ in range(H)])[None]
    k[0, 0, 2] = 0.0
    q = rng.standard_normal((1, H, L, d_k))
    v = rng.standard_normal((1, H, L, d_v))
    beta = rng.uniform(0.2, 0.9, (1, H, L))
    s0 = 0.5 * rng.standard_normal((1, H, d_k, d_v))
    do = rng.standard_normal((1, H, L, d_v))
    dsf = rng.standard_normal((1, H, d_k, d_v))
    return q, k, v, beta, s0, do, dsf


def check_bwd_finite_differences(orc):
    """Every gradient against central differences of the forward's loss sum(o * do) + sum(S_L * dS_L)."""
    rng = np.random.default_rng(41)
    for gate in (0, 3):
        q, k, v, beta, s0, do, dsf = _bwd_problem(rng)
        x = dict(q=q, k=k, v=v, beta=beta, s0=s0)

        def loss(xx):
            o, S, _ = orc.fwd(xx["q"], xx["k"], xx["v"], xx["beta"], xx["s0"], n_threads=1, gate=gate)
            return float(np.sum(o * do) + np.sum(S * dsf))

        g = dict(zip(("q", "k", "v", "beta", "s0"), orc.bwd(q, k, v, beta, s0, do, dsf, gate=gate)))
        for name, arr in x.items():
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                h = 1e-6 * max(1.0, abs(arr[idx]))
                xp = {n: a.copy() for n, a in x.items()}
                xm = {n: a.copy() for n, a in x.items()}
                xp[name][idx] += h
                xm[name][idx] -= h
                fd[idx] = (loss(xp) - loss(xm)) / (2 * h)
            scale = max(1.0, np.abs(fd).max())
            assert np.abs(g[name] - fd).max() <= 2e-7 * scale, (gate, name, np.abs(g[name] - fd).max())


def check_bwd_one_token(orc):
    """One token from S_0 = 0: o = alpha (k.q) v, so every gradient has a closed form."""
    rng = np.random.default_rng(42)
    for kscale in (0.1, 1.0, 3.0):
        d_k, d_v = 4, 3
        k = kscale * rng.standard_normal(d_k)
        q, v, do = rng.standard_normal(d_k), rng.standard_normal(d_v), rng.standard_normal(d_v)
        beta = 0.7
        lam = k @ k
        ex = np.exp(-beta * lam)
        a = (1 - ex) / lam
        da_db, da_dl = ex, -(a - beta * ex) / lam
        kq, vdo = k @ q, v @ do
        dq, dk, dv, db, ds0 = orc.bwd(q.reshape(1, 1, 1, d_k), k.reshape(1, 1, 1, d_k), v.reshape(1, 1, 1, d_v),
                                      np.array([[[beta]]]), None, do.reshape(1, 1, 1, d_v))
        np.testing.assert_allclose(dq[0, 0, 0], a * vdo * k, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dv[0, 0, 0], a * kq * do, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(db[0, 0, 0], kq * vdo * da_db, rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(dk[0, 0, 0], a * vdo * q + kq * vdo * 2 * k * da_dl, rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(ds0[0, 0], np.outer(q - a * kq * k, do), rtol=1e-12, atol=1e-13)


def check_bwd_linearity(orc):
    """The gradients are linear in the incoming gradients (do, dS_L)."""
    rng = np.random.default_rng(43)
    q, k, v, beta, s0, do1, ds1 = _bwd_problem(rng)
    do2, ds2 = rng.standard_normal(do1.shape), rng.standard_normal(ds1.shape)
    g1 = orc.bwd(q, k, v, beta, s0, do1, ds1)
    g2 = orc.bwd(q, k, v, beta, s0, do2, ds2)
    g3 = orc.bwd(q, k, v, beta, s0, 2 * do1 - 3 * do2, 2 * ds1 - 3 * ds2)
    for a1, a2, a3 in zip(g1, g2, g3):
        np.testing.assert_allclose(a3, 2 * a1 - 3 * a2, rtol=1e-10, atol=1e-11)


def check_bwd_state_chaining(orc):
    """Gradients over [0, L) equal those of the second half (from the first half's final state) followed by
    the first half with the second half's initial-state gradient as its final-state gradient."""
    rng = np.random.default_rng(44)
    q, k, v, beta, s0, do, dsf = _bwd_problem(rng, L=10)
    full = orc.bwd(q, k, v, beta, s0, do, dsf)
    m = 4
    _, Sm, _ = orc.fwd(q[:, :, :m], k[:, :, :m], v[:, :, :m], beta[:, :, :m], s0)
    second = orc.bwd(q[:, :, m:], k[:, :, m:], v[:, :, m:], beta[:, :, m:], Sm, do[:, :, m:], dsf)
    first = orc.bwd(q[:, :, :m], k[:, :, :m], v[:, :, :m], beta[:, :, :m], s0, do[:, :, :m], second[4])
    for i in range(4):
        np.testing.assert_allclose(full[i], np.concatenate([first[i], second[i]], axis=2), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(full[4], first[4], rtol=1e-11, atol=1e-12)


PINS = [check_worked_example, check_expm_erase, check_van_loan, check_rk4_sequence, check_alpha_extremes,
        check_euler_limit, check_directional_decay, check_stiff_overwrite, check_contractive,
        check_linearity, check_chunk_identity, check_state_chaining, check_zero_initial_state,
        check_ut_chunk_identity, check_ut_orthogonal_keys, check_gate_rk_tableaus, check_gate_limits,
        check_gate_chunk_identity, check_bwd_one_token, check_bwd_state_chaining, check_bwd_linearity,
        check_bwd_finite_differences]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle.default())


def test_oracle_mpmath_recurrence():
    """Rounding of the fp64 recurrence: a 40-digit mpmath run of the same tokens agrees to ~1e-14."""
    mpmath.mp.dps = 40
    rng = np.random.default_rng(22)
    L, d_k, d_v = 24, 4, 3
    k = _mixed_keys(rng, L, d_k, 1e-3, 8.0)
    q = rng.standard_normal((L, d_k))
    v = rng.standard_normal((L, d_v))
    beta = rng.uniform(0, 1, L)
    o, Sf, _ = oracle.fwd(q[None, None], k[None, None], v[None, None], beta[None, None])
    S = mpmath.zeros(d_k, d_v)
    for t in range(L):
        kt = mpmath.matrix([mpmath.mpf(x) for x in k[t]])
        lam = sum(x * x for x in kt)
        a = (1 - mpmath.exp(-mpmath.mpf(beta[t]) * lam)) / lam
        vt = mpmath.matrix([mpmath.mpf(x) for x in v[t]])
        kS = kt.T * S
        S = S - a * kt * kS + a * kt * vt.T
        ot = S.T * mpmath.matrix([mpmath.mpf(x) for x in q[t]])
        for j in range(d_v):
            assert abs(o[0, 0, t, j] - float(ot[j])) <= 1e-13
    for i in range(d_k):
        for j in range(d_v):
            assert abs(Sf[0, 0, i, j] - float(S[i, j])) <= 1e-13


def test_oracle_threads_do_not_change_results():
    w = W.workload(2, B=2, H=2, L=96)
    x = W.make_fwd_inputs(w)
    o1, s1, n1 = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["initial_state"], n_threads=1)
    o4, s4, n4 = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["initial_state"], n_threads=4)
    assert n1 == 1
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(s1, s4)


# ----------------------------------------------------------------------------------------------
# the pins must be able to fail: plausible mistakes planted in a copy of the oracle's C source
# ----------------------------------------------------------------------------------------------

MUTANTS = {
    "erase_sign": ("S[(size_t)i * d_v + j] - alpha * k[i] * kS[j]", "S[(size_t)i * d_v + j] + alpha * k[i] * kS[j]"),
    "write_dropped": ("- alpha * k[i] * kS[j] + alpha * k[i] * v[j];", "- alpha * k[i] * kS[j];"),
    "euler_alpha": ("return -expm1(-beta * lambda) / lambda;", "return beta;"),
    "no_divide": ("return -expm1(-beta * lambda) / lambda;", "return -expm1(-beta * lambda);"),
    "lambda_off_by_one": ("for (int i = 0; i < d_k; ++i)\n        lambda", "for (int i = 1; i < d_k; ++i)\n        lambda"),
    "readout_with_key": ("o[j] += S[(size_t)i * d_v + j] * q[i];", "o[j] += S[(size_t)i * d_v + j] * k[i];"),
    "readout_before_update": ("o[j] += S[(size_t)i * d_v + j] * q[i];",
                              "o[j] += (S[(size_t)i * d_v + j] + alpha * k[i] * kS[j] - alpha * k[i] * v[j]) * q[i];"),
    "exp_sign": ("return -expm1(-beta * lambda) / lambda;", "return expm1(beta * lambda) / lambda;"),
    "initial_state_ignored": ("memcpy(S, initial_state + bh * ssz, sizeof(double) * ssz);",
                              "memset(S, 0, sizeof(double) * ssz);"),
    "ut_substitution_sign": ("x -= A[(size_t)i * C + m] * T[(size_t)m * C + j];",
                             "x += A[(size_t)i * C + m] * T[(size_t)m * C + j];"),
    "ut_alpha_on_rows": ("T[(size_t)i * C + j] *= alpha[j];", "T[(size_t)i * C + j] *= alpha[i];"),
    "ut_gram_without_alpha": ("A[(size_t)i * C + j] = alpha[i] * dot;", "A[(size_t)i * C + j] = dot;"),
    "ut_gram_alpha_of_column": ("A[(size_t)i * C + j] = alpha[i] * dot;", "A[(size_t)i * C + j] = alpha[j] * dot;"),
    "ut_gram_wrong_key": ("dot += kc[(size_t)i * d_k + e] * kc[(size_t)j * d_k + e];",
                          "dot += kc[(size_t)i * d_k + e] * kc[(size_t)i * d_k + e];"),
    "ut_substitution_range": ("for (int m = 0; m < i; ++m)\n                        x -=",
                              "for (int m = 0; m + 1 < i; ++m)\n                        x -="),
    "rk_sign": ("(n % 2 == 1) ? 1.0 : -1.0", "(n % 2 == 0) ? 1.0 : -1.0"),
    "rk_order_short": ("for (int n = 1; n <= p; ++n)", "for (int n = 1; n < p; ++n)"),
    "rk_order_long": ("for (int n = 1; n <= p; ++n)", "for (int n = 1; n <= p + 1; ++n)"),
    "rk_factorial": ("factorial *= n;", "factorial *= (n > 1 ? n - 1 : 1);"),
    "rk_lambda_power": ("pow(lambda, n - 1)", "pow(lambda, n)"),
    "gate_ignored": ("    if (gate > 0)\n        return oracle_alpha_rk(beta, lambda, gate);\n", ""),
    "bwd_da_sign": ("da[j] = -alpha * w[j];", "da[j] = alpha * w[j];"),
    "bwd_state_grad_dropped": ("G[(size_t)i * d_v + j] += kt[i] * da[j];", ";"),
    "bwd_lambda_factor": ("dk[tok * d_k + i] = s + 2.0 * kt[i] * dlambda;", "dk[tok * d_k + i] = s + kt[i] * dlambda;"),
    "bwd_readout_previous_state": ("s += St[(size_t)i * d_v + j] * dot[j];", "s += Sp[(size_t)i * d_v + j] * dot[j];"),
    "bwd_dalpha_without_erase": ("dalpha += w[j] * e[j];", "dalpha += w[j] * vt[j];"),
    "bwd_dbeta_without_decay": ("*da_dbeta = exp(-x);", "*da_dbeta = 1.0;"),
    "bwd_series_sign": ("const double sign = (m % 2 == 1) ? 1.0 : -1.0;", "const double sign = (m % 2 == 0) ? 1.0 : -1.0;"),
    "bwd_closed_form_sign": ("g = (x * exp(-x) + expm1(-x)) / (x * x);", "g = (x * exp(-x) - expm1(-x)) / (x * x);"),
    "bwd_rk_lambda_power": ("pow(beta, n) * pow(lambda, n - 2)", "pow(beta, n) * pow(lambda, n - 1)"),
    "bwd_direct_dk_dropped": ("s += alpha * G[(size_t)i * d_v + j] * e[j] + Sp[(size_t)i * d_v + j] * da[j];",
                              "s += Sp[(size_t)i * d_v + j] * da[j];"),
    "bwd_readout_state_grad_dropped": ("G[(size_t)i * d_v + j] += qt[i] * dot[j];", ";"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutants(name):
    src_path = os.path.join(os.path.dirname(oracle.__file__), "efla_oracle.c")
    src = open(src_path).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor not found: " + name
    tmp = tempfile.mkdtemp(prefix="efla_mutant_")
    try:
        mpath = os.path.join(tmp, "mutant.c")
        with open(mpath, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.build(force=True, src=mpath, out=os.path.join(tmp, "libmutant.so"))
        orc = oracle.Oracle(lib)
        failed = []
        for pin in PINS:   # the first pin that fails is enough
            try:
                with np.errstate(all="ignore"):
                    pin(orc)
            except AssertionError:
                failed.append(pin.__name__)
                break
        assert failed, "no pin detects mutant " + name
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
