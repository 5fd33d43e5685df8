"""Pins of the CPU oracle against things other than itself.

Every check here compares the oracle with something it does not share code
with: brute force at 50 digits from the definition, closed forms of special
inputs, invariants of softmax attention, an independent library routine
(scipy's logsumexp) and central finite differences for the backward.  The
mutation tests at the end plant plausible mistakes in the oracle (on the
CPU) and show that at least one pin catches each of them.
"""

import itertools

import mpmath
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from oracle import attention as oatt

mpmath.mp.dps = 50

# ---------------------------------------------------------------- helpers


def _brute_force(q, k, v, scale, causal):
    """o_i = sum_j e^{s_ij} v_j / sum_j e^{s_ij}, L_i = ln sum_j e^{s_ij}, s = scale q_i.k_j.

    Plain Python loops over mpmath numbers at 50 digits; no max subtraction
    is needed at this precision.  q, k, v: [N, D] float arrays.
    """
    n, d = q.shape
    sc = mpmath.mpf(float(scale))
    o = np.empty((n, d))
    lse = np.empty(n)
    for i in range(n):
        weights = []
        for j in range(n):
            if causal and j > i:
                continue
            dot = mpmath.fsum(mpmath.mpf(float(q[i, t])) * mpmath.mpf(float(k[j, t])) for t in range(d))
            weights.append((j, mpmath.e ** (sc * dot)))
        z = mpmath.fsum(w for _, w in weights)
        for t in range(d):
            o[i, t] = float(mpmath.fsum(w * mpmath.mpf(float(v[j, t])) for j, w in weights) / z)
        lse[i] = float(mpmath.log(z))
    return o, lse


def _rand(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


def check_bruteforce(fwd=oracle.forward):
    """Oracle forward against brute force on tiny shapes, both causal modes."""
    for (n, d, mult), causal in itertools.product([(1, 1, 1.0), (3, 2, 1.0), (5, 4, 3.0), (6, 3, 8.0)], [False, True]):
        q, k, v = (_rand((n, d), 100 * n + 10 * d + s, mult) for s in range(3))
        scale = 1.0 / np.sqrt(d)
        o_ref, l_ref = _brute_force(q, k, v, scale, causal)
        o, l = fwd(q, k, v, scale, causal)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)
    # batched [B, H, N, D] entry: every slice is its own problem
    q, k, v = (_rand((2, 2, 4, 3), 7 + s) for s in range(3))
    o, l = fwd(q, k, v, 0.5, True)
    for b, h in itertools.product(range(2), range(2)):
        o_ref, l_ref = _brute_force(q[b, h], k[b, h], v[b, h], 0.5, True)
        np.testing.assert_allclose(o[b, h], o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l[b, h], l_ref, rtol=0, atol=1e-12)


def check_lse_library(fwd=oracle.forward):
    """L equals scipy's logsumexp of the (masked) score rows."""
    for causal in (False, True):
        q, k, v = (_rand((40, 16), 11 + s, 2.0) for s in range(3))
        scale = 0.25
        _, l = fwd(q, k, v, scale, causal)
        s = scale * (q @ k.T)
        if causal:
            s = np.where(np.tri(40, dtype=bool), s, -np.inf)
        np.testing.assert_allclose(l, logsumexp(s, axis=1), rtol=0, atol=1e-12)


def check_closed_forms(fwd=oracle.forward):
    n, d = 24, 8
    scale = 1.0 / np.sqrt(d)
    q = _rand((n, d), 21, 2.0)
    k = _rand((n, d), 22)
    v = _rand((n, d), 23)
    for causal in (False, True):
        # constant V: every output row is that row
        vc = np.tile(_rand((1, d), 24), (n, 1))
        o, _ = fwd(q, k, vc, scale, causal)
        np.testing.assert_allclose(o, vc, rtol=0, atol=1e-13)
        # identical keys: plain (prefix) mean of V; L = scale q.k + ln(count)
        kc = np.tile(_rand((1, d), 25), (n, 1))
        o, l = fwd(q, kc, v, scale, causal)
        counts = np.arange(1, n + 1) if causal else np.full(n, n)
        mean = np.cumsum(v, axis=0) / counts[:, None] if causal else np.tile(v.mean(axis=0), (n, 1))
        np.testing.assert_allclose(o, mean, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, scale * (q @ kc[0]) + np.log(counts), rtol=0, atol=1e-12)
        # Q = 0: uniform weights
        o, l = fwd(np.zeros_like(q), k, v, scale, causal)
        np.testing.assert_allclose(o, mean, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, np.log(counts), rtol=0, atol=1e-13)
    # causal row 0 sees only key 0
    o, l = fwd(q, k, v, scale, True)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(l[0], scale * q[0] @ k[0], rtol=0, atol=1e-13)


def check_invariants(fwd=oracle.forward):
    n, d = 32, 8
    scale = 0.3
    q, k, v = (_rand((n, d), 31 + s, 2.0) for s in range(3))
    u = _rand((d,), 34, 5.0)
    for causal in (False, True):
        o, l = fwd(q, k, v, scale, causal)
        # shift of every key by u: O unchanged, L_i moves by scale q_i.u
        o2, l2 = fwd(q, k + u, v, scale, causal)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, l + scale * (q @ u), rtol=0, atol=1e-11)
        # permuting query rows permutes the outputs (keys fixed)
        if not causal:
            perm = np.random.default_rng(35).permutation(n)
            o3, l3 = fwd(q[perm], k, v, scale, causal)
            np.testing.assert_allclose(o3, o[perm], rtol=0, atol=1e-13)
            np.testing.assert_allclose(l3, l[perm], rtol=0, atol=1e-13)
            # joint permutation of key and value rows changes nothing
            o4, l4 = fwd(q, k[perm], v[perm], scale, causal)
            np.testing.assert_allclose(o4, o, rtol=0, atol=1e-13)
            np.testing.assert_allclose(l4, l, rtol=0, atol=1e-13)
        # causal prefix: rows < m only see keys < m
        if causal:
            m = 13
            o5, l5 = fwd(q[:m], k[:m], v[:m], scale, causal)
            np.testing.assert_allclose(o5, o[:m], rtol=0, atol=1e-13)
            np.testing.assert_allclose(l5, l[:m], rtol=0, atol=1e-13)


def check_probabilities(probs=oracle.probabilities):
    n, d = 20, 6
    q, k = _rand((n, d), 41, 3.0), _rand((n, d), 42)
    for causal in (False, True):
        p = probs(q, k, 0.4, causal)
        assert p.shape == (n, n)
        assert (p >= 0).all()
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        if causal:
            assert (p[np.triu_indices(n, 1)] == 0).all()
        s = 0.4 * (q @ k.T)
        if causal:
            s = np.where(np.tri(n, dtype=bool), s, -np.inf)
        np.testing.assert_allclose(p, np.exp(s - logsumexp(s, axis=1)[:, None]), rtol=0, atol=1e-13)


def _fd_grad(f, x, h=1e-6):
    g = np.empty_like(x)
    for idx in np.ndindex(*x.shape):
        old = x[idx]
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


def check_backward_fd(bwd=oracle.backward, fwd=oracle.forward):
    """dQ, dK, dV against central differences of F = sum(O * dO)."""
    n, d = 16, 8
    scale = 1.0 / np.sqrt(d)
    for causal in (False, True):
        q, k, v, do = (_rand((n, d), 51 + s + 10 * causal) for s in range(4))
        g = bwd(q, k, v, do, scale, causal)

        def f():
            return float((fwd(q, k, v, scale, causal)[0] * do).sum())

        for name, x in (("dq", q), ("dk", k), ("dv", v)):
            num = _fd_grad(f, x)
            err = np.abs(g[name] - num).max() / np.abs(num).max()
            assert err <= 1e-6, (name, causal, err)
        # the backward's own O and L agree with the forward's
        o, l = fwd(q, k, v, scale, causal)
        np.testing.assert_allclose(g["o"], o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(g["lse"], l, rtol=0, atol=1e-13)


def check_backward_identities(bwd=oracle.backward, probs=oracle.probabilities):
    n, d = 24, 8
    scale = 0.35
    q, k, v, do = (_rand((n, d), 61 + s, 1.5) for s in range(4))
    for causal in (False, True):
        g = bwd(q, k, v, do, scale, causal)
        # sum_j dK_j = 0 (each row of dS sums to 0) and sum_j dV_j = sum_i dO_i
        np.testing.assert_allclose(g["dk"].sum(axis=0), 0.0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(g["dv"].sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-12)
        # delta_i = sum_d dO_id O_id = sum_j P_ij (dO V^T)_ij
        p = probs(q, k, scale, causal)
        np.testing.assert_allclose(g["delta"], (p * (do @ v.T)).sum(axis=1), rtol=0, atol=1e-12)
        np.testing.assert_allclose(g["delta"], (do * (p @ v)).sum(axis=1), rtol=0, atol=1e-12)
        # identical keys: the scores do not depend on q, so dQ = 0
        kc = np.tile(k[:1], (n, 1))
        g2 = bwd(q, kc, v, do, scale, causal)
        np.testing.assert_allclose(g2["dq"], 0.0, rtol=0, atol=1e-13)
        # constant V: O does not depend on q or k, so dQ = dK = 0
        vc = np.tile(v[:1], (n, 1))
        g3 = bwd(q, k, vc, do, scale, causal)
        np.testing.assert_allclose(g3["dq"], 0.0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(g3["dk"], 0.0, rtol=0, atol=1e-12)
    # batched entry equals per-head calls
    q4, k4, v4, do4 = (_rand((1, 2, 8, 4), 70 + s) for s in range(4))
    gb = bwd(q4, k4, v4, do4, 0.5, True)
    for h in range(2):
        gh = bwd(q4[0, h], k4[0, h], v4[0, h], do4[0, h], 0.5, True)
        for name in ("dq", "dk", "dv", "delta", "lse"):
            np.testing.assert_allclose(gb[name][0, h], gh[name], rtol=0, atol=0)


def check_online(fwd=oracle.forward, online=oracle.online_forward):
    """The streaming recurrence reaches the two-pass definition."""
    for causal, (qt, kt) in itertools.product((False, True), ((8, 4), (5, 7), (64, 64), (1, 1))):
        q, k, v = (_rand((37, 12), 81 + s, 4.0) for s in range(3))
        o_ref, l_ref = fwd(q, k, v, 0.2, causal)
        o, l = online(q, k, v, 0.2, causal, q_tile=qt, k_tile=kt)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ tests


def test_forward_bruteforce():
    check_bruteforce()


def test_lse_against_scipy():
    check_lse_library()


def test_closed_forms():
    check_closed_forms()


def test_invariants():
    check_invariants()


def test_probabilities():
    check_probabilities()


def test_backward_finite_differences():
    check_backward_fd()


def test_backward_identities():
    check_backward_identities()


def test_online_recurrence_matches_definition():
    check_online()


def test_forward_rows_subset_matches_full():
    q, k, v = (_rand((1, 2, 300, 16), 90 + s) for s in range(3))
    for causal in (False, True):
        o, l = oracle.forward(q, k, v, 0.25, causal, row_block=64)
        o2, l2 = oracle.forward(q, k, v, 0.25, causal, row_block=1000)
        np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)
        rows = np.array([0, 1, 63, 64, 150, 299])
        o3, l3 = oracle.forward_rows(q[0, 1], k[0, 1], v[0, 1], rows, 0.25, causal)
        np.testing.assert_allclose(o3, o[0, 1, rows], rtol=0, atol=1e-14)
        np.testing.assert_allclose(l3, l[0, 1, rows], rtol=0, atol=1e-14)


# --------------------------------------------------------- planted mistakes
#
# Each mutant is a plausible slip in the oracle.  The test installs it on
# the CPU, runs the pins and requires that at least one of them fails.


def _mut_no_scale(q_rows, k, rows, scale, causal):
    return _ORIG_SCORES(q_rows, k, rows, 1.0, causal)


def _mut_causal_flipped(q_rows, k, rows, scale, causal):
    s = _ORIG_SCORES(q_rows, k, rows, scale, False)
    if causal:
        cols = np.arange(s.shape[1])
        s = np.where(cols[None, :] < rows[:, None], s, -np.inf)
        s[:, 0] = scale * (q_rows @ k[0])  # keep row 0 finite
    return s


def _mut_transposed(q_rows, k, rows, scale, causal):
    s = _ORIG_SCORES(q_rows, k, rows, scale, causal)
    if s.shape[0] == s.shape[1]:
        s = s.T.copy()
    return s


def _mut_lse_no_max(s):
    p, m, l = _ORIG_SOFTMAX(s)
    return p, np.zeros_like(m), l


def _mut_max_sign(s):
    m = s.max(axis=1)
    e = np.exp(s + m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def _mut_unnormalised(s):
    p, m, l = _ORIG_SOFTMAX(s)
    return p * l[:, None] / l.max(), m, l


_ORIG_SCORES = oatt._scores
_ORIG_SOFTMAX = oatt._softmax_two_pass


@pytest.mark.parametrize(
    "target,mutant",
    [
        ("_scores", _mut_no_scale),
        ("_scores", _mut_causal_flipped),
        ("_scores", _mut_transposed),
        ("_softmax_two_pass", _mut_lse_no_max),
        ("_softmax_two_pass", _mut_max_sign),
        ("_softmax_two_pass", _mut_unnormalised),
    ],
)
def test_forward_pins_catch_planted_mistake(monkeypatch, target, mutant):
    monkeypatch.setattr(oatt, target, mutant)
    caught = 0
    for check in (check_bruteforce, check_closed_forms, check_lse_library, check_probabilities):
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught >= 1, "no pin caught the planted mistake"


def _bwd_mutant(kind):
    orig = oatt.backward

    def wrapped(q, k, v, do, scale, causal=False):
        g = orig(q, k, v, do, scale, causal)
        if kind == "dk_no_scale":
            g["dk"] = g["dk"] / scale
        elif kind == "dv_transposed_p":  # dV = P dO instead of P^T dO
            p = oatt.probabilities(q, k, scale, causal)
            g["dv"] = p @ np.asarray(do, dtype=np.float64)
        elif kind == "ds_sign":  # dS = P (delta - dP)
            g["dq"] = -g["dq"]
        elif kind == "delta_dropped":  # dS = P dP
            p = oatt.probabilities(q, k, scale, causal)
            ds = p * (np.asarray(do, dtype=np.float64) @ np.asarray(v, dtype=np.float64).T)
            g["dq"] = scale * ds @ np.asarray(k, dtype=np.float64)
        return g

    return wrapped


@pytest.mark.parametrize("kind", ["dk_no_scale", "dv_transposed_p", "ds_sign", "delta_dropped"])
def test_backward_pins_catch_planted_mistake(kind):
    mutant = _bwd_mutant(kind)
    caught = 0
    for check in (lambda: check_backward_fd(bwd=mutant), lambda: check_backward_identities(bwd=mutant)):
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught >= 1
