"""Pins of ``oracle.forward_kv`` (query and key lengths apart).

The pins compare the oracle with things it shares no code with: brute force
at 50 digits from the definition, the square oracle (itself pinned in
test_oracle_pins.py) through the suffix property that defines the causal
alignment, closed forms, and the exact merge of results over disjoint key
ranges.  Planted mistakes at the end (a top-left alignment, an alignment
off by one, keys cut to the query length) are each caught.
"""

import itertools

import mpmath
import numpy as np
import pytest

import oracle

mpmath.mp.dps = 50


def _rand(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


def _brute_force_kv(q, k, v, scale, causal):
    """Plain loops at 50 digits: query i sees key j iff (not causal) or
    j <= i + (Nk - Nq); o_i = sum_j e^{s_ij} v_j / sum_j e^{s_ij},
    L_i = ln sum_j e^{s_ij}, s_ij = scale q_i . k_j."""
    nq, d = q.shape
    nk = k.shape[0]
    sc = mpmath.mpf(float(scale))
    o = np.empty((nq, d))
    lse = np.empty(nq)
    for i in range(nq):
        weights = []
        for j in range(nk):
            if causal and j > i + (nk - nq):
                continue
            dot = mpmath.fsum(mpmath.mpf(float(q[i, t])) * mpmath.mpf(float(k[j, t])) for t in range(d))
            weights.append((j, mpmath.e ** (sc * dot)))
        z = mpmath.fsum(w for _, w in weights)
        for t in range(d):
            o[i, t] = float(mpmath.fsum(w * mpmath.mpf(float(v[j, t])) for j, w in weights) / z)
        lse[i] = float(mpmath.log(z))
    return o, lse


def check_kv_bruteforce(fwd=oracle.forward_kv):
    shapes = [(1, 1, 2), (1, 5, 3), (2, 5, 4), (3, 4, 2), (4, 4, 3), (6, 2, 3)]  # (Nq, Nk, D)
    for (nq, nk, d), causal in itertools.product(shapes, [False, True]):
        if causal and nq > nk:
            continue
        q = _rand((nq, d), 300 + 10 * nq + nk, 2.0)
        k = _rand((nk, d), 400 + 10 * nq + nk)
        v = _rand((nk, d), 500 + 10 * nq + nk)
        scale = 1.0 / np.sqrt(d)
        o_ref, l_ref = _brute_force_kv(q, k, v, scale, causal)
        o, l = fwd(q, k, v, scale, causal)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)


def check_kv_square_and_suffix(fwd=oracle.forward_kv):
    """Nq = Nk is the square definition; under either mask the rows of a
    query suffix are the last rows of the square problem over all keys."""
    n, d = 37, 8
    q, k, v = (_rand((2, 1, n, d), 60 + s, 1.5) for s in range(3))
    for causal in (False, True):
        o_sq, l_sq = oracle.forward(q, k, v, 0.35, causal)
        o, l = fwd(q, k, v, 0.35, causal)
        np.testing.assert_allclose(o, o_sq, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, l_sq, rtol=0, atol=1e-13)
        for nq in (1, 2, 9, 36):
            o, l = fwd(q[:, :, n - nq :], k, v, 0.35, causal)
            np.testing.assert_allclose(o, o_sq[:, :, n - nq :], rtol=0, atol=1e-13)
            np.testing.assert_allclose(l, l_sq[:, :, n - nq :], rtol=0, atol=1e-13)


def check_kv_closed_forms(fwd=oracle.forward_kv):
    nq, nk, d = 5, 19, 4
    scale = 0.5
    q = _rand((nq, d), 71, 2.0)
    k = _rand((nk, d), 72)
    v = _rand((nk, d), 73)
    # one decoded row under the causal mask sees every key
    o1, l1 = fwd(q[-1:], k, v, scale, True)
    o2, l2 = fwd(q[-1:], k, v, scale, False)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-15)
    for causal in (False, True):
        counts = np.arange(nk - nq + 1, nk + 1) if causal else np.full(nq, nk)
        # constant V
        vc = np.tile(_rand((1, d), 74), (nk, 1))
        o, _ = fwd(q, k, vc, scale, causal)
        np.testing.assert_allclose(o, vc[:nq], rtol=0, atol=1e-13)
        # identical keys: mean of the visible V rows, L = scale q.k + ln(count)
        kc = np.tile(_rand((1, d), 75), (nk, 1))
        o, l = fwd(q, kc, v, scale, causal)
        mean = np.stack([v[:c].mean(axis=0) for c in counts])
        np.testing.assert_allclose(o, mean, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, scale * (q @ kc[0]) + np.log(counts), rtol=0, atol=1e-12)


def check_kv_range_merge(fwd=oracle.forward_kv):
    """Results over disjoint key ranges merge exactly:
    L = ln sum_s e^{L_s}, O = sum_s e^{L_s - L} O_s (the combination a
    key-split kernel performs)."""
    nq, nk, d = 7, 50, 6
    q, k, v = _rand((nq, d), 81, 2.0), _rand((nk, d), 82), _rand((nk, d), 83)
    o_all, l_all = fwd(q, k, v, 0.4, False)
    for cuts in ([0, 50], [0, 1, 50], [0, 13, 26, 49, 50], list(range(0, 51, 5))):
        parts = [fwd(q, k[a:b], v[a:b], 0.4, False) for a, b in zip(cuts[:-1], cuts[1:])]
        ls = np.stack([p[1] for p in parts])
        l = np.log(np.exp(ls).sum(axis=0))
        o = sum(np.exp(p[1] - l)[:, None] * p[0] for p in parts)
        np.testing.assert_allclose(l, l_all, rtol=0, atol=1e-13)
        np.testing.assert_allclose(o, o_all, rtol=0, atol=1e-13)


def test_kv_bruteforce():
    check_kv_bruteforce()


def test_kv_square_and_suffix():
    check_kv_square_and_suffix()


def test_kv_closed_forms():
    check_kv_closed_forms()


def test_kv_range_merge():
    check_kv_range_merge()


def test_kv_rejects_causal_with_more_queries_than_keys():
    with pytest.raises(ValueError):
        oracle.forward_kv(np.zeros((4, 2)), np.zeros((3, 2)), np.zeros((3, 2)), 1.0, True)


# --------------------------------------------------------- planted mistakes


def _kv_mutant(kind):
    """forward_kv with one plausible slip in its mask."""

    def f(q, k, v, scale, causal=False):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        single = q.ndim == 2
        if single:
            q, k, v = q[None, None], k[None, None], v[None, None]
        nq, nk = q.shape[2], k.shape[2]
        if kind == "keys_cut":
            k, v, nk = k[:, :, :nq], v[:, :, :nq], min(nk, nq)
        offset = {"top_left": 0, "off_by_one": nk - nq - 1}.get(kind, nk - nq)
        s = scale * np.einsum("bhid,bhjd->bhij", q, k)
        if causal:
            vis = np.arange(nk)[None, :] <= np.arange(nq)[:, None] + offset
            vis[:, 0] = True  # keep every row finite
            s = np.where(vis, s, -np.inf)
        m = s.max(axis=-1, keepdims=True)
        e = np.exp(s - m)
        lsum = e.sum(axis=-1, keepdims=True)
        o = (e / lsum) @ v
        lse = (m + np.log(lsum))[..., 0]
        return (o[0, 0], lse[0, 0]) if single else (o, lse)

    return f


@pytest.mark.parametrize("kind", ["top_left", "off_by_one", "keys_cut"])
def test_kv_pins_catch_planted_mistake(kind):
    mutant = _kv_mutant(kind)
    caught = 0
    for check in (check_kv_bruteforce, check_kv_square_and_suffix, check_kv_closed_forms, check_kv_range_merge):
        try:
            check(fwd=mutant)
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1, "no pin caught the planted mistake"


def test_kv_mutant_harness_is_faithful():
    """The mutant harness with no slip passes every pin (so a caught
    mutant is caught for its slip, not for the harness)."""
    exact = _kv_mutant("none")
    for check in (check_kv_bruteforce, check_kv_square_and_suffix, check_kv_closed_forms, check_kv_range_merge):
        check(fwd=exact)
