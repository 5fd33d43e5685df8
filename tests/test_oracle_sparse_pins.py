"""Pins of ``oracle.forward_block_sparse`` (attention restricted to the
(query block, key block) pairs of a block mask).

The pins compare the oracle with things it shares no code with: brute force
at 50 digits from the definition with the mask applied element by element,
the square oracle (pinned in test_oracle_pins.py) for the all-ones mask and
the block-causal mask, ``forward_kv`` (pinned in test_oracle_kv_pins.py) for
a mask that keeps one key block, the independence of query blocks, rows
that see no key, and the exact merge of two disjoint masks.  Planted
mistakes at the end are each caught.
"""

import itertools

import mpmath
import numpy as np
import pytest

import oracle

mpmath.mp.dps = 50


def _rand(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


def _brute_force_sparse(q, k, v, scale, causal, mask, block):
    """Plain loops at 50 digits: key j is visible to query i iff
    mask[i // block][j // block] != 0 and (not causal or j <= i); a row with
    no visible key gives O = 0, L = -inf."""
    n, d = q.shape
    sc = mpmath.mpf(float(scale))
    o = np.zeros((n, d))
    lse = np.full(n, -np.inf)
    for i in range(n):
        weights = []
        for j in range(n):
            if not mask[i // block][j // block] or (causal and j > i):
                continue
            dot = mpmath.fsum(mpmath.mpf(float(q[i, t])) * mpmath.mpf(float(k[j, t])) for t in range(d))
            weights.append((j, mpmath.e ** (sc * dot)))
        if not weights:
            continue
        z = mpmath.fsum(w for _, w in weights)
        for t in range(d):
            o[i, t] = float(mpmath.fsum(w * mpmath.mpf(float(v[j, t])) for j, w in weights) / z)
        lse[i] = float(mpmath.log(z))
    return o, lse


def _masks(nb, seed):
    rng = np.random.default_rng(seed)
    yield np.ones((nb, nb), dtype=np.uint8)
    yield (rng.random((nb, nb)) < 0.5).astype(np.uint8)
    m = (rng.random((nb, nb)) < 0.6).astype(np.uint8)
    m[0] = 0  # a query block that sees nothing
    yield m
    yield np.triu(np.ones((nb, nb), dtype=np.uint8), 1)  # only blocks above the diagonal


def check_sparse_bruteforce(fwd=oracle.forward_block_sparse):
    for (n, d, block), causal in itertools.product([(5, 3, 2), (7, 2, 3), (6, 4, 2)], [False, True]):
        q = _rand((n, d), 900 + n, 2.0)
        k = _rand((n, d), 910 + n)
        v = _rand((n, d), 920 + n)
        nb = -(-n // block)
        for mi, mask in enumerate(_masks(nb, 930 + n)):
            o_ref, l_ref = _brute_force_sparse(q, k, v, 0.5, causal, mask, block)
            o, l = fwd(q, k, v, 0.5, causal, mask, block=block)
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
            np.testing.assert_array_equal(np.isinf(l), np.isinf(l_ref))
            fin = np.isfinite(l_ref)
            np.testing.assert_allclose(l[fin], l_ref[fin], rtol=0, atol=1e-12)


def check_sparse_special_masks(fwd=oracle.forward_block_sparse):
    n, d, block = 40, 8, 8
    nb = n // block
    q, k, v = (_rand((2, 3, n, d), 940 + s, 1.5) for s in range(3))
    for causal in (False, True):
        # every block kept: the square definition
        o_sq, l_sq = oracle.forward(q, k, v, 0.3, causal)
        o, l = fwd(q, k, v, 0.3, causal, np.ones((nb, nb)), block=block)
        np.testing.assert_allclose(o, o_sq, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, l_sq, rtol=0, atol=1e-13)
    # blocks on and below the diagonal with the causal mask: the causal definition
    o_c, l_c = oracle.forward(q, k, v, 0.3, True)
    o, l = fwd(q, k, v, 0.3, True, np.tril(np.ones((nb, nb))), block=block)
    np.testing.assert_allclose(o, o_c, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, l_c, rtol=0, atol=1e-13)
    # one key block kept for every query block: attention over that key slice
    for c in (0, 2, nb - 1):
        mask = np.zeros((nb, nb))
        mask[:, c] = 1
        o, l = fwd(q, k, v, 0.3, False, mask, block=block)
        sl = slice(c * block, (c + 1) * block)
        o_kv, l_kv = oracle.forward_kv(q, k[:, :, sl], v[:, :, sl], 0.3, False)
        np.testing.assert_allclose(o, o_kv, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, l_kv, rtol=0, atol=1e-13)
    # no block kept: O = 0, L = -inf everywhere
    o, l = fwd(q, k, v, 0.3, False, np.zeros((nb, nb)), block=block)
    assert (o == 0).all() and np.isneginf(l).all()


def check_sparse_rows_and_heads(fwd=oracle.forward_block_sparse):
    """Query block a depends on mask row a only; per-head masks act per head."""
    n, d, block = 48, 4, 16
    nb = n // block
    q, k, v = (_rand((1, 2, n, d), 950 + s) for s in range(3))
    rng = np.random.default_rng(955)
    m1 = (rng.random((nb, nb)) < 0.5).astype(np.uint8)
    m1[:, 0] = 1
    m2 = m1.copy()
    m2[1] = 1 - m2[1]  # change row 1 only
    for causal in (False, True):
        o1, l1 = fwd(q, k, v, 0.4, causal, m1, block=block)
        o2, l2 = fwd(q, k, v, 0.4, causal, m2, block=block)
        keep = np.r_[0:block, 2 * block : n]
        np.testing.assert_array_equal(o1[:, :, keep], o2[:, :, keep])
        np.testing.assert_array_equal(l1[:, :, keep], l2[:, :, keep])
        # a [B*H, nb, nb] mask: head h uses its own mask
        o_h, l_h = fwd(q, k, v, 0.4, causal, np.stack([m1, m2]), block=block)
        np.testing.assert_array_equal(o_h[:, 0], o1[:, 0])
        np.testing.assert_array_equal(o_h[:, 1], o2[:, 1])


def check_sparse_merge(fwd=oracle.forward_block_sparse):
    """Two disjoint masks merge by log-sum-exp into their union."""
    n, d, block = 36, 5, 6
    nb = n // block
    q, k, v = (_rand((n, d), 960 + s, 2.0) for s in range(3))
    rng = np.random.default_rng(965)
    for causal in (False, True):
        m = (rng.random((nb, nb)) < 0.7).astype(np.uint8)
        split = (rng.random((nb, nb)) < 0.5).astype(np.uint8)
        m1, m2 = m * split, m * (1 - split)
        o, l = fwd(q, k, v, 0.5, causal, m, block=block)
        o1, l1 = fwd(q, k, v, 0.5, causal, m1, block=block)
        o2, l2 = fwd(q, k, v, 0.5, causal, m2, block=block)
        with np.errstate(invalid="ignore"):
            mx = np.maximum(l1, l2)
            fin = np.isfinite(mx)
            lm = np.full(n, -np.inf)
            lm[fin] = mx[fin] + np.log(np.exp(l1[fin] - mx[fin]) + np.exp(l2[fin] - mx[fin]))
            w1 = np.where(np.isfinite(l1), np.exp(l1 - np.where(fin, lm, 0)), 0.0)
            w2 = np.where(np.isfinite(l2), np.exp(l2 - np.where(fin, lm, 0)), 0.0)
        om = w1[:, None] * o1 + w2[:, None] * o2
        np.testing.assert_allclose(om, o, rtol=0, atol=1e-13)
        np.testing.assert_array_equal(np.isinf(lm), np.isinf(l))
        np.testing.assert_allclose(lm[fin], l[fin], rtol=0, atol=1e-13)


CHECKS = (check_sparse_bruteforce, check_sparse_special_masks, check_sparse_rows_and_heads, check_sparse_merge)


def test_sparse_bruteforce():
    check_sparse_bruteforce()


def test_sparse_special_masks():
    check_sparse_special_masks()


def test_sparse_rows_and_heads():
    check_sparse_rows_and_heads()


def test_sparse_merge():
    check_sparse_merge()


# --------------------------------------------------------- planted mistakes


def _sparse_mutant(kind):
    exact = oracle.forward_block_sparse

    def f(q, k, v, scale, causal, block_mask, block=64):
        mask = np.asarray(block_mask)
        if kind == "transposed_mask":
            mask = np.swapaxes(mask, -1, -2)
        elif kind == "causal_ignored":
            causal = False
        elif kind == "block_shift":  # rows of block a use mask row a+1
            mask = np.roll(mask, -1, axis=-2)
        o, l = exact(q, k, v, scale, causal, mask, block=block)
        if kind == "empty_rows_nan":
            o = np.where(np.isinf(l)[..., None], np.nan, o)
        return o, l

    return f


@pytest.mark.parametrize("kind", ["transposed_mask", "causal_ignored", "block_shift", "empty_rows_nan"])
def test_sparse_pins_catch_planted_mistake(kind):
    mutant = _sparse_mutant(kind)
    caught = 0
    for check in CHECKS:
        try:
            check(fwd=mutant)
        except AssertionError:
            caught += 1
    assert caught >= 1, "no pin caught the planted mistake"
