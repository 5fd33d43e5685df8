"""GPU parity of ``fa_fwd_kv`` (query and key lengths apart, split key
ranges merged on the GPU) against the float64 oracle ``forward_kv``.

Inputs are the seeded draws of ``fa_inputs.make_inputs`` at the key length;
the query rows are the last Nq rows of the drawn Q (the positions a causal
query block holds when it is the end of the sequence).  Cases cover one
decoded row over long key sequences, ragged lengths, fewer keys than a tile,
more key ranges than key tiles (empty ranges), causal ranges that some rows
of a block do not reach, more queries than keys without a mask, peaked rows,
each head dimension, the vector decode kernel that serves up to four query
rows, and the pages' benchmark shape with the library's own split count.
"""

import numpy as np
import pytest

import oracle
from fa_inputs import WORKLOADS, make_inputs
from tests._gpu import TOL_BF16_L, TOL_BF16_O, dev_bf16, host, log

pytestmark = pytest.mark.gpu


def _fa():
    import exact_attention_51_amd as fa

    return fa


def _inputs(B, H, Nq, Nk, D, seed, q_mult=1.0):
    w = WORKLOADS["c3"].with_(B=B, H=H, N=Nk, D=D, q_mult=q_mult)
    x = make_inputs(w, seed=seed, with_do=False)
    qb = np.ascontiguousarray(x.q_bits[:, :, Nk - Nq :]) if Nq <= Nk else None
    q = np.ascontiguousarray(x.q[:, :, Nk - Nq :]) if Nq <= Nk else None
    if Nq > Nk:  # more queries than keys: draw the queries at their own length
        wq = w.with_(N=Nq)
        xq = make_inputs(wq, seed=seed + 1000, with_do=False)
        q, qb = xq.q, xq.q_bits
    return w.scale, q, qb, x.k, x.k_bits, x.v, x.v_bits


def _run_and_check(B, H, Nq, Nk, D, causal, splits, seed=21, q_mult=1.0):
    import torch

    log(f"fwd_kv B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} splits={splits} seed={seed}")
    scale, q, qb, k, kb, v, vb = _inputs(B, H, Nq, Nk, D, seed, q_mult)
    o, lse = _fa().fwd_kv(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), scale, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward_kv(q, k, v, scale, causal)
    oh, lh = host(o), host(lse)
    assert np.isfinite(oh).all() and np.isfinite(lh).all()
    eo = float(np.abs(oh - o_ref).max())
    el = float(np.abs(lh - l_ref).max())
    log(f"  max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= TOL_BF16_O and el <= TOL_BF16_L, (eo, el)
    return o, lse


CASES = [
    # (B, H, Nq, Nk, D, causal, splits)
    (2, 4, 1, 4096, 128, True, 0),  # one decoded row, the library's split count
    (1, 3, 1, 5000, 128, False, 16),  # ragged key length
    (2, 2, 7, 1000, 64, True, 5),
    (1, 2, 5, 333, 256, True, 3),
    (1, 2, 3, 40, 64, False, 2),  # fewer keys than a tile
    (1, 1, 1, 1, 128, True, 1),  # one key
    (1, 2, 16, 100, 128, True, 8),  # more ranges than key tiles: empty ranges
    (1, 2, 300, 1000, 128, True, 8),  # ranges some rows of a block do not reach
    (1, 2, 300, 1000, 64, True, 6),
    (1, 2, 130, 700, 256, True, 4),
    (1, 2, 300, 100, 128, False, 3),  # more queries than keys, no mask
    (1, 2, 512, 512, 128, True, 4),  # equal lengths, split
    (1, 4, 200, 3000, 64, False, 0),
    (1, 2, 64, 4096, 128, True, 12),  # more than 8 ranges: the wide merge
    (2, 1, 33, 3000, 256, False, 20),
    # up to four query rows run on the vector decode kernel
    (1, 2, 4, 777, 64, True, 3),  # causal: the last three keys are partly masked
    (2, 2, 2, 1500, 256, True, 0),
    (1, 2, 3, 2049, 128, True, 1),  # one key range: O and L written directly
    (1, 2, 2, 130, 128, False, 12),  # more ranges than 64-key chunks: empty ranges
    (1, 1, 4, 4, 256, True, 2),  # as many keys as rows: row r sees keys 0..r
    (3, 5, 1, 20000, 64, True, 0),
    # head dims 96 and 160 (matrix-core kernel also for up to four rows)
    (1, 2, 300, 1000, 96, True, 6),
    (1, 2, 2, 3000, 96, True, 0),
    (1, 2, 130, 700, 160, True, 4),
    (2, 1, 1, 5000, 160, False, 0),
    (1, 2, 40, 3000, 160, False, 12),
    (1, 2, 300, 1000, 32, True, 6),
    (2, 2, 3, 2500, 32, False, 0),
]


@pytest.mark.parametrize("B,H,Nq,Nk,D,causal,splits", CASES)
def test_forward_kv(B, H, Nq, Nk, D, causal, splits):
    _run_and_check(B, H, Nq, Nk, D, causal, splits)


@pytest.mark.parametrize("splits", [1, 2, 7])
def test_forward_kv_peaked_rows(splits):
    """Q x 3 (peaked softmax rows): the merge rescales ranges whose maxima
    differ by a lot."""
    _run_and_check(1, 2, 64, 4096, 128, True, splits, seed=4, q_mult=3.0)


@pytest.mark.parametrize("D,causal,H", [(64, False, 60), (128, True, 256), (256, True, 256)])
def test_forward_kv_unsplit_equals_square_forward(D, causal, H):
    """With Nq = Nk and one key range the kernel does the square forward's
    arithmetic in the same order: the results are bitwise equal.  (At D =
    128, enough heads that the square forward keeps its full-size
    workgroups: small D = 128 grids take 128-row workgroups, which visit the
    causal diagonal tiles in another order.  At D = 64, a grid smaller than
    the device: larger ones run the square forward's own D = 64 kernel,
    whose row sums add the rounded P in another order.)"""
    import torch

    scale, _, qb, _, kb, _, vb = _inputs(2, H, 300, 300, D, 31)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o1, l1 = _fa().fwd(q, k, v, scale, causal=causal)
    o2, l2 = _fa().fwd_kv(q, k, v, scale, causal=causal, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_kv_pages_shape(causal):
    """The pages' benchmark shape, B=2 H=4 N=2048 D=128, with the library's
    split count (its grid of 64 query blocks fills a quarter of the CUs)."""
    fa = _fa()
    s = fa.kv_splits(2, 4, 2048, 2048, 128, causal)
    log(f"library split count for the pages' shape: {s}")
    assert s > 1
    _run_and_check(2, 4, 2048, 2048, 128, causal, 0, seed=51)


def test_forward_kv_workspace_reuse():
    """One caller-owned workspace serves two calls in a row, the second
    smaller; results match the oracle both times."""
    import torch

    fa = _fa()
    need = fa._lib.load().fa_fwd_kv_workspace_bytes(2, 2, 40, 128, 6)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for Nq, Nk, seed in ((40, 2000, 61), (9, 900, 62)):
        scale, q, qb, k, kb, v, vb = _inputs(2, 2, Nq, Nk, 128, seed)
        o, lse = fa.fwd_kv(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), scale, causal=True, num_splits=6, workspace=ws)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.forward_kv(q, k, v, scale, True)
        assert float(np.abs(host(o) - o_ref).max()) <= TOL_BF16_O
        assert float(np.abs(host(lse) - l_ref).max()) <= TOL_BF16_L


def test_forward_kv_long_decode_sampled_heads():
    """One decoded row per head over 32768 keys (the long-context key
    length), B=1 H=8, with the library's split count."""
    _run_and_check(1, 8, 1, 32768, 128, True, 0, seed=4, q_mult=3.0)


@pytest.mark.parametrize("Nq,Nk,D,splits", [(1, 9000, 128, 0), (300, 2000, 64, 7), (3, 4000, 96, 0)])
def test_forward_kv_deterministic(Nq, Nk, D, splits):
    """Two runs on the same inputs give bitwise equal O and L (no atomics; the
    merge sums the ranges in a fixed order)."""
    import torch

    scale, _, qb, _, kb, _, vb = _inputs(2, 3, Nq, Nk, D, 91)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o1, l1 = _fa().fwd_kv(q, k, v, scale, causal=True, num_splits=splits)
    o2, l2 = _fa().fwd_kv(q, k, v, scale, causal=True, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
