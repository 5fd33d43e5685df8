"""GPU parity of ``fa_fwd_sparse`` (block-sparse forward) against the float64
oracle ``forward_block_sparse``.

Masks are over (64-row query block, 64-key block) pairs: random patterns at
several densities (shared by all heads and per head), a band with a first
column (a local window with a sink block), patterns that leave whole query
blocks with no key, and the all-ones mask.  Lengths cover one tile, a ragged
tail and several workgroups.  At the c3 shape the check is on sampled rows:
each row's reference is the oracle over exactly the keys the mask and the
causal mask leave it (attention over a subset of keys is the same
definition).
"""

import numpy as np
import pytest

import oracle
from fa_inputs import WORKLOADS, make_inputs
from tests._gpu import TOL_BF16_L, TOL_BF16_O, dev_bf16, host, log, sample_rows

pytestmark = pytest.mark.gpu

BLOCK = 64


def _fa():
    import exact_attention_51_amd as fa

    return fa


def _mask(kind, nb, seed, heads=None):
    rng = np.random.default_rng(seed)
    shape = (nb, nb) if heads is None else (heads, nb, nb)
    if kind == "ones":
        return np.ones(shape, np.uint8)
    if kind.startswith("rand"):
        return (rng.random(shape) < float(kind[4:])).astype(np.uint8)
    if kind == "band":  # each query block sees itself, the two blocks before it and block 0
        m = np.zeros((nb, nb), np.uint8)
        for a in range(nb):
            m[a, max(0, a - 2) : a + 1] = 1
            m[a, 0] = 1
        return m if heads is None else np.broadcast_to(m, shape).copy()
    if kind == "holes":  # random, with every third query block seeing nothing
        m = (rng.random(shape) < 0.5).astype(np.uint8)
        m[..., ::3, :] = 0
        return m
    raise ValueError(kind)


def _run(B, H, N, D, causal, kind, per_head, seed=71):
    import torch

    log(f"fwd_sparse B={B} H={H} N={N} D={D} causal={causal} mask={kind} per_head={per_head} seed={seed}")
    w = WORKLOADS["c3"].with_(B=B, H=H, N=N, D=D, causal=causal)
    x = make_inputs(w, seed=seed, with_do=False)
    nb = -(-N // BLOCK)
    m = _mask(kind, nb, seed + 1, B * H if per_head else None)
    o, lse = _fa().fwd_sparse(
        dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits), torch.from_numpy(m).cuda(), w.scale, causal
    )
    torch.cuda.synchronize()
    return w, x, m, host(o), host(lse)


CASES = [
    # (B, H, N, D, causal, mask kind, per-head masks)
    (1, 2, 1000, 128, False, "rand0.5", False),
    (1, 2, 1000, 128, True, "rand0.5", False),
    (2, 2, 1024, 64, False, "rand0.3", True),
    (2, 2, 1024, 64, True, "band", False),
    (1, 3, 777, 128, True, "holes", True),
    (1, 2, 777, 64, False, "holes", False),
    (1, 2, 50, 128, False, "ones", False),  # one short tile
    (1, 2, 50, 64, True, "rand0.5", True),
    (1, 1, 64, 128, True, "ones", False),
    (1, 2, 2048, 128, True, "ones", False),
    (1, 2, 2048, 128, False, "rand0.1", False),
    (1, 1, 300, 128, False, "rand0.0", False),  # nothing kept: O = 0, L = -inf everywhere
    (1, 2, 1000, 96, True, "rand0.5", True),
    (1, 2, 777, 96, False, "band", False),
    (1, 2, 1000, 32, True, "holes", False),
    (1, 2, 1000, 256, True, "rand0.5", True),
    (1, 2, 777, 256, False, "holes", False),
    (1, 2, 50, 256, True, "ones", False),
    (1, 2, 900, 160, True, "band", False),
]


@pytest.mark.parametrize("B,H,N,D,causal,kind,per_head", CASES)
def test_forward_sparse(B, H, N, D, causal, kind, per_head):
    w, x, m, oh, lh = _run(B, H, N, D, causal, kind, per_head)
    o_ref, l_ref = oracle.forward_block_sparse(x.q, x.k, x.v, w.scale, causal, m, block=BLOCK)
    assert np.isfinite(oh).all()
    empty = np.isneginf(l_ref)
    assert (np.isneginf(lh) == empty).all(), "rows with no key must get L = -inf, the others a finite L"
    assert (oh[empty] == 0).all()
    eo = float(np.abs(oh - o_ref).max())
    el = float(np.abs(lh[~empty] - l_ref[~empty]).max()) if (~empty).any() else 0.0
    log(f"  max|dO|={eo:.3e} max|dL|={el:.3e} rows with no key: {int(empty.sum())}")
    assert eo <= TOL_BF16_O and el <= TOL_BF16_L, (eo, el)


@pytest.mark.parametrize("kind", ["band", "rand0.5"])
def test_forward_sparse_c3_shape_sampled_rows(kind):
    """B=2 H=16 N=8192 D=128 causal with a block mask, on sampled rows of
    every head."""
    w, x, m, oh, lh = _run(2, 16, 8192, 128, True, kind, False, seed=3)
    eo = el = 0.0
    for b in range(w.B):
        for h in range(w.H):
            for i in sample_rows(w.N, 8, seed=100 * b + h):
                keys = np.arange(i + 1)
                keys = keys[m[i // BLOCK, keys // BLOCK] != 0]
                if keys.size == 0:
                    assert np.isneginf(lh[b, h, i]) and (oh[b, h, i] == 0).all()
                    continue
                o_ref, l_ref = oracle.forward_kv(x.q[b, h, i : i + 1], x.k[b, h, keys], x.v[b, h, keys], w.scale, False)
                eo = max(eo, float(np.abs(oh[b, h, i] - o_ref[0]).max()))
                el = max(el, abs(float(lh[b, h, i] - l_ref[0])))
    log(f"  c3 shape, mask {kind}: max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= TOL_BF16_O and el <= TOL_BF16_L, (eo, el)


def test_forward_sparse_deterministic():
    """Two runs on the same inputs and mask give bitwise equal O and L."""
    import torch

    w = WORKLOADS["c3"].with_(B=1, H=4, N=3000, D=128, causal=True)
    x = make_inputs(w, seed=93, with_do=False)
    m = torch.from_numpy(_mask("rand0.5", -(-w.N // BLOCK), 94)).cuda()
    q, k, v = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits)
    o1, l1 = _fa().fwd_sparse(q, k, v, m, w.scale, True)
    o2, l2 = _fa().fwd_sparse(q, k, v, m, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
