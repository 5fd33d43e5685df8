"""The streaming (online-softmax) recurrence in float64 (test infrastructure).

Only ``tests/`` may use this module.  It is not the oracle's definition of
the result (that is ``oracle.attention``); it is a second, independent CPU
computation that follows the tiled algorithm, so a test can show that the
algorithm the GPU kernels use reaches the definition to float64 rounding
before any GPU result is looked at.

The recurrence ("Learning Metal with FlashAttention", section
FlashAttention, tiled pseudocode; "Flash Attention" page, kernel anatomy;
metal-flash-attention README, "Quantifying performance", forward
pseudocode): for a block of query rows, keep a running row max m, a running
normaliser Z and an unnormalised output accumulator A.  For every block of
keys, take the block's scores s, raise m to m' = max(m, rowmax s), shrink
the old state by a = exp(m - m'), add the block's exp(s - m') to Z and
exp(s - m') V_block to A.  After the last block, O = A / Z and the saved
statistic is L = m + ln Z.

Causal masking skips key blocks that lie wholly above the diagonal and
masks the entries above it inside a block that straddles it.
"""

from __future__ import annotations

import numpy as np

__all__ = ["online_forward"]


def online_forward(q, k, v, scale: float, causal: bool = False, q_tile: int = 8, k_tile: int = 4):
    """Run the recurrence for one head.  q, k, v: [N, D].  Returns (O, L)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    o = np.empty((n, d))
    lse = np.empty(n)
    for q0 in range(0, n, q_tile):
        qi = np.arange(q0, min(n, q0 + q_tile))
        m = np.full(qi.size, -np.inf)
        z = np.zeros(qi.size)
        acc = np.zeros((qi.size, d))
        for k0 in range(0, n, k_tile):
            if causal and k0 > qi[-1]:
                break  # this block and every later one lies above the diagonal
            kj = np.arange(k0, min(n, k0 + k_tile))
            s = scale * (q[qi] @ k[kj].T)
            if causal:
                s = np.where(kj[None, :] <= qi[:, None], s, -np.inf)
            m_next = np.maximum(m, s.max(axis=1))
            shrink = np.exp(m - m_next)  # exp(-inf) = 0 on the first block
            e = np.exp(s - m_next[:, None])
            z = shrink * z + e.sum(axis=1)
            acc = shrink[:, None] * acc + e @ v[kj]
            m = m_next
        o[qi] = acc / z[:, None]
        lse[qi] = m + np.log(z)
    return o, lse
