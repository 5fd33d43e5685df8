"""CPU oracle for exact attention (forward and backward), in float64.

This package is TEST INFRASTRUCTURE.  Only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import it.  The GPU library
never imports, links or calls anything here, and nothing here imports the
GPU library: the two share no code.  The only thing both sides consume is
the seeded inputs produced by ``fa_inputs``, which holds none of the
method's arithmetic.

What the oracle computes is the plain definition of attention, not the
tiled algorithm: FlashAttention is exact, so the tiled GPU kernels must
reach the same numbers up to rounding order ("Flash Attention" page,
opening definition; "Learning Metal with FlashAttention", section
FlashAttention).  The score matrix is materialised in float64 and the
softmax is taken in two passes (row max, then exp / sum).

Modules
-------
attention
    ``forward`` / ``forward_rows`` (O and the per-row log-sum-exp L),
    ``forward_kv`` (the same with query and key lengths apart, causal
    masking aligned to the last query rows), ``forward_block_sparse`` (the
    same restricted to the (query block, key block) pairs of a block mask),
    ``probabilities`` (the softmax matrix P) and ``backward`` (dQ, dK, dV
    and delta = rowsum(dO * O)).
online
    A float64 run of the streaming recurrence (running max m, running sum
    Z, unnormalised accumulator) in the order the pages give it.  It exists
    only to pin the definition above against the algorithm the kernels use.

Pins: every public function is pinned by ``tests/test_oracle_pins.py``
against brute force at 50 digits (mpmath), closed forms, invariants,
finite differences and an independent library routine
(``scipy.special.logsumexp``).  No function here is "parity unpinned".
"""

from .attention import backward, forward, forward_block_sparse, forward_kv, forward_rows, probabilities  # noqa: F401
from .online import online_forward  # noqa: F401
