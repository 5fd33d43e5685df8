"""Exact attention in float64: the definition written out (test infrastructure).

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the GPU library.

Notation (shared by the three pages this follows):

* Q, K, V are N x D per (batch, head); batched arrays are [B, H, N, D].
* S = scale * Q K^T, with scale = 1/sqrt(D) for every configuration used
  here ("Learning Metal with FlashAttention", FlashAttention section,
  tiled pseudocode; "Flash Attention" page, opening definition).
* P = softmax over each row of S; O = P V.
* L = m + ln(l), the natural-log log-sum-exp of a row of S, where m is the
  row max and l the sum of exp(S - m) (metal-flash-attention README,
  "Quantifying performance", forward pseudocode, last step).
* Causal masking keeps key j for query i iff j <= i (top-left alignment,
  equal query and key lengths): the tiles "above the diagonal" of the
  "Flash Attention" page's kernel anatomy are exactly the masked entries.

The two-pass softmax (first the row max, then exp and sum) is the stable
form the "Learning Metal with FlashAttention" page describes before it
introduces the running maximum.  Nothing here is tiled over keys: every
needed score of a row is materialised before its softmax is taken.
"""

from __future__ import annotations

import numpy as np

__all__ = ["probabilities", "forward_rows", "forward", "forward_kv", "forward_block_sparse", "backward"]


def _as_f64(x) -> np.ndarray:
    """Upcast to float64.  bf16 and fp32 inputs convert exactly."""
    return np.asarray(x, dtype=np.float64)


def _scores(q_rows: np.ndarray, k: np.ndarray, rows: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    """S for the query rows ``rows`` of one head, with -inf where masked.

    q_rows: [R, D] (the Q rows with indices ``rows``); k: [N, D].
    Under causal masking only columns 0 .. max(rows) can be visible, so the
    columns past it are not formed: they would all be -inf and contribute
    exp(-inf) = 0 exactly.
    """
    ncols = k.shape[0]
    if causal:
        ncols = int(rows.max()) + 1
    s = scale * (q_rows @ k[:ncols].T)
    if causal:
        cols = np.arange(ncols)
        s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
    return s


def _softmax_two_pass(s: np.ndarray):
    """Row softmax in two passes.  Returns (P, m, l).

    Pass 1 finds m_i = max_j s_ij; pass 2 forms E = exp(s - m), its row sum
    l_i and P = E / l.  Every row has at least one finite entry (the
    diagonal under causal masking), so m is finite.
    """
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def probabilities(q, k, scale: float, causal: bool = False) -> np.ndarray:
    """The softmax matrix P = softmax(scale * Q K^T) for one head, [N, N].

    q, k: [N, D].  Masked entries are exactly 0.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    n = q.shape[0]
    rows = np.arange(n)
    s = _scores(q, k, rows, scale, causal)
    p, _, _ = _softmax_two_pass(s)
    if p.shape[1] < k.shape[0]:  # causal: pad the never-visible columns with 0
        p = np.concatenate([p, np.zeros((n, k.shape[0] - p.shape[1]))], axis=1)
    return p


def forward_rows(q, k, v, rows, scale: float, causal: bool = False):
    """O and L for the query rows ``rows`` of one head.

    q: [N, D] (all rows; only ``rows`` are read), k, v: [N, D].
    Returns (O_rows [R, D], L_rows [R]).  Rows of attention are independent
    of one another, so any subset can be computed on its own; this is what
    makes sampled checks at large N possible.
    """
    rows = np.asarray(rows, dtype=np.int64)
    k = _as_f64(k)
    v = _as_f64(v)
    q_rows = _as_f64(np.asarray(q)[rows])
    s = _scores(q_rows, k, rows, scale, causal)
    p, m, l = _softmax_two_pass(s)
    o = p @ v[: s.shape[1]]
    lse = m + np.log(l)
    return o, lse


def forward(q, k, v, scale: float, causal: bool = False, row_block: int = 256):
    """O = softmax(scale Q K^T) V and L = logsumexp per row, all heads.

    q, k, v: [B, H, N, D] (or [N, D] for a single head).  Returns
    (O [B, H, N, D] float64, L [B, H, N] float64).  Rows are processed in
    blocks of ``row_block`` only to bound memory; each row's arithmetic is
    the same whatever the block size.
    """
    q = np.asarray(q)
    single = q.ndim == 2
    if single:
        q, k, v = q[None, None], np.asarray(k)[None, None], np.asarray(v)[None, None]
    b_, h_, n, d = q.shape
    o = np.empty((b_, h_, n, d), dtype=np.float64)
    lse = np.empty((b_, h_, n), dtype=np.float64)
    for b in range(b_):
        for h in range(h_):
            for r0 in range(0, n, row_block):
                rows = np.arange(r0, min(n, r0 + row_block))
                o[b, h, rows], lse[b, h, rows] = forward_rows(q[b, h], k[b, h], v[b, h], rows, scale, causal)
    if single:
        return o[0, 0], lse[0, 0]
    return o, lse


def forward_kv(q, k, v, scale: float, causal: bool = False):
    """Attention of Nq query rows over Nk keys (Nq and Nk may differ).

    q: [B, H, Nq, D] (or [Nq, D]); k, v: [B, H, Nk, D] (or [Nk, D]).
    Returns (O [.., Nq, D], L [.., Nq]) in float64.

    This is the definition above with the two lengths apart: the case of a
    block of new query rows attending to a longer key sequence, and of
    decoding one row at a time, which the "Flash Attention" page's section
    on the technique's boundaries sets apart from the square case.  The
    pages do not say how a causal mask lines up when Nq < Nk; the reading
    taken here is that the query rows are the LAST Nq positions of the key
    sequence (bottom-right alignment): query i sees key j iff
    j <= i + (Nk - Nq).  With Nq = Nk this is the square mask of
    ``forward``.  Under causal masking Nq must not exceed Nk (the first
    rows would see no key at all).
    """
    q = np.asarray(q)
    single = q.ndim == 2
    if single:
        q, k, v = q[None, None], np.asarray(k)[None, None], np.asarray(v)[None, None]
    else:
        k, v = np.asarray(k), np.asarray(v)
    b_, h_, nq, d = q.shape
    nk = k.shape[2]
    if k.shape != (b_, h_, nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Nk, D] with the batch, heads and D of q")
    if causal and nq > nk:
        raise ValueError("causal attention with more query rows than keys leaves rows with no key")
    offset = nk - nq
    o = np.empty((b_, h_, nq, d), dtype=np.float64)
    lse = np.empty((b_, h_, nq), dtype=np.float64)
    cols = np.arange(nk)
    for b in range(b_):
        for h in range(h_):
            qh, kh, vh = (_as_f64(x[b, h]) for x in (q, k, v))
            s = scale * (qh @ kh.T)
            if causal:
                s = np.where(cols[None, :] <= np.arange(nq)[:, None] + offset, s, -np.inf)
            p, m, l = _softmax_two_pass(s)
            o[b, h] = p @ vh
            lse[b, h] = m + np.log(l)
    if single:
        return o[0, 0], lse[0, 0]
    return o, lse


def forward_block_sparse(q, k, v, scale: float, causal: bool, block_mask, block: int = 64):
    """Attention restricted to the (query block, key block) pairs a block mask keeps.

    q, k, v: [B, H, N, D] (or [N, D]).  block_mask: array of shape
    [nb, nb] or [B*H, nb, nb] (or [B, H, nb, nb]) with nb = ceil(N / block); a nonzero entry
    (a, c) lets the queries of rows a*block .. a*block+block-1 see the keys
    of rows c*block .. c*block+block-1.  With causal masking a key must in
    addition satisfy j <= i.  Returns (O, L) in float64.

    The pages name skipping whole blocks beyond the causal ones as the
    natural extension of the tile skip (metal-flash-attention README,
    closing sections; "Flash Attention" page, kernel anatomy) without fixing
    a format; this is the plainest reading: the definition of ``forward``
    with the scores of dropped blocks set to -inf.  A row that sees no key
    at all has no softmax; it is given O = 0 and L = -inf (the limit of a
    row whose scores all tend to -inf contributes nothing, and L = -inf
    gives it weight 0 in any merge by log-sum-exp).
    """
    q = np.asarray(q)
    single = q.ndim == 2
    if single:
        q, k, v = q[None, None], np.asarray(k)[None, None], np.asarray(v)[None, None]
    else:
        k, v = np.asarray(k), np.asarray(v)
    b_, h_, n, d = q.shape
    nb = -(-n // block)
    mask = np.asarray(block_mask)
    if mask.ndim == 2:
        mask = np.broadcast_to(mask, (b_ * h_, nb, nb))
    mask = mask.reshape(b_ * h_, nb, nb) != 0
    blk = np.arange(n) // block
    o = np.zeros((b_, h_, n, d), dtype=np.float64)
    lse = np.full((b_, h_, n), -np.inf, dtype=np.float64)
    for b in range(b_):
        for h in range(h_):
            vis = mask[b * h_ + h][blk[:, None], blk[None, :]]
            if causal:
                vis = vis & (np.arange(n)[None, :] <= np.arange(n)[:, None])
            qh, kh, vh = (_as_f64(x[b, h]) for x in (q, k, v))
            s = np.where(vis, scale * (qh @ kh.T), -np.inf)
            rows = vis.any(axis=1)
            if rows.any():
                p, m, l = _softmax_two_pass(s[rows])
                o[b, h, rows] = p @ vh
                lse[b, h, rows] = m + np.log(l)
    if single:
        return o[0, 0], lse[0, 0]
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool = False):
    """Gradients of attention for one head, dense, in float64.

    Given the upstream gradient dO of O = P V with P = softmax(S),
    S = scale Q K^T (masked entries constant -inf), the chain rule gives

        dV = P^T dO
        dP = dO V^T
        delta_i = sum_d dO_id O_id   (= sum_j P_ij dP_ij)
        dS = P * (dP - delta 1^T)    (elementwise; softmax Jacobian)
        dQ = scale dS K,   dK = scale dS^T Q.

    These are the quantities the split backward kernels of the
    metal-flash-attention README ("Quantifying performance", backward-query
    and backward-key-value pseudocode) accumulate, there with P rebuilt as
    exp(S - L) from the saved L.  Here P comes straight from the definition.

    q, k, v, do: [N, D] or [B, H, N, D].  Returns a dict with float64
    arrays dq, dk, dv (input shape), delta and lse (shape without D), and
    o (input shape).
    """
    q = np.asarray(q)
    single = q.ndim == 2
    if single:
        q, k, v, do = (np.asarray(x)[None, None] for x in (q, k, v, do))
    else:
        k, v, do = (np.asarray(x) for x in (k, v, do))
    b_, h_, n, d = q.shape
    out = {name: np.empty((b_, h_, n, d)) for name in ("dq", "dk", "dv", "o")}
    out["delta"] = np.empty((b_, h_, n))
    out["lse"] = np.empty((b_, h_, n))
    rows = np.arange(n)
    for b in range(b_):
        for h in range(h_):
            qh, kh, vh, doh = (_as_f64(x[b, h]) for x in (q, k, v, do))
            s = _scores(qh, kh, rows, scale, causal)
            p, m, l = _softmax_two_pass(s)
            oh = p @ vh
            dv = p.T @ doh
            dp = doh @ vh.T
            delta = (doh * oh).sum(axis=1)
            ds = p * (dp - delta[:, None])
            out["dq"][b, h] = scale * (ds @ kh)
            out["dk"][b, h] = scale * (ds.T @ qh)
            out["dv"][b, h] = dv
            out["o"][b, h] = oh
            out["delta"][b, h] = delta
            out["lse"][b, h] = m + np.log(l)
    if single:
        return {name: val[0, 0] for name, val in out.items()}
    return out
