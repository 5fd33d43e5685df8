"""GPU parity of the forward kernels against the float64 oracle, through the C ABI.

Every full-size workload (c1 .. c5) is checked element by element on every
row of every head; for c3 and c4 the oracle runs over (batch, head, row
block) units on a thread pool (attention rows are independent).  The N =
65536 runs are checked on sampled rows (the ends, tile boundaries and random
rows).  Small shapes cover ragged lengths,
several tiles and both masking modes, for every head dimension of the bf16
forward (32, 64, 96, 128, 160, 256).
"""

import numpy as np
import pytest

import oracle
from fa_inputs import WORKLOADS, make_inputs
from tests._gpu import (
    TOL_BF16_L,
    TOL_BF16_O,
    TOL_F32,
    dev_bf16,
    forward_errors_all_rows,
    host,
    inputs_on_device,
    log,
    sample_rows,
)

pytestmark = pytest.mark.gpu


def _fa():
    import exact_attention_51_amd as fa

    return fa


def _run(w, x):
    import torch

    q, k, v = inputs_on_device(w, x)
    o, lse = _fa().fwd(q, k, v, w.scale, causal=w.causal)
    torch.cuda.synchronize()
    return o, lse


def _tols(w):
    return (TOL_F32, TOL_F32) if w.dtype == "fp32" else (TOL_BF16_O, TOL_BF16_L)


def _check_full(w, x, o, lse):
    o_ref, l_ref = oracle.forward(x.q, x.k, x.v, w.scale, w.causal)
    eo = float(np.abs(host(o) - o_ref).max())
    el = float(np.abs(host(lse) - l_ref).max())
    to, tl = _tols(w)
    log(f"  {w.name} B={w.B} H={w.H} N={w.N} D={w.D} causal={w.causal}: max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= to and el <= tl, (eo, el)
    assert np.isfinite(host(o)).all() and np.isfinite(host(lse)).all()


def _check_rows(w, x, o, lse, count=24):
    oh, lh = host(o), host(lse)
    assert np.isfinite(lh).all()
    eo = el = 0.0
    for b in range(w.B):
        for h in range(w.H):
            rows = sample_rows(w.N, count, seed=1000 * b + h)
            o_ref, l_ref = oracle.forward_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, w.scale, w.causal)
            eo = max(eo, float(np.abs(oh[b, h, rows] - o_ref).max()))
            el = max(el, float(np.abs(lh[b, h, rows] - l_ref).max()))
    to, tl = _tols(w)
    log(f"  {w.name} sampled rows: max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= to and el <= tl, (eo, el)


def _check_all_rows(w, x, o, lse):
    oh, lh = host(o), host(lse)
    assert np.isfinite(oh).all() and np.isfinite(lh).all()
    eo, el = forward_errors_all_rows(w, x, oh, lh)
    to, tl = _tols(w)
    log(f"  {w.name} B={w.B} H={w.H} N={w.N} D={w.D} causal={w.causal}, all rows: max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= to and el <= tl, (eo, el)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_forward(name):
    w = WORKLOADS[name]
    log(f"test_workload_forward[{name}] start")
    x = make_inputs(w, with_do=False)
    o, lse = _run(w, x)
    if name in ("c3", "c4"):
        _check_all_rows(w, x, o, lse)
    else:
        _check_full(w, x, o, lse)


@pytest.mark.parametrize("D,causal", [(128, True), (64, False), (256, True), (96, True), (160, False), (32, True)])
def test_forward_long_sequence(D, causal):
    """N = 65536 (twice c4's length: 1024 key tiles per row, 32-bit tile
    offsets within a head up to 32 MiB), checked on sampled rows."""
    w = WORKLOADS["c4"].with_(name="long", B=1, H=1, N=65536, D=D, causal=causal, q_mult=1.0, seed=65536 + D)
    log(f"test_forward_long_sequence N={w.N} D={D} causal={causal}")
    x = make_inputs(w, with_do=False)
    o, lse = _run(w, x)
    _check_rows(w, x, o, lse, count=16)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [32, 64, 96, 128, 160, 256])
@pytest.mark.parametrize("N", [1, 5, 64, 65, 130, 256, 300, 520])
def test_forward_bf16_shapes(N, D, causal):
    w = WORKLOADS["c2"].with_(name="edge", B=1, H=2, N=N, D=D, causal=causal, seed=N * 7 + D)
    log(f"test_forward_bf16_shapes N={N} D={D} causal={causal}")
    x = make_inputs(w, with_do=False)
    _check_full(w, x, *_run(w, x))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [96, 128])
def test_forward_bf16_many_heads(D, causal):
    """B*H = 512 heads of N = 300: enough 256-row blocks that D = 96 and 128
    run their 8-wave workgroups (the small shapes above run the 4-wave,
    128-row workgroups the forward picks for grids smaller than the GPU)."""
    w = WORKLOADS["c3"].with_(name="heads", B=4, H=128, N=300, D=D, causal=causal, seed=300 + D)
    log(f"test_forward_bf16_many_heads D={D} causal={causal}")
    x = make_inputs(w, with_do=False)
    o, lse = _run(w, x)
    _check_full(w, x, o, lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [(3, 37, 1000), (2, 20, 3000), (2, 64, 1000)])
@pytest.mark.parametrize("D", [64, 128])
def test_forward_persistent_rounds(D, B, H, N, causal):
    """D = 64 and 128 grids larger than the GPU run one persistent workgroup
    per compute unit, which carries its K/V ring from one 256-row block into
    the next.  The shapes take a full round of blocks and a partial one,
    with a ragged last key tile: 111 heads of N = 1000 (444 blocks; heads not
    a multiple of the eight XCDs, so no per-XCD head groups) and 40 heads of
    N = 3000 (480 blocks, 5 heads per XCD, blocks of 4 to 47 key tiles).
    Under the causal mask those grids take the 128-row workgroups of smaller
    grids; 128 heads of N = 1000 (512 blocks) run the persistent kernels
    with the mask too."""
    w = WORKLOADS["c3"].with_(name="rounds", B=B, H=H, N=N, D=D, causal=causal, seed=N + H + D)
    log(f"test_forward_persistent_rounds D={D} B={B} H={H} N={N} causal={causal}")
    x = make_inputs(w, with_do=False)
    o, lse = _run(w, x)
    _check_full(w, x, o, lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [64, 130, 200])
def test_forward_d64_short_many_heads(N, causal):
    """520 heads of N < 256: one 256-row block per head, enough blocks for
    the D = 64 assembly kernel (also under the causal mask), too short for
    its persistent walk: one block per workgroup, 1 to 4 key tiles, a ragged
    last tile at 130 and 200."""
    w = WORKLOADS["c2"].with_(name="short", B=2, H=260, N=N, D=64, causal=causal, seed=N + 7)
    log(f"test_forward_d64_short_many_heads N={N} causal={causal}")
    x = make_inputs(w, with_do=False)
    o, lse = _run(w, x)
    _check_full(w, x, o, lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 33, 256, 300])
def test_forward_f32_shapes(N, D, causal):
    w = WORKLOADS["c1"].with_(name="edge32", B=2, H=1, N=N, D=D, causal=causal, seed=N + D)
    log(f"test_forward_f32_shapes N={N} D={D} causal={causal}")
    x = make_inputs(w, with_do=False)
    _check_full(w, x, *_run(w, x))


@pytest.mark.parametrize("D", [32, 64, 96, 128, 160, 256])
def test_forward_peaked_rows(D):
    """Q scaled by 3 (and by 8): nearly one-hot rows stress the rescale path."""
    for mult in (3.0, 8.0):
        w = WORKLOADS["c4"].with_(name="peaked", B=1, H=2, N=1024, D=D, q_mult=mult, seed=int(mult) + D)
        log(f"test_forward_peaked_rows D={D} q_mult={mult}")
        x = make_inputs(w, with_do=False)
        _check_full(w, x, *_run(w, x))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [32, 64, 96, 128, 160, 256])
def test_forward_growing_scores(D, causal):
    """Scores that grow from key tile to key tile by G (exp2 units) along the
    processing order, so a later tile's exponentials against the running max
    exceed any fixed bound (G = 200 overflows float32 before the max is
    raised), and the same keys in falling order."""
    import torch

    from fa_inputs import Inputs, bf16_round

    n = 512
    rng = np.random.default_rng(11 + D)
    scale = 1.0 / np.sqrt(D)
    for growth in (4.0, 30.0, 200.0):
        for rising in (True, False):
            log(f"test_forward_growing_scores D={D} causal={causal} growth={growth} rising={rising}")
            q = 0.1 * rng.standard_normal((1, 1, n, D)).astype(np.float32)
            q[..., 0] = 1.0
            k = 0.1 * rng.standard_normal((1, 1, n, D)).astype(np.float32)
            j = np.arange(n) if rising else np.arange(n)[::-1]
            k[0, 0, :, 0] = j * growth / (64 * scale * np.log2(np.e))
            v = rng.standard_normal((1, 1, n, D)).astype(np.float32)
            (qv, qb), (kv, kb), (vv, vb) = bf16_round(q), bf16_round(k), bf16_round(v)
            x = Inputs(q=qv, k=kv, v=vv, do=None, q_bits=qb, k_bits=kb, v_bits=vb)
            w = WORKLOADS["c2"].with_(name="growing", B=1, H=1, N=n, D=D, causal=causal)
            _check_full(w, x, *_run(w, x))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_forward_persistent_growing_scores(D, causal):
    """The growing-score inputs above on a D = 64 or 128 grid large enough to
    run persistently (260 heads of N = 512: 520 blocks), so the out-of-line
    rescale path runs in blocks that took their first K/V tiles from the
    ring of the block before."""
    from fa_inputs import Inputs, bf16_round

    n, h = 512, 260
    rng = np.random.default_rng(97 + D)
    scale = 1.0 / np.sqrt(D)
    for growth in (30.0, 200.0):
        for rising in (True, False):
            log(f"test_forward_persistent_growing_scores D={D} causal={causal} growth={growth} rising={rising}")
            q = 0.1 * rng.standard_normal((1, h, n, D)).astype(np.float32)
            q[..., 0] = 1.0
            k = 0.1 * rng.standard_normal((1, h, n, D)).astype(np.float32)
            j = np.arange(n) if rising else np.arange(n)[::-1]
            k[0, :, :, 0] = j * growth / (64 * scale * np.log2(np.e))
            v = rng.standard_normal((1, h, n, D)).astype(np.float32)
            (qv, qb), (kv, kb), (vv, vb) = bf16_round(q), bf16_round(k), bf16_round(v)
            x = Inputs(q=qv, k=kv, v=vv, do=None, q_bits=qb, k_bits=kb, v_bits=vb)
            w = WORKLOADS["c3"].with_(name="growing_persistent", B=1, H=h, N=n, D=D, causal=causal)
            _check_full(w, x, *_run(w, x))


@pytest.mark.parametrize("D", [32, 64, 96, 128, 160, 256])
def test_forward_invariants(D):
    import torch

    fa = _fa()
    n = 384
    w = WORKLOADS["c2"].with_(B=1, H=1, N=n, D=D, seed=D)
    x = make_inputs(w, with_do=False)
    q, k, v = inputs_on_device(w, x)
    log(f"test_forward_invariants D={D}")
    for causal in (False, True):
        # constant V: every output row equals that row
        vc = v[:, :, :1, :].expand(-1, -1, n, -1).contiguous()
        o, _ = fa.fwd(q, k, vc, w.scale, causal)
        torch.cuda.synchronize()
        np.testing.assert_allclose(host(o), host(vc), rtol=0, atol=1e-2)
        # identical keys: plain mean (prefix mean under causal) of V, and L = scale q.k + ln(count)
        kc = k[:, :, :1, :].expand(-1, -1, n, -1).contiguous()
        o, lse = fa.fwd(q, kc, v, w.scale, causal)
        torch.cuda.synchronize()
        vh = x.v[0, 0].astype(np.float64)
        counts = np.arange(1, n + 1) if causal else np.full(n, n)
        mean = np.cumsum(vh, axis=0) / counts[:, None] if causal else np.tile(vh.mean(axis=0), (n, 1))
        np.testing.assert_allclose(host(o)[0, 0], mean, rtol=0, atol=2e-2)
        l_ref = w.scale * (x.q[0, 0].astype(np.float64) @ x.k[0, 0, 0].astype(np.float64)) + np.log(counts)
        np.testing.assert_allclose(host(lse)[0, 0], l_ref, rtol=0, atol=1e-2)
    # causal row 0 sees key 0 only: O_0 = V_0 exactly
    o, lse = fa.fwd(q, k, v, w.scale, True)
    torch.cuda.synchronize()
    assert np.array_equal(host(o)[0, 0, 0], host(v)[0, 0, 0])


def test_forward_deterministic():
    import torch

    w = WORKLOADS["c3"].with_(B=1, H=4, N=2048)
    x = make_inputs(w, with_do=False)
    q, k, v = inputs_on_device(w, x)
    fa = _fa()
    o1, l1 = fa.fwd(q, k, v, w.scale, True)
    o2, l2 = fa.fwd(q, k, v, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_forward_causal_prefix():
    """Causal rows < n do not depend on keys >= n: a length-n run agrees."""
    import torch

    fa = _fa()
    w = WORKLOADS["c3"].with_(B=1, H=2, N=1024)
    x = make_inputs(w, with_do=False)
    q, k, v = inputs_on_device(w, x)
    o, lse = fa.fwd(q, k, v, w.scale, True)
    for n in (1, 100, 256, 700):
        op, lp = fa.fwd(q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous(), w.scale, True)
        torch.cuda.synchronize()
        np.testing.assert_allclose(host(op), host(o)[:, :, :n], rtol=0, atol=2e-2)
        np.testing.assert_allclose(host(lp), host(lse)[:, :, :n], rtol=0, atol=1e-3)


def test_forward_batch_slices_independent():
    """A [B, H] batch equals separate single-head calls, bit for bit."""
    import torch

    fa = _fa()
    w = WORKLOADS["c2"].with_(B=2, H=3, N=320)
    x = make_inputs(w, with_do=False)
    q, k, v = inputs_on_device(w, x)
    o, lse = fa.fwd(q, k, v, w.scale, False)
    for b in range(2):
        for h in range(3):
            sl = lambda t: t[b : b + 1, h : h + 1].contiguous()  # noqa: E731
            o1, l1 = fa.fwd(sl(q), sl(k), sl(v), w.scale, False)
            torch.cuda.synchronize()
            assert torch.equal(o1[0, 0], o[b, h]) and torch.equal(l1[0, 0], lse[b, h])


def test_forward_writes_only_its_outputs():
    """Outputs of a ragged call stay inside [B, H, N, D]: guard words around them are untouched."""
    import torch

    fa = _fa()
    w = WORKLOADS["c3"].with_(B=1, H=1, N=77, D=128)
    x = make_inputs(w, with_do=False)
    q, k, v = (dev_bf16(b) for b in (x.q_bits, x.k_bits, x.v_bits))
    n_o = w.N * w.D
    o_buf = torch.full((n_o + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((w.N + 1024,), 7.0, dtype=torch.float32, device="cuda")
    o = o_buf[:n_o].view(1, 1, w.N, w.D)
    lse = l_buf[: w.N].view(1, 1, w.N)
    fa.fwd(q, k, v, w.scale, True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((o_buf[n_o:] == 7.0).all()) and bool((l_buf[w.N :] == 7.0).all())
