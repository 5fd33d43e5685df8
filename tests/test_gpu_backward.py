"""GPU parity of the split backward (fa_bwd_dq then fa_bwd_dkdv) against the
float64 oracle's dense backward, through the C ABI.

The GPU backward consumes the GPU forward's O and L (as a caller would); the
oracle backward uses its own float64 forward.  Gradients are compared by
max absolute error and by max absolute error relative to the largest
reference magnitude (gradient entries are small, so the relative form is
the one with teeth).
"""

import numpy as np
import pytest

import oracle
from fa_inputs import WORKLOADS, make_inputs
from tests._gpu import TOL_BF16_GRAD, dev_bf16, host, log

pytestmark = pytest.mark.gpu

# delta = rowsum(dO * O) is formed from the forward's stored bf16 O (as the
# backward-query pseudocode forms it from the stored output), so its error is
# that of O's rounding, about 2^-9 |O| per term: bound it relative to max|delta|.
TOL_DELTA_REL = 1e-2
# Below this reference magnitude a gradient is exactly zero in the oracle
# (for instance N = 1, where the softmax is constant): only the absolute bound applies.
TINY = 1e-6


def _run_bwd(w, x):
    import torch

    import exact_attention_51_amd as fa

    q, k, v, do = (dev_bf16(b) for b in (x.q_bits, x.k_bits, x.v_bits, x.do_bits))
    o, lse = fa.fwd(q, k, v, w.scale, w.causal)
    dq, dk, dv, delta = fa.bwd(q, k, v, o, do, lse, w.scale, w.causal)
    torch.cuda.synchronize()
    return dq, dk, dv, delta


def _check(w, x, got, rel_tol=TOL_BF16_GRAD, heads=None):
    """Gradients: max abs error <= 2e-2 * max(1, max |reference|) and, unless
    the oracle's gradient is exactly zero, max abs error / max |reference|
    <= 2e-2.  bf16 rounding errors scale with the magnitude of what is
    rounded; the absolute 2e-2 is the bound for entries up to 1 (the
    D = 256 workload's are about 0.03), and where a gradient's largest entry
    exceeds 1 (small head dims, scale 1/sqrt(32)) it scales with it.
    heads: the (batch, head) pairs to compare (default: all)."""
    dq, dk, dv, delta = got
    gh = {"dq": host(dq), "dk": host(dk), "dv": host(dv)}
    delta_h = host(delta)
    errs = {}
    refmax = {}
    zero = set()
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in heads:
        ref = oracle.backward(x.q[b, h], x.k[b, h], x.v[b, h], x.do[b, h], w.scale, w.causal)
        for name in ("dq", "dk", "dv"):
            g = gh[name][b, h]
            assert np.isfinite(g).all(), name
            ea = float(np.abs(g - ref[name]).max())
            er = ea / max(float(np.abs(ref[name]).max()), 1e-30)
            pa, pr = errs.get(name, (0.0, 0.0))
            errs[name] = (max(pa, ea), max(pr, er))
            refmax[name] = max(refmax.get(name, 0.0), float(np.abs(ref[name]).max()))
        ed = float(np.abs(delta_h[b, h] - ref["delta"]).max())
        edr = ed / max(float(np.abs(ref["delta"]).max()), TINY)
        pa, pr = errs.get("delta", (0.0, 0.0))
        errs["delta"] = (max(pa, ed), max(pr, edr))
        for name in ("dq", "dk", "dv"):
            if float(np.abs(ref[name]).max()) < TINY:
                zero.add(name)
    log(f"  {w.name} B={w.B} H={w.H} N={w.N} D={w.D} causal={w.causal}: " + ", ".join(f"{k}: abs {a:.2e} rel {r:.2e}" for k, (a, r) in errs.items()))
    for name in ("dq", "dk", "dv"):
        a, r = errs[name]
        assert a <= TOL_BF16_GRAD * max(1.0, refmax[name]), (name, a, refmax[name])
        assert name in zero or r <= rel_tol, (name, r)
    assert errs["delta"][1] <= TOL_DELTA_REL, errs["delta"]


def test_workload_backward_c5():
    w = WORKLOADS["c5"]
    log("test_workload_backward_c5 start")
    x = make_inputs(w)
    _check(w, x, _run_bwd(w, x))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [32, 64, 96, 128, 160, 256])
@pytest.mark.parametrize("N", [1, 40, 64, 100, 160, 256, 320, 333])
def test_backward_shapes(N, D, causal):
    w = WORKLOADS["c5"].with_(name="edge", B=1, H=2, N=N, D=D, causal=causal, seed=3 * N + D)
    log(f"test_backward_shapes N={N} D={D} causal={causal}")
    x = make_inputs(w, with_do=True)
    _check(w, x, _run_bwd(w, x))


@pytest.mark.parametrize("D", [96, 128, 160, 256])
def test_backward_causal_long(D):
    w = WORKLOADS["c5"].with_(name="causal_long", B=1, H=2, N=1024, D=D, causal=True, seed=D + 1)
    log(f"test_backward_causal_long D={D}")
    x = make_inputs(w, with_do=True)
    _check(w, x, _run_bwd(w, x))


def test_backward_c3_shape():
    """The causal backward on the whole c3 grid (B = 2, H = 16, N = 8192,
    D = 128): both kernels run over all 32 heads, and eight of them are
    compared with the dense oracle.  The tile scheduler gives each of the
    eight XCDs a contiguous group of B*H/8 = 4 heads, so the heads checked,
    bh = 0, 5, 10, 15, 16, 21, 26, 31, are one per XCD group and each
    position within a group."""
    w = WORKLOADS["c3"].with_(name="c3_bwd", backward=True, seed=13)
    log(f"test_backward_c3_shape B={w.B} H={w.H} N={w.N} D={w.D} causal={w.causal}")
    x = make_inputs(w, with_do=True)
    got = _run_bwd(w, x)
    heads = [divmod(bh, w.H) for bh in (0, 5, 10, 15, 16, 21, 26, 31)]
    _check(w, x, got, heads=heads)


def test_backward_deterministic():
    """No atomics anywhere: two runs agree bit for bit."""
    import torch

    w = WORKLOADS["c5"].with_(B=1, H=2, N=512, D=128)
    x = make_inputs(w, with_do=True)
    a = _run_bwd(w, x)
    b = _run_bwd(w, x)
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)


def test_backward_identical_keys_give_zero_dq():
    """With every key equal the scores do not depend on q, so dQ = 0."""
    import torch

    import exact_attention_51_amd as fa

    w = WORKLOADS["c5"].with_(B=1, H=1, N=256, D=128)
    x = make_inputs(w, with_do=True)
    q, k, v, do = (dev_bf16(b) for b in (x.q_bits, x.k_bits, x.v_bits, x.do_bits))
    kc = k[:, :, :1].expand(-1, -1, w.N, -1).contiguous()
    for causal in (False, True):
        o, lse = fa.fwd(q, kc, v, w.scale, causal)
        dq, dk, dv, delta = fa.bwd(q, kc, v, o, do, lse, w.scale, causal)
        torch.cuda.synchronize()
        ref = oracle.backward(x.q[0, 0], np.tile(x.k[0, 0, :1], (w.N, 1)), x.v[0, 0], x.do[0, 0], w.scale, causal)
        scale_ref = float(np.abs(ref["dv"]).max())
        assert float(np.abs(host(dq)).max()) <= 2e-2 * scale_ref + 1e-3
