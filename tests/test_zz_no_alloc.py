"""fa_fwd_kv_noalloc (the entry point that allocates nothing: key-range
partials in the library's per-device scratch array) against fa_fwd_kv with
a caller workspace, through the C ABI, and both against the float64 oracle.

Two calls in a row, the second on a smaller input, for each path: the
matrix-core range kernel with the narrow merge, the same with more than
eight ranges (wide merge), the vector decode kernel, and D = 256.
"""

import numpy as np
import pytest

import oracle
from fa_inputs import WORKLOADS, make_inputs
from tests._gpu import TOL_BF16_L, TOL_BF16_O, dev_bf16, host, log

pytestmark = pytest.mark.gpu


def _inputs(B, H, Nq, Nk, D, seed):
    w = WORKLOADS["c3"].with_(B=B, H=H, N=Nk, D=D, seed=seed)
    x = make_inputs(w, with_do=False)
    q = np.ascontiguousarray(x.q[:, :, Nk - Nq :])
    qb = np.ascontiguousarray(x.q_bits[:, :, Nk - Nq :])
    return w.scale, q, x.k, x.v, dev_bf16(qb), dev_bf16(x.k_bits), dev_bf16(x.v_bits)


# (first call, second smaller call): (B, H, Nq, Nk, D, causal, splits)
CASES = [
    ((2, 4, 300, 2048, 128, True, 4), (1, 2, 70, 520, 128, True, 3)),
    ((1, 4, 200, 4096, 64, False, 12), (1, 2, 64, 1500, 64, False, 10)),
    ((2, 8, 1, 8192, 128, True, 16), (1, 3, 2, 1000, 128, True, 5)),
    ((1, 2, 130, 1024, 256, True, 4), (1, 1, 33, 300, 256, False, 2)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_fwd_kv(first, second):
    import torch

    import exact_attention_51_amd as fa

    for i, (B, H, Nq, Nk, D, causal, splits) in enumerate((first, second)):
        log(f"test_noalloc call {i}: B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} splits={splits}")
        scale, q, k, v, qd, kd, vd = _inputs(B, H, Nq, Nk, D, seed=31 * Nq + Nk + D)
        o_ref_gpu, l_ref_gpu = fa.fwd_kv(qd, kd, vd, scale, causal, splits)
        o = torch.full_like(qd, 7.0)
        lse = torch.full((B, H, Nq), 7.0, dtype=torch.float32, device=qd.device)
        fa.fwd_kv_noalloc(qd, kd, vd, o, lse, scale, causal, splits)
        torch.cuda.synchronize()
        # same kernels, same ranges: identical bits
        assert torch.equal(o, o_ref_gpu) and torch.equal(lse, l_ref_gpu)
        o_ref, l_ref = oracle.forward_kv(q, k, v, scale, causal)
        eo = float(np.abs(host(o) - o_ref).max())
        el = float(np.abs(host(lse) - l_ref).max())
        log(f"  max|dO|={eo:.3e} max|dL|={el:.3e}")
        assert eo <= TOL_BF16_O and el <= TOL_BF16_L


def test_noalloc_library_split_count_and_limit():
    """num_splits = 0 takes the library's count; a range count whose partials
    exceed the scratch array is refused with FA_ERR_INVALID_ARG, nothing
    launched (the outputs keep their fill)."""
    import torch

    import exact_attention_51_amd as fa

    scale, q, k, v, qd, kd, vd = _inputs(1, 8, 1, 16384, 128, seed=5)
    o = torch.empty_like(qd)
    lse = torch.empty((1, 8, 1), dtype=torch.float32, device=qd.device)
    fa.fwd_kv_noalloc(qd, kd, vd, o, lse, scale, True, 0)
    o2, l2 = fa.fwd_kv(qd, kd, vd, scale, True, 0)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)

    B, H, Nq, Nk, D = 1, 64, 512, 1024, 128
    lib = fa._lib.load()
    assert lib.fa_fwd_kv_workspace_bytes(B, H, Nq, D, 8) > fa._lib.FA_FWD_KV_NOALLOC_MAX_BYTES
    qd = torch.zeros((B, H, Nq, D), dtype=torch.bfloat16, device="cuda")
    kd = torch.zeros((B, H, Nk, D), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(qd, 3.0)
    lse = torch.full((B, H, Nq), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError) as ei:
        fa.fwd_kv_noalloc(qd, kd, kd, o, lse, None, False, 8)
    assert ei.value.code == fa._lib.FA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((lse == 3.0).all())
