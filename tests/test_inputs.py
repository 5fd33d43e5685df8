"""The seeded input generator: determinism, shapes and bf16 rounding."""

import numpy as np
import torch

import fa_inputs
from fa_inputs import WORKLOADS, bf16_bits_to_f32, bf16_round, make_inputs


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate(
        [
            rng.standard_normal(100000, dtype=np.float32) * 3,
            np.array([0.0, -0.0, 1.0, -1.0, 1e-40, 3.0e38, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-9], np.float32),
        ]
    )
    vals, bits = bf16_round(x)
    t = torch.from_numpy(x).to(torch.bfloat16)
    np.testing.assert_array_equal(bits, t.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(vals, t.float().numpy())
    np.testing.assert_array_equal(bf16_bits_to_f32(bits), vals)


def test_inputs_deterministic_and_shaped():
    w = WORKLOADS["c2"].with_(B=1, H=2, N=64)
    a = make_inputs(w)
    b = make_inputs(w)
    for name in ("q", "k", "v", "q_bits", "k_bits", "v_bits"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    assert a.q.shape == (1, 2, 64, 64) and a.q.dtype == np.float32 and a.q_bits.dtype == np.uint16
    assert a.do is None
    c = make_inputs(w, seed=99)
    assert not np.array_equal(a.q, c.q)


def test_q_multiplier_and_backward_inputs():
    w4 = WORKLOADS["c4"].with_(N=256, H=1)
    x = make_inputs(w4)
    base = make_inputs(w4.with_(q_mult=1.0))
    np.testing.assert_array_equal(x.k, base.k)
    assert 2.5 < x.q.std() / base.q.std() < 3.5
    w5 = WORKLOADS["c5"].with_(N=128)
    y = make_inputs(w5)
    assert y.do is not None and y.do_bits is not None and y.do.shape == y.q.shape


def test_flop_counts():
    assert WORKLOADS["c3"].fwd_flop() == 549755813888
    assert WORKLOADS["c2"].fwd_flop() == 68719476736
    assert WORKLOADS["c4"].fwd_flop() == 2199023255552
    assert WORKLOADS["c5"].fwd_flop() == 68719476736
    assert WORKLOADS["c5"].bwd_flop() == 6 * 4096**2 * 256 * 4 + 8 * 4096**2 * 256 * 4
    assert fa_inputs.workload("c1").fwd_flop() == 16777216
