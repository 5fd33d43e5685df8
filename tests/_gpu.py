"""Helpers for the GPU parity tests: move seeded inputs to the device, run
the library through its C ABI and compare with the float64 oracle."""

import sys

import numpy as np

# Tolerances (max absolute error) for the forward: bf16 inputs with float32
# accumulation, and float32 throughout.
TOL_BF16_O = 2e-2
TOL_BF16_L = 1e-2
TOL_F32 = 1e-4
# Backward, bf16: the forward's output bound carried over to dQ, dK, dV,
# plus the same bound relative to the largest reference magnitude.
TOL_BF16_GRAD = 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_f32(arr):
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def host(t):
    import torch

    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def inputs_on_device(w, x):
    """(q, k, v) device tensors in the workload's dtype, from seeded inputs x."""
    if w.dtype == "fp32":
        return dev_f32(x.q), dev_f32(x.k), dev_f32(x.v)
    return dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits)


def sample_rows(n, count, seed):
    """Rows to check at large N: the ends, tile boundaries and random rows."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, n // 2, n - 257, n - 256, n - 65, n - 64, n - 2, n - 1]
    rows = [r for r in fixed if 0 <= r < n]
    rows += list(rng.integers(0, n, size=count))
    return np.unique(np.array(rows, dtype=np.int64))
