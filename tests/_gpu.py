"""Helpers for the GPU parity tests: move seeded inputs to the device, run
the library through its C ABI and compare with the float64 oracle."""

import os
import sys
from concurrent.futures import ThreadPoolExecutor

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


def pool_workers(cap=16):
    """Worker threads for the CPU oracle: the host cores this process may use,
    at most ``cap`` (one GPU's share of a shared host)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(n, cap))


def forward_errors_all_rows(w, x, o_host, l_host, row_block=256):
    """Max |O - O_ref| and max |L - L_ref| over EVERY row of every (batch,
    head), the oracle run on (batch, head, row block) units over a thread
    pool (one BLAS thread per worker).  o_host, l_host: the GPU results as
    float64 host arrays [B, H, N, D] and [B, H, N]."""
    import oracle
    from threadpoolctl import threadpool_limits

    def unit(args):
        b, h, r0 = args
        rows = np.arange(r0, min(w.N, r0 + row_block))
        o_ref, l_ref = oracle.forward_rows(x.q[b, h], x.k[b, h], x.v[b, h], rows, w.scale, w.causal)
        return (float(np.abs(o_host[b, h, rows] - o_ref).max()), float(np.abs(l_host[b, h, rows] - l_ref).max()))

    units = [(b, h, r0) for b in range(w.B) for h in range(w.H) for r0 in range(0, w.N, row_block)]
    with threadpool_limits(1), ThreadPoolExecutor(pool_workers()) as ex:
        res = list(ex.map(unit, units))
    return max(r[0] for r in res), max(r[1] for r in res)
