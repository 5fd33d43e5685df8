"""Seeded synthetic inputs for exact attention, shared by the tests, the
benchmark and the smoke check.

This module holds no arithmetic of the attention method.  It only draws
random numbers, rounds them to the storage type and describes the
workloads.  Both the CPU oracle and the GPU library consume exactly the
bits produced here: the GPU gets the bf16 bit patterns, the oracle gets the
same values widened (exactly) to float64.

Workloads (all i.i.d. N(0, 1) draws, BHND contiguous, scale = 1/sqrt(D)):

=====  =====  ==  =====  ===  ======  ======================================
name   B      H   N      D    dtype   notes
=====  =====  ==  =====  ===  ======  ======================================
c1     1      1   256    64   fp32    non-causal
c2     4      16  2048   64   bf16    non-causal
c3     2      16  8192   128  bf16    causal
c4     1      8   32768  128  bf16    causal, Q drawn then multiplied by 3
c5     1      4   4096   256  bf16    non-causal, forward and backward (dO)
=====  =====  ==  =====  ===  ======  ======================================

Draw order is Q, K, V, then dO, each as float32 ``standard_normal`` from
``numpy.random.default_rng(seed)``; the Q multiplier is applied to the
float32 draw and the result is rounded once to bf16 (round to nearest,
ties to even).  The default seed of each workload is its index (1..5).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "bf16_round", "bf16_bits_to_f32", "make_inputs", "Inputs"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str  # "bf16" or "fp32"
    causal: bool
    q_mult: float = 1.0
    backward: bool = False
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def fwd_flop(self) -> int:
        """4 N^2 D per (batch, head) for the two products, halved under causal."""
        f = 4 * self.N * self.N * self.D * self.B * self.H
        return f // 2 if self.causal else f

    def bwd_flop(self) -> int:
        """Split backward: 3 products in the dQ kernel and 4 in the dK/dV kernel.

        That is 6 N^2 D + 8 N^2 D = 14 N^2 D per (batch, head), halved under
        causal masking (metal-flash-attention README, "Quantifying
        performance": the split design costs seven products instead of five).
        """
        f = 14 * self.N * self.N * self.D * self.B * self.H
        return f // 2 if self.causal else f


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 256, 64, "fp32", False, seed=1),
    "c2": Workload("c2", 4, 16, 2048, 64, "bf16", False, seed=2),
    "c3": Workload("c3", 2, 16, 8192, 128, "bf16", True, seed=3),
    "c4": Workload("c4", 1, 8, 32768, 128, "bf16", True, q_mult=3.0, seed=4),
    "c5": Workload("c5", 1, 4, 4096, 256, "bf16", False, backward=True, seed=5),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def bf16_round(x: np.ndarray):
    """Round float32 to bf16, nearest-even.  Returns (values as float32, uint16 bits).

    NaN is not expected from normal draws and is not handled specially.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    vals = (rounded.astype(np.uint32) << 16).view(np.float32)
    return vals, rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32, exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    """Values as float32 (exactly representable in the storage dtype) and,
    for bf16, the bit patterns the GPU receives."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray | None
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None
    do_bits: np.ndarray | None = None


def make_inputs(w: Workload, seed: int | None = None, with_do: bool | None = None) -> Inputs:
    """Draw Q, K, V (and dO) for workload ``w`` with the given seed."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.D)
    with_do = w.backward if with_do is None else with_do
    raw = []
    for i, name in enumerate(("q", "k", "v", "do")):
        if name == "do" and not with_do:
            raw.append(None)
            continue
        a = rng.standard_normal(shape, dtype=np.float32)
        if name == "q" and w.q_mult != 1.0:
            a *= np.float32(w.q_mult)
        raw.append(a)
    if w.dtype == "fp32":
        return Inputs(*raw)
    vals, bits = [], []
    for a in raw:
        if a is None:
            vals.append(None)
            bits.append(None)
        else:
            fv, b = bf16_round(a)
            vals.append(fv)
            bits.append(b)
    return Inputs(*vals, *bits)
