"""Seeded synthetic workloads for the Laplacian-kernel Nystrom attention forward.

This module is shared by the CPU oracle's tests, the GPU parity tests, the
smoke check and the benchmark.  It holds the workload shapes and the seeded
input draws only: it contains none of the attention method's arithmetic, so
sharing it does not couple the oracle to the GPU path.

Inputs stand in for the heavy-tailed query/key statistics that the
LaplacianFormer pages report for vision transformers (each page's problem
statement, section 1): Q, K and V are i.i.d. Student-t with 3 degrees of
freedom, scaled by 0.25, drawn in float64 from numpy's PCG64 generator, then
rounded to nearest-even float32, then (for bf16 workloads) rounded to
nearest-even bfloat16.  The draw order is Q, then K, then V.
"""

from __future__ import annotations

import dataclasses
from typing import Dict

import numpy as np

SEED_BASE = 20260423


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic forward problem set: B*H independent (batch, head) problems."""

    name: str
    B: int
    H: int
    grid_h: int
    grid_w: int
    d: int
    pool: int
    lam: float = 4.0
    eps: float = 1e-3
    ns_iters: int = 20
    dtype: str = "f32"  # storage type of Q, K, V: "f32" or "bf16"
    whiten: bool = True
    seed_index: int = 0
    refine: bool = False  # one float64-residual correction after the Newton-Schulz steps
    kernel: str = "laplacian"  # or "gaussian"
    solver: str = "ns"  # or "cg" (conjugate gradient for W^-1 (B V))
    ns_plain: bool = False  # every Newton-Schulz product in float32 (m <= 64: as a launch of its own)
    # > 0: every odd pooled window of each landmark row of K is replaced by its
    # left neighbour's tokens plus near_dup-scaled normal noise (see
    # make_inputs), so pairs of landmarks nearly coincide and W is close to
    # singular.
    near_dup: float = 0.0

    @property
    def N(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def m(self) -> int:
        return (self.grid_h // self.pool) * (self.grid_w // self.pool)

    @property
    def P(self) -> int:
        return self.B * self.H

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.N

    @property
    def seed(self) -> int:
        return SEED_BASE + self.seed_index

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five forward workloads, plus the stage-1 shape with bf16 storage (the
# headline throughput workload) and the two smaller points of the sequence
# length sweep at 256 landmarks.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32", B=1, H=1, grid_h=14, grid_w=14, d=32, pool=2,
                 dtype="f32", seed_index=1),
        Workload("stage1_56x56_f32", B=32, H=1, grid_h=56, grid_w=56, d=64, pool=8,
                 dtype="f32", seed_index=2),
        Workload("stage2_28x28_bf16", B=32, H=2, grid_h=28, grid_w=28, d=64, pool=4,
                 dtype="bf16", seed_index=3),
        Workload("stage3_14x14_bf16", B=64, H=5, grid_h=14, grid_w=14, d=64, pool=2,
                 dtype="bf16", seed_index=4),
        Workload("long_256x256_bf16", B=1, H=8, grid_h=256, grid_w=256, d=64, pool=16,
                 ns_iters=24, dtype="bf16", seed_index=5),
        Workload("stage1_56x56_bf16", B=32, H=1, grid_h=56, grid_w=56, d=64, pool=8,
                 dtype="bf16", seed_index=6),
        Workload("sweep_64x64_bf16", B=1, H=8, grid_h=64, grid_w=64, d=64, pool=4,
                 ns_iters=24, dtype="bf16", seed_index=7),
        Workload("sweep_128x128_bf16", B=1, H=8, grid_h=128, grid_w=128, d=64, pool=8,
                 ns_iters=24, dtype="bf16", seed_index=8),
    ]
}

# The workload the throughput metric is quoted on: N=3136, d=64, m=49, bf16.
HEADLINE = "stage1_56x56_bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """Q, K, V of one workload.

    ``q``/``k``/``v`` hold the storage form handed to the device (float32 arrays,
    or uint16 arrays of bfloat16 bit patterns); ``qf``/``kf``/``vf`` hold the
    same values widened exactly to float64.  Shapes are [B, H, N, d], C order.
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    qf: np.ndarray
    kf: np.ndarray
    vf: np.ndarray


def _draw(rng: np.random.Generator, shape, dtype: str):
    x64 = rng.standard_t(3.0, size=shape) * 0.25
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32, x32.astype(np.float64)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_grad_out(w: Workload, seed: int = 99) -> np.ndarray:
    """A float32 output gradient dO of shape [B, H, N, d] (standard normal, PCG64(seed))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((w.B, w.H, w.N, w.d)).astype(np.float32)


def near_duplicate_keys(k32: np.ndarray, w: Workload, delta: float, rng: np.random.Generator) -> np.ndarray:
    """K (float32, [B, H, N, d]) with every odd pooled window column of the
    token grid replaced by the window to its left plus delta * N(0, 1) noise
    (float32): the landmarks of windows 2c and 2c + 1 then differ by about
    delta, which makes the landmark kernel matrix nearly singular.  A
    structural recipe for ill-conditioned inputs; it computes nothing of the
    attention method."""
    k = np.array(k32, dtype=np.float32, copy=True)
    p, gw = w.pool, w.grid_w // w.pool
    g = k.reshape(w.B, w.H, w.grid_h, w.grid_w, w.d)
    for j in range(1, gw, 2):
        src = g[:, :, :, (j - 1) * p:j * p, :]
        g[:, :, :, j * p:(j + 1) * p, :] = src + np.float32(delta) * rng.standard_normal(src.shape).astype(np.float32)
    return g.reshape(k.shape)


def make_inputs(w: Workload, seed: int | None = None) -> Inputs:
    """Draw Q, K, V for workload ``w`` from PCG64(seed) (default: the workload's seed).

    With ``w.near_dup > 0`` the float32 K is then made near-duplicate
    (``near_duplicate_keys``, noise from PCG64(seed + 1000)) before any
    rounding to bf16."""
    s = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(s))
    shape = (w.B, w.H, w.N, w.d)
    if w.near_dup > 0:
        x64 = [rng.standard_t(3.0, size=shape) * 0.25 for _ in range(3)]
        x32 = [a.astype(np.float32) for a in x64]
        x32[1] = near_duplicate_keys(x32[1], w, w.near_dup, np.random.Generator(np.random.PCG64(s + 1000)))
        out = []
        for a in x32:
            if w.dtype == "f32":
                out.append((a, a.astype(np.float64)))
            else:
                bits = f32_to_bf16_bits(a)
                out.append((bits, bf16_bits_to_f32(bits).astype(np.float64)))
        (q, qf), (k, kf), (v, vf) = out
        return Inputs(q, k, v, qf, kf, vf)
    q, qf = _draw(rng, shape, w.dtype)
    k, kf = _draw(rng, shape, w.dtype)
    v, vf = _draw(rng, shape, w.dtype)
    return Inputs(q, k, v, qf, kf, vf)
