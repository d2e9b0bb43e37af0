"""Seeded synthetic inputs for the attention forward workloads.

This module only draws numbers and rounds them to the storage type the
device receives; it contains none of the attention arithmetic, so both the
HIP path and the CPU oracle can be fed from it.

Tensors are C-order ``[B, H, N, d]`` (batch, heads, sequence, head dim), the
layout the attention pages use for Q, K and V ("Flash Attention" tag page,
excerpt on the standard attention listing).

Recipe (numpy ``Generator(PCG64(seed))``, ``standard_normal`` in float32):

* Q, K, V are drawn in that order, each over the whole ``[B, H, N, d]``.
* ``qk_gain`` multiplies Q and K (the sharpened-softmax workload uses 2).
* ``spike_frac`` > 0 then picks, per (b, h) in order,
  ``round(spike_frac * N)`` distinct key rows with ``rng.choice`` and
  multiplies them by ``spike_gain`` (8 for the long-sequence workload).
* Powers of two are exact under the later rounding, so the gains commute
  with it.
* ``dtype="bf16"`` rounds every value to the nearest bfloat16 (ties to
  even); the arrays stay float32 so the same array can be handed to torch
  (``.to(torch.bfloat16)`` is then exact) and, widened to float64, to the
  oracle.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even.

    Returns float32 whose low 16 bits are zero.  Inputs here are finite
    normals, so no NaN/Inf special-casing is needed; those are rejected.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_to_bf16 expects finite inputs")
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


@dataclass(frozen=True)
class Workload:
    """One attention-forward workload: shapes, storage type and value recipe."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32", "bf16" or "fp8" (fp8 = e4m3 Q/K built on the device from bf16)
    causal: bool
    seed: int
    qk_gain: float = 1.0
    spike_frac: float = 0.0
    spike_gain: float = 8.0
    note: str = field(default="", compare=False)

    @property
    def shape(self) -> tuple[int, int, int, int]:
        return (self.B, self.H, self.N, self.d)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def flops(self) -> float:
        """Attention FLOPs by the usual convention: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * float(self.N) ** 2 * self.d
        return f / 2.0 if self.causal else f

    def compulsory_bytes(self) -> int:
        """Bytes that must cross HBM once: Q, K, V read, O and lse written (+ fp8 scales)."""
        elems = self.B * self.H * self.N * self.d
        if self.dtype == "f32":
            io = 4 * elems * 4
        elif self.dtype == "bf16":
            io = 4 * elems * 2
        elif self.dtype == "fp8":  # fp8 Q/K codes, bf16 V and O, one fp32 scale per 64-row tile of Q and of K
            tiles = self.B * self.H * ((self.N + 63) // 64)
            io = 2 * elems * 1 + 2 * elems * 2 + 2 * tiles * 4
        else:  # fp8pv: fp8 Q/K/V codes, bf16 O, Q/K tile scales and one exponent byte per (tile, column) of V
            tiles = self.B * self.H * ((self.N + 63) // 64)
            io = 3 * elems * 1 + elems * 2 + 2 * tiles * 4 + tiles * self.d
        return io + self.B * self.H * self.N * 4


# The five workloads the forward pass is measured and checked on.  The
# 1024/d_model-512 shape is the one the Triton-walkthrough page times on its
# RTX 4090 (section 6.1); N = 32768 is where it quotes its FP8 speed-up.
WORKLOADS: dict[str, Workload] = {
    "c1_f32": Workload("c1_f32", 1, 2, 128, 64, "f32", False, 1,
                       note="fp32, N(0,1), non-causal"),
    "c2_bf16": Workload("c2_bf16", 8, 16, 1024, 32, "bf16", False, 2,
                        note="bf16, d_model 512, non-causal"),
    "c2_bf16_causal": Workload("c2_bf16_causal", 8, 16, 1024, 32, "bf16", True, 2,
                               note="bf16, d_model 512, causal (same tensors)"),
    "c3_bf16": Workload("c3_bf16", 4, 32, 4096, 128, "bf16", True, 3, qk_gain=2.0,
                        note="bf16 causal, Q and K scaled by 2"),
    "c4_bf16": Workload("c4_bf16", 1, 32, 16384, 128, "bf16", True, 4, spike_frac=0.01,
                        note="bf16 causal long sequence, 1% of K rows x8"),
    "c5_fp8": Workload("c5_fp8", 1, 16, 32768, 128, "fp8", True, 5,
                       note="fp8 e4m3 Q/K with per-64-row scales, bf16 V, causal"),
    # the same tensors with P*V on e4m3 as well (the next row after the five)
    "c5_fp8pv": Workload("c5_fp8pv", 1, 16, 32768, 128, "fp8pv", True, 5,
                         note="fp8 e4m3 Q/K (per-64-row scales) and V, P (power-of-two block scales), causal"),
}


def make_inputs(w: Workload, seed: int | None = None, shape: tuple | None = None):
    """Draw (q, k, v) as float32 numpy arrays following ``w``'s recipe.

    ``shape`` overrides ``w.shape`` (the same recipe at another size, for
    small parity cases); ``seed`` overrides ``w.seed``.  For "bf16" and "fp8"
    the values are rounded to bfloat16 (fp8 Q/K are produced from these bf16
    tensors on the device).
    """
    shp = tuple(shape) if shape is not None else w.shape
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    q = rng.standard_normal(shp, dtype=np.float32)
    k = rng.standard_normal(shp, dtype=np.float32)
    v = rng.standard_normal(shp, dtype=np.float32)
    if w.qk_gain != 1.0:
        q *= np.float32(w.qk_gain)
        k *= np.float32(w.qk_gain)
    if w.spike_frac > 0.0:
        B, H, N, _ = shp
        n_spike = int(round(w.spike_frac * N))
        for b in range(B):
            for h in range(H):
                rows = rng.choice(N, n_spike, replace=False)
                k[b, h, rows, :] *= np.float32(w.spike_gain)
    if w.dtype in ("bf16", "fp8", "fp8pv"):
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


def digest(*arrays: np.ndarray) -> str:
    """SHA-256 over the raw bytes of the given arrays (input provenance)."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def make_grad(w: Workload, seed: int | None = None, shape: tuple | None = None):
    """Upstream gradient dO for the backward pass: standard normal, rounded to
    bf16, from its own stream (PCG64 seeded with ``seed`` or ``w.seed``
    + 1_000_003), so the forward inputs of a workload stay unchanged."""
    shp = tuple(shape) if shape is not None else w.shape
    rng = np.random.Generator(np.random.PCG64((w.seed if seed is None else seed) + 1_000_003))
    return round_to_bf16(rng.standard_normal(shp, dtype=np.float32))


def band_global_block_mask(nb: int, window: int = 16, n_global: int = 2) -> np.ndarray:
    """0/1 table [nb, nb] of 64x64 blocks: every query block sees the ``window``
    key blocks ending at its own (a sliding window) plus the first ``n_global``
    key blocks (global tokens) -- the sliding-window-plus-global pattern the
    pages cite for sparse attention.  Blocks above the diagonal are left to the
    causal flag."""
    qb = np.arange(nb)[:, None]
    kb = np.arange(nb)[None, :]
    m = ((kb <= qb) & (kb > qb - window)) | (kb < n_global)
    return m.astype(np.uint8)


def random_block_mask(nb: int, density: float, seed: int, shape_prefix: tuple = ()) -> np.ndarray:
    """Seeded 0/1 block table with about ``density`` of the blocks set."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.random(tuple(shape_prefix) + (nb, nb)) < density).astype(np.uint8)
