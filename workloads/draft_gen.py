"""Seeded synthetic inputs for the draft model's sliding-window self-attention.

The draft keeps a ring of the last ``W`` positions' keys and values (slot =
position mod W) and adds ``Tn`` new tokens per step. Recipe (one
``numpy.random.default_rng(seed)``), drawn in this order, all float32 N(0, 1):
``q[B, Hq, Tn, D]``, ``k_ring[B, Hkv, W, D]``, ``v_ring``, ``k_new[B, Hkv, Tn,
D]``, ``v_new``. ``pos[B]`` (tokens written before the step) is given by the
caller. Ring slots that hold no position yet (slot >= pos when pos < W) are
zero, or NaN with ``poison_unused`` so tests can show they are never read.
bf16 cases round to bfloat16 (nearest, ties to even) and keep the bit
patterns. This module draws numbers only; it holds none of the attention
arithmetic.
"""

from __future__ import annotations

import dataclasses
from typing import Sequence

import numpy as np

from .gen import bf16_bits_to_f32, f32_to_bf16_bits


@dataclasses.dataclass
class WindowCase:
    dtype: str
    B: int
    Hq: int
    Hkv: int
    D: int
    W: int
    Tn: int
    q: np.ndarray        # [B, Hq, Tn, D]
    k_ring: np.ndarray   # [B, Hkv, W, D]
    v_ring: np.ndarray
    k_new: np.ndarray    # [B, Hkv, Tn, D]
    v_new: np.ndarray
    pos: np.ndarray      # int32 [B]
    scale: float

    def as_f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return np.asarray(a, dtype=np.float64)


def make_window_case(*, B: int, Hq: int, Hkv: int, D: int, W: int, Tn: int, pos: Sequence[int],
                     dtype: str = "bf16", seed: int = 0, poison_unused: bool = False) -> WindowCase:
    rng = np.random.default_rng(seed)
    pos = np.asarray(pos, dtype=np.int32).reshape(B)
    draw = lambda *shape: rng.standard_normal(shape, dtype=np.float32)
    q = draw(B, Hq, Tn, D)
    kr, vr = draw(B, Hkv, W, D), draw(B, Hkv, W, D)
    kn, vn = draw(B, Hkv, Tn, D), draw(B, Hkv, Tn, D)
    for b in range(B):
        if pos[b] < W:
            fill = np.nan if poison_unused else 0.0
            kr[b, :, pos[b]:] = fill
            vr[b, :, pos[b]:] = fill
    if dtype == "bf16":
        q, kr, vr, kn, vn = (_bits_keep_nan(a) for a in (q, kr, vr, kn, vn))
    return WindowCase(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, W=W, Tn=Tn, q=q, k_ring=kr, v_ring=vr,
                      k_new=kn, v_new=vn, pos=pos, scale=1.0 / float(np.sqrt(D)))


def _bits_keep_nan(a: np.ndarray) -> np.ndarray:
    bits = f32_to_bf16_bits(np.nan_to_num(a, nan=0.0))
    bits[np.isnan(a)] = 0x7FC0
    return bits
