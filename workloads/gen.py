"""Seeded synthetic workloads: draft trees, KV caches and tree-token tensors.

The five named workloads are layer shapes of the target models the LongSpec
page lists in its experimental setup (Vicuna-7B, Llama-3.1-8B, QwQ-32B), with
the draft tree that a verification step attends to (LongSpec, "fast tree
attention"; LogitSpec, "draft tree construction and verification"). Token
content does not change the cost of the attention, so N(0,1) tensors stand in
for the long-context and math-reasoning datasets the pages measure on.

Recipe (one ``numpy.random.default_rng(seed)`` per workload, default seed
``1000 + k`` for workload k), drawn in this fixed order:

1. prefix lengths ``prefix_len[B]``;
2. parent arrays ``parent[B, T]`` (node 0 is the root, ``parent[b, 0] = -1``,
   ``-1 <= parent[b, i] < i``);
3. ``q[B, Hq, T, D]``, 4. ``k_cache[B, Hkv, Lcap, D]``, 5. ``v_cache``,
6. ``k_tree[B, Hkv, T, D]``, 7. ``v_tree``; all float32 N(0, 1).

bf16 workloads round every float32 sample to bfloat16 (round to nearest,
ties to even) and keep the 16-bit patterns; the exact float values of those
patterns are what every consumer sees. Cache rows at positions
``>= prefix_len[b]`` are zero (or NaN when ``poison_tail`` is set, so tests
can show that no kernel reads them into a result).

Tree shapes:
* ``uniform``: node i picks its parent uniformly in ``[0, i-1]``.
* ``bounded(d, f)``: node i picks its parent uniformly among the earlier nodes
  j with ``depth(j) < d`` and fewer than ``f`` children (``f`` unbounded when
  not given). The root has depth 0.

Key drift (the 131k workload): every component of a key at absolute position
``pos`` gets ``0.5 * sin(pos / 1000)`` added before rounding; prefix keys sit
at ``pos = 0 .. L-1`` and tree node i at ``pos = L + depth(i)``.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# bf16 bit patterns
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Finite inputs only (the generators never produce NaN before poisoning).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Trees
# ----------------------------------------------------------------------------

def tree_uniform(T: int, rng: np.random.Generator) -> np.ndarray:
    """parent[i] uniform in [0, i-1]; parent[0] = -1."""
    p = np.full(T, -1, dtype=np.int32)
    for i in range(1, T):
        p[i] = int(rng.integers(0, i))
    return p


def tree_bounded(T: int, rng: np.random.Generator, max_depth: int,
                 max_fanout: Optional[int] = None) -> np.ndarray:
    """Random tree with depth <= max_depth and at most max_fanout children per node."""
    p = np.full(T, -1, dtype=np.int32)
    depth = [0]
    children = [0]
    for i in range(1, T):
        elig = [j for j in range(i)
                if depth[j] < max_depth and (max_fanout is None or children[j] < max_fanout)]
        if not elig:
            raise ValueError("tree bounds leave no eligible parent")
        j = elig[int(rng.integers(0, len(elig)))]
        p[i] = j
        depth.append(depth[j] + 1)
        children[j] += 1
        children.append(0)
    return p


def tree_chain(T: int) -> np.ndarray:
    """parent[i] = i - 1: the tree is one path (plain causal decoding of T tokens)."""
    return np.arange(-1, T - 1, dtype=np.int32)


def tree_star(T: int) -> np.ndarray:
    """Every node but the root hangs off the root."""
    p = np.zeros(T, dtype=np.int32)
    p[0] = -1
    return p


def tree_depths(parent: np.ndarray) -> np.ndarray:
    """Depth of each node of a topologically ordered parent array (roots have depth 0)."""
    d = np.zeros(len(parent), dtype=np.int32)
    for i, pi in enumerate(parent):
        d[i] = 0 if pi < 0 else d[pi] + 1
    return d


# ----------------------------------------------------------------------------
# Workload descriptions
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    key: int
    name: str
    dtype: str               # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    D: int
    Lcap: int
    T: int
    prefix: tuple            # ("fixed", L) or ("uniform", lo, hi) inclusive
    tree: tuple              # ("uniform",) or ("bounded", max_depth, max_fanout|None)
    drift: bool = False

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


CONFIGS = {
    1: WorkloadConfig(1, "tiny-f32-mha4-d64-L256-T8", "f32", 1, 4, 4, 64, 256, 8,
                      ("fixed", 256), ("uniform",)),
    2: WorkloadConfig(2, "vicuna7b-bf16-mha32-d128-L4096-T26", "bf16", 1, 32, 32, 128, 4096, 26,
                      ("fixed", 4096), ("bounded", 5, 4)),
    3: WorkloadConfig(3, "llama31-8b-bf16-gqa32x8-d128-L32768-T64", "bf16", 1, 32, 8, 128, 32768, 64,
                      ("fixed", 32768), ("bounded", 6, None)),
    4: WorkloadConfig(4, "qwq32b-bf16-gqa40x8-d128-B4-L8k..32k-T32", "bf16", 4, 40, 8, 128, 32768, 32,
                      ("uniform", 8192, 32768), ("uniform",)),
    5: WorkloadConfig(5, "llama31-8b-bf16-gqa32x8-d128-L131072-T64-drift", "bf16", 1, 32, 8, 128, 131072, 64,
                      ("fixed", 131072), ("bounded", 8, None), drift=True),
}


@dataclasses.dataclass
class Workload:
    """One batch of inputs. Float tensors are float32 arrays (f32) or uint16 bf16 bits."""
    dtype: str
    B: int
    Hq: int
    Hkv: int
    D: int
    Lcap: int
    T: int
    scale: float
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    k_tree: np.ndarray
    v_tree: np.ndarray
    parent: np.ndarray        # int32 [B, T]
    prefix_len: np.ndarray    # int32 [B]
    name: str = "custom"

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def as_f64(self, name: str) -> np.ndarray:
        """Exact float64 values of one of the float tensors."""
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _draw_tensors(rng, dtype, B, Hq, Hkv, D, Lcap, T, prefix_len, parents, drift, poison_tail,
                  v_tree_override=None):
    q = rng.standard_normal((B, Hq, T, D), dtype=np.float32)
    kc = rng.standard_normal((B, Hkv, Lcap, D), dtype=np.float32)
    vc = rng.standard_normal((B, Hkv, Lcap, D), dtype=np.float32)
    kt = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    vt = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    if drift:
        pos = np.arange(Lcap, dtype=np.float64)
        kc += (0.5 * np.sin(pos / 1000.0)).astype(np.float32)[None, None, :, None]
        for b in range(B):
            tpos = prefix_len[b] + tree_depths(parents[b]).astype(np.float64)
            kt[b] += (0.5 * np.sin(tpos / 1000.0)).astype(np.float32)[None, :, None]
    q, kc, vc, kt, vt = (_round(a, dtype) for a in (q, kc, vc, kt, vt))
    for b in range(B):
        L = int(prefix_len[b])
        if 0 <= L < Lcap:
            if poison_tail:
                fill = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
            else:
                fill = 0
            kc[b, :, L:, :] = fill
            vc[b, :, L:, :] = fill
    return q, kc, vc, kt, vt


def make_workload(key: int, seed: Optional[int] = None, poison_tail: bool = False) -> Workload:
    """Inputs for one of the five named workloads (seed defaults to 1000 + key)."""
    c = CONFIGS[key]
    rng = np.random.default_rng(1000 + key if seed is None else seed)
    if c.prefix[0] == "fixed":
        prefix_len = np.full(c.B, c.prefix[1], dtype=np.int32)
    else:
        prefix_len = rng.integers(c.prefix[1], c.prefix[2], size=c.B, endpoint=True).astype(np.int32)
    parents = np.stack([
        tree_uniform(c.T, rng) if c.tree[0] == "uniform"
        else tree_bounded(c.T, rng, c.tree[1], c.tree[2])
        for _ in range(c.B)
    ]).astype(np.int32)
    q, kc, vc, kt, vt = _draw_tensors(rng, c.dtype, c.B, c.Hq, c.Hkv, c.D, c.Lcap, c.T,
                                      prefix_len, parents, c.drift, poison_tail)
    return Workload(c.dtype, c.B, c.Hq, c.Hkv, c.D, c.Lcap, c.T, c.scale,
                    q, kc, vc, kt, vt, parents, prefix_len, name=c.name)


def make_custom(*, B: int, Hq: int, Hkv: int, D: int, Lcap: int, T: int,
                prefix_len: Sequence[int], parents: Optional[Sequence[Sequence[int]]] = None,
                dtype: str = "bf16", seed: int = 0, drift: bool = False,
                poison_tail: bool = False, scale: Optional[float] = None,
                tree: tuple = ("uniform",)) -> Workload:
    """Inputs of any shape, for edge cases (explicit trees, ragged or empty prefixes)."""
    rng = np.random.default_rng(seed)
    prefix_len = np.asarray(prefix_len, dtype=np.int32).reshape(B)
    if parents is None:
        parents = np.stack([
            tree_uniform(T, rng) if tree[0] == "uniform" else tree_bounded(T, rng, tree[1], tree[2])
            for _ in range(B)
        ])
    parents = np.asarray(parents, dtype=np.int32).reshape(B, T)
    q, kc, vc, kt, vt = _draw_tensors(rng, dtype, B, Hq, Hkv, D, Lcap, T, prefix_len, parents,
                                      drift, poison_tail)
    return Workload(dtype, B, Hq, Hkv, D, Lcap, T,
                    (1.0 / math.sqrt(D)) if scale is None else float(scale),
                    q, kc, vc, kt, vt, parents, prefix_len)
