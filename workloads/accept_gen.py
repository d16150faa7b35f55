"""Seeded synthetic inputs for accepting a verified draft tree.

Recipe (one ``numpy.random.default_rng(seed)``), drawn in this order:

1. parent arrays ``parent[B, T]`` (same tree shapes as ``gen``);
2. draft tokens ``tree_tokens[B, T]`` int32: the root gets a uniform token in
   ``[0, V)``; the children of each node get distinct tokens drawn without
   replacement from ``[0, V)`` (with ``dup_siblings`` set, each child after the
   first copies an earlier sibling's token with probability 0.3);
3. target logits ``logits[B, T, V]``, float32 N(0, 1);
4. a planted path per sequence: from the root, for ``depth[b]`` steps (or
   until a leaf), pick a uniform child c of the current node j and set
   ``logits[b, j, tree_tokens[b, c]] = 8`` (above any N(0, 1) draw at these
   vocabulary sizes), then move to c. ``depth[b]`` is uniform in
   ``[0, max_depth]`` unless given.

bf16 cases round the logits to bfloat16 (nearest, ties to even) and keep the
16-bit patterns. Token content of real models is not needed: the step's cost
depends on B, T and V only, and the planted path fixes how much it accepts.
This module draws numbers and tree shapes only; it holds none of the accept
arithmetic.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

from .gen import bf16_bits_to_f32, f32_to_bf16_bits, tree_bounded, tree_chain, tree_star, tree_uniform


@dataclasses.dataclass
class AcceptCase:
    dtype: str                 # logits dtype: "f32" or "bf16"
    B: int
    T: int
    V: int
    parent: np.ndarray         # int32 [B, T]
    tree_tokens: np.ndarray    # int32 [B, T]
    logits: np.ndarray         # float32 or uint16 bf16 bits [B, T, V]
    depth: np.ndarray          # int32 [B]: planted steps

    def logits_f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.logits).astype(np.float64)
        return self.logits.astype(np.float64)


def _tree(kind, T, rng):
    if kind[0] == "uniform":
        return tree_uniform(T, rng)
    if kind[0] == "bounded":
        return tree_bounded(T, rng, kind[1], kind[2] if len(kind) > 2 else None)
    if kind[0] == "chain":
        return tree_chain(T)
    if kind[0] == "star":
        return tree_star(T)
    raise ValueError(kind)


def make_accept_case(*, B: int, T: int, V: int, dtype: str = "bf16", seed: int = 0,
                     tree: tuple = ("bounded", 6, None), max_depth: int = 6,
                     depth: Optional[Sequence[int]] = None, dup_siblings: bool = False,
                     parents: Optional[Sequence[Sequence[int]]] = None) -> AcceptCase:
    rng = np.random.default_rng(seed)
    if parents is not None:
        parent = np.asarray(parents, dtype=np.int32).reshape(B, T)
    else:
        parent = np.stack([_tree(tree, T, rng) for _ in range(B)]).astype(np.int32)
    tokens = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        tokens[b, 0] = rng.integers(V)
        for j in range(T):
            kids = [c for c in range(T) if parent[b, c] == j]
            if not kids:
                continue
            draw = rng.choice(V, size=len(kids), replace=False)
            for n, c in enumerate(kids):
                tokens[b, c] = draw[n]
                if dup_siblings and n > 0 and rng.random() < 0.3:
                    tokens[b, c] = tokens[b, kids[rng.integers(n)]]
    logits = rng.standard_normal((B, T, V), dtype=np.float32)
    d = np.asarray(depth, dtype=np.int32) if depth is not None else rng.integers(0, max_depth + 1, size=B).astype(np.int32)
    for b in range(B):
        j = 0
        for _ in range(int(d[b])):
            kids = [c for c in range(T) if parent[b, c] == j]
            if not kids or parent[b, 0] != -1:
                break
            c = kids[rng.integers(len(kids))]
            logits[b, j, tokens[b, c]] = 8.0
            j = c
    if dtype == "bf16":
        logits = f32_to_bf16_bits(logits)
    return AcceptCase(dtype=dtype, B=B, T=T, V=V, parent=parent, tree_tokens=tokens, logits=logits, depth=d)
