"""fp64 CPU oracle for tree-verification attention (Hybrid Tree Attention).

TEST INFRASTRUCTURE ONLY. This module exists to check the GPU library. Only
the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it; the library and its Python binding never do, and it shares no
code with them.

What it computes. LongSpec ("fast tree attention" on its summary pages)
splits the target model's attention over a draft tree into a cached part
(the KV prefix, which every tree token sees without a mask) and a
speculative part (the tree tokens, under a tree mask), and combines the two
with the log-sum-exp trick without changing the result. LogitSpec's draft
tree section says what the tree mask does: a tree token sees only the
tokens on its own root path, so every branch is verified in one pass. The
combined result is therefore ordinary softmax attention of each tree
token over one visible set; that plain definition is what this oracle
writes out, with no split, no online softmax and no bitmask:

* visible set of tree node i of sequence b: every prefix position
  ``0 <= p < prefix_len[b]``, node i itself, and every node reached from i
  by following ``parent`` until -1;
* score ``s = scale * <q, k>`` in float64 over that set, for query head h
  and the key/value head ``h // (Hq // Hkv)``;
* one pass over the concatenated [prefix || tree] row:
  ``lse = max(s) + ln(sum(exp(s - max(s))))`` (natural log, scaled scores),
  ``out = sum(exp(s - lse) * v)``.

Readings of points the pages leave open (listed with the rest in the
design notes): the LSE is the natural log of the summed exponentials of the
scaled scores; a node sees itself; query head h uses KV head ``h // G``;
an extra -1 in ``parent`` starts another root (a forest); rows with an empty
visible set (only possible when the tree part is excluded and the prefix is
empty) have ``lse = -inf`` and ``out = 0``.

Pins: every function here is checked against something other than itself in
``tests/test_oracle_pins.py`` (brute force, closed forms, library attention,
and invariants).
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np


class BadTree(ValueError):
    """parent[] breaks -1 <= parent[i] < i."""


def check_parent(parent: Sequence[int]) -> None:
    for i, p in enumerate(parent):
        if not (-1 <= int(p) < i):
            raise BadTree(f"parent[{i}] = {int(p)} is not in [-1, {i - 1}]")


def tree_visible_nodes(parent: Sequence[int]) -> list:
    """For each node i: i and its ancestors, found by walking parent pointers up to -1."""
    check_parent(parent)
    out = []
    for i in range(len(parent)):
        chain = []
        j = i
        while j != -1:
            chain.append(j)
            j = int(parent[j])
        out.append(sorted(chain))
    return out


def tree_mask_bits(parent: Sequence[int]) -> np.ndarray:
    """uint64 word per node: bit j set iff tree node j is visible to node i (T <= 64)."""
    T = len(parent)
    if T > 64:
        raise ValueError("one 64-bit word per node holds at most 64 nodes")
    words = np.zeros(T, dtype=np.uint64)
    for i, vis in enumerate(tree_visible_nodes(parent)):
        w = 0
        for j in vis:
            w |= 1 << j
        words[i] = np.uint64(w)
    return words


def attend_rows(q_rows: np.ndarray, keys: np.ndarray, vals: np.ndarray,
                visible: np.ndarray, scale: float):
    """Softmax attention of R query rows over N keys with a boolean visibility matrix.

    q_rows [R, D], keys/vals [N, D], visible [R, N]; all float64. Returns
    (out [R, D], lse [R]) with the natural-log LSE of the scaled scores.
    """
    R = q_rows.shape[0]
    D = vals.shape[1]
    if keys.shape[0] == 0:
        return np.zeros((R, D)), np.full(R, -np.inf)
    s = scale * (q_rows @ keys.T)
    s = np.where(visible, s, -np.inf)
    mu = s.max(axis=1)
    empty = ~np.isfinite(mu)
    mu_safe = np.where(empty, 0.0, mu)
    e = np.exp(s - mu_safe[:, None])
    tot = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, mu_safe + np.log(tot))
    w = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, tot)[:, None])
    return w @ vals, lse


def verify_attn(w, parts: Iterable[str] = ("prefix", "tree"), scale: Optional[float] = None,
                heads: Optional[Sequence[int]] = None, batches: Optional[Sequence[int]] = None,
                prefix_range: Optional[tuple] = None):
    """Attention of every tree token over its visible set.

    ``w`` is a ``workloads.Workload`` (or anything with the same fields).
    ``parts`` chooses which keys exist: "prefix" (the cached KV, no mask),
    "tree" (tree tokens under the ancestor mask) or both. ``prefix_range``
    ``(lo, hi)`` restricts the prefix to positions ``lo <= p < min(hi, L_b)``
    (used to check that splitting the prefix and merging gives the same
    answer). ``heads``/``batches`` restrict which outputs are computed
    (others are left NaN), so large shapes can be sampled.

    Returns ``(out [B, Hq, T, D], lse [B, Hq, T])`` in float64.
    """
    parts = tuple(parts)
    sc = w.scale if scale is None else scale
    B, Hq, Hkv, T, D = w.B, w.Hq, w.Hkv, w.T, w.D
    G = Hq // Hkv
    out = np.full((B, Hq, T, D), np.nan)
    lse = np.full((B, Hq, T), np.nan)
    q = w.as_f64("q")
    kt = w.as_f64("k_tree")
    vt = w.as_f64("v_tree")
    want_heads = set(range(Hq) if heads is None else heads)
    for b in (range(B) if batches is None else batches):
        L = int(w.prefix_len[b])
        lo, hi = (0, L) if prefix_range is None else (max(0, prefix_range[0]), min(L, prefix_range[1]))
        hi = max(lo, hi)
        vis_tree = np.zeros((T, T), dtype=bool)
        for i, nodes in enumerate(tree_visible_nodes(w.parent[b])):
            vis_tree[i, nodes] = True
        for g in range(Hkv):
            group = [h for h in range(g * G, (g + 1) * G) if h in want_heads]
            if not group:
                continue
            keys, vals, vis = [], [], []
            if "prefix" in parts:
                keys.append(_exact_f64(w, w.k_cache[b, g, lo:hi]))
                vals.append(_exact_f64(w, w.v_cache[b, g, lo:hi]))
                vis.append(np.ones((T, hi - lo), dtype=bool))
            if "tree" in parts:
                keys.append(kt[b, g])
                vals.append(vt[b, g])
                vis.append(vis_tree)
            K = np.concatenate(keys, axis=0) if keys else np.zeros((0, D))
            V = np.concatenate(vals, axis=0) if vals else np.zeros((0, D))
            M = np.concatenate(vis, axis=1) if vis else np.zeros((T, 0), dtype=bool)
            for h in group:
                o, l = attend_rows(q[b, h], K, V, M, sc)
                out[b, h] = o
                lse[b, h] = l
    return out, lse


def lse_merge(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]):
    """Combine normalised partial attentions over disjoint key sets.

    With ``lse = ln(sum_k exp(lse_k))`` the merged output is
    ``sum_k exp(lse_k - lse) * out_k``; parts with ``lse_k = -inf`` add nothing.
    Rows where every part is empty keep ``lse = -inf``, ``out = 0``.
    """
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lses])
    O = np.stack([np.asarray(x, dtype=np.float64) for x in outs])
    mx = L.max(axis=0)
    empty = ~np.isfinite(mx)
    mxs = np.where(empty, 0.0, mx)
    wts = np.exp(L - mxs[None])
    tot = wts.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, mxs + np.log(np.where(empty, 1.0, tot)))
    coef = np.where(empty[None], 0.0, wts / np.where(empty, 1.0, tot)[None])
    # an empty part (lse = -inf) adds nothing, whatever its o holds
    O = np.where(np.isneginf(L)[..., None], 0.0, O)
    out = (coef[..., None] * O).sum(axis=0)
    return out, lse


def _exact_f64(w, a: np.ndarray) -> np.ndarray:
    """Exact float64 values of a slice of one of the workload's float tensors."""
    if w.dtype == "bf16":
        return (np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)) \
            .view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
