"""fp64 CPU oracle for the draft model's attention (LongSpec's memory-efficient drafter).

TEST INFRASTRUCTURE ONLY: used by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg; the GPU library and its binding never import it.

What it computes. The LongSpec summary pages (§2.A "memory-efficient
architecture" in the Korean summary; item 1 of the methodology in the Dutch
one) give the drafter two attentions whose memory does not grow with the
context:

* cross-attention straight over the target model's KV cache, which exists
  anyway: every draft query row sees all ``prefix_len[b]`` cached positions of
  its KV head, with no mask (``cross_attn``);
* self-attention over a sliding window of 512 positions: the drafter keeps a
  fixed-size cache of the last ``W`` positions. Reading taken: the window
  includes the query's own position, so a new token at absolute position
  ``t`` sees positions ``max(0, t - W + 1) .. t``. The fixed-size cache is a
  ring, slot = position mod W, holding positions ``max(0, P - W) .. P - 1``
  before a step that adds ``Tn`` new tokens at positions ``P .. P + Tn - 1``;
  the new tokens' keys and values come separately and are causal among
  themselves (``window_attn``), and ``window_append`` then writes them into
  the ring.

Both are plain softmax attention over one visible set per row, written out
with ``attend_rows`` (one pass, natural-log LSE, fp64 on the exact input
values). Pins: ``tests/test_draft_pins.py``.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .hta_oracle import attend_rows


def cross_attn(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, prefix_len: np.ndarray,
               scale: float):
    """q [B, Hq, Tq, D], caches [B, Hkv, Lcap, D] (float64 values), prefix_len [B].

    Returns (out [B, Hq, Tq, D], lse [B, Hq, Tq]); a sequence with an empty
    prefix gets out = 0, lse = -inf.
    """
    B, Hq, Tq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Tq, D))
    lse = np.zeros((B, Hq, Tq))
    for b in range(B):
        L = int(prefix_len[b])
        for h in range(Hq):
            g = h // G
            K, V = k_cache[b, g, :L], v_cache[b, g, :L]
            o, l = attend_rows(q[b, h], K, V, np.ones((Tq, L), dtype=bool), scale)
            out[b, h], lse[b, h] = o, l
    return out, lse


def window_visible(P: int, W: int, Tn: int) -> np.ndarray:
    """Boolean [Tn, W + Tn]: which ring slots and which new tokens new token j sees (Tn <= W)."""
    if Tn > W:
        raise ValueError("more new tokens than the window holds")
    vis = np.zeros((Tn, W + Tn), dtype=bool)
    for j in range(Tn):
        t = P + j  # absolute position of new token j
        for x in range(max(0, t - W + 1), P):  # window positions already in the ring
            vis[j, x % W] = True
        vis[j, W:W + j + 1] = True  # new tokens 0 .. j (itself included)
    return vis


def window_attn(q: np.ndarray, k_ring: np.ndarray, v_ring: np.ndarray, k_new: np.ndarray,
                v_new: np.ndarray, pos: np.ndarray, scale: float, W: Optional[int] = None):
    """Sliding-window self-attention of Tn new tokens.

    q [B, Hq, Tn, D]; k_ring/v_ring [B, Hkv, W, D]; k_new/v_new [B, Hkv, Tn, D];
    pos [B] = positions written before this step. float64 values. Returns
    (out [B, Hq, Tn, D], lse [B, Hq, Tn]).
    """
    B, Hq, Tn, D = q.shape
    Hkv = k_ring.shape[1]
    W = k_ring.shape[2] if W is None else W
    G = Hq // Hkv
    out = np.zeros((B, Hq, Tn, D))
    lse = np.zeros((B, Hq, Tn))
    for b in range(B):
        vis = window_visible(int(pos[b]), W, Tn)
        for h in range(Hq):
            g = h // G
            K = np.concatenate([k_ring[b, g], k_new[b, g]])
            V = np.concatenate([v_ring[b, g], v_new[b, g]])
            # slots the row does not see may hold anything (even NaN): give them
            # zero values so that a zero weight stays zero
            K = np.where(vis.any(axis=0)[:, None], K, 0.0)
            V = np.where(vis.any(axis=0)[:, None], V, 0.0)
            o, l = attend_rows(q[b, h], K, V, vis, scale)
            out[b, h], lse[b, h] = o, l
    return out, lse


def window_append(k_ring: np.ndarray, v_ring: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                  pos: np.ndarray):
    """Write the Tn new tokens into the ring (slot = position mod W); returns copies
    of the rings and pos + Tn. Tn <= W."""
    kr, vr = k_ring.copy(), v_ring.copy()
    W = kr.shape[2]
    Tn = k_new.shape[2]
    assert Tn <= W
    for b in range(kr.shape[0]):
        for j in range(Tn):
            s = (int(pos[b]) + j) % W
            kr[b, :, s] = k_new[b, :, j]
            vr[b, :, s] = v_new[b, :, j]
    return kr, vr, np.asarray(pos, dtype=np.int64) + Tn
