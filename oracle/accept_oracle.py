"""fp64 / integer CPU oracle for accepting a verified draft tree and committing it.

TEST INFRASTRUCTURE ONLY, like ``hta_oracle``: the test suite, the smoke
check and the benchmark may use it; the GPU library and its binding never do,
and it shares no code with them.

What it computes. Speculative decoding is lossless: the target model checks
the draft, and only draft tokens the target itself would have produced are
kept (LongSpec summary pages, problem statement; LogitSpec summary pages,
section 1). LogitSpec's draft tree is rooted at x_{i+1}, with its branches for
the guessed next-next tokens, and the target verifies all branches at once
under the tree mask (LogitSpec, "draft tree construction and verification").
The pages do not spell out the acceptance rule; the plainest lossless reading
for greedy decoding, taken here, is:

* the target's prediction at tree node j is the token with the largest logit
  at j (``target[j] = argmax_v logits[j, v]``, the lowest index among equal
  maxima), compared on the exact values of the stored logits;
* the root (node 0, x_{i+1}, produced by the target at the previous step) is
  always accepted; from an accepted node j the walk moves to its child whose
  draft token equals ``target[j]`` -- the lowest-numbered such child when
  several match -- and stops at a node none of whose children match;
* ``accept_len`` counts the accepted nodes (root included), ``path`` lists
  them root first, and the bonus token is ``target[last accepted node]``,
  the target's own next token, which becomes the next step's root.

Committing appends the accepted nodes' keys and values, in path order, to the
sequence's KV cache at position ``prefix_len`` and advances ``prefix_len`` by
``accept_len``; a sequence whose cache cannot hold them is left unchanged and
reported.

Pins: ``tests/test_accept_pins.py`` checks these functions against brute force
(every root path enumerated), closed forms for chain and star trees, a
hand-worked example and invariants.
"""

from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .hta_oracle import check_parent


def target_tokens(logits: np.ndarray) -> np.ndarray:
    """Greedy prediction per tree node: index of the largest logit, lowest index on ties.

    ``logits`` [..., V] holds the exact values (float64 of the stored
    bf16 / float32 numbers). Returns int64 [...].
    """
    return np.argmax(np.asarray(logits, dtype=np.float64), axis=-1)


def accept_path(parent: Sequence[int], tree_tokens: Sequence[int], target: Sequence[int]) -> Tuple[int, list, int]:
    """Greedy walk from the root of one sequence's draft tree.

    Returns (accept_len, path, bonus): the accepted nodes root first, and the
    target's token at the last of them.
    """
    check_parent(parent)
    T = len(parent)
    path = [0]
    cur = 0
    while True:
        nxt = None
        for c in range(T):  # children in index order; the first match is taken
            if int(parent[c]) == cur and int(tree_tokens[c]) == int(target[cur]):
                nxt = c
                break
        if nxt is None:
            break
        path.append(nxt)
        cur = nxt
    return len(path), path, int(target[cur])


def accept(parent: np.ndarray, tree_tokens: np.ndarray, logits: np.ndarray):
    """Batched accept: parent, tree_tokens [B, T], logits [B, T, V].

    Returns dict with target [B, T], accept_len [B], path [B, T] (-1 past the
    accepted length), bonus [B]; a sequence with a bad parent array gets
    accept_len 0, an all -1 path and bonus -1.
    """
    B, T = parent.shape
    target = target_tokens(logits)
    n = np.zeros(B, dtype=np.int64)
    path = np.full((B, T), -1, dtype=np.int64)
    bonus = np.full(B, -1, dtype=np.int64)
    bad = np.zeros(B, dtype=bool)
    for b in range(B):
        try:
            nb, pb, bb = accept_path(parent[b], tree_tokens[b], target[b])
        except ValueError:
            bad[b] = True
            continue
        n[b] = nb
        path[b, :nb] = pb
        bonus[b] = bb
    return dict(target=target, accept_len=n, path=path, bonus=bonus, bad=bad)


def commit(k_cache: np.ndarray, v_cache: np.ndarray, prefix_len: np.ndarray, k_tree: np.ndarray,
           v_tree: np.ndarray, accept_len: np.ndarray, path: np.ndarray):
    """Append the accepted nodes' K/V rows to the caches (copies; inputs untouched).

    k_cache, v_cache [B, Hkv, Lcap, D]; k_tree, v_tree [B, Hkv, T, D]; any
    element dtype (rows are copied as they are). Returns (k_cache', v_cache',
    prefix_len', overflow [B] bool). A sequence with accept_len <= 0 or whose
    cache would overflow keeps its rows and length.
    """
    kc, vc = k_cache.copy(), v_cache.copy()
    L = prefix_len.astype(np.int64).copy()
    Lcap = k_cache.shape[2]
    B = k_cache.shape[0]
    over = np.zeros(B, dtype=bool)
    for b in range(B):
        nb = int(accept_len[b])
        if nb <= 0:
            continue
        if L[b] < 0 or L[b] + nb > Lcap:
            over[b] = True
            continue
        for k in range(nb):
            kc[b, :, L[b] + k, :] = k_tree[b, :, int(path[b, k]), :]
            vc[b, :, L[b] + k, :] = v_tree[b, :, int(path[b, k]), :]
        L[b] += nb
    return kc, vc, L, over
