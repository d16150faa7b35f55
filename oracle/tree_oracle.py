"""CPU oracle for building the draft tree from the last logits (LogitSpec).

TEST INFRASTRUCTURE ONLY: used by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg; the GPU library and its binding never import it.

What it computes (LogitSpec summary pages, §2 "LogitSpec workflow"): the
target's last logits give the next token x_{i+1} (the greedy choice) and,
with x_{i+1} excluded, the top-k entries are taken as guesses for the
next-next token. Two kinds of n-gram query then look up the sequence's own
history: query 1 is the m tokens ending with x_{i+1}; query 2, one per guess,
is the m tokens ending with x_{i+1} followed by that guess (so its last m-1
history-side tokens end with x_{i+1}). The retrieved tokens form a draft tree
rooted at x_{i+1} whose branches correspond to the guesses, and a rank-based
rule keeps more retrieved tokens for higher-ranked (more confident) guesses.

Readings taken where the pages leave the step open (listed with the rest in
the design notes):

* the reference text searched is the sequence's own tokens (its history
  followed by x_{i+1}); a match is the most recent earlier occurrence of the
  query n-gram, and the retrieved tokens are the ones that follow it;
* the top-k order is by logit value, lower vocabulary index first among
  equal values, and x_{i+1} is the first entry of that order (so "excluding
  x_{i+1}" means entries 2 .. k+1);
* tree layout, in node order: node 0 = x_{i+1} (parent -1); then the tokens
  retrieved for query 1 as a chain under node 0 (at most keep_first); then
  for each guess by rank r: a child of node 0 holding the guess, and the
  tokens retrieved for its query 2 as a chain under it (at most keep[r]); a
  guess without a match is still a node. Nodes past the tree size are
  dropped in that order; unused slots hold token -1 under the root;
* the kept lengths keep_first and keep[r] (non-increasing in r: the pages
  give the shape of the rule, not its constants), k and m are parameters.

Pins: ``tests/test_tree_pins.py``.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np


def ranked_tokens(logits: np.ndarray, n: int) -> list:
    """Vocabulary indices of the n largest logits, by value then lower index."""
    v = np.asarray(logits, dtype=np.float64)
    order = np.lexsort((np.arange(v.shape[0]), -v))  # primary key: -value; ties: index
    return [int(t) for t in order[:n]]


def most_recent_match(seq: Sequence[int], gram: Sequence[int], before: int) -> int:
    """Largest end position p < before with seq[p-len(gram)+1 .. p] == gram, or -1."""
    m = len(gram)
    for p in range(min(before, len(seq)) - 1, m - 2, -1):
        if all(seq[p - m + 1 + t] == gram[t] for t in range(m)):
            return p
    return -1


def build_tree(history: Sequence[int], logits: np.ndarray, k: int, m: int, keep_first: int,
               keep: Sequence[int], T: int):
    """One sequence: returns (tokens [T], parent [T], n_nodes)."""
    hist = [int(t) for t in history]
    top = ranked_tokens(logits, k + 1)
    x1 = top[0]
    guesses = top[1:k + 1]
    seq = hist + [x1]
    n = len(seq)
    tokens, parent = [x1], [-1]

    def add(tok, par):
        if len(tokens) < T:
            tokens.append(int(tok))
            parent.append(par)
            return len(tokens) - 1
        return None

    # query 1: the m tokens ending with x1; an earlier occurrence must end before x1
    if m <= n:
        p = most_recent_match(seq, seq[n - m:], n - 1)
        if p >= 0:
            par = 0
            for t in seq[p + 1:p + 1 + keep_first]:
                par = add(t, par)
                if par is None:
                    break
    # query 2 per guess: the m-1 tokens ending with x1, then the guess
    for r, gtok in enumerate(guesses):
        node = add(gtok, 0)
        if node is None:
            break
        if m - 1 > n:
            continue
        gram = seq[n - (m - 1):] + [gtok] if m > 1 else [gtok]
        p = most_recent_match(seq, gram, n)
        if p < 0:
            continue
        par = node
        for t in seq[p + 1:p + 1 + int(keep[r])]:
            par = add(t, par)
            if par is None:
                break
    used = len(tokens)
    while len(tokens) < T:
        tokens.append(-1)
        parent.append(0)
    return np.array(tokens, dtype=np.int64), np.array(parent, dtype=np.int64), used


def build_trees(history: np.ndarray, history_len: np.ndarray, logits: np.ndarray, k: int, m: int,
                keep_first: int, keep: Sequence[int], T: int):
    """Batched: history [B, cap] int, history_len [B], logits [B, V]."""
    B = history.shape[0]
    tok = np.zeros((B, T), dtype=np.int64)
    par = np.zeros((B, T), dtype=np.int64)
    n = np.zeros(B, dtype=np.int64)
    for b in range(B):
        tok[b], par[b], n[b] = build_tree(history[b, :int(history_len[b])], logits[b], k, m, keep_first, keep, T)
    return tok, par, n
