"""Pins of the tree-construction oracle (CPU only).

The ranking is checked against a plain repeated-maximum loop, the n-gram
search against a forward scan that keeps the last hit, the whole construction
against a hand-worked example (tests/golden/tree_hand_example.json) and
against structural invariants; two planted mistakes must fail the example.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import tree_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_hand_example.json")
GOLDEN_M2 = os.path.join(os.path.dirname(__file__), "golden", "tree_hand_example_m2.json")


def _loop_ranking(v, n):
    left = list(range(len(v)))
    out = []
    for _ in range(n):
        best = left[0]
        for i in left[1:]:
            if v[i] > v[best]:  # strict: an equal later value does not win
                best = i
        out.append(best)
        left.remove(best)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_ranking_matches_repeated_maximum(seed):
    rng = np.random.default_rng(seed)
    v = np.round(rng.standard_normal(50) * 2) / 2  # many ties
    assert oracle.ranked_tokens(v, 12) == _loop_ranking(list(v), 12)


def _forward_last_match(seq, gram, before):
    m, last = len(gram), -1
    for p in range(m - 1, min(before, len(seq))):
        if list(seq[p - m + 1:p + 1]) == list(gram):
            last = p
    return last


@pytest.mark.parametrize("seed", range(6))
def test_most_recent_match_matches_forward_scan(seed):
    rng = np.random.default_rng(100 + seed)
    seq = list(rng.integers(0, 4, size=80))
    for m in (1, 2, 3, 4):
        for _ in range(20):
            gram = list(rng.integers(0, 4, size=m))
            before = int(rng.integers(0, 81))
            assert oracle.most_recent_match(seq, gram, before) == _forward_last_match(seq, gram, before)


def _golden_inputs(g):
    if "logits" in g:
        return g["history"], np.array(g["logits"], dtype=np.float64)
    logits = np.zeros(g["vocab"])
    for t, val in g["logits_nonzero"].items():
        logits[int(t)] = val
    return g["history"], logits


@pytest.mark.parametrize("path", [GOLDEN, GOLDEN_M2])
def test_hand_example(path):
    g = json.load(open(path))
    hist, logits = _golden_inputs(g)
    tok, par, n = oracle.build_tree(hist, logits, g["k"], g["m"], g["keep_first"], g["keep"], g["T"])
    assert list(tok) == g["tokens"] and list(par) == g["parent"] and n == g["n_nodes"]


def test_planted_mistakes_fail_the_hand_example(monkeypatch):
    g = json.load(open(GOLDEN))
    hist, logits = _golden_inputs(g)
    args = (hist, logits, g["k"], g["m"], g["keep_first"], g["keep"], g["T"])
    good = oracle.build_tree(*args)
    real = tree_oracle.most_recent_match
    # (1) query 1 allowed to match itself (its own end, the last position)
    monkeypatch.setattr(tree_oracle, "most_recent_match", lambda s, gr, before: real(s, gr, len(s)))
    bad = tree_oracle.build_tree(*args)
    assert list(bad[0]) != list(good[0])
    # (2) retrieved tokens start at the match's last token instead of after it
    monkeypatch.setattr(tree_oracle, "most_recent_match", lambda s, gr, before: max(-1, real(s, gr, before) - 1)
                        if real(s, gr, before) >= 0 else -1)
    bad = tree_oracle.build_tree(*args)
    assert list(bad[0]) != list(good[0])


@pytest.mark.parametrize("seed", range(8))
def test_structure_and_truncation(seed):
    rng = np.random.default_rng(200 + seed)
    hist = list(rng.integers(0, 6, size=int(rng.integers(1, 120))))
    logits = rng.standard_normal(6 + 20)
    k, m = int(rng.integers(1, 8)), int(rng.integers(1, 5))
    keep = sorted(rng.integers(0, 6, size=k).tolist(), reverse=True)
    kf = int(rng.integers(0, 6))
    tok, par, n = oracle.build_tree(hist, logits, k, m, kf, keep, 64)
    seq = hist + [int(tok[0])]
    assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, 64))
    assert n <= 1 + kf + k + sum(keep)
    assert all(tok[i] == -1 and par[i] == 0 for i in range(n, 64))
    # the guesses are the children of the root that are not on query 1's chain
    ranked = oracle.ranked_tokens(logits, k + 1)
    assert tok[0] == ranked[0]
    root_kids = [i for i in range(1, n) if par[i] == 0]
    chain1 = 1 if (n > 1 and par[1] == 0 and (len(root_kids) > k)) else 0
    assert [int(tok[i]) for i in root_kids[chain1:]] == ranked[1:1 + len(root_kids) - chain1]
    # every retrieved chain is a run of consecutive tokens of the sequence
    for i in range(1, n):
        kids = [c for c in range(n) if par[c] == i]
        assert len(kids) <= 1
    # a smaller tree is a prefix of the larger one
    for T in (1, 2, 5, 17):
        t2, p2, n2 = oracle.build_tree(hist, logits, k, m, kf, keep, T)
        assert list(t2[:min(T, n)]) == list(tok[:min(T, n)]) and n2 == min(T, n)
        assert list(p2[:n2]) == list(par[:n2])


def test_signed_zeros_rank_equal():
    # -0 and +0 tie, so they rank by index like any other tie
    v = np.array([-1.0, -0.0, 0.0, -0.0, -3.0])
    assert oracle.ranked_tokens(v, 4) == [1, 2, 3, 0]


def test_planted_mistakes_fail_the_bigram_example(monkeypatch):
    g = json.load(open(GOLDEN_M2))
    hist, logits = _golden_inputs(g)
    args = (hist, logits, g["k"], g["m"], g["keep_first"], g["keep"], g["T"])
    good = tree_oracle.build_tree(*args)
    # (1) ties ranked by higher index first
    monkeypatch.setattr(tree_oracle, "ranked_tokens",
                        lambda v, n: [int(t) for t in np.lexsort((-np.arange(len(v)), -np.asarray(v)))[:n]])
    assert list(tree_oracle.build_tree(*args)[0]) != list(good[0])
    monkeypatch.undo()
    # (2) query 1 searched up to the last position (x_{i+1}'s own n-gram counts as a match)
    real = tree_oracle.most_recent_match
    monkeypatch.setattr(tree_oracle, "most_recent_match",
                        lambda s, gr, before: real(s, gr, len(s)) if gr == s[len(s) - len(gr):] else real(s, gr, before))
    assert list(tree_oracle.build_tree(*args)[0]) != list(good[0])


@pytest.mark.parametrize("seed", range(6))
def test_latest_gram_index_answers_the_scan_queries(seed):
    """The reading behind hta_build_tree_indexed: a map from each distinct m-gram
    of the history alone to the latest position where it ends, filled as the
    history grows, gives exactly the oracle's most recent earlier match for
    query 1 (the m tokens ending with x1, searched before x1) and for every
    query 2 (m-1 tokens ending with x1, then a guess other than x1) over the
    sequence history + [x1]."""
    rng = np.random.default_rng(500 + seed)
    alphabet = int(rng.integers(1, 6))
    L = int(rng.integers(0, 300))
    hist = [int(t) for t in rng.integers(0, alphabet, size=L)]
    for m in range(1, 9):
        index = {}
        covered = 0
        for cut in sorted(set([int(c) for c in rng.integers(0, L + 1, size=3)] + [L])):
            for e in range(max(covered, m - 1), cut):  # grams ending at the new positions
                index[tuple(hist[e - m + 1:e + 1])] = e
            covered = cut
            h = hist[:cut]
            for x1 in range(alphabet + 1):
                seq = h + [x1]
                n = len(seq)
                if m <= n:
                    want = tree_oracle.most_recent_match(seq, seq[n - m:], n - 1)
                    got = index.get(tuple(seq[n - m:]), -1)
                    assert got == want, (m, cut, x1)
                for g in range(alphabet + 1):
                    if g == x1 or m - 1 > n:
                        continue
                    gram = (seq[n - (m - 1):] if m > 1 else []) + [g]
                    want = tree_oracle.most_recent_match(seq, gram, n)
                    assert index.get(tuple(gram), -1) == want, (m, cut, x1, g)
