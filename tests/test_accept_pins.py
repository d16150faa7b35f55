"""Pins of the accept / commit oracle (CPU only).

Each check compares the oracle with something other than itself: a
brute-force search over every root path (walking up from each node, where the
oracle walks down from the root), a plain loop for the argmax, closed forms on
chain and star trees, a hand-worked example, and invariants of the commit.
"""

import numpy as np
import pytest

import oracle
from workloads import tree_bounded, tree_chain, tree_star, tree_uniform


# ----------------------------------------------------------------------------
# target prediction: largest logit, lowest index among equal maxima
# ----------------------------------------------------------------------------

def _argmax_loop(row):
    best, idx = -np.inf, -1
    for v, x in enumerate(row):
        if x > best:  # strict: an equal later value does not replace the first
            best, idx = x, v
    return idx


@pytest.mark.parametrize("seed", range(5))
def test_target_tokens_is_first_maximum(seed):
    rng = np.random.default_rng(seed)
    # coarse values so that maxima repeat
    logits = np.round(rng.standard_normal((3, 5, 40)) * 2) / 2
    got = oracle.target_tokens(logits)
    for b in range(3):
        for i in range(5):
            assert got[b, i] == _argmax_loop(logits[b, i])


def test_target_tokens_ties_take_lowest_index():
    row = np.array([0.0, 3.0, -1.0, 3.0, 3.0])
    assert oracle.target_tokens(row[None])[0] == 1


# ----------------------------------------------------------------------------
# accepted path: brute force over every root path
# ----------------------------------------------------------------------------

def _random_case(rng, T, kind, vocab=None, p_match=0.6):
    vocab = vocab or max(12, T + 1)
    parent = {"uniform": tree_uniform, "chain": lambda T, r: tree_chain(T),
              "star": lambda T, r: tree_star(T)}.get(kind, None)
    par = parent(T, rng) if parent else tree_bounded(T, rng, 4, 3)
    tokens = np.zeros(T, dtype=np.int64)
    kids = {j: [c for c in range(T) if par[c] == j] for j in range(T)}
    for j, cs in kids.items():  # distinct tokens among siblings
        perm = rng.permutation(vocab)
        for n, c in enumerate(cs):
            tokens[c] = perm[n]
    tokens[0] = rng.integers(vocab)
    target = np.zeros(T, dtype=np.int64)
    for j in range(T):
        cs = kids[j]
        if cs and rng.random() < p_match:
            target[j] = tokens[cs[rng.integers(len(cs))]]
        else:
            used = {int(tokens[c]) for c in cs}
            target[j] = next(v for v in range(vocab + T) if v not in used)
    return par, tokens, target


def _brute_force(par, tokens, target):
    """Longest root path whose every edge p -> c has tokens[c] == target[p]."""
    best = [0]
    for i in range(len(par)):
        chain = []
        j = i
        while j != -1:
            chain.append(j)
            j = int(par[j])
        chain.reverse()
        if chain[0] != 0:
            continue  # another root of a forest: not reachable from node 0
        if all(tokens[c] == target[p] for p, c in zip(chain, chain[1:])) and len(chain) > len(best):
            best = chain
    return best


@pytest.mark.parametrize("kind", ["uniform", "bounded", "chain", "star"])
@pytest.mark.parametrize("T", [1, 2, 7, 33, 64])
def test_accept_path_is_longest_matching_root_path(kind, T):
    rng = np.random.default_rng(T * 31 + len(kind))
    for _ in range(30):
        par, tokens, target = _random_case(rng, T, kind)
        n, path, bonus = oracle.accept_path(par, tokens, target)
        want = _brute_force(par, tokens, target)
        assert path == want and n == len(want)
        assert bonus == target[want[-1]]


def test_chain_all_matching_accepts_everything():
    T = 9
    par = tree_chain(T)
    tokens = np.arange(100, 100 + T)
    target = np.append(tokens[1:], 7)  # target at node i is the token of node i+1
    n, path, bonus = oracle.accept_path(par, tokens, target)
    assert n == T and path == list(range(T)) and bonus == 7


def test_no_matching_child_accepts_the_root_only():
    par = tree_star(6)
    tokens = np.array([3, 10, 11, 12, 13, 14])
    target = np.array([99, 0, 0, 0, 0, 0])
    assert oracle.accept_path(par, tokens, target) == (1, [0], 99)


def test_star_takes_the_matching_leaf():
    par = tree_star(6)
    tokens = np.array([3, 10, 11, 12, 13, 14])
    target = np.array([13, 5, 6, 7, 8, 9])
    assert oracle.accept_path(par, tokens, target) == (2, [0, 4], 8)


def test_hand_example_duplicate_siblings_take_lowest_index():
    # Nodes:      0    1    2    3    4    5    6
    # parent:    -1    0    0    1    2    2    5
    # token:      1    5    5    7    8    6    9
    # target:     5    7    6    4    0    9    2
    # Root: target 5; children 1 and 2 both carry 5 -> the lower-numbered, 1.
    # Node 1: target 7; child 3 carries 7 -> accept 3.
    # Node 3: target 4; no children -> stop. (Through node 2 the walk would
    # have gone 2 -> 5 -> 6, deeper, but the first matching child is taken.)
    par = [-1, 0, 0, 1, 2, 2, 5]
    tokens = [1, 5, 5, 7, 8, 6, 9]
    target = [5, 7, 6, 4, 0, 9, 2]
    assert oracle.accept_path(par, tokens, target) == (3, [0, 1, 3], 4)


def test_forest_roots_after_the_first_are_never_accepted():
    par = [-1, 0, -1, 2]
    tokens = [0, 1, 2, 3]
    target = [2, 0, 3, 0]  # root's target is node 2's token, but node 2 is a separate root
    assert oracle.accept_path(par, tokens, target) == (1, [0], 2)


def test_batched_accept_marks_bad_trees():
    parent = np.array([[-1, 0, 1], [-1, 2, 0]])
    tokens = np.array([[1, 2, 3], [1, 2, 3]])
    logits = np.zeros((2, 3, 5))
    logits[0, 0, 2] = 1.0  # target(0) = 2 -> node 1
    logits[0, 1, 3] = 1.0  # target(1) = 3 -> node 2
    out = oracle.accept(parent, tokens, logits)
    assert list(out["accept_len"]) == [3, 0]
    assert list(out["path"][0]) == [0, 1, 2] and list(out["path"][1]) == [-1, -1, -1]
    assert out["bonus"][0] == 0 and out["bonus"][1] == -1
    assert list(out["bad"]) == [False, True]


# ----------------------------------------------------------------------------
# commit
# ----------------------------------------------------------------------------

def test_commit_appends_path_rows_and_advances_length():
    rng = np.random.default_rng(5)
    B, Hkv, Lcap, T, D = 3, 2, 20, 6, 4
    kc = rng.standard_normal((B, Hkv, Lcap, D))
    vc = rng.standard_normal((B, Hkv, Lcap, D))
    kt = rng.standard_normal((B, Hkv, T, D))
    vt = rng.standard_normal((B, Hkv, T, D))
    L = np.array([5, 17, 0])
    n = np.array([3, 4, 1])  # sequence 1 overflows: 17 + 4 > 20
    path = np.array([[0, 2, 5, -1, -1, -1], [0, 1, 2, 3, -1, -1], [0, -1, -1, -1, -1, -1]])
    kc2, vc2, L2, over = oracle.commit(kc, vc, L, kt, vt, n, path)
    assert list(L2) == [8, 17, 1] and list(over) == [False, True, False]
    for k, node in enumerate([0, 2, 5]):
        assert np.array_equal(kc2[0, :, 5 + k], kt[0, :, node]) and np.array_equal(vc2[0, :, 5 + k], vt[0, :, node])
    assert np.array_equal(kc2[2, :, 0], kt[2, :, 0])
    # every other row is untouched
    touched = np.zeros((B, Lcap), dtype=bool)
    touched[0, 5:8] = True
    touched[2, 0] = True
    rows = lambda a: a.transpose(0, 2, 1, 3)  # [B, Lcap, Hkv, D]
    assert np.array_equal(rows(kc2)[~touched], rows(kc)[~touched])
    assert np.array_equal(rows(vc2)[~touched], rows(vc)[~touched])
    assert L[1] == 17  # inputs untouched


def test_signed_zeros_rank_equal():
    # -0 and +0 are equal values: the lower index wins whichever sign it has
    assert oracle.target_tokens(np.array([[-1.0, -0.0, 0.0, -2.0]]))[0] == 1
    assert oracle.target_tokens(np.array([[-1.0, 0.0, -0.0, -2.0]]))[0] == 1
