"""Pins for the fp64 oracle: each check compares it with something other than itself.

* brute force: pure-Python loops with math.exp, visible sets built top-down
  (a child's set is its parent's set plus itself) rather than by walking up;
* the tree mask, exhaustively over every parent array of up to 6 nodes
  (forests included), against reachability from powers of the adjacency matrix;
* closed forms: all-zero keys give uniform weights, so lse = ln(#visible)
  and out = mean of the visible values; one tree node with no prefix gives
  out = v and lse = scale * q.k; a hand-derived example in tests/golden;
* a library routine: torch's scaled_dot_product_attention in float64;
* invariants: a chain tree is causal attention; splitting the prefix and
  merging with log-sum-exp equals the unsplit result; a star tree; grouped
  query heads equal multi-head attention with repeated KV heads; permuting
  prefix positions changes nothing.

The mutation tests at the end plant plausible mistakes in the oracle (on the
CPU) and check that at least one pin catches each of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.hta_oracle as O
from workloads import make_custom, tree_chain, tree_star

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# independent helpers
# ----------------------------------------------------------------------------

def visible_top_down(parent):
    """Visible tree nodes per node, built from the roots down (parents precede children)."""
    sets = []
    for i, p in enumerate(parent):
        s = {i} if p < 0 else set(sets[p]) | {i}
        sets.append(s)
    return sets


def visible_by_closure(parent):
    """Visible tree nodes per node from reachability: (I + A)^T, A[i, j] = [parent[i] == j]."""
    T = len(parent)
    A = np.zeros((T, T), dtype=np.int64)
    for i, p in enumerate(parent):
        if p >= 0:
            A[i, p] = 1
    R = np.eye(T, dtype=np.int64)
    step = np.eye(T, dtype=np.int64)
    for _ in range(T):
        step = np.minimum(step @ A, 1)
        R = np.minimum(R + step, 1)
    return [set(np.nonzero(R[i])[0].tolist()) for i in range(T)]


def all_parent_arrays(T):
    ranges = [range(-1, i) for i in range(1, T)]
    for rest in itertools.product(*ranges):
        yield [-1] + list(rest)


def brute_force(w, scale=None):
    """Pure-Python loops with math.exp; returns out [B][Hq][T][D], lse [B][Hq][T]."""
    sc = w.scale if scale is None else scale
    q, kc, vc = w.as_f64("q"), w.as_f64("k_cache"), w.as_f64("v_cache")
    kt, vt = w.as_f64("k_tree"), w.as_f64("v_tree")
    G = w.Hq // w.Hkv
    out = np.zeros((w.B, w.Hq, w.T, w.D))
    lse = np.zeros((w.B, w.Hq, w.T))
    for b in range(w.B):
        vis = visible_top_down([int(x) for x in w.parent[b]])
        for h in range(w.Hq):
            g = h // G
            for i in range(w.T):
                items = [(kc[b, g, p], vc[b, g, p]) for p in range(int(w.prefix_len[b]))]
                items += [(kt[b, g, j], vt[b, g, j]) for j in sorted(vis[i])]
                scores = [sc * sum(float(q[b, h, i, d]) * float(k[d]) for d in range(w.D))
                          for k, _ in items]
                mx = max(scores)
                z = sum(math.exp(s - mx) for s in scores)
                lse[b, h, i] = mx + math.log(z)
                for d in range(w.D):
                    out[b, h, i, d] = sum(math.exp(s - mx) / z * float(v[d])
                                          for s, (_, v) in zip(scores, items))
    return out, lse


def f64_workload(**kw):
    kw.setdefault("dtype", "f32")
    return make_custom(**kw)


def zero_keys(w):
    if w.dtype == "bf16":
        w.k_cache[...] = 0
        w.k_tree[...] = 0
    else:
        w.k_cache[...] = 0.0
        w.k_tree[...] = 0.0
    return w


# ----------------------------------------------------------------------------
# pin checks, written as functions so the mutation tests can reuse them
# ----------------------------------------------------------------------------

def pin_mask_exhaustive(max_T=6):
    for T in range(1, max_T + 1):
        for par in all_parent_arrays(T):
            want = visible_by_closure(par)
            got = oracle.tree_visible_nodes(par)
            if [set(x) for x in got] != want:
                return False
            bits = oracle.tree_mask_bits(par)
            for i in range(T):
                if int(bits[i]) != sum(1 << j for j in want[i]):
                    return False
    return True


def pin_brute_force(seed=3):
    w = f64_workload(B=2, Hq=4, Hkv=2, D=5, Lcap=9, T=5, prefix_len=[7, 0], seed=seed)
    o, l = oracle.verify_attn(w)
    bo, bl = brute_force(w)
    return max(np.abs(o - bo).max(), np.abs(l - bl).max())


def pin_closed_form_uniform(seed=4):
    w = zero_keys(f64_workload(B=2, Hq=2, Hkv=1, D=6, Lcap=11, T=7, prefix_len=[11, 3], seed=seed))
    o, l = oracle.verify_attn(w)
    err = 0.0
    vc, vt = w.as_f64("v_cache"), w.as_f64("v_tree")
    for b in range(w.B):
        L = int(w.prefix_len[b])
        vis = visible_top_down([int(x) for x in w.parent[b]])
        for h in range(w.Hq):
            for i in range(w.T):
                n = L + len(vis[i])
                mean = (vc[b, 0, :L].sum(axis=0) + sum(vt[b, 0, j] for j in vis[i])) / n
                err = max(err, abs(l[b, h, i] - math.log(n)), np.abs(o[b, h, i] - mean).max())
    return err


def pin_single_node(seed=5):
    w = f64_workload(B=1, Hq=3, Hkv=3, D=8, Lcap=4, T=1, prefix_len=[0], seed=seed)
    o, l = oracle.verify_attn(w)
    q, kt, vt = w.as_f64("q"), w.as_f64("k_tree"), w.as_f64("v_tree")
    err = 0.0
    for h in range(3):
        err = max(err, np.abs(o[0, h, 0] - vt[0, h, 0]).max(),
                  abs(l[0, h, 0] - w.scale * float(q[0, h, 0] @ kt[0, h, 0])))
    return err


def pin_golden():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))

    class W:
        pass
    w = W()
    w.dtype = "f32"
    for key in ("B", "Hq", "Hkv", "D", "T", "Lcap"):
        setattr(w, key, g[key])
    w.scale = g["scale"]
    for key in ("q", "k_cache", "v_cache", "k_tree", "v_tree"):
        setattr(w, key, np.asarray(g[key], dtype=np.float64))
    w.parent = np.asarray(g["parent"], dtype=np.int32)
    w.prefix_len = np.asarray(g["prefix_len"], dtype=np.int32)
    w.as_f64 = lambda name: np.asarray(getattr(w, name), dtype=np.float64)
    o, l = oracle.verify_attn(w)
    bits = [int(x) for x in oracle.tree_mask_bits(w.parent[0])]
    if bits != g["expected_mask_bits"][0]:
        return float("inf")
    return max(np.abs(o - np.asarray(g["expected_out"])).max(),
               np.abs(l - np.asarray(g["expected_lse"])).max())


def sdpa_reference(w):
    """out via torch's SDPA in float64 with an explicit boolean mask (no LSE)."""
    q, kc, vc = w.as_f64("q"), w.as_f64("k_cache"), w.as_f64("v_cache")
    kt, vt = w.as_f64("k_tree"), w.as_f64("v_tree")
    G = w.Hq // w.Hkv
    out = np.zeros((w.B, w.Hq, w.T, w.D))
    for b in range(w.B):
        L = int(w.prefix_len[b])
        vis = visible_by_closure([int(x) for x in w.parent[b]])
        mask = torch.zeros(w.T, L + w.T, dtype=torch.bool)
        mask[:, :L] = True
        for i in range(w.T):
            for j in vis[i]:
                mask[i, L + j] = True
        K = torch.from_numpy(np.concatenate([kc[b, :, :L], kt[b]], axis=1))
        V = torch.from_numpy(np.concatenate([vc[b, :, :L], vt[b]], axis=1))
        K = K.repeat_interleave(G, dim=0).contiguous()
        V = V.repeat_interleave(G, dim=0).contiguous()
        Q = torch.from_numpy(q[b])
        out[b] = F.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=mask,
                                                scale=w.scale)[0].numpy()
    return out


def pin_sdpa(seed=6):
    w = f64_workload(B=2, Hq=8, Hkv=2, D=16, Lcap=40, T=13, prefix_len=[40, 17], seed=seed)
    o, _ = oracle.verify_attn(w)
    return np.abs(o - sdpa_reference(w)).max()


def pin_chain_is_causal(seed=7):
    T, L = 9, 23
    w = f64_workload(B=1, Hq=4, Hkv=2, D=16, Lcap=L, T=T, prefix_len=[L], parents=[tree_chain(T)],
                     seed=seed)
    o, _ = oracle.verify_attn(w)
    q, kc, vc = w.as_f64("q"), w.as_f64("k_cache"), w.as_f64("v_cache")
    kt, vt = w.as_f64("k_tree"), w.as_f64("v_tree")
    K = torch.from_numpy(np.concatenate([kc[0], kt[0]], axis=1)).repeat_interleave(2, dim=0)
    V = torch.from_numpy(np.concatenate([vc[0], vt[0]], axis=1)).repeat_interleave(2, dim=0)
    Qf = torch.zeros(4, L + T, 16, dtype=torch.float64)
    Qf[:, L:] = torch.from_numpy(q[0])
    ref = F.scaled_dot_product_attention(Qf[None], K[None].contiguous(), V[None].contiguous(),
                                         is_causal=True, scale=w.scale)[0, :, L:]
    return np.abs(o[0] - ref.numpy()).max()


def pin_split_merge(seed=8):
    rng = np.random.default_rng(seed)
    w = f64_workload(B=2, Hq=4, Hkv=2, D=8, Lcap=50, T=6, prefix_len=[50, 31], seed=seed)
    full_o, full_l = oracle.verify_attn(w)
    err = 0.0
    for _ in range(4):
        cuts = sorted(set([0, 50] + rng.integers(0, 51, size=3).tolist()))
        outs, lses = [], []
        for lo, hi in zip(cuts[:-1], cuts[1:]):
            o, l = oracle.verify_attn(w, parts=("prefix",), prefix_range=(lo, hi))
            outs.append(o)
            lses.append(l)
        o, l = oracle.verify_attn(w, parts=("tree",))
        outs.append(o)
        lses.append(l)
        mo, ml = oracle.lse_merge(outs, lses)
        err = max(err, np.abs(mo - full_o).max(), np.abs(ml - full_l).max())
    return err


def pin_star(seed=9):
    T = 6
    w = f64_workload(B=1, Hq=2, Hkv=2, D=4, Lcap=5, T=T, prefix_len=[5], parents=[tree_star(T)],
                     seed=seed)
    o, l = oracle.verify_attn(w)
    bo, bl = brute_force(w)
    vis_ok = all(set(v) == ({0, i} if i else {0})
                 for i, v in enumerate(oracle.tree_visible_nodes(tree_star(T))))
    return max(np.abs(o - bo).max(), np.abs(l - bl).max()) if vis_ok else float("inf")


def pin_gqa_is_repeated_mha(seed=10):
    w = f64_workload(B=1, Hq=6, Hkv=2, D=8, Lcap=12, T=5, prefix_len=[12], seed=seed)
    o, l = oracle.verify_attn(w)
    m = f64_workload(B=1, Hq=6, Hkv=6, D=8, Lcap=12, T=5, prefix_len=[12], seed=seed,
                     parents=w.parent)
    m.q = w.q.copy()
    for name in ("k_cache", "v_cache", "k_tree", "v_tree"):
        setattr(m, name, np.repeat(getattr(w, name), 3, axis=1))
    mo, ml = oracle.verify_attn(m)
    return max(np.abs(o - mo).max(), np.abs(l - ml).max())


def pin_prefix_permutation(seed=11):
    w = f64_workload(B=1, Hq=2, Hkv=1, D=8, Lcap=20, T=4, prefix_len=[20], seed=seed)
    o, l = oracle.verify_attn(w)
    perm = np.random.default_rng(seed).permutation(20)
    w.k_cache = w.k_cache[:, :, perm].copy()
    w.v_cache = w.v_cache[:, :, perm].copy()
    po, pl = oracle.verify_attn(w)
    return max(np.abs(o - po).max(), np.abs(l - pl).max())


def pin_merge_closed_forms(seed=12):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((3, 5))
    l = rng.standard_normal(3)
    o2, l2 = oracle.lse_merge([o, o], [l, l])
    e1 = max(np.abs(o2 - o).max(), np.abs(l2 - (l + math.log(2))).max())
    o3, l3 = oracle.lse_merge([o, rng.standard_normal((3, 5))], [l, np.full(3, -np.inf)])
    e2 = max(np.abs(o3 - o).max(), np.abs(l3 - l).max())
    # weights e^1 and e^2 over e^1 + e^2: a weighted mean with known coefficients
    a, b = rng.standard_normal((4, 3)), rng.standard_normal((4, 3))
    o4, l4 = oracle.lse_merge([a, b], [np.ones(4), np.full(4, 2.0)])
    want = (math.e * a + math.e ** 2 * b) / (math.e + math.e ** 2)
    e3 = max(np.abs(o4 - want).max(), np.abs(l4 - math.log(math.e + math.e ** 2)).max())
    return max(e1, e2, e3)


PINS = {
    "brute_force": pin_brute_force,
    "closed_form_uniform": pin_closed_form_uniform,
    "single_node": pin_single_node,
    "golden": pin_golden,
    "sdpa": pin_sdpa,
    "chain_is_causal": pin_chain_is_causal,
    "split_merge": pin_split_merge,
    "star": pin_star,
    "gqa_is_repeated_mha": pin_gqa_is_repeated_mha,
    "prefix_permutation": pin_prefix_permutation,
    "merge_closed_forms": pin_merge_closed_forms,
}


# ----------------------------------------------------------------------------
# the pins themselves
# ----------------------------------------------------------------------------

def test_mask_exhaustive_small_trees():
    assert pin_mask_exhaustive()


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    assert PINS[name]() < 1e-12


def test_bad_tree_rejected():
    for bad in ([0], [-1, 1], [-1, 0, 3], [-1, -2]):
        with pytest.raises(oracle.BadTree):
            oracle.tree_visible_nodes(bad)


def test_forest_roots_see_only_their_own_path():
    par = [-1, 0, -1, 2, 1]
    vis = [set(v) for v in oracle.tree_visible_nodes(par)]
    assert vis == [{0}, {0, 1}, {2}, {2, 3}, {0, 1, 4}]


def test_empty_visible_rows_follow_the_convention():
    w = f64_workload(B=1, Hq=1, Hkv=1, D=4, Lcap=3, T=2, prefix_len=[0], seed=1)
    o, l = oracle.verify_attn(w, parts=("prefix",))
    assert np.all(l == -np.inf) and np.all(o == 0)


def test_bf16_inputs_are_used_exactly():
    """The oracle sees the rounded bf16 values, not the float32 samples."""
    w = make_custom(B=1, Hq=2, Hkv=1, D=8, Lcap=10, T=3, prefix_len=[10], seed=2, dtype="bf16")
    o, l = oracle.verify_attn(w)
    bo, bl = brute_force(w)
    assert max(np.abs(o - bo).max(), np.abs(l - bl).max()) < 1e-12


# ----------------------------------------------------------------------------
# mutation tests: a planted mistake must trip some pin
# ----------------------------------------------------------------------------

def _mut_no_self(parent):
    O.check_parent(parent)
    out = []
    for i in range(len(parent)):
        chain, j = [], int(parent[i])
        while j != -1:
            chain.append(j)
            j = int(parent[j])
        out.append(sorted(chain) if chain else [i])
    return out


def _mut_skip_root(parent):
    O.check_parent(parent)
    out = []
    for i in range(len(parent)):
        chain, j = [], i
        while j != -1 and int(parent[j]) != -1:
            chain.append(j)
            j = int(parent[j])
        out.append(sorted(chain) if chain else [i])
    return out


_orig_attend = O.attend_rows


def _mut_log2_lse(q, k, v, vis, scale):
    o, l = _orig_attend(q, k, v, vis, scale)
    return o, l / math.log(2)


def _mut_no_scale(q, k, v, vis, scale):
    return _orig_attend(q, k, v, vis, 1.0)


def _mut_transposed_values(q, k, v, vis, scale):
    o, l = _orig_attend(q, k, v, vis, scale)
    return o[::-1].copy(), l


_orig_merge = O.lse_merge


def _mut_merge_unweighted(outs, lses):
    o, l = _orig_merge(outs, lses)
    return np.mean(np.stack(outs), axis=0), l


MUTANTS = [
    ("tree_visible_nodes", _mut_no_self),
    ("tree_visible_nodes", _mut_skip_root),
    ("attend_rows", _mut_log2_lse),
    ("attend_rows", _mut_no_scale),
    ("attend_rows", _mut_transposed_values),
    ("lse_merge", _mut_merge_unweighted),
]


@pytest.mark.parametrize("attr,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(O, attr, mutant)
    monkeypatch.setattr(oracle, attr, mutant)
    caught = []
    if attr == "tree_visible_nodes":
        try:
            caught.append(not pin_mask_exhaustive(max_T=4))
        except Exception:
            caught.append(True)
    for name, pin in PINS.items():
        try:
            caught.append(not (pin() < 1e-12))
        except Exception:
            caught.append(True)
    assert any(caught), f"no pin caught mutant {mutant.__name__}"
