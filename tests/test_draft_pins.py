"""Pins of the draft-attention oracle (CPU only).

Cross-attention is checked against torch's fp64 attention and closed forms;
the sliding window against one-hot values that reveal exactly which slots a
row sees (counted by an independent age formula), against the verification
oracle's chain tree (causal attention) when the window covers everything,
against torch's fp64 attention with a band mask over the unrolled positions,
and against closed forms (a window of 1) and invariants.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import make_custom, make_window_case, tree_chain


def _sdpa(q, k, v, mask, scale):
    """torch fp64 attention (and its natural-log LSE) of rows q [R, D] over k, v [N, D]."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    m = torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], attn_mask=m[None],
                                                           scale=scale)[0]
    s = (qt @ kt.T) * scale
    lse = torch.logsumexp(s.masked_fill(~m, -math.inf), dim=-1)
    return out.numpy(), lse.numpy()


# ----------------------------------------------------------------------------
# cross-attention over the target's cache
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cross_attn_matches_torch(dtype):
    w = make_custom(B=2, Hq=8, Hkv=2, D=32, Lcap=70, T=3, prefix_len=[70, 33], dtype=dtype, seed=3)
    q, kc, vc = w.as_f64("q"), w.as_f64("k_cache"), w.as_f64("v_cache")
    out, lse = oracle.cross_attn(q, kc, vc, w.prefix_len, w.scale)
    for b in range(2):
        L = int(w.prefix_len[b])
        for h in range(8):
            o, l = _sdpa(q[b, h], kc[b, h // 4, :L], vc[b, h // 4, :L], np.ones((3, L), dtype=bool), w.scale)
            np.testing.assert_allclose(out[b, h], o, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], l, atol=1e-12)


def test_cross_attn_closed_forms():
    rng = np.random.default_rng(0)
    B, Hq, Hkv, T, D, L = 2, 4, 2, 2, 8, 9
    q = rng.standard_normal((B, Hq, T, D))
    kc = np.zeros((B, Hkv, L, D))
    vc = rng.standard_normal((B, Hkv, L, D))
    out, lse = oracle.cross_attn(q, kc, vc, np.array([L, 0]), 0.3)
    # zero keys: uniform weights over the L positions
    np.testing.assert_allclose(lse[0], np.log(L), atol=1e-14)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], np.broadcast_to(vc[0, h // 2].mean(axis=0), (T, D)), atol=1e-14)
    # empty prefix: nothing to attend to
    assert np.all(np.isneginf(lse[1])) and np.all(out[1] == 0)


def test_cross_attn_is_the_prefix_part_of_verification():
    w = make_custom(B=2, Hq=4, Hkv=1, D=16, Lcap=40, T=5, prefix_len=[40, 17], dtype="bf16", seed=8)
    o1, l1 = oracle.cross_attn(w.as_f64("q"), w.as_f64("k_cache"), w.as_f64("v_cache"), w.prefix_len, w.scale)
    o2, l2 = oracle.verify_attn(w, parts=("prefix",))
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


# ----------------------------------------------------------------------------
# sliding-window self-attention
# ----------------------------------------------------------------------------

def _visible_by_age(P, W, j):
    """Slots new token j sees, by age (0 = newest ring entry): it keeps the W - 1 - j
    newest entries that exist (age < P)."""
    return sorted(s for s in range(W) if (P - 1 - s) % W <= W - 2 - j and (P - 1 - s) % W < P)


@pytest.mark.parametrize("P,W,Tn", [(0, 8, 3), (3, 8, 2), (8, 8, 4), (13, 8, 5), (100, 8, 8), (5, 1, 1),
                                    (37, 16, 1)])
def test_window_sees_exactly_the_last_w_positions(P, W, Tn):
    # zero keys and one-hot values: out * count is the indicator of the visible keys
    D = W + Tn
    q = np.ones((1, 1, Tn, D))
    kr, kn = np.zeros((1, 1, W, D)), np.zeros((1, 1, Tn, D))
    vr = np.eye(D)[:W][None, None]
    vn = np.eye(D)[W:][None, None]
    out, lse = oracle.window_attn(q, kr, vr, kn, vn, np.array([P]), 0.5)
    for j in range(Tn):
        count = min(W, P + j + 1)
        assert lse[0, 0, j] == pytest.approx(math.log(count), abs=1e-14)
        seen = np.flatnonzero(out[0, 0, j] * count > 0.5)
        want = _visible_by_age(P, W, j) + [W + i for i in range(j + 1)]
        assert list(seen) == want
        assert len(want) == count


def test_window_covering_everything_is_causal_attention():
    # W >= P + Tn: the ring holds positions 0..P-1 at slots 0..P-1 and the window
    # hides nothing, so the new tokens do causal attention = a chain-shaped tree
    P, W, Tn, D = 11, 32, 5, 16
    w = make_custom(B=1, Hq=4, Hkv=2, D=D, Lcap=W, T=Tn, prefix_len=[P], dtype="f32", seed=4)
    w.parent = tree_chain(Tn)[None].astype(np.int32)
    want_o, want_l = oracle.verify_attn(w)
    q, kc, vc, kt, vt = (w.as_f64(n) for n in ("q", "k_cache", "v_cache", "k_tree", "v_tree"))
    out, lse = oracle.window_attn(q, kc, vc, kt, vt, np.array([P]), w.scale)
    np.testing.assert_allclose(out, want_o, atol=1e-13)
    np.testing.assert_allclose(lse, want_l, atol=1e-13)


@pytest.mark.parametrize("P", [0, 5, 24, 61])
def test_window_matches_torch_band_attention(P):
    W, Tn = 24, 6
    c = make_window_case(B=1, Hq=6, Hkv=2, D=16, W=W, Tn=Tn, pos=[P], dtype="bf16", seed=P)
    q, kr, vr, kn, vn = (c.as_f64(n) for n in ("q", "k_ring", "v_ring", "k_new", "v_new"))
    out, lse = oracle.window_attn(q, kr, vr, kn, vn, c.pos, c.scale)
    # unroll: positions max(0, P - W) .. P + Tn - 1 in order
    first = max(0, P - W)
    positions = list(range(first, P + Tn))
    for h in range(6):
        g = h // 3
        K = np.stack([kr[0, g, x % W] if x < P else kn[0, g, x - P] for x in positions])
        V = np.stack([vr[0, g, x % W] if x < P else vn[0, g, x - P] for x in positions])
        mask = np.array([[P + j - W < x <= P + j for x in positions] for j in range(Tn)])
        o, l = _sdpa(q[0, h], K, V, mask, c.scale)
        np.testing.assert_allclose(out[0, h], o, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], l, atol=1e-12)


def test_window_of_one_is_the_token_itself():
    c = make_window_case(B=2, Hq=2, Hkv=1, D=8, W=1, Tn=1, pos=[0, 9], dtype="f32", seed=2)
    q, kr, vr, kn, vn = (c.as_f64(n) for n in ("q", "k_ring", "v_ring", "k_new", "v_new"))
    out, lse = oracle.window_attn(q, kr, vr, kn, vn, c.pos, c.scale)
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(out[b, h, 0], vn[b, 0, 0], atol=1e-15)
            assert lse[b, h, 0] == pytest.approx(c.scale * q[b, h, 0] @ kn[b, 0, 0], abs=1e-13)


def test_window_shift_by_w_changes_nothing_and_unused_slots_are_not_read():
    c = make_window_case(B=1, Hq=4, Hkv=2, D=8, W=16, Tn=3, pos=[20], dtype="f32", seed=6)
    args = [c.as_f64(n) for n in ("q", "k_ring", "v_ring", "k_new", "v_new")]
    o1, l1 = oracle.window_attn(*args, np.array([20]), c.scale)
    o2, l2 = oracle.window_attn(*args, np.array([36]), c.scale)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    p = make_window_case(B=1, Hq=4, Hkv=2, D=8, W=16, Tn=3, pos=[5], dtype="bf16", seed=6, poison_unused=True)
    assert np.isnan(p.as_f64("k_ring")[0, :, 5:]).all()
    o, l = oracle.window_attn(*(p.as_f64(n) for n in ("q", "k_ring", "v_ring", "k_new", "v_new")), p.pos, p.scale)
    assert np.isfinite(o).all() and np.isfinite(l).all()


def test_window_is_ring_part_merged_with_new_part():
    c = make_window_case(B=1, Hq=2, Hkv=1, D=8, W=10, Tn=4, pos=[23], dtype="f32", seed=1)
    q, kr, vr, kn, vn = (c.as_f64(n) for n in ("q", "k_ring", "v_ring", "k_new", "v_new"))
    out, lse = oracle.window_attn(q, kr, vr, kn, vn, c.pos, c.scale)
    vis = oracle.window_visible(23, 10, 4)
    for h in range(2):
        o1, l1 = oracle.attend_rows(q[0, h], kr[0, 0], vr[0, 0], vis[:, :10], c.scale)
        o2, l2 = oracle.attend_rows(q[0, h], kn[0, 0], vn[0, 0], vis[:, 10:], c.scale)
        o, l = oracle.lse_merge([o1, o2], [l1, l2])
        np.testing.assert_allclose(out[0, h], o, atol=1e-13)
        np.testing.assert_allclose(lse[0, h], l, atol=1e-13)


def test_window_append_places_tokens_by_position():
    c = make_window_case(B=2, Hq=2, Hkv=1, D=4, W=5, Tn=3, pos=[3, 9], dtype="f32", seed=0)
    kr, vr, pos = oracle.window_append(c.k_ring, c.v_ring, c.k_new, c.v_new, c.pos)
    assert list(pos) == [6, 12]
    # sequence 0: positions 3, 4, 5 -> slots 3, 4, 0; sequence 1: positions 9, 10, 11 -> slots 4, 0, 1
    for b, slots in ((0, [3, 4, 0]), (1, [4, 0, 1])):
        for j, s in enumerate(slots):
            np.testing.assert_array_equal(kr[b, 0, s], c.k_new[b, 0, j])
            np.testing.assert_array_equal(vr[b, 0, s], c.v_new[b, 0, j])
        rest = [s for s in range(5) if s not in slots]
        np.testing.assert_array_equal(kr[b, 0, rest], c.k_ring[b, 0, rest])
    # one token at a time gives the same rings
    k1, v1, p1 = c.k_ring, c.v_ring, c.pos
    for j in range(3):
        k1, v1, p1 = oracle.window_append(k1, v1, c.k_new[:, :, j:j + 1], c.v_new[:, :, j:j + 1], p1)
    np.testing.assert_array_equal(k1, kr)
    np.testing.assert_array_equal(v1, vr)


def test_planted_window_mistakes_are_caught():
    # a window that drops the query's own position from its count, or maps
    # position x to slot (x + 1) mod W, must fail the one-hot pin
    P, W, Tn = 13, 8, 3
    def wrong_visible(P, W, Tn, kind):
        vis = np.zeros((Tn, W + Tn), dtype=bool)
        for j in range(Tn):
            t = P + j
            lo = max(0, t - W + (2 if kind == "short" else 1))
            for x in range(lo, P):
                vis[j, ((x + 1) if kind == "slot" else x) % W] = True
            vis[j, W:W + j + 1] = True
        return vis
    for kind in ("short", "slot"):
        vis = wrong_visible(P, W, Tn, kind)
        ok = all(sorted(np.flatnonzero(vis[j, :W])) == _visible_by_age(P, W, j)
                 and vis[j].sum() == min(W, P + j + 1) for j in range(Tn))
        assert not ok, kind
    vis = oracle.window_visible(P, W, Tn)
    assert all(sorted(np.flatnonzero(vis[j, :W])) == _visible_by_age(P, W, j) for j in range(Tn))
