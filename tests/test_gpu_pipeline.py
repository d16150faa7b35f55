"""The rows composed as one decoding step, checked against the oracle chain, and
the stateless calls replayed from a HIP graph.

Step: hta_build_tree (tree from the last logits and the history) -> its parent
array feeds hta_verify_attn -> its tokens and parents feed hta_accept (on
per-node target logits) -> hta_commit appends the accepted rows. Every stage is
compared with the oracle run on the oracle's own previous outputs (trees,
acceptance and commit exactly, attention within the usual tolerances).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_LSE_REL, TOL_OUT, say
from speculative_decoding_verification_hybrid_amd import hta
from workloads import make_accept_case, make_custom, make_tree_case

pytestmark = pytest.mark.gpu

B, HQ, HKV, D, T, LCAP, V = 2, 8, 2, 128, 16, 1024, 1000
K, M, KEEP_FIRST, KEEP = 5, 2, 4, [4, 3, 2, 2, 1]


def _inputs():
    w = make_custom(B=B, Hq=HQ, Hkv=HKV, D=D, Lcap=LCAP, T=T, prefix_len=[1000, 555], dtype="bf16", seed=31)
    tc = make_tree_case(B=B, V=V, cap=600, history_len=[600, 321], alphabet=12, seed=32)
    return w, tc


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def test_decoding_step_matches_oracle_chain():
    w, tc = _inputs()
    say("pipeline: build_tree -> verify_attn -> accept -> commit")
    cfg = hta.make_config(batch=B, n_q_heads=HQ, n_kv_heads=HKV, head_dim=D, tree_nodes=T, kv_capacity=LCAP,
                          dtype="bf16", softmax_scale=w.scale)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    with hta.hta_create(cfg) as h:
        # 1. the tree
        tok = torch.empty(B, T, dtype=torch.int32, device="cuda")
        par = torch.empty(B, T, dtype=torch.int32, device="cuda")
        nn = torch.empty(B, dtype=torch.int32, device="cuda")
        hta.hta_build_tree(h, _bf16(tc.logits), i32(tc.history), i32(tc.history_len),
                           hta.make_tree_params(K, M, KEEP_FIRST, KEEP), tok, par, nn)
        rt, rp, rn = oracle.build_trees(tc.history, tc.history_len, tc.logits_f64(), K, M, KEEP_FIRST, KEEP, T)
        assert np.array_equal(tok.cpu().numpy(), rt) and np.array_equal(par.cpu().numpy(), rp)
        assert np.array_equal(nn.cpu().numpy(), rn)
        # 2. verification attention over that tree
        w.parent = rp.astype(np.int32)
        out = torch.empty(B, HQ, T, D, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, HQ, T, dtype=torch.float32, device="cuda")
        kc, vc = _bf16(w.k_cache), _bf16(w.v_cache)
        kt, vt = _bf16(w.k_tree), _bf16(w.v_tree)
        plen = i32(w.prefix_len)
        hta.hta_verify_attn(h, _bf16(w.q), kc, vc, kt, vt, par, plen, out, lse)
        ro, rl = oracle.verify_attn(w)
        assert np.abs(out.float().cpu().numpy() - ro).max() <= TOL_OUT["bf16"]
        assert (np.abs(lse.cpu().numpy() - rl) / np.maximum(1, np.abs(rl))).max() <= TOL_LSE_REL
        # 3. acceptance of the tree's tokens (per-node target logits, a path planted)
        ac = make_accept_case(B=B, T=T, V=V, dtype="bf16", seed=33, parents=rp, depth=[3, 2])
        target = torch.empty(B, T, dtype=torch.int32, device="cuda")
        n_acc = torch.empty(B, dtype=torch.int32, device="cuda")
        path = torch.empty(B, T, dtype=torch.int32, device="cuda")
        bonus = torch.empty(B, dtype=torch.int32, device="cuda")
        hta.hta_accept(h, _bf16(ac.logits), par, tok, target, n_acc, path, bonus)
        ra = oracle.accept(rp, rt, ac.logits_f64())
        assert np.array_equal(n_acc.cpu().numpy(), ra["accept_len"])
        assert np.array_equal(path.cpu().numpy(), ra["path"]) and np.array_equal(bonus.cpu().numpy(), ra["bonus"])
        # 4. commit of the accepted rows
        hta.hta_commit(h, kt, vt, n_acc, path, kc, vc, plen)
        assert hta.hta_get_status(h) == 0
        kc2, vc2, L2, over = oracle.commit(w.k_cache, w.v_cache, w.prefix_len, w.k_tree, w.v_tree,
                                           ra["accept_len"], ra["path"])
        assert not over.any()
        assert np.array_equal(plen.cpu().numpy(), L2)
        host = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(host(kc), kc2) and np.array_equal(host(vc), vc2)


def test_stateless_calls_replay_from_a_graph():
    """build_tree, verify_attn, accept, cross_attn captured once; replayed three
    times with eager work in between; every replay equals the eager results."""
    w, tc = _inputs()
    say("pipeline graph replays")
    cfg = hta.make_config(batch=B, n_q_heads=HQ, n_kv_heads=HKV, head_dim=D, tree_nodes=T, kv_capacity=LCAP,
                          dtype="bf16", softmax_scale=w.scale)
    cfg1 = hta.make_config(batch=B, n_q_heads=HQ, n_kv_heads=HKV, head_dim=D, tree_nodes=1, kv_capacity=LCAP,
                           dtype="bf16", softmax_scale=w.scale)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    lg, hist, hl = _bf16(tc.logits), i32(tc.history), i32(tc.history_len)
    q, kc, vc, kt, vt, plen = _bf16(w.q), _bf16(w.k_cache), _bf16(w.v_cache), _bf16(w.k_tree), _bf16(w.v_tree), \
        i32(w.prefix_len)
    q1 = _bf16(w.q[:, :, :1])
    ac_logits = _bf16(make_accept_case(B=B, T=T, V=V, dtype="bf16", seed=34, parents=[[-1] + [0] * (T - 1)] * B).logits)
    prm = hta.make_tree_params(K, M, KEEP_FIRST, KEEP)
    bufs = dict(tok=torch.empty(B, T, dtype=torch.int32, device="cuda"),
                par=torch.empty(B, T, dtype=torch.int32, device="cuda"),
                nn=torch.empty(B, dtype=torch.int32, device="cuda"),
                out=torch.empty(B, HQ, T, D, dtype=torch.bfloat16, device="cuda"),
                lse=torch.empty(B, HQ, T, dtype=torch.float32, device="cuda"),
                tgt=torch.empty(B, T, dtype=torch.int32, device="cuda"),
                n=torch.empty(B, dtype=torch.int32, device="cuda"),
                path=torch.empty(B, T, dtype=torch.int32, device="cuda"),
                bonus=torch.empty(B, dtype=torch.int32, device="cuda"),
                cout=torch.empty(B, HQ, 1, D, dtype=torch.bfloat16, device="cuda"),
                clse=torch.empty(B, HQ, 1, dtype=torch.float32, device="cuda"))
    with hta.hta_create(cfg) as h, hta.hta_create(cfg1) as h1:
        def step(s):
            hta.hta_build_tree(h, lg, hist, hl, prm, bufs["tok"], bufs["par"], bufs["nn"], s)
            hta.hta_verify_attn(h, q, kc, vc, kt, vt, bufs["par"], plen, bufs["out"], bufs["lse"], s)
            hta.hta_accept(h, ac_logits, bufs["par"], bufs["tok"], bufs["tgt"], bufs["n"], bufs["path"],
                           bufs["bonus"], s)
            hta.hta_cross_attn(h1, q1, kc, vc, plen, bufs["cout"], bufs["clse"], s)

        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        eager = {k: v.clone() for k, v in bufs.items()}
        for v in bufs.values():
            v.zero_()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(torch.cuda.current_stream())
        for rep in range(3):
            for v in bufs.values():
                v.fill_(3)  # eager work between replays, and stale contents to overwrite
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for k in bufs:
                assert torch.equal(bufs[k], eager[k]), f"replay {rep}: {k} differs from the eager result"
        assert hta.hta_get_status(h) == 0 and hta.hta_get_status(h1) == 0
