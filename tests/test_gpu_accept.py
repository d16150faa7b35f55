"""GPU parity of hta_accept / hta_commit against the oracle (exact: integer and byte results).

Accept: target tokens, accepted length, path and bonus token must equal the
oracle's (argmax ties resolve to the lowest index on both sides, on the same
exact logit values). Commit: the caches must equal the oracle's byte for
byte, and prefix_len must advance by the accepted length.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import say
from speculative_decoding_verification_hybrid_amd import hta
from workloads import f32_to_bf16_bits, make_accept_case, make_custom

pytestmark = pytest.mark.gpu


def _logits_tensor(case, misalign=False):
    if case.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(case.logits).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(case.logits, dtype=np.float32))
    t = t.cuda()
    if misalign:  # same values, data pointer off 16-byte alignment
        flat = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        flat[1:] = t.reshape(-1)
        t = flat[1:].view(t.shape)
    return t


def _run_accept(h, case, misalign=False):
    B, T = case.B, case.T
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    out = dict(target=torch.full((B, T), -7, dtype=torch.int32, device="cuda"),
               accept_len=torch.full((B,), -7, dtype=torch.int32, device="cuda"),
               path=torch.full((B, T), -7, dtype=torch.int32, device="cuda"),
               bonus=torch.full((B,), -7, dtype=torch.int32, device="cuda"))
    hta.hta_accept(h, _logits_tensor(case, misalign), dev(case.parent), dev(case.tree_tokens), out["target"],
                   out["accept_len"], out["path"], out["bonus"])
    status = hta.hta_get_status(h)
    return {k: v.cpu().numpy().astype(np.int64) for k, v in out.items()}, status


def _cfg(B, T, D=128, Hkv=2, Lcap=256, dtype="bf16"):
    return hta.make_config(batch=B, n_q_heads=2 * Hkv, n_kv_heads=Hkv, head_dim=D, tree_nodes=T,
                           kv_capacity=Lcap, dtype=dtype)


def _check(case, got, status):
    ref = oracle.accept(case.parent, case.tree_tokens, case.logits_f64())
    assert status == (hta.HTA_STATUS_BAD_TREE if ref["bad"].any() else 0)
    assert np.array_equal(got["target"], ref["target"])
    assert np.array_equal(got["accept_len"], ref["accept_len"])
    assert np.array_equal(got["path"], ref["path"])
    assert np.array_equal(got["bonus"], ref["bonus"])
    return ref


CASES = {
    # name: make_accept_case kwargs
    "cfg3_llama_vocab": dict(B=1, T=64, V=128256, dtype="bf16", tree=("bounded", 6, None), depth=[5]),
    "batch4_bounded": dict(B=4, T=32, V=32000, dtype="bf16", tree=("uniform",), max_depth=8),
    "f32_logits": dict(B=3, T=26, V=5000, dtype="f32", tree=("bounded", 5, 4)),
    "odd_vocab_scalar_path": dict(B=2, T=17, V=1003, dtype="bf16", tree=("uniform",)),
    "chain_all_accepted": dict(B=2, T=64, V=4096, dtype="bf16", tree=("chain",), depth=[63, 40]),
    "star": dict(B=3, T=40, V=2048, dtype="bf16", tree=("star",), depth=[1, 0, 1]),
    "single_node": dict(B=2, T=1, V=512, dtype="bf16", tree=("uniform",)),
    "duplicate_siblings": dict(B=4, T=48, V=64, dtype="bf16", tree=("bounded", 4, 6), dup_siblings=True,
                               max_depth=4),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_accept_parity(name):
    kw = CASES[name]
    case = make_accept_case(seed=sum(map(ord, name)), **kw)
    say(f"hta_accept {name}")
    with hta.hta_create(_cfg(case.B, case.T)) as h:
        got, status = _run_accept(h, case)
    ref = _check(case, got, status)
    assert np.all(ref["accept_len"] >= 1)


def test_accept_misaligned_logits_take_the_scalar_path():
    case = make_accept_case(B=2, T=20, V=4096, dtype="bf16", seed=5)
    say("hta_accept misaligned logits")
    with hta.hta_create(_cfg(case.B, case.T)) as h:
        got, status = _run_accept(h, case, misalign=True)
    _check(case, got, status)


def test_accept_ties_resolve_to_lowest_index():
    # coarse logits: every row has many equal maxima
    case = make_accept_case(B=2, T=12, V=300, dtype="f32", seed=9)
    case.logits = (np.round(case.logits * 0.5) / 0.5).astype(np.float32)
    case.logits[:, :, 7] = case.logits.max(axis=2)  # an early index among the maxima of every row
    say("hta_accept ties")
    with hta.hta_create(_cfg(case.B, case.T)) as h:
        got, status = _run_accept(h, case)
    _check(case, got, status)
    assert np.all(got["target"] <= 7)



@pytest.mark.parametrize("dtype,V", [("bf16", 4096), ("bf16", 1003), ("f32", 4096)])
def test_accept_signed_zero_maxima(dtype, V):
    # every row's maximum is zero, held by -0 and +0 at two or more indices
    case = make_accept_case(B=2, T=10, V=V, dtype="f32", seed=31)
    rng = np.random.default_rng(32)
    lg = -1.0 - np.abs(case.logits.astype(np.float64))
    for b in range(case.B):
        for i in range(case.T):
            pos = np.sort(rng.choice(V, size=3, replace=False))
            lg[b, i, pos] = [-0.0, 0.0, -0.0] if (b + i) % 2 == 0 else [0.0, -0.0, 0.0]
    case.logits = lg.astype(np.float32)
    if dtype == "bf16":
        case.logits = f32_to_bf16_bits(case.logits)
        case.dtype = "bf16"
    say(f"hta_accept signed zeros {dtype} V={V}")
    with hta.hta_create(_cfg(case.B, case.T)) as h:
        got, status = _run_accept(h, case, misalign=V % 8 != 0)
    _check(case, got, status)
    assert np.array_equal(got["target"], np.argmax(case.logits_f64() == 0.0, axis=2))  # first zero of each row

def test_accept_bad_tree_and_forest():
    case = make_accept_case(B=3, T=8, V=256, dtype="bf16", seed=11,
                            parents=[[-1, 0, 0, 1, 1, 2, 3, 4],
                                     [-1, 0, -1, 2, 0, 4, 2, 6],   # a forest: nodes 2, 3, 6, 7 under root 2
                                     [-1, 0, 3, 1, 1, 2, 3, 4]])   # bad: parent[2] = 3 >= 2
    say("hta_accept bad tree / forest")
    with hta.hta_create(_cfg(case.B, case.T)) as h:
        got, status = _run_accept(h, case)
    ref = _check(case, got, status)
    assert list(ref["bad"]) == [False, False, True]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_commit_parity(dtype):
    B, Hkv, D, T, Lcap = 4, 2, 128, 24, 300
    w = make_custom(B=B, Hq=2 * Hkv, Hkv=Hkv, D=D, Lcap=Lcap, T=T, prefix_len=[10, 299, 0, 150], dtype=dtype,
                    seed=21)
    case = make_accept_case(B=B, T=T, V=3000, dtype="bf16", seed=22, parents=w.parent, depth=[6, 5, 3, 23])
    say(f"hta_accept + hta_commit {dtype}")
    dev = lambda a: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
                     if dtype == "bf16" else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))).cuda()
    kc, vc, kt, vt = dev(w.k_cache), dev(w.v_cache), dev(w.k_tree), dev(w.v_tree)
    plen = torch.from_numpy(w.prefix_len.astype(np.int32)).cuda()
    with hta.hta_create(_cfg(B, T, D=D, Hkv=Hkv, Lcap=Lcap, dtype=dtype)) as h:
        got, status = _run_accept(h, case)
        ref = _check(case, got, status)
        n = torch.from_numpy(got["accept_len"].astype(np.int32)).cuda()
        path = torch.from_numpy(got["path"].astype(np.int32)).cuda()
        hta.hta_commit(h, kt, vt, n, path, kc, vc, plen)
        status = hta.hta_get_status(h)
    kc2, vc2, L2, over = oracle.commit(w.k_cache, w.v_cache, w.prefix_len, w.k_tree, w.v_tree,
                                       ref["accept_len"], ref["path"])
    assert status == (hta.HTA_STATUS_COMMIT_OVERFLOW if over.any() else 0)
    assert list(over) == [False, True, False, False]  # 299 + (at least 2) > 300
    assert np.array_equal(plen.cpu().numpy(), L2)
    host = lambda t: (t.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16"
                      else t.cpu().numpy())
    assert np.array_equal(host(kc), kc2) and np.array_equal(host(vc), vc2)


def test_commit_bad_prefix_len():
    # prefix_len outside [0, Lcap] is a bad prefix, not an overflow; the sequence is left as it is
    B, Hkv, D, T, Lcap = 4, 2, 128, 8, 64
    w = make_custom(B=B, Hq=2 * Hkv, Hkv=Hkv, D=D, Lcap=Lcap, T=T, prefix_len=[5, 5, 5, 5], dtype="bf16", seed=23)
    bad_len = np.array([-3, 10, Lcap + 1, 62], dtype=np.int32)  # 62 + 3 > 64 overflows
    accept_len = np.array([3, 3, 2, 3], dtype=np.int32)
    path = np.full((B, T), -1, dtype=np.int32)
    path[:, :3] = [0, 1, 3]
    say("hta_commit bad prefix_len")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    kc, vc, kt, vt = dev(w.k_cache), dev(w.v_cache), dev(w.k_tree), dev(w.v_tree)
    plen = torch.from_numpy(bad_len.copy()).cuda()
    i32 = lambda a: torch.from_numpy(a).cuda()
    with hta.hta_create(_cfg(B, T, D=D, Hkv=Hkv, Lcap=Lcap)) as h:
        hta.hta_commit(h, kt, vt, i32(accept_len), i32(path), kc, vc, plen)
        status = hta.hta_get_status(h)
        hta.hta_commit(h, kt, vt, i32(np.zeros(B, np.int32)), i32(path), kc, vc, plen)  # nothing accepted
        status_empty = hta.hta_get_status(h)
    assert status == hta.HTA_STATUS_BAD_PREFIX | hta.HTA_STATUS_COMMIT_OVERFLOW
    assert status_empty == hta.HTA_STATUS_BAD_PREFIX  # a bad length is reported even with nothing to commit
    kc2, vc2, L2, _ = oracle.commit(w.k_cache, w.v_cache, bad_len, w.k_tree, w.v_tree, accept_len, path)
    assert list(plen.cpu().numpy()) == list(L2) == [-3, 13, Lcap + 1, 62]
    host = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(host(kc), kc2) and np.array_equal(host(vc), vc2)
