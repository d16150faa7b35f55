"""GPU parity of hta_build_tree against the oracle (exact: token ids, parents, node counts).

Both sides rank on the same exact logit values (lower index first on ties)
and search the same token sequence, so every output must be identical.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import say
from speculative_decoding_verification_hybrid_amd import hta
from workloads import f32_to_bf16_bits, make_tree_case

pytestmark = pytest.mark.gpu


def _run(case, k, m, keep_first, keep, T, hist_len=None):
    B = case.B
    if case.dtype == "bf16":
        lg = torch.from_numpy(np.ascontiguousarray(case.logits).view(np.int16)).view(torch.bfloat16).cuda()
    else:
        lg = torch.from_numpy(np.ascontiguousarray(case.logits, dtype=np.float32)).cuda()
    hist = torch.from_numpy(case.history).cuda()
    hl = torch.from_numpy(np.asarray(case.history_len if hist_len is None else hist_len, dtype=np.int32)).cuda()
    tok = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    par = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    nn = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    cfg = hta.make_config(batch=B, n_q_heads=8, n_kv_heads=2, head_dim=128, tree_nodes=T, kv_capacity=64)
    with hta.hta_create(cfg) as h:
        hta.hta_build_tree(h, lg, hist, hl, hta.make_tree_params(k, m, keep_first, keep), tok, par, nn)
        status = hta.hta_get_status(h)
    return tok.cpu().numpy(), par.cpu().numpy(), nn.cpu().numpy(), status


def _check(case, k, m, keep_first, keep, T):
    say(f"hta_build_tree B={case.B} V={case.V} k={k} m={m} T={T} lens={list(case.history_len)[:4]}")
    tok, par, nn, status = _run(case, k, m, keep_first, keep, T)
    assert status == 0
    rt, rp, rn = oracle.build_trees(case.history, case.history_len, case.logits_f64(), k, m, keep_first, keep, T)
    assert np.array_equal(nn, rn)
    assert np.array_equal(tok, rt)
    assert np.array_equal(par, rp)
    return rn


def test_llama_vocab_32k_history():
    case = make_tree_case(B=1, V=128256, cap=32768, history_len=[32768], alphabet=40, seed=1)
    keep = [8, 6, 5, 4, 4, 3, 3, 2, 2, 2, 1, 1, 1, 1, 1]
    n = _check(case, 15, 3, 8, keep, 64)
    assert n[0] > 16  # the planted repeats give matches


@pytest.mark.parametrize("m", [1, 2, 3, 4, 8])
def test_ngram_lengths_ragged_batch(m):
    case = make_tree_case(B=5, V=1000, cap=9000, history_len=[0, 1, 2, 8200, 9000], alphabet=6, seed=m)
    _check(case, 7, m, 4, [5, 4, 3, 3, 2, 1, 1], 64)


@pytest.mark.parametrize("k", [0, 1, 31])
def test_guess_counts(k):
    case = make_tree_case(B=2, V=300, cap=3000, history_len=[3000, 1234], alphabet=10, seed=10 + k)
    keep = [max(0, 4 - r // 4) for r in range(k)]
    _check(case, k, 2, 3, keep, 64)


@pytest.mark.parametrize("T", [1, 2, 5, 33])
def test_truncated_trees(T):
    case = make_tree_case(B=2, V=500, cap=2000, history_len=[2000, 700], alphabet=5, seed=T)
    _check(case, 9, 3, 6, [6, 5, 5, 4, 3, 3, 2, 2, 1], T)


def test_ties_and_float_logits():
    case = make_tree_case(B=3, V=257, cap=1500, history_len=[1500, 100, 10], alphabet=8, dtype="f32", seed=3)
    case.logits = (np.round(case.logits) ).astype(np.float32)  # many equal values
    _check(case, 12, 2, 3, [3] * 12, 64)


def test_odd_vocab_and_no_matches():
    # alphabet larger than the history: few or no repeats
    case = make_tree_case(B=2, V=70001, cap=64, history_len=[64, 30], alphabet=60000, seed=4)
    _check(case, 5, 3, 4, [4, 3, 2, 1, 1], 16)


def test_bad_history_len_gives_empty_tree_and_status():
    case = make_tree_case(B=2, V=200, cap=100, history_len=[100, 50], alphabet=5, seed=2)
    say("hta_build_tree bad history_len")
    tok, par, nn, status = _run(case, 3, 2, 2, [2, 2, 2], 8, hist_len=[100, 101])
    assert status == hta.HTA_STATUS_BAD_PREFIX
    assert nn[1] == 0 and np.all(tok[1] == -1) and par[1, 0] == -1 and np.all(par[1, 1:] == 0)
    rt, rp, rn = oracle.build_trees(case.history[:1], case.history_len[:1], case.logits_f64()[:1], 3, 2, 2,
                                    [2, 2, 2], 8)
    assert np.array_equal(tok[:1], rt) and np.array_equal(par[:1], rp) and nn[0] == rn[0]


@pytest.mark.parametrize("dtype,V", [("bf16", 5000), ("f32", 257)])
def test_signed_zero_ties(dtype, V):
    # the largest logits are zeros of both signs: they rank as equals, by index
    case = make_tree_case(B=2, V=V, cap=800, history_len=[800, 300], alphabet=6, dtype="f32", seed=41)
    rng = np.random.default_rng(42)
    lg = -1.0 - np.abs(case.logits.astype(np.float64))
    for b in range(case.B):
        pos = rng.choice(V, size=10, replace=False)
        lg[b, pos] = np.where(np.arange(10) % 2 == 0, -0.0, 0.0)
    case.logits = lg.astype(np.float32)
    if dtype == "bf16":
        case.logits = f32_to_bf16_bits(case.logits)
        case.dtype = "bf16"
    _check(case, 8, 2, 6, [4, 3, 2, 2, 1, 1, 1, 1], 64)
