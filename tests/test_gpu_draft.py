"""GPU parity of the small-row (DOT) split-KV kernel: the drafter's cross-attention
over the target's cache (hta_cross_attn) and verification of very small trees.

The oracle is ``oracle.cross_attn`` / ``oracle.verify_attn`` on the exact input
values; tolerances as for the other kernels (bf16: max-abs 2e-2 on outputs,
1e-3 relative on the LSE).
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, config_for, io_dtype, run_verify, say, to_device
from speculative_decoding_verification_hybrid_amd import hta
from workloads import make_custom, tree_chain

pytestmark = pytest.mark.gpu


def run_cross(w, **cfg_kw):
    dev = to_device(w)
    with hta.hta_create(config_for(w, **cfg_kw)) as h:
        plan = hta.hta_get_plan(h)
        out = torch.full((w.B, w.Hq, w.T, w.D), 7.0, dtype=io_dtype(w), device="cuda")
        lse = torch.full((w.B, w.Hq, w.T), 7.0, dtype=torch.float32, device="cuda")
        hta.hta_cross_attn(h, dev["q"], dev["k_cache"], dev["v_cache"], dev["prefix_len"], out, lse)
        status = hta.hta_get_status(h)
        torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), status, plan


CROSS = {
    # name: make_custom kwargs; T = draft query tokens per sequence, M = (Hq/Hkv)*T rows per KV head
    "llama8b_t1_4k": dict(B=1, Hq=32, Hkv=8, D=128, Lcap=4096, T=1, prefix_len=[4096]),       # M = 4
    "mha_t1": dict(B=2, Hq=8, Hkv=8, D=128, Lcap=1000, T=1, prefix_len=[1000, 333]),          # M = 1
    "m2": dict(B=1, Hq=4, Hkv=2, D=128, Lcap=500, T=1, prefix_len=[433]),                     # M = 2
    "m3_ragged": dict(B=6, Hq=6, Hkv=2, D=128, Lcap=1000, T=1, prefix_len=[1, 63, 64, 65, 1000, 0]),
    "qwq_gqa5_t1": dict(B=4, Hq=40, Hkv=8, D=128, Lcap=2000, T=1, prefix_len=[2000, 1, 64, 1500]),  # M = 5
    "gqa4_t2_m8": dict(B=2, Hq=16, Hkv=4, D=128, Lcap=900, T=2, prefix_len=[900, 65]),        # M = 8
    "gqa4_t3_m12": dict(B=2, Hq=16, Hkv=4, D=128, Lcap=1200, T=3, prefix_len=[1200, 97]),     # M = 12: 2 groups
    "gqa5_t3_m15": dict(B=1, Hq=40, Hkv=8, D=128, Lcap=700, T=3, prefix_len=[700]),          # M = 15
    "mha_t9_ragged": dict(B=3, Hq=2, Hkv=2, D=128, Lcap=300, T=9, prefix_len=[300, 1, 65]),  # M = 9
    "d64_m4_gqa4": dict(B=2, Hq=16, Hkv=4, D=64, Lcap=1500, T=1, prefix_len=[1500, 333]),      # D = 64
    "d64_m1_mha_ragged": dict(B=4, Hq=4, Hkv=4, D=64, Lcap=300, T=1, prefix_len=[1, 63, 64, 300]),
    "d64_m8_t2": dict(B=1, Hq=8, Hkv=2, D=64, Lcap=900, T=2, prefix_len=[899]),
    "d64_m12_t3": dict(B=2, Hq=16, Hkv=4, D=64, Lcap=700, T=3, prefix_len=[700, 65]),          # two row groups
    "d64_poison_tail": dict(B=2, Hq=8, Hkv=2, D=64, Lcap=400, T=1, prefix_len=[97, 1], poison_tail=True),
    "poison_tail": dict(B=3, Hq=8, Hkv=2, D=128, Lcap=500, T=1, prefix_len=[77, 500, 1], poison_tail=True),
    "unit_tails": dict(B=5, Hq=8, Hkv=2, D=128, Lcap=200, T=1, prefix_len=[31, 32, 33, 95, 97]),
    "drift_keys": dict(B=1, Hq=32, Hkv=8, D=128, Lcap=5000, T=1, prefix_len=[5000], drift=True),
}


@pytest.mark.parametrize("name", sorted(CROSS))
def test_cross_attn_parity(name):
    w = make_custom(seed=zlib.crc32(name.encode()) % 1000, dtype="bf16", **CROSS[name])
    say(f"hta_cross_attn {name}")
    out, lse, status, plan = run_cross(w)
    assert plan["path"] == hta.HTA_PATH_DOT
    assert status == 0
    ref_out, ref_lse = oracle.cross_attn(w.as_f64("q"), w.as_f64("k_cache"), w.as_f64("v_cache"), w.prefix_len,
                                         w.scale)
    empty = w.prefix_len == 0
    assert np.all(np.isneginf(lse[empty])) and np.all(out[empty] == 0)
    eo, el = assert_close(w, out, lse, ref_out, ref_lse, sel=~empty[:, None, None] & np.ones(lse.shape, bool))
    say(f"hta_cross_attn {name}: out err {eo:.2e}, lse rel err {el:.2e}")


def test_cross_attn_full_size_llama8b_32k():
    """The benchmarked shape: one draft token per step, 32 q / 8 kv heads, 32k-token cache."""
    w = make_custom(B=1, Hq=32, Hkv=8, D=128, Lcap=32768, T=1, prefix_len=[32768], dtype="bf16", seed=77)
    say("hta_cross_attn llama8b 32k")
    out, lse, status, plan = run_cross(w)
    assert plan["path"] == hta.HTA_PATH_DOT and status == 0
    ref_out, ref_lse = oracle.cross_attn(w.as_f64("q"), w.as_f64("k_cache"), w.as_f64("v_cache"), w.prefix_len,
                                         w.scale)
    assert_close(w, out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("nwg", [1, 5, 64, 999])
def test_cross_attn_any_split(nwg):
    w = make_custom(B=3, Hq=16, Hkv=4, D=128, Lcap=1200, T=1, prefix_len=[1200, 5, 640], dtype="bf16", seed=nwg)
    say(f"hta_cross_attn num_workgroups={nwg}")
    out, lse, status, _ = run_cross(w, num_workgroups=nwg)
    assert status == 0
    ref_out, ref_lse = oracle.cross_attn(w.as_f64("q"), w.as_f64("k_cache"), w.as_f64("v_cache"), w.prefix_len,
                                         w.scale)
    assert_close(w, out, lse, ref_out, ref_lse)


def test_cross_attn_matches_prefix_attn_of_other_paths():
    """Same inputs through the VALU path's hta_prefix_attn: the two kernels agree."""
    w = make_custom(B=2, Hq=8, Hkv=2, D=128, Lcap=700, T=1, prefix_len=[700, 200], dtype="bf16", seed=4)
    say("hta_cross_attn vs forced VALU hta_prefix_attn")
    out, lse, _, _ = run_cross(w)
    dev = to_device(w)
    with hta.hta_create(config_for(w, force_path=hta.HTA_PATH_VALU)) as h:
        o2 = torch.empty(w.B, w.Hq, w.T, w.D, dtype=torch.float32, device="cuda")
        l2 = torch.empty(w.B, w.Hq, w.T, dtype=torch.float32, device="cuda")
        hta.hta_prefix_attn(h, dev["q"], dev["k_cache"], dev["v_cache"], dev["prefix_len"], o2, l2)
        torch.cuda.synchronize()
    assert np.abs(out - o2.cpu().numpy()).max() <= 2e-2
    assert np.abs(lse - l2.cpu().numpy()).max() <= 1e-3 * max(1.0, np.abs(lse).max())


SMALL_TREES = {
    "t1_gqa4": dict(B=2, Hq=8, Hkv=2, D=128, Lcap=600, T=1, prefix_len=[600, 3]),
    "t2_gqa4": dict(B=2, Hq=32, Hkv=8, D=128, Lcap=900, T=2, prefix_len=[900, 1]),
    "t8_mha": dict(B=2, Hq=4, Hkv=4, D=128, Lcap=500, T=8, prefix_len=[500, 0]),
    "t5_chain_mha": dict(B=1, Hq=2, Hkv=2, D=128, Lcap=300, T=5, prefix_len=[257], parents=[tree_chain(5)]),
    "t4_gqa2_forest": dict(B=1, Hq=4, Hkv=2, D=128, Lcap=128, T=4, prefix_len=[128], parents=[[-1, 0, -1, 2]]),
    "t9_mha": dict(B=2, Hq=2, Hkv=2, D=128, Lcap=700, T=9, prefix_len=[700, 65]),
    "d64_t6_mha_forest": dict(B=2, Hq=2, Hkv=2, D=64, Lcap=500, T=6, prefix_len=[500, 70],
                              parents=[[-1, 0, 1, -1, 3, 0], [-1, 0, 0, 1, 2, 4]]),
    "d64_t3_gqa4_m12": dict(B=1, Hq=8, Hkv=2, D=64, Lcap=1000, T=3, prefix_len=[999]),
    "d64_t1_gqa4": dict(B=3, Hq=8, Hkv=2, D=64, Lcap=256, T=1, prefix_len=[256, 0, 17]),
    "t3_gqa4_m12": dict(B=2, Hq=8, Hkv=2, D=128, Lcap=1000, T=3, prefix_len=[1000, 64]),
    "t5_gqa3_m15_chain": dict(B=1, Hq=6, Hkv=2, D=128, Lcap=400, T=5, prefix_len=[399], parents=[tree_chain(5)]),
    "t7_gqa2_m14_forest": dict(B=1, Hq=4, Hkv=2, D=128, Lcap=256, T=7, prefix_len=[130],
                               parents=[[-1, 0, -1, 2, 1, 3, -1]]),
}


@pytest.mark.parametrize("name", sorted(SMALL_TREES))
def test_small_tree_verify_on_dot_path(name):
    w = make_custom(seed=zlib.crc32(name.encode()) % 1000, dtype="bf16", **SMALL_TREES[name])
    say(f"hta_verify_attn on the DOT path: {name}")
    with hta.hta_create(config_for(w)) as h:
        assert hta.hta_get_plan(h)["path"] == hta.HTA_PATH_DOT
        out, lse, status = run_verify(w, handle=h)
    assert status == 0
    ref_out, ref_lse = oracle.verify_attn(w)
    assert_close(w, out, lse, ref_out, ref_lse)


def test_small_tree_bad_parent_on_dot_path():
    w = make_custom(B=3, Hq=8, Hkv=2, D=128, Lcap=300, T=2, prefix_len=[300, 200, 100], dtype="bf16", seed=9)
    w.parent[1, 1] = 1  # parent[i] must be < i
    say("hta_verify_attn DOT path, bad tree")
    out, lse, status = run_verify(w)
    assert status == hta.HTA_STATUS_BAD_TREE
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    ref_out, ref_lse = oracle.verify_attn(w, batches=[0, 2])
    assert_close(w, out, lse, ref_out, ref_lse)
