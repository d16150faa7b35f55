"""hta_verify_attn_noalloc (no handle, no allocation) against hta_verify_attn.

Both run the same plan and kernels, so the outputs must be identical bit for
bit; each is also held to the oracle's tolerance. Calls follow one another
on the one scratch array, each with a smaller input than the one before.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, config_for, io_dtype, run_verify, say, to_device
from speculative_decoding_verification_hybrid_amd import hta
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _noalloc(w, dev, **cfg_kw):
    out = torch.full((w.B, w.Hq, w.T, w.D), 7.0, dtype=io_dtype(w), device="cuda")
    lse = torch.full((w.B, w.Hq, w.T), 7.0, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    hta.hta_verify_attn_noalloc(config_for(w, **cfg_kw), dev["q"], dev["k_cache"], dev["v_cache"], dev["k_tree"],
                                dev["v_tree"], dev["parent"], dev["prefix_len"], out, lse, status)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            int(status.cpu().item()))


SEQUENCE = [
    # each call smaller than the one before; paths MFMA, MFMA, DOT, VALU (f32)
    ("mfma_32q8kv_t64", dict(B=2, Hq=32, Hkv=8, D=128, Lcap=4096, T=64, prefix_len=[4096, 3001], dtype="bf16")),
    ("mfma_gqa4_t16", dict(B=1, Hq=8, Hkv=2, D=128, Lcap=700, T=16, prefix_len=[650], dtype="bf16")),
    ("dot_m12", dict(B=1, Hq=4, Hkv=1, D=128, Lcap=300, T=3, prefix_len=[299], dtype="bf16")),
    ("valu_f32", dict(B=1, Hq=2, Hkv=1, D=64, Lcap=100, T=5, prefix_len=[77], dtype="f32")),
]


def test_noalloc_matches_handle_path_on_calls_in_a_row():
    for i, (name, kw) in enumerate(SEQUENCE):
        w = make_custom(seed=100 + i, **kw)
        dev = to_device(w)
        say(f"hta_verify_attn_noalloc {name}")
        out, lse, status = _noalloc(w, dev)
        assert status == 0
        say(f"hta_verify_attn {name}")
        ref = run_verify(w, dev=dev)
        assert ref[2] == 0
        assert np.array_equal(out, ref[0]) and np.array_equal(lse, ref[1]), name
        ro, rl = oracle.verify_attn(w)
        assert_close(w, out, lse, ro, rl)


def test_noalloc_second_call_smaller_reuses_scratch():
    big = make_custom(seed=7, B=4, Hq=16, Hkv=4, D=128, Lcap=2048, T=32, prefix_len=[2048, 1500, 1, 999],
                      dtype="bf16")
    small = make_custom(seed=8, B=1, Hq=16, Hkv=4, D=128, Lcap=2048, T=32, prefix_len=[700], dtype="bf16")
    for w in (big, small, big):
        dev = to_device(w)
        say(f"hta_verify_attn_noalloc B={w.B} L={list(w.prefix_len)}")
        out, lse, status = _noalloc(w, dev, num_workgroups=96)
        ref = run_verify(w, dev=dev, num_workgroups=96)
        assert status == 0 and ref[2] == 0
        assert np.array_equal(out, ref[0]) and np.array_equal(lse, ref[1])


def test_noalloc_reports_bad_tree_and_prefix_in_its_status():
    w = make_custom(seed=9, B=3, Hq=8, Hkv=2, D=128, Lcap=300, T=8, prefix_len=[300, 200, 100], dtype="bf16")
    w.parent[1, 3] = 5  # parent[i] must be < i
    dev = to_device(w)
    dev["prefix_len"][2] = 301  # beyond the capacity
    say("hta_verify_attn_noalloc bad tree + bad prefix")
    out, lse, status = _noalloc(w, dev)
    assert status == hta.HTA_STATUS_BAD_TREE | hta.HTA_STATUS_BAD_PREFIX
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all() and np.isfinite(out[0]).all()


def test_noalloc_rejects_shapes_beyond_its_scratch():
    w = make_custom(seed=10, B=1, Hq=8, Hkv=2, D=128, Lcap=64, T=64, prefix_len=[64], dtype="bf16")
    dev = to_device(w)
    big_cfg = dict(num_workgroups=4096)  # 4097 slots x 256 rows x 128 dims x 2 B > 32 MiB
    say("hta_verify_attn_noalloc beyond its scratch")
    with pytest.raises(hta.HtaError) as e:
        _noalloc(w, dev, **big_cfg)
    assert e.value.code == hta.HTA_ERR_TOO_LARGE


def test_noalloc_under_graph_capture():
    """Captured once, replayed with other no-allocation calls (sharing the scratch array) in between."""
    w = make_custom(seed=11, B=2, Hq=16, Hkv=4, D=128, Lcap=1500, T=16, prefix_len=[1500, 612], dtype="bf16")
    w2 = make_custom(seed=12, B=1, Hq=4, Hkv=1, D=128, Lcap=900, T=2, prefix_len=[900], dtype="bf16")  # DOT path
    dev, dev2 = to_device(w), to_device(w2)
    say("hta_verify_attn_noalloc graph: eager")
    ref_o, ref_l, st = _noalloc(w, dev)
    assert st == 0
    ref2_o, ref2_l, st2 = _noalloc(w2, dev2)
    assert st2 == 0
    cfg = config_for(w)
    out = torch.empty(w.B, w.Hq, w.T, w.D, dtype=io_dtype(w), device="cuda")
    lse = torch.empty(w.B, w.Hq, w.T, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["k_tree"], dev["v_tree"], dev["parent"], dev["prefix_len"])
    say("hta_verify_attn_noalloc graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hta.hta_verify_attn_noalloc(cfg, *args, out, lse, status, torch.cuda.current_stream())
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        say(f"hta_verify_attn_noalloc graph: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.float().cpu().numpy().astype(np.float64), ref_o)
        assert np.array_equal(lse.cpu().numpy().astype(np.float64), ref_l)
        o2, l2, s2 = _noalloc(w2, dev2)  # another shape through the same scratch array
        assert s2 == 0 and np.array_equal(o2, ref2_o) and np.array_equal(l2, ref2_l)
    assert int(status.item()) == 0
