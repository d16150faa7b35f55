"""GPU: hta_verify_attn captured in a HIP graph gives the eager result on every replay.

The benchmark times the attention layer as a graph replay, so the captured
launches must reproduce the eager ones bit for bit (the kernels are
deterministic for a fixed plan). The graph is replayed several times with
unrelated eager work and synchronisations in between; every replay is
compared with the eager output, and the eager output with the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, config_for, io_dtype, say, to_device
from speculative_decoding_verification_hybrid_amd import hta
from workloads import make_custom

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_graph_replay_matches_eager(dtype):
    w = make_custom(B=3, Hq=8, Hkv=2, D=128, Lcap=1100, T=21, prefix_len=[1100, 0, 333], dtype=dtype,
                    seed=77)
    w2 = make_custom(B=3, Hq=8, Hkv=2, D=128, Lcap=1100, T=21, prefix_len=[5, 700, 1099], dtype=dtype,
                     seed=78)
    dev, dev2 = to_device(w), to_device(w2)
    h = hta.hta_create(config_for(w))
    h2 = hta.hta_create(config_for(w2))
    try:
        out = torch.empty(w.B, w.Hq, w.T, w.D, dtype=io_dtype(w), device="cuda")
        lse = torch.empty(w.B, w.Hq, w.T, dtype=torch.float32, device="cuda")
        out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
        args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["k_tree"], dev["v_tree"], dev["parent"],
                dev["prefix_len"])
        args2 = (dev2["q"], dev2["k_cache"], dev2["v_cache"], dev2["k_tree"], dev2["v_tree"],
                 dev2["parent"], dev2["prefix_len"])
        say(f"graph {dtype}: eager")
        hta.hta_verify_attn(h, *args, out, lse)
        torch.cuda.synchronize()
        ref_o, ref_l = out.clone(), lse.clone()
        ro, rl = oracle.verify_attn(w)
        assert_close(w, ref_o.float().cpu().numpy().astype(np.float64), ref_l.cpu().numpy().astype(np.float64),
                     ro, rl)

        say(f"graph {dtype}: capture")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            hta.hta_verify_attn(h, *args, out, lse, torch.cuda.current_stream())
        for rep in range(4):
            out.fill_(float("nan"))
            lse.fill_(0.0)
            torch.cuda.synchronize()
            say(f"graph {dtype}: replay {rep}")
            g.replay()
            # unrelated eager work on another handle between replays
            hta.hta_verify_attn(h2, *args2, out2, lse2)
            _ = (out2.float() * 2).sum().item()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o), f"replay {rep}: out differs from eager"
            assert torch.equal(lse, ref_l), f"replay {rep}: lse differs from eager"
            assert hta.hta_get_status(h) == 0
        del g
    finally:
        hta.hta_destroy(h)
        hta.hta_destroy(h2)
