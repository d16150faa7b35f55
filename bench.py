"""Benchmark: tree-verification attention at the Llama-3.1-8B layer shape.

One step = one hta_verify_attn call (split-KV kernel with the tree part fused
in, then the LSE merge) over one batch of synthetic inputs: 32 query / 8 KV
heads, head_dim 128, a 32768-token bf16 KV prefix and a 64-node draft tree.
Inputs are resident in HBM before the timed region; the KV cache is rotated
over enough replicas (>= 512 MB) that the 256 MB Infinity Cache cannot hold
the next step's KV, so every step streams its KV from HBM.

The K timed steps are captured once into a HIP graph and replayed once
between two events on the replay stream, so the figure is GPU time, not the
cost of launching from Python. The warm-up is W eager steps plus one untimed
replay of the graph. The graph's outputs are checked bit for bit against an
eager step on the same inputs.

Prints one JSON line. ``value`` is the layer's achieved HBM bandwidth on its
algorithmic bytes (valid KV read once + q, tree K/V, out, lse, tree shape);
beside it: the per-layer latency, verified tokens/s, the split-KV kernel's
roofline (its K launches captured and timed the same way, alone; against the
HBM peak, and in "mfma" against the bf16 matrix-core peak with the busy
fractions of a committed rocprofv3 counter pass) and the fp64 CPU oracle's
throughput on a bounded sample of the same workload. A second
leg ("accept_commit") times hta_accept + hta_commit on the same draft tree
with bf16 target logits over a 128256-token vocabulary, the same way, with
the oracle's accept + commit on the same inputs beside it. A third leg
("draft_cross_attn") times the drafter's cross-attention over the same 32k
cache with one draft token (hta_cross_attn, the small-row DOT kernel), and a
fourth ("tree_build") the construction of the next draft tree from the last
logits and a 32k-token history (hta_build_tree; its "indexed" object times
hta_build_tree_indexed in a decoding loop that adds 3 tokens per call). "configs" reports the layer
at all five configurations (p10/p50/p90 over graph replays, each against the
HBM peak and against a measured device copy, with one oracle run each), and
"copy_bw_gbs" that copy's bandwidth.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --copy-calibration   (adds 8 launches of a plain elementwise
           kernel that reads 256 MiB and writes 256 MiB before the timed region:
           the reference dispatches that HBM byte counters are scaled by)
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("verify-attn layer µs + achieved HBM GB/s (% peak), 8B GQA shape, 32k ctx, "
          "64-node tree")
PEAK_HBM_GBS = 8000.0
WORKLOAD_KEY = 3
CSRC = os.path.join(ROOT, "speculative_decoding_verification_hybrid_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefix_mfma_llama8b_32k_traffic.txt")
PREFIX_SRC = os.path.join(CSRC, "prefix_mfma.hip")
ACCEPT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "argmax_accept_llama8b_vocab128k_traffic.txt")
ACCEPT_SRC = os.path.join(CSRC, "accept.hip")
DOT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefix_dot_llama8b_draft_32k_traffic.txt")
DOT_SRC = os.path.join(CSRC, "prefix_dot.hip")
MFMA_COUNTERS_FILE = os.path.join(ROOT, "profiles", "prefix_mfma_llama8b_32k_mfma_lds_counters.txt")
PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replica-bytes", type=float, default=512e6,
                    help="total KV bytes to rotate over (cold-cache protocol)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum wall time of the CPU oracle baseline")
    ap.add_argument("--no-accept", action="store_true", help="skip the accept + commit leg")
    ap.add_argument("--no-draft", action="store_true", help="skip the draft cross-attention leg")
    ap.add_argument("--no-tree", action="store_true", help="skip the tree-construction leg")
    ap.add_argument("--no-configs", action="store_true", help="skip the five-configuration sweep")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run 8 copy-like 256 MiB elementwise kernels before timing")
    return ap.parse_args()


def algorithmic_bytes(w):
    s = 2 if w.dtype == "bf16" else 4
    kv = 2 * w.Hkv * w.D * int(w.prefix_len.sum()) * s
    tree_kv = 2 * w.B * w.Hkv * w.T * w.D * s
    q_out = 2 * w.B * w.Hq * w.T * w.D * s
    lse = w.B * w.Hq * w.T * 4
    meta = w.B * w.T * 4 + w.B * 4
    return kv, kv + tree_kv + q_out + lse + meta


def source_hash(src):
    """sha256 (first 16 hex) of a kernel source and the repository headers it includes, in
    include order, so a change to any of them marks counter summaries taken before as stale."""
    h, seen = hashlib.sha256(), set()

    def add(path):
        if path in seen or not os.path.exists(path):
            return
        seen.add(path)
        text = open(path, "rb").read()
        h.update(text)
        for ln in text.decode("utf-8", "replace").splitlines():
            ln = ln.strip()
            if ln.startswith('#include "'):
                add(os.path.join(os.path.dirname(path), ln.split('"')[1]))

    add(src)
    return h.hexdigest()[:16]


def traffic_from_profile(path=TRAFFIC_FILE, src=PREFIX_SRC, key="hbm_bytes_per_launch"):
    """HBM bytes per launch of a kernel from a committed rocprofv3 counter summary, if
    it was taken on the current kernel source and headers; else None."""
    if not os.path.exists(path):
        return None
    fields = {}
    for ln in open(path):
        if "=" in ln and not ln.startswith("#"):
            k, v = ln.split("=", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != source_hash(src):
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, min_seconds):
    """The fp64 oracle on the same workload, repeated until min_seconds of wall time."""
    import oracle
    cores = _cores()
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.verify_attn(w)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    _, total = algorithmic_bytes(w)
    gbs = total * reps / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"the whole workload (all {w.Hq} query heads, {w.T} tree nodes, "
                      f"{int(w.prefix_len[0])}-token prefix) {reps} times, {dt:.2f} s wall, "
                      f"{dt / reps * 1e3:.1f} ms per layer"}


VOCAB = 128256  # Llama-3.1-8B vocabulary


def accept_commit_row(w, steps, warmup, replica_bytes, cpu_seconds):
    """hta_accept + hta_commit on the same draft tree with bf16 target logits over a
    Llama-3.1-8B vocabulary: [B, T, V] logits rotated over >= replica_bytes of copies
    (cold in the Infinity Cache), a fresh prefix_len per step so every step commits
    at the same place, and a cache with room behind the prefix for two replays of the
    graph of steps (each step's prefix_len advances once per replay)."""
    import torch
    from speculative_decoding_verification_hybrid_amd import hta
    from workloads import make_accept_case

    case = make_accept_case(B=w.B, T=w.T, V=VOCAB, dtype="bf16", seed=1234, parents=w.parent,
                            depth=[5] * w.B)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    lg0 = torch.from_numpy(case.logits.view(np.int16)).view(torch.bfloat16).cuda()
    logit_bytes = lg0.numel() * 2
    R = max(1, int(np.ceil(replica_bytes / logit_bytes)))
    lgs = [lg0] + [lg0.clone() for _ in range(R - 1)]
    parent, tokens = i32(case.parent), i32(case.tree_tokens)
    Lcap = int(w.prefix_len.max()) + 2 * w.T  # the graph of steps replays twice (upload, timed)
    kc = torch.zeros(w.B, w.Hkv, Lcap, w.D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    kt, vt = bits(w.k_tree), bits(w.v_tree)
    target = torch.empty(w.B, w.T, dtype=torch.int32, device="cuda")
    n = torch.empty(w.B, dtype=torch.int32, device="cuda")
    path = torch.empty(w.B, w.T, dtype=torch.int32, device="cuda")
    bonus = torch.empty(w.B, dtype=torch.int32, device="cuda")
    plen0 = i32(w.prefix_len)
    plens = [plen0.clone() for _ in range(warmup + steps)]
    cfg = hta.make_config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, tree_nodes=w.T,
                          kv_capacity=Lcap, dtype="bf16", softmax_scale=w.scale)
    h = hta.hta_create(cfg)

    def accept(i, s):
        hta.hta_accept(h, lgs[i % R], parent, tokens, target, n, path, bonus, s)

    def accept_commit(i, s):
        accept(i, s)
        hta.hta_commit(h, kt, vt, n, path, kc, vc, plens[i], s)

    def timed(fn):
        s = torch.cuda.current_stream()
        for i in range(warmup):
            fn(i, s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(warmup + i, torch.cuda.current_stream())
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s = torch.cuda.current_stream()
        e0.record(s)
        g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    both_ms = timed(accept_commit)
    status = hta.hta_get_status(h)
    got = [t.cpu().numpy() for t in (target, n, path, bonus)]
    last_len = plens[warmup + steps - 1].cpu().numpy()
    acc_ms = timed(accept)
    hta.hta_destroy(h)
    acc_n = int(got[1].sum())
    accept_bytes = logit_bytes + w.B * w.T * 4 * 4 + w.B * 4 * 2  # logits, parent/tokens/target/path, len/bonus
    commit_bytes = 2 * 2 * acc_n * w.Hkv * w.D * 2 + w.B * 4 * 3  # K and V rows read + written, lengths
    gbs = accept_bytes / (acc_ms * 1e-3) / 1e9
    ok = status == 0 and np.array_equal(last_len, w.prefix_len + 2 * got[1]) and bool((got[1] >= 1).all())
    row = {
        "workload": f"accept+commit over {w.B}x{w.T} tree nodes, bf16 logits V={VOCAB}",
        "us_per_step": round(both_ms * 1e3, 3),
        "accept_us": round(acc_ms * 1e3, 3),
        "accepted_tokens": acc_n,
        "logit_replicas": R,
        "status_ok_lengths_advanced": ok,
        "roofline": {
            "kernel": "argmax_kernel + accept_kernel (hta_accept)",
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic_from_profile(ACCEPT_TRAFFIC_FILE, ACCEPT_SRC),
            "avg_launch_us": round(acc_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": accept_bytes,
            "commit_bytes_per_launch": commit_bytes,
        },
    }
    if cpu_seconds > 0:
        row["cpu_baseline"] = accept_cpu_baseline(case, w, cpu_seconds, accept_bytes)
    del lgs
    torch.cuda.synchronize()
    return row


def draft_cross_row(w, steps, warmup, replica_bytes, cpu_seconds):
    """The drafter's cross-attention over the target's cache (hta_cross_attn): one draft
    token per sequence (T = 1) at the same Llama-3.1-8B layer shape and 32k cache, the
    cache rotated over >= replica_bytes of copies; the split-KV (DOT) kernel alone is
    timed the same way for its roofline."""
    import torch
    from speculative_decoding_verification_hybrid_amd import hta
    from workloads import make_custom

    L = int(w.prefix_len[0])
    d = make_custom(B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, Lcap=w.Lcap, T=1, prefix_len=list(w.prefix_len),
                    dtype="bf16", seed=4321)
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    q, plen = bits(d.q), torch.from_numpy(d.prefix_len).cuda()
    kv_bytes = 2 * d.Hkv * d.D * int(d.prefix_len.sum()) * 2
    R = max(1, int(np.ceil(replica_bytes / kv_bytes)))
    kc0, vc0 = bits(d.k_cache), bits(d.v_cache)
    kcs = [kc0] + [kc0.clone() for _ in range(R - 1)]
    vcs = [vc0] + [vc0.clone() for _ in range(R - 1)]
    out = torch.empty(d.B, d.Hq, 1, d.D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(d.B, d.Hq, 1, dtype=torch.float32, device="cuda")
    h = hta.hta_create(hta.make_config(batch=d.B, n_q_heads=d.Hq, n_kv_heads=d.Hkv, head_dim=d.D, tree_nodes=1,
                                       kv_capacity=d.Lcap, dtype="bf16", softmax_scale=d.scale))
    plan = hta.hta_get_plan(h)

    def timed(fn):
        s = torch.cuda.current_stream()
        for i in range(warmup):
            fn(i, s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(warmup + i, torch.cuda.current_stream())
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s = torch.cuda.current_stream()
        e0.record(s)
        g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    hta.hta_cross_attn(h, q, kc0, vc0, plen, out, lse)
    torch.cuda.synchronize()
    out_eager, lse_eager = out.clone(), lse.clone()
    ms = timed(lambda i, s: hta.hta_cross_attn(h, q, kcs[i % R], vcs[i % R], plen, out, lse, s))
    same = bool(torch.equal(out, out_eager)) and bool(torch.equal(lse, lse_eager))
    pms = timed(lambda i, s: hta.hta_prefix_partials(h, q, kcs[i % R], vcs[i % R], plen, s))
    status = hta.hta_get_status(h)
    hta.hta_destroy(h)
    # the drafter's own self-attention: a 512-slot ring (sliding window) plus the new token
    from workloads import make_window_case
    wc = make_window_case(B=d.B, Hq=d.Hq, Hkv=d.Hkv, D=d.D, W=512, Tn=1, pos=[L] * d.B, dtype="bf16", seed=99)
    wt = {n: bits(getattr(wc, n)) for n in ("q", "k_ring", "v_ring", "k_new", "v_new")}
    wpos = torch.from_numpy(wc.pos).cuda()
    hw = hta.hta_create(hta.make_config(batch=d.B, n_q_heads=d.Hq, n_kv_heads=d.Hkv, head_dim=d.D, tree_nodes=1,
                                        kv_capacity=512, dtype="bf16", softmax_scale=d.scale))
    wms = timed(lambda i, s: hta.hta_window_attn(hw, wt["q"], wt["k_ring"], wt["v_ring"], wt["k_new"], wt["v_new"],
                                                 wpos, out, lse, s))
    ams = timed(lambda i, s: hta.hta_window_append(hw, wt["k_new"], wt["v_new"], wt["k_ring"], wt["v_ring"],
                                                   wpos, s))
    status |= hta.hta_get_status(hw)
    hta.hta_destroy(hw)
    gbs = kv_bytes / (pms * 1e-3) / 1e9
    row = {
        "workload": f"draft cross-attention, {d.Hq} q / {d.Hkv} kv heads, D {d.D}, 1 draft token, {L}-token cache",
        "us_per_call": round(ms * 1e3, 3),
        "tokens_per_s": round(d.B / (ms * 1e-3), 1),
        "window_attn_us": round(wms * 1e3, 3),
        "window_append_us": round(ams * 1e3, 3),
        "window": "512-slot ring, 1 new token (hta_window_attn, hta_window_append)",
        "path": plan["path"],
        "num_workgroups": plan["num_workgroups"],
        "kv_replicas": R,
        "outputs_match_eager_status_ok": same and status == 0,
        "roofline": {
            "kernel": "prefix_dot_kernel<4> (split-KV, v_dot2; hta_prefix_partials)",
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic_from_profile(DOT_TRAFFIC_FILE, DOT_SRC),
            "avg_launch_us": round(pms * 1e3, 3),
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }
    if cpu_seconds > 0:
        import oracle
        args = [d.as_f64(n) for n in ("q", "k_cache", "v_cache")]
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.cross_attn(*args, d.prefix_len, d.scale)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= cpu_seconds:
                break
        row["cpu_baseline"] = {"value": round(kv_bytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": _cores(),
                               "kind": "oracle", "us_per_call": round(dt / reps * 1e6, 1),
                               "sample": f"the whole call (all {d.Hq} heads, {L}-token cache) {reps} times, "
                                         f"{dt:.2f} s wall"}
    del kcs, vcs
    torch.cuda.synchronize()
    return row


TREE_KEEP = [8, 6, 5, 4, 4, 3, 3, 2, 2, 2, 1, 1, 1, 1, 1]  # tokens kept per guess rank (non-increasing)


def tree_indexed_leg(h, case, lg, hist, params, m, steps, warmup):
    """hta_build_tree_indexed in a decoding loop: each call finds 3 more history
    tokens than the last (the accepted ones), adds their grams to the index and
    answers the queries from it. Before every timed graph replay the index is
    reset and brought to the length just below the first call's (untimed), so
    every replayed call inserts exactly 3 positions."""
    import torch
    from speculative_decoding_verification_hybrid_amd import hta

    B, cap = case.history.shape
    T = int(h.dims[4])
    add = 3
    L0 = cap - add * steps
    lens = [torch.tensor([L0 + add * i], dtype=torch.int32, device="cuda") for i in range(steps)]
    pre = torch.tensor([L0 - add], dtype=torch.int32, device="cuda")
    tok = torch.empty(1, T, dtype=torch.int32, device="cuda")
    par = torch.empty(1, T, dtype=torch.int32, device="cuda")
    nn = torch.empty(1, dtype=torch.int32, device="cuda")
    idx = hta.hta_ngram_index_create(B, cap, m)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def prime():
        hta.hta_ngram_index_reset(idx, -1, s)
        e0.record(s)
        hta.hta_build_tree_indexed(h, idx, lg, hist, pre, params, tok, par, nn, s)
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    for _ in range(max(1, warmup)):
        build_us = prime()
        for i in range(steps):
            hta.hta_build_tree_indexed(h, idx, lg, hist, lens[i], params, tok, par, nn, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream()
        for i in range(steps):
            hta.hta_build_tree_indexed(h, idx, lg, hist, lens[i], params, tok, par, nn, cs)
    build_us = prime()
    g.replay()
    prime()
    e0.record(s)
    g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    hta.hta_ngram_index_destroy(idx)
    return {"us_per_call": round(ms * 1e3, 3), "new_tokens_per_call": add,
            "history_len": f"{L0}..{L0 + add * (steps - 1)}", "n_nodes_last": int(nn.item()),
            "index_first_build_us": round(build_us, 1),
            "index_first_build": f"{L0 - add} positions into an empty index (one call)"}


def tree_build_row(w, steps, warmup, cpu_seconds):
    """hta_build_tree for one sequence: the last logits over the Llama-3.1-8B vocabulary
    (bf16), a 32k-token history, 15 next-next guesses, 3-grams, a 64-node tree. The
    inputs are a few hundred KB, so they stay in the caches: the figure is the call's
    latency, not a stream."""
    import torch
    from speculative_decoding_verification_hybrid_amd import hta
    from workloads import make_tree_case

    cap = int(w.prefix_len[0])
    case = make_tree_case(B=1, V=VOCAB, cap=cap, history_len=[cap], alphabet=40, seed=7)
    lg = torch.from_numpy(case.logits.view(np.int16)).view(torch.bfloat16).cuda()
    hist = torch.from_numpy(case.history).cuda()
    hl = torch.from_numpy(case.history_len).cuda()
    tok = torch.empty(1, w.T, dtype=torch.int32, device="cuda")
    par = torch.empty(1, w.T, dtype=torch.int32, device="cuda")
    nn = torch.empty(1, dtype=torch.int32, device="cuda")
    k, m, kf = len(TREE_KEEP), 3, 8
    params = hta.make_tree_params(k, m, kf, TREE_KEEP)
    h = hta.hta_create(hta.make_config(batch=1, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, tree_nodes=w.T,
                                       kv_capacity=w.Lcap))
    s = torch.cuda.current_stream()
    for _ in range(warmup):
        hta.hta_build_tree(h, lg, hist, hl, params, tok, par, nn, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            hta.hta_build_tree(h, lg, hist, hl, params, tok, par, nn, torch.cuda.current_stream())
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s = torch.cuda.current_stream()
    e0.record(s)
    g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    status = hta.hta_get_status(h)
    n_scan = int(nn.item())
    indexed = tree_indexed_leg(h, case, lg, hist, params, m, steps, warmup)
    status_ix = hta.hta_get_status(h)
    hta.hta_destroy(h)
    nbytes = VOCAB * 2 + cap * 4 + w.T * 8 + 4
    row = {
        "workload": f"tree construction: bf16 logits V={VOCAB}, {cap}-token history, k={k} guesses, {m}-grams, "
                    f"{w.T}-node tree",
        "us_per_call": round(ms * 1e3, 3),
        "n_nodes": n_scan,
        "status_ok": status == 0 and status_ix == 0,
        "bytes_per_call": nbytes,
        "achieved_gbs": round(nbytes / (ms * 1e-3) / 1e9, 2),
        "indexed": indexed,
    }
    if cpu_seconds > 0:
        import oracle
        lf = case.logits_f64()
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.build_trees(case.history, case.history_len, lf, k, m, kf, TREE_KEEP, w.T)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= cpu_seconds:
                break
        row["cpu_baseline"] = {"value": round(dt / reps * 1e6, 1), "unit": "µs per call", "cores": 1,
                               "kind": "oracle",
                               "sample": f"the same call {reps} times, {dt:.2f} s wall (pure Python search)"}
    return row


def copy_bandwidth():
    """Device-to-device copy of 512 MiB (read + write bytes / time): the measured
    bandwidth the layer figures are also compared with."""
    import torch
    n = 256 << 20  # int16 elements = 512 MiB
    src = torch.ones(n, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 2 / (ms * 1e-3) / 1e9


def all_configs_row(copy_gbs, cpu):
    """hta_verify_attn at each of the five layer configurations: KV rotated over
    >= 512 MB of replicas, 10 graph replays of 20 calls each; p10/p50/p90 of the
    per-call time over the replays. With cpu, one oracle run per configuration."""
    import torch
    from speculative_decoding_verification_hybrid_amd import hta
    from workloads import CONFIGS, make_workload

    rows = {}
    for key in sorted(CONFIGS):
        w = make_workload(key)
        kv_bytes, total_bytes = algorithmic_bytes(w)
        if w.dtype == "bf16":
            dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
            odt = torch.bfloat16
        else:
            dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
            odt = torch.float32
        R = max(1, int(np.ceil(512e6 / kv_bytes)))
        kc0, vc0 = dev(w.k_cache), dev(w.v_cache)
        kcs = [kc0] + [kc0.clone() for _ in range(R - 1)]
        vcs = [vc0] + [vc0.clone() for _ in range(R - 1)]
        q, kt, vt = dev(w.q), dev(w.k_tree), dev(w.v_tree)
        parent, plen = torch.from_numpy(w.parent).cuda(), torch.from_numpy(w.prefix_len).cuda()
        out = torch.empty(w.B, w.Hq, w.T, w.D, dtype=odt, device="cuda")
        lse = torch.empty(w.B, w.Hq, w.T, dtype=torch.float32, device="cuda")
        h = hta.hta_create(hta.make_config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D,
                                           tree_nodes=w.T, kv_capacity=w.Lcap, dtype=w.dtype,
                                           softmax_scale=w.scale))
        path = hta.hta_get_plan(h)["path"]
        n_call = 20
        for i in range(5):
            hta.hta_verify_attn(h, q, kcs[i % R], vcs[i % R], kt, vt, parent, plen, out, lse)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_call):
                hta.hta_verify_attn(h, q, kcs[i % R], vcs[i % R], kt, vt, parent, plen, out, lse,
                                    torch.cuda.current_stream())
        g.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / n_call * 1e3)
        status = hta.hta_get_status(h)
        hta.hta_destroy(h)
        del g, kcs, vcs
        torch.cuda.empty_cache()
        p10, p50, p90 = (float(np.percentile(per, x)) for x in (10, 50, 90))
        gbs = total_bytes / (p50 * 1e-6) / 1e9
        row = {"workload": CONFIGS[key].name, "path": path, "kv_replicas": R,
               "layer_us_p10_p50_p90": [round(p10, 3), round(p50, 3), round(p90, 3)],
               "gbs": round(gbs, 1), "pct_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
               "pct_copy_bw": round(100 * gbs / copy_gbs, 2),
               "tokens_per_s_verified": round(w.B * w.T / (p50 * 1e-6), 1), "status_ok": status == 0}
        if cpu:
            import oracle
            t0 = time.perf_counter()
            oracle.verify_attn(w)
            row["oracle_s"] = round(time.perf_counter() - t0, 3)
        rows[str(key)] = row
    return rows


def accept_cpu_baseline(case, w, min_seconds, accept_bytes):
    """The oracle's accept + commit on the same logits and tree; the commit writes into a
    cache of room T behind a T-row prefix (its cost does not depend on the prefix)."""
    import oracle
    logits = case.logits_f64()
    kc = np.zeros((w.B, w.Hkv, 2 * w.T, w.D), dtype=np.uint16)
    vc = np.zeros_like(kc)
    L = np.full(w.B, w.T, dtype=np.int64)
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref = oracle.accept(case.parent, case.tree_tokens, logits)
        oracle.commit(kc, vc, L, w.k_tree, w.v_tree, ref["accept_len"], ref["path"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(dt / reps * 1e6, 1), "unit": "µs per step", "cores": _cores(), "kind": "oracle",
            "gbs_on_accept_bytes": round(accept_bytes * reps / dt / 1e9, 4),
            "sample": f"accept over the same {w.B}x{w.T}x{VOCAB} fp64 logits + commit of its rows, "
                      f"{reps} times, {dt:.2f} s wall"}


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] + [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the split-KV path "
              "shards across GPUs by KV head or context, which this build does not launch.")
        sys.exit(2)

    import torch
    from speculative_decoding_verification_hybrid_amd import hta
    from workloads import CONFIGS, make_workload

    c = CONFIGS[WORKLOAD_KEY]
    w = make_workload(WORKLOAD_KEY)
    kv_bytes, total_bytes = algorithmic_bytes(w)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    q, kt, vt = dev(w.q), dev(w.k_tree), dev(w.v_tree)
    parent = torch.from_numpy(w.parent).cuda()
    plen = torch.from_numpy(w.prefix_len).cuda()
    kc0, vc0 = dev(w.k_cache), dev(w.v_cache)
    R = max(1, int(np.ceil(args.replica_bytes / kv_bytes)))
    kcs = [kc0] + [kc0.clone() for _ in range(R - 1)]
    vcs = [vc0] + [vc0.clone() for _ in range(R - 1)]
    out = torch.empty(w.B, w.Hq, w.T, w.D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.B, w.Hq, w.T, dtype=torch.float32, device="cuda")
    cfg = hta.make_config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, tree_nodes=w.T,
                          kv_capacity=w.Lcap, dtype="bf16", softmax_scale=w.scale)
    h = hta.hta_create(cfg)
    plan = hta.hta_get_plan(h)

    def step(i, s):
        hta.hta_verify_attn(h, q, kcs[i % R], vcs[i % R], kt, vt, parent, plen, out, lse, s)

    def prefix_only(i, s):
        hta.hta_prefix_partials(h, q, kcs[i % R], vcs[i % R], plen, s)

    def timed(fn, steps, warmup):
        """Average GPU time of one fn step: `steps` steps captured in one graph,
        replayed once between two events on the stream the graph runs on."""
        s = torch.cuda.current_stream()
        for i in range(warmup):
            fn(i, s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream()
            for i in range(steps):
                fn(warmup + i, cs)
        g.replay()  # untimed: uploads the graph
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s = torch.cuda.current_stream()
        e0.record(s)
        g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, g

    if args.copy_calibration:
        src = torch.empty(128 << 20, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(8):
            torch.bitwise_not(src, out=dst)  # one elementwise kernel: 256 MiB in, 256 MiB out
        torch.cuda.synchronize()
        del src, dst

    # eager reference step, then the whole layer as a graph of K steps
    step(0, torch.cuda.current_stream())
    torch.cuda.synchronize()
    out_eager, lse_eager = out.clone(), lse.clone()
    out.zero_()
    lse.zero_()
    ms, g_layer = timed(step, args.steps, args.warmup)
    status = hta.hta_get_status(h)
    same = bool(torch.equal(out, out_eager)) and bool(torch.equal(lse, lse_eager))
    ok = same and bool(torch.isfinite(out.float()).all().item()) and status == 0
    del g_layer
    # the split-KV kernel alone, same rotation
    pms, g_prefix = timed(prefix_only, args.steps, args.warmup)
    del g_prefix
    torch.cuda.synchronize()
    hta.hta_destroy(h)

    layer_us = ms * 1e3
    value = total_bytes / (ms * 1e-3) / 1e9
    prefix_gbs = kv_bytes / (pms * 1e-3) / 1e9
    traffic = traffic_from_profile()
    # bf16 MFMA work of one prefix launch: QK^T and PV, 2 flops per multiply-add each
    mfma_flops = 4 * w.Hq * w.T * w.D * int(w.prefix_len.sum())
    mfma_tflops = mfma_flops / (pms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": c.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "prefix_len": int(w.prefix_len[0]), "tree_nodes": w.T,
                   "kv_replicas": R},
        "layer_us": round(layer_us, 3),
        "pct_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "tokens_per_s_verified": round(w.B * w.T / (ms * 1e-3), 1),
        "outputs_match_eager_finite_status_ok": ok,
        "plan": {k: plan[k] for k in ("path", "num_workgroups", "waves_per_workgroup",
                                      "qblocks_per_wave", "row_groups", "compute_units")},
        "roofline": {
            "kernel": "prefix_mfma_kernel (split-KV prefix, hta_prefix_partials)",
            "bound": "hbm",
            "achieved": round(prefix_gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(prefix_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(pms * 1e3, 3),
            "algorithmic_bytes_per_launch": kv_bytes,
            # the same launches against the bf16 matrix-core peak; busy fractions from a
            # committed rocprofv3 counter pass on the current kernel source (else null)
            "mfma": {
                "flops_per_launch": mfma_flops,
                "achieved_tflops": round(mfma_tflops, 1),
                "peak_tflops": PEAK_BF16_MFMA_TFLOPS,
                "frac": round(mfma_tflops / PEAK_BF16_MFMA_TFLOPS, 4),
                "busy_counters": traffic_from_profile(MFMA_COUNTERS_FILE, PREFIX_SRC, "mfma_busy"),
                "lds_util_counters": traffic_from_profile(MFMA_COUNTERS_FILE, PREFIX_SRC, "lds_util"),
            },
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    if not args.no_draft:
        res["draft_cross_attn"] = draft_cross_row(w, args.steps, args.warmup, args.replica_bytes,
                                                  0 if args.no_cpu_baseline else args.cpu_seconds / 4)
    if not args.no_configs:
        cgbs = copy_bandwidth()
        res["copy_bw_gbs"] = round(cgbs, 1)
        res["pct_copy_bw"] = round(100 * value / cgbs, 2)
        res["configs"] = all_configs_row(cgbs, not args.no_cpu_baseline)
    if not args.no_tree:
        res["tree_build"] = tree_build_row(w, args.steps, args.warmup,
                                           0 if args.no_cpu_baseline else args.cpu_seconds / 4)
    if not args.no_accept:
        res["accept_commit"] = accept_commit_row(w, args.steps, args.warmup, args.replica_bytes,
                                                 0 if args.no_cpu_baseline else args.cpu_seconds / 2)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
