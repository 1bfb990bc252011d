#!/usr/bin/env python3
"""Decode throughput per layer at a 1M-token context on one MI355X.

One step is one decode token per sequence through
  * a CSA layer (compression m = 4, top-k 1024, window 128), 8 sequences of
    2^20 tokens: the compress step (the new token's window row, the entry it
    completes and that entry's pooled indexer key), indexer scores over all
    262,144 entries, top-k, sparse attention;
  * then an HCA layer (compression m' = 128, window 128), 32 sequences of
    2^20 tokens: the compress step, dense attention over all 8,192 entries;
the calls in that order on one stream, as layers of a stack run.  All inputs
are seeded synthetic N(0,1) data resident in HBM before timing.  The HCA
caches rotate over several copies so successive steps do not hit the 256 MB
Infinity Cache (each model layer has its own cache).

Prints ONE JSON line: value = query-token-layers per second ((8 + 32) query
tokens / (CSA layer time + HCA layer time)); per_layer = each layer's query
tokens/s, algorithmic bytes and fraction of the HBM roofline; the per-kernel
timing breakdown from HIP events; the roofline of the dominant kernel; the
same calls with the two independent batches overlapped on two streams (and
as a HIP graph replay), labelled as such; the CSA layer at a 128K context
(16 sequences); 8 sequences through an alternating CSA/HCA layer stack; and
the float64 oracle timed on the host cores on bounded samples (decode with
the thread pool and with one thread, the prefill chunk extrapolated from a
stratified sample).

A "prefill" section times the 4096-token chunk appended to a 2^20-token
context (both layers) and reports MFMA fractions for scoring and attention.
"fp8_indexer" and "mxfp4_indexer" sections run the same CSA decode layer and
prefill indexer with the FP8 (E4M3, one scale per row) and MXFP4 lightning
indexers; the headline value keeps the bf16 indexer keys of the workload
definition.  An "nsa_variant" section times the NSA-style compress-select-
window layer at the same 1M-token decode shape.  A "ragged_decode" section
runs the same step with each sequence at its own position (128K to 1M).  A
"backward" section times the CSA layer's training step on the prefill chunk
(attention, indexer KL and compressor backward).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-prefill]
                    [--no-fp8] [--no-nsa] [--nsa-only] [--no-ragged] [--no-extra-decode]
                    [--no-backward] [--backward-only] [--prefill-only] [--counters]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 matrix peak, published
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense FP4/FP6 matrix peak, published
COPY_BYTES = 1 << 30           # calibration copy for the HBM byte counters

# HBM bytes of one index_score launch at the decode shape, from two
# rocprofv3 --pmc passes over `bench.py --counters` (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads
# for torch's elementwise kernel over 1 GiB in and 1 GiB out (FETCH 524,318
# KiB -> x2.0; WRITE 1,048,576 KiB -> x1.0).  Valid only for the kernel
# sources they were taken with (hash below); otherwise reported as null.
TRAFFIC = {"sources_sha256_16": "cc2d1ee3cd142591",
           "fetch_kib": 262708.0, "fetch_scale": 2.0,
           "write_kib": 8192.0, "write_scale": 1.0}
TRAFFIC_SOURCES = ("long_context_sparse_csa_amd/csrc/indexer.hip",
                   "long_context_sparse_csa_amd/csrc/common.hpp")
METRIC = "decode query-tokens/s per layer at 1M ctx (CSA, HCA); % of HBM/MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_inputs(dev, rotate):
    from long_context_sparse_csa_amd import decode
    from long_context_sparse_csa_amd.configs import CSA_1M, HCA_1M
    return decode.build_inputs(CSA_1M, HCA_1M, dev, rotate)


# The calls of one layer, in dependency order: a layer's compress step
# writes the rows its indexer and attention read.
CSA_LAYER = ("csa_compress", "index_score", "topk_select", "csa_attend")
HCA_LAYER = ("hca_compress", "hca_attend")


def make_step(inp, dev, csa_pos=None, hca_pos=None, names=CSA_LAYER + HCA_LAYER):
    """(name, fn) launches of one eager step -- the CSA layer's calls, then
    the HCA layer's, one stream (HCA cache copies rotate) -- and the
    DecodeStep behind them (optionally a ragged batch)."""
    from long_context_sparse_csa_amd import decode
    from long_context_sparse_csa_amd.configs import CSA_1M, HCA_1M
    st = decode.DecodeStep(inp, CSA_1M, HCA_1M, dev, csa_pos=csa_pos, hca_pos=hca_pos)
    state = {"i": 0}
    calls = [st.calls(r) for r in range(len(inp["hca"]["entries"]))]

    def mk(name):
        def fn():
            calls[state["i"] % len(calls)][name]()
            if name == "hca_attend":
                state["i"] += 1
        return fn
    return [(n, mk(n)) for n in names], st


def algorithmic_bytes():
    """Bytes each call must move by the method's definition (per step)."""
    from long_context_sparse_csa_amd.configs import CSA_1M as c, HCA_1M as h
    Nc, Nh = c.T // c.m, h.T // h.m
    row = c.D + c.R
    out = {
        "index_score": c.B * (Nc * c.dI * 2 + c.HI * c.dI * 2 + c.HI * 4),
        "csa_attend": c.B * ((c.k + c.W) * row + c.H * c.D * 2 * 2 + c.k * 4),
        "hca_attend": h.B * ((Nh + h.W) * row + h.H * h.D * 2 * 2),
        "csa_compress": c.B * (2 * c.m * (c.D * 2 + 4 + c.dI * 2) + row + c.D * 2 + row + c.dI * 2),
        "hca_compress": h.B * (2 * h.m * (h.D * 2 + 4) + row + h.D * 2 + row),
    }
    out["compress"] = out["csa_compress"] + out["hca_compress"]   # both layers, one launch
    flops = {
        "index_score": c.B * 2 * c.HI * c.dI * Nc,
        "csa_attend": c.B * 4 * c.H * c.D * (c.k + c.W),
        "hca_attend": h.B * 4 * h.H * h.D * (Nh + h.W),
    }
    return out, flops


def measured_traffic():
    """Counter-measured HBM bytes per index_score launch, or None when the
    kernel sources differ from the ones the counters were taken with."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != TRAFFIC["sources_sha256_16"]:
        return None
    return int(1024 * (TRAFFIC["fetch_kib"] * TRAFFIC["fetch_scale"] +
                       TRAFFIC["write_kib"] * TRAFFIC["write_scale"]))


def run_timed(launches, steps, warmup):
    import torch
    for _ in range(warmup):
        for _, fn in launches:
            fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        for _, fn in launches:
            fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return e0.elapsed_time(e1) / steps, wall


def run_timed_concurrent(st, rotate, steps, warmup):
    """Steps of DecodeStep.run_concurrent (HCA attention on a second stream),
    HCA cache copies used in turn; events on the launching stream, which
    waits for the second stream every step."""
    import torch
    for i in range(warmup):
        st.run_concurrent(i % rotate)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        st.run_concurrent(i % rotate)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return e0.elapsed_time(e1) / steps, wall


def run_timed_graphs(st, rotate, steps, warmup):
    """Steps replayed from HIP graphs of the concurrent schedule, one graph
    per HCA cache copy (used in turn)."""
    import torch
    for r in range(rotate):
        st.run_concurrent(r)
    torch.cuda.synchronize()
    graphs = [st.capture(r) for r in range(rotate)]
    for i in range(warmup):
        graphs[i % rotate].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        graphs[i % rotate].replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return e0.elapsed_time(e1) / steps, wall


def run_timed_replays(graphs, steps, warmup):
    """Replays of HIP graphs used in turn, between two HIP events on the
    current stream: milliseconds per replay."""
    import torch
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def one_stream_graphs(st, rotate):
    """One HIP graph per HCA cache copy of the headline step's one-stream
    calls (the CSA layer's, then the HCA layer's)."""
    import torch
    from long_context_sparse_csa_amd import decode
    graphs = []
    for r in range(rotate):
        f = st.calls(r)
        lr = [(n, f[n]) for n in CSA_LAYER + HCA_LAYER]
        for _, fn in lr:
            fn()
        torch.cuda.synchronize()
        graphs.append(decode.capture_launches(lr))
    return graphs


def run_breakdown(launches, steps):
    """Per-call HIP-event durations on the launching (current) stream."""
    import torch
    names = [n for n, _ in launches]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        evs[s][0].record()
        for i, (_, fn) in enumerate(launches):
            fn()
            evs[s][i + 1].record()
    torch.cuda.synchronize()
    tot = {n: 0.0 for n in names}
    for s in range(steps):
        for i, n in enumerate(names):
            tot[n] += evs[s][i].elapsed_time(evs[s][i + 1])
    return {n: tot[n] / steps * 1e3 for n in names}   # microseconds


def run_back_to_back(fn, n, warmup=3):
    """Average duration of one launch of fn: n launches back to back between
    two HIP events on the launching (current) stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3   # microseconds


def prefill_section(dev, reps):
    """The 4096-token prefill chunk appended to a 2^20-token context (one
    sequence): CSA layer = compress the 1024 new m=4 entries, pack the window
    rows, indexer + top-k over ~263K entries, sparse attention; HCA layer =
    compress the 32 new m'=128 entries, dense attention over ~8.2K entries.
    Timed with HIP events on the launching stream."""
    import torch
    from long_context_sparse_csa_amd import ops, synth
    from long_context_sparse_csa_amd.configs import PREFILL_1M as p
    P, Tq, H, D, R = p.T, p.Tq, p.H, p.D, p.R
    HI, dI, k, W, mh, seed = p.HI, p.dI, p.k, p.W, p.extra["m_hca"], p.seed
    Nc, Nh = P // p.m + Tq // p.m, P // mh + Tq // mh
    ent_c = synth.packed_rows((1, Nc), D, R, seed, "entries", dev, chunk_rows=1 << 18)
    ent_h = synth.packed_rows((1, Nh), D, R, seed, "entries_h", dev)
    k_idx = synth.normal((1, Nc, dI), seed, "kI", dev, dtype=torch.bfloat16)
    q_idx = synth.normal((1, Tq, HI, dI), seed, "qI", dev, dtype=torch.bfloat16)
    w_idx = synth.normal((1, Tq, HI), seed, "w", dev)
    q = synth.normal((1, Tq, H, D), seed, "q", dev, dtype=torch.bfloat16)
    raw_c = synth.normal((1, Tq + p.m, D), seed, "raw", dev, dtype=torch.bfloat16)
    raw_h = synth.normal((1, Tq + mh, D), seed, "raw_h", dev, dtype=torch.bfloat16)
    s_c = synth.normal((1, Tq + p.m), seed, "score", dev)
    s_h = synth.normal((1, Tq + mh), seed, "score_h", dev)
    b_c = synth.normal((2 * p.m,), seed, "bias", dev, std=0.1)
    b_h = synth.normal((2 * mh,), seed, "bias_h", dev, std=0.1)
    raw_w = synth.normal((1, Tq + W - 1, D), seed, "rawwin", dev, dtype=torch.bfloat16)
    gamma = torch.ones(D, device=dev)
    sink = synth.normal((H,), seed, "sink", dev)
    win = torch.empty((1, Tq + W - 1, D + R), dtype=torch.uint8, device=dev)
    topk = torch.empty((1, Tq, k), dtype=torch.int32, device=dev)
    ws = torch.empty(ops.index_topk_workspace_bytes(1, Tq, Nc, P, p.m, k), dtype=torch.uint8,
                     device=dev)
    calls = {
        "compress_m4": lambda: ops.compress_pool(raw_c, s_c, b_c, gamma, ent_c, raw_pos0=P - p.m,
                                                 m=p.m, entry0=P // p.m, n_out=Tq // p.m,
                                                 out_row0=P // p.m),
        "pack_window": lambda: ops.compress_pack(raw_w, gamma, win, raw_pos0=P - W + 1),
        "index_topk": lambda: ops.index_topk(q_idx, w_idx, k_idx, n_entries=Nc, q_pos0=P, m=p.m,
                                             k=k, topk=topk, workspace=ws),
        "csa_attend": lambda: ops.csa_attend(q, ent_c, topk, win, gamma, sink, q_pos0=P, W=W),
        "compress_m128": lambda: ops.compress_pool(raw_h, s_h, b_h, gamma, ent_h, raw_pos0=P - mh,
                                                   m=mh, entry0=P // mh, n_out=Tq // mh,
                                                   out_row0=P // mh),
        "hca_attend": lambda: ops.hca_attend(q, ent_h, win, gamma, sink, n_entries=Nh, m=mh,
                                             q_pos0=P, W=W),
    }
    for fn in calls.values():   # warm-up
        fn()
    torch.cuda.synchronize()
    ms = {}
    for name, fn in calls.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms[name] = e0.elapsed_time(e1) / reps
    # algorithmic FLOPs: every (query, visible key) pair once
    vis_c = sum(min(Nc, (P + r + 1) // p.m) for r in range(Tq))
    vis_h = sum(min(Nh, (P + r + 1) // mh) for r in range(Tq))
    fl_idx = 2 * HI * dI * vis_c
    fl_csa = 4 * H * D * (k + W) * Tq
    fl_hca = 4 * H * D * (vis_h + W * Tq)
    mfma_peak = 2500.0   # TFLOP/s, dense bf16, published
    t_csa = ms["compress_m4"] + ms["pack_window"] + ms["index_topk"] + ms["csa_attend"]
    t_hca = ms["compress_m128"] + ms["hca_attend"]

    def tf(fl, t):
        return round(fl / (t * 1e-3) / 1e12, 1)
    return {
        "workload": "prefill_4096_on_1m: 4096 new tokens after 2^20 cached, one sequence, "
                    "H=64 D=512 HI=64 dI=128 k=1024 W=128, m=4 (CSA) and m'=128 (HCA)",
        "ms": {n: round(v, 3) for n, v in ms.items()},
        "csa_layer_tokens_per_s": round(Tq / (t_csa * 1e-3), 1),
        "hca_layer_tokens_per_s": round(Tq / (t_hca * 1e-3), 1),
        "index_topk_TFLOPs": tf(fl_idx, ms["index_topk"]),
        "index_topk_mfma_frac": round(tf(fl_idx, ms["index_topk"]) / mfma_peak, 4),
        "csa_attend_TFLOPs": tf(fl_csa, ms["csa_attend"]),
        "hca_attend_TFLOPs": tf(fl_hca, ms["hca_attend"]),
        "hca_attend_mfma_frac": round(tf(fl_hca, ms["hca_attend"]) / mfma_peak, 4),
        "mfma_peak_TFLOPs": mfma_peak,
        "reps": reps,
    }


def low_precision_indexer_section(dev, st, launches, reps, fmt):
    """The lightning indexer with FP8 (E4M3, one fp32 scale per row) or MXFP4
    (E2M1 with an E8M0 scale per 32 dims) queries and keys, on the same
    workloads: the decode CSA layer with it in place of the bf16 indexer
    (8 x 262,144 entries), and the 4096-query prefill indexer + top-k over
    ~263K entries.  Inputs: N(0,1) rows quantised by synth.e4m3_rows /
    synth.mxfp4_rows."""
    import torch
    from long_context_sparse_csa_amd import ops, synth
    from long_context_sparse_csa_amd.configs import CSA_1M as c, PREFILL_1M as p
    fp8 = fmt == "fp8"
    a = st.inp["csa"]
    Nc, tc = a["N"], a["t"]
    if fp8:
        q, qs = synth.e4m3_rows((c.B, 1, c.HI, c.dI), c.seed, "q8", dev)
        kk, ks = synth.e4m3_rows((c.B, Nc, c.dI), c.seed, "k8", dev, chunk_rows=1 << 18)
        score, topk_fn, peak = ops.index_score_fp8, ops.index_topk_fp8, FP8_PEAK_TFLOPS
        key_bytes = c.dI + 4
    else:
        q, qs = synth.mxfp4_rows((c.B, 1, c.HI, c.dI), c.seed, "q4", dev)
        kk, ks = synth.mxfp4_rows((c.B, Nc, c.dI), c.seed, "k4", dev)
        score, topk_fn, peak = ops.index_score_mxfp4, ops.index_topk_mxfp4, FP4_PEAK_TFLOPS
        key_bytes = c.dI // 2 + c.dI // 32
    fn = dict(st.calls(0))   # the per-layer calls (the CSA layer alone)
    fn["index_score"] = lambda: score(q, qs, a["w_idx"], kk, ks, n_entries=Nc, q_pos0=tc, m=c.m,
                                      scores=st.scores)
    names = ("csa_compress", "index_score", "topk_select", "csa_attend")
    csa = [(n, fn[n]) for n in names]
    for _ in range(3):
        for _, f in csa:
            f()
    br = run_breakdown(csa, 20)
    t_layer = sum(br.values())
    idx_bytes = c.B * Nc * key_bytes + q.numel() + qs.numel() * qs.element_size() + c.B * c.HI * 4
    dec = {
        "index_score_us": round(br["index_score"], 2),
        "index_score_GBps": round(idx_bytes / (br["index_score"] * 1e-6) / 1e9, 1),
        "index_score_hbm_frac": round(idx_bytes / (br["index_score"] * 1e-6) / 1e9 /
                                      HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_launch": idx_bytes,
        "csa_layer_us": round(t_layer, 2),
        "csa_query_tokens_per_s": round(c.B / (t_layer * 1e-6), 1),
    }
    del kk, ks
    P, Tq, HI, dI, k = p.T, p.Tq, p.HI, p.dI, p.k
    Np = P // p.m + Tq // p.m
    if fp8:
        pq, pqs = synth.e4m3_rows((1, Tq, HI, dI), p.seed, "q8", dev)
        pk, pks = synth.e4m3_rows((1, Np, dI), p.seed, "k8", dev)
    else:
        pq, pqs = synth.mxfp4_rows((1, Tq, HI, dI), p.seed, "q4", dev)
        pk, pks = synth.mxfp4_rows((1, Np, dI), p.seed, "k4", dev)
    pw = synth.normal((1, Tq, HI), p.seed, "w", dev)
    topk = torch.empty((1, Tq, k), dtype=torch.int32, device=dev)
    ws = torch.empty(ops.index_topk_workspace_bytes(1, Tq, Np, P, p.m, k), dtype=torch.uint8,
                     device=dev)
    call = lambda: topk_fn(pq, pqs, pw, pk, pks, n_entries=Np, q_pos0=P, m=p.m, k=k, topk=topk,
                           workspace=ws)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    vis = sum(min(Np, (P + r + 1) // p.m) for r in range(Tq))
    tf = 2 * HI * dI * vis / (ms * 1e-3) / 1e12
    return {
        "workload": ("indexer keys and queries E4M3 with one fp32 scale per row" if fp8 else
                     "indexer keys and queries MXFP4 (E2M1, E8M0 scale per 32 dims)") +
                    "; decode: the CSA layer of decode_1m_csa_hca with this indexer; prefill: "
                    "prefill_4096_on_1m indexer + top-k",
        "decode": dec,
        "prefill_index_topk_ms": round(ms, 3),
        "prefill_index_topk_TFLOPs": round(tf, 1),
        "prefill_index_topk_mfma_frac": round(tf / peak, 4),
        "mfma_peak_TFLOPs": peak,
    }


def nsa_section(dev, reps):
    """The NSA-style variant at the 1M-token decode shape: 8 sequences, 64
    heads x 512 dims, 16,384 compressed entries of 64-token blocks, 16 blocks
    (1,024 tokens) selected, 128-token window, gates U(0,1).  One call =
    compressed branch (logits kept), block scores, top-16, selected branch,
    window branch, gated sum; timed with HIP events on the launching stream.
    Inputs: N(0,1) packed rows for entries and the full token cache."""
    import torch
    from long_context_sparse_csa_amd import ops, synth
    from long_context_sparse_csa_amd.configs import NSA_1M as c
    B, H, D, R, m, W, n_sel = c.B, c.H, c.D, c.R, c.m, c.W, c.extra["n_sel"]
    V, t = c.n_entries, c.q_pos0
    q = synth.normal((B, 1, H, D), c.seed, "q", dev, dtype=torch.bfloat16)
    ent = synth.packed_rows((B, V), D, R, c.seed, "entries", dev)
    tok = synth.packed_rows((B, c.T), D, R, c.seed, "tokens", dev)
    win = tok[:, t - (W - 1): t + 1].contiguous()
    gq = synth.normal((D,), c.seed, "gamma_q", dev, mean=1.0, std=0.1)
    gates = torch.rand((B, 1, H, 3), generator=torch.Generator().manual_seed(c.seed)).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(ops.nsa_attend_workspace_bytes(B, 1, H, D, V, m, t, W, n_sel),
                     dtype=torch.uint8, device=dev)
    call = lambda: ops.nsa_attend(q, ent, tok, win, gq, gates, n_entries=V, m=m, q_pos0=t, W=W,
                                  n_sel=n_sel, out=out, workspace=ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    row = D + R
    # per query: entries, logits written and read back, block scores written
    # and read, selected token rows, window rows, q, three branch outputs
    # written and read, out
    per_q = (V * row + 2 * H * V * 4 + 2 * V * 4 + n_sel * m * row + W * row + H * D * 2 +
             6 * H * D * 2 + H * D * 2)
    gbs = B * per_q / (us * 1e-6) / 1e9
    del tok
    return {
        "workload": f"nsa_decode_1m: B={B} T=2^20 m={m} N={V} n_sel={n_sel} "
                    f"(selected tokens {n_sel * m}) H={H} D={D} R={R} W={W}",
        "layer_us": round(us, 2),
        "query_tokens_per_s": round(B / (us * 1e-6), 1),
        "algorithmic_bytes_per_call": B * per_q,
        "GBps": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
    }


def backward_section(dev, reps):
    """Training step of the CSA layer on the 4096-token prefill chunk of a
    2^20-token context (one sequence): attention backward over each query's
    1024 selected entries + its 128-token window (64 heads x 512 dims), the
    indexer KL loss backward over the same 1024 entries (64 x 128 indexer
    heads), and the compressor backward for the chunk's 1024 new entries
    (m = 4).  Inputs: N(0,1) packed rows and latents, random sorted top-k
    sets, dout N(0,1).  Timed with HIP events; the attention backward is
    reported against the bf16 matrix peak with its algorithmic FLOPs
    10 H n D per query (n = k + W rows): [S; dP] 4, dq 2, dX 4."""
    import torch
    from long_context_sparse_csa_amd import ops, synth
    from long_context_sparse_csa_amd.configs import PREFILL_1M as p
    P, Tq, H, D, R, W, k, seed = p.T, p.Tq, p.H, p.D, p.R, p.W, p.k, p.seed
    HI, dI, m = p.HI, p.dI, p.m
    Nc = P // m + Tq // m
    q = synth.normal((1, Tq, H, D), seed, "q", dev, dtype=torch.bfloat16)
    ent = synth.packed_rows((1, Nc), D, R, seed, "entries", dev, chunk_rows=1 << 18)
    win = synth.packed_rows((1, Tq + W - 1), D, R, seed, "win", dev)
    gq = torch.ones(D, device=dev)
    sink = synth.normal((H,), seed, "sink", dev)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    # sorted random k-subsets of each query's visible entries
    vis = torch.minimum(torch.full((Tq,), Nc, device=dev),
                        (P + torch.arange(Tq, device=dev) + 1) // m)
    r = torch.rand((Tq, k), generator=g, device=dev)
    topk = (r * vis[:, None].float()).long().clamp(max=Nc - 1)
    topk = torch.sort(topk, dim=1).values.to(torch.int32)[None].contiguous()
    out, lse = ops.csa_attend(q, ent, topk, win, gq, sink, q_pos0=P, W=W, want_lse=True)
    dout = synth.normal((1, Tq, H, D), seed, "dout", dev, dtype=torch.bfloat16)
    p_sel = torch.empty((1, Tq, k), dtype=torch.float32, device=dev)
    grads = {"dq": torch.empty((1, Tq, H, D), dtype=torch.float32, device=dev),
             "d_entries": torch.zeros((1, Nc, D), dtype=torch.float32, device=dev),
             "d_win": torch.zeros((1, Tq + W - 1, D), dtype=torch.float32, device=dev),
             "d_sink": torch.zeros(H, dtype=torch.float32, device=dev),
             "d_gamma_q": torch.zeros(D, dtype=torch.float32, device=dev)}
    ws = torch.empty(ops.lib().v4attn_csa_attend_backward_workspace(1, Tq, H, D, k, W, Nc),
                     dtype=torch.uint8, device=dev)
    att = lambda: ops.csa_attend_backward(q, ent, topk, win, gq, sink, out, lse, dout, q_pos0=P,
                                          W=W, grads=grads, p_sel=p_sel, workspace=ws)
    qi = synth.normal((1, Tq, HI, dI), seed, "qI", dev, dtype=torch.bfloat16)
    wi = synth.normal((1, Tq, HI), seed, "w", dev)
    ki = synth.normal((1, Nc, dI), seed, "kI", dev, dtype=torch.bfloat16)
    dk = torch.zeros((1, Nc, dI), dtype=torch.float32, device=dev)
    kws = torch.empty(ops.lib().v4attn_index_kl_backward_workspace(1, Tq, dI, k, Nc),
                      dtype=torch.uint8, device=dev)
    kl = lambda: ops.index_kl_backward(qi, wi, ki, topk, p_sel, dk=dk, workspace=kws)
    raw = synth.normal((1, Tq + m, D), seed, "raw", dev, dtype=torch.bfloat16)
    sc = synth.normal((1, Tq + m), seed, "score", dev)
    bias = synth.normal((2 * m,), seed, "bias", dev, std=0.1)
    de = synth.normal((1, Tq // m, D), seed, "de", dev)
    cgr = {"d_raw": torch.zeros((1, Tq + m, D), dtype=torch.float32, device=dev),
           "d_score": torch.zeros((1, Tq + m), dtype=torch.float32, device=dev),
           "d_bias": torch.zeros(2 * m, dtype=torch.float32, device=dev),
           "d_gamma": torch.zeros(D, dtype=torch.float32, device=dev)}
    cmp = lambda: ops.compress_backward(raw, sc, bias, gq, de, raw_pos0=P - m, m=m,
                                        entry0=P // m, grads=cgr)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_att, ms_kl, ms_cmp = timed(att), timed(kl), timed(cmp)
    flops = 10.0 * H * (k + W) * D * Tq
    tf = flops / (ms_att * 1e-3) / 1e12
    return {
        "workload": f"csa_layer_backward_4096_on_1m: Tq={Tq} k={k} W={W} H={H} D={D} "
                    f"HI={HI} dI={dI} m={m}",
        "ms": {"attend_backward": round(ms_att, 3), "index_kl_backward": round(ms_kl, 3),
               "compress_backward": round(ms_cmp, 3)},
        "layer_backward_ms": round(ms_att + ms_kl + ms_cmp, 3),
        "tokens_per_s": round(Tq / ((ms_att + ms_kl + ms_cmp) * 1e-3), 1),
        "attend_backward_TFLOPs": round(tf, 1),
        "attend_backward_mfma_frac": round(tf / 2500.0, 4),
    }


def ragged_section(dev, inp, reps):
    """The decode step with a ragged batch: the same caches and calls, each
    sequence's new token at its own position -- CSA sequence b at
    (b + 1) 2^17 - 1, HCA sequence b at (b + 1) 2^15 - 1 (lengths 128K to 1M,
    mean 0.56M) -- timed like the headline (one stream, CSA layer then HCA
    layer) and with the two batches overlapped on two streams.  The indexer
    reads only each sequence's visible keys, so its algorithmic bytes are
    sum_b V_b (256 + ...) per step."""
    from long_context_sparse_csa_amd.configs import CSA_1M as c, HCA_1M as h
    csa_pos = [(b + 1) * (1 << 17) - 1 for b in range(c.B)]
    hca_pos = [(b + 1) * (1 << 15) - 1 for b in range(h.B)]
    launches, st = make_step(inp, dev, csa_pos=csa_pos, hca_pos=hca_pos)
    rot = len(inp["hca"]["entries"])
    blocks = [run_timed(launches, reps, 5)[0] for _ in range(3)]
    blocks2 = [run_timed_concurrent(st, rot, reps, 5)[0] for _ in range(3)]
    br = run_breakdown(launches, 20)
    vis = sum(min(c.T // c.m, (p + 1) // c.m) for p in csa_pos)
    idx_bytes = vis * c.dI * 2 + c.B * (c.HI * c.dI * 2 + c.HI * 4 + 0)
    t_csa = sum(br[k] for k in CSA_LAYER)
    t_hca = sum(br[k] for k in HCA_LAYER)
    ms = sum(blocks) / 3
    return {
        "workload": "decode_ragged: CSA B=8 at positions (b+1) 2^17 - 1, HCA B=32 at "
                    "(b+1) 2^15 - 1 (the decode_1m_csa_hca caches)",
        "step_us": round(ms * 1e3, 2),
        "step_us_blocks": [round(x * 1e3, 2) for x in blocks],
        "query_token_layers_per_s": round((c.B + h.B) / (ms * 1e-3), 1),
        "two_stream_overlap_step_us_blocks": [round(x * 1e3, 2) for x in blocks2],
        "csa_layer_us": round(t_csa, 2), "hca_layer_us": round(t_hca, 2),
        "csa_query_tokens_per_s": round(c.B / (t_csa * 1e-6), 1),
        "hca_query_tokens_per_s": round(h.B / (t_hca * 1e-6), 1),
        "kernels_us": {k: round(v, 2) for k, v in br.items()},
        "index_score_GBps": round(idx_bytes / (br["index_score"] * 1e-6) / 1e9, 1),
        "index_score_hbm_frac": round(idx_bytes / (br["index_score"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
    }


def csa_128k_section(dev, steps, rotate=4):
    """The CSA layer at a 128K context (16 sequences, 32,768 entries each):
    compress step with the pooled indexer key, indexer over every entry,
    top-1024, sparse attention; one stream.  One step's bytes (~147 MB) fit
    the 256 MB Infinity Cache, so the entry and indexer-key caches rotate
    over `rotate` copies."""
    import torch
    from long_context_sparse_csa_amd import ops, synth
    from long_context_sparse_csa_amd.configs import CSA_128K as c
    B, N, t, m = c.B, c.T // c.m, c.T - 1, c.m
    ents = [synth.packed_rows((B, N), c.D, c.R, c.seed + 100 * i, "entries", dev) for i in range(rotate)]
    kids = [synth.normal((B, N, c.dI), c.seed + 100 * i, "kI", dev, dtype=torch.bfloat16)
            for i in range(rotate)]
    qI = synth.normal((B, 1, c.HI, c.dI), c.seed, "qI", dev, dtype=torch.bfloat16)
    wI = synth.normal((B, 1, c.HI), c.seed, "w", dev)
    q = synth.normal((B, 1, c.H, c.D), c.seed, "q", dev, dtype=torch.bfloat16)
    win = synth.packed_rows((B, c.W), c.D, c.R, c.seed, "win", dev)
    raw = synth.normal((B, 2 * m, c.D), c.seed, "raw", dev, dtype=torch.bfloat16)
    raw_idx = synth.normal((B, 2 * m, c.dI), c.seed, "rawI", dev, dtype=torch.bfloat16)
    score = synth.normal((B, 2 * m), c.seed, "score", dev)
    bias = synth.normal((2 * m,), c.seed, "bias", dev, std=0.1)
    sink = synth.normal((c.H,), c.seed, "sink", dev)
    gamma = torch.ones(c.D, device=dev)
    scores = torch.empty((B, ops.score_stride(1, N, t, m)), dtype=torch.float32, device=dev)
    topk = torch.empty((B, 1, c.k), dtype=torch.int32, device=dev)
    tk_ws = torch.empty(max(ops.topk_select_workspace_bytes(B, 1, N, t, m, c.k), 16),
                        dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    a_ws = torch.empty(max(ops.csa_attend_workspace_bytes(B, 1, c.H, c.D, c.k, c.W), 16),
                       dtype=torch.uint8, device=dev)
    state = {"i": 0}

    def copy():
        return state["i"] % rotate
    calls = [
        ("csa_compress", lambda: ops.compress_step(raw, score, bias, gamma, ents[copy()], win,
                                                   raw_pos0=t + 1 - 2 * m, m=m, t=t,
                                                   win_row=c.W - 1, raw_idx=raw_idx,
                                                   k_idx=kids[copy()])),
        ("index_score", lambda: ops.index_score(qI, wI, kids[copy()], n_entries=N, q_pos0=t, m=m,
                                                scores=scores)),
        ("topk_select", lambda: ops.topk_select(scores, B=B, Tq=1, n_entries=N, q_pos0=t, m=m,
                                                k=c.k, topk=topk, workspace=tk_ws)),
        ("csa_attend", lambda: ops.csa_attend(q, ents[copy()], topk, win, gamma, sink, q_pos0=t,
                                              W=c.W, out=out, workspace=a_ws)),
    ]

    def bump():
        state["i"] += 1
    launches = calls + [("next_copy", bump)]
    ms, _ = run_timed(launches, steps, 5)
    br = run_breakdown(launches, 20)
    br.pop("next_copy")
    row = c.D + c.R
    per_q = (N * c.dI * 2 + c.HI * c.dI * 2 + c.HI * 4 + (c.k + c.W) * row + c.H * c.D * 2 * 2 +
             c.k * 4)
    gbs = B * per_q / (ms * 1e-3) / 1e9
    return {
        "workload": f"csa_decode_128k: B={B} T=2^17 m={m} N={N} H={c.H} D={c.D} HI={c.HI} "
                    f"dI={c.dI} k={c.k} W={c.W}; entry and indexer-key caches rotate over "
                    f"{rotate} copies",
        "layer_us": round(ms * 1e3, 2),
        "query_tokens_per_s": round(B / (ms * 1e-3), 1),
        "algorithmic_bytes_per_query": per_q,
        "GBps": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline_query_tokens_per_s": round(HBM_PEAK_GBS * 1e9 / per_q, 1),
        "kernels_us": {k: round(v, 2) for k, v in br.items()},
    }


def stack_section(dev, steps, pairs=2):
    """8 sequences at a 2^20-token context through an alternating stack of
    CSA and HCA layers (2 x `pairs` layers, each with its own caches), one
    decode token: every layer's calls in order on one stream, as a dependent
    stack would run them (a layer's compress step needs that layer's input)."""
    import torch
    from long_context_sparse_csa_amd import decode
    from long_context_sparse_csa_amd.configs import CSA_1M, HCA_1M
    sts = []
    for i in range(pairs):
        c = CSA_1M.with_(seed=CSA_1M.seed + 1000 * (i + 1))
        h = HCA_1M.with_(B=CSA_1M.B, seed=HCA_1M.seed + 1000 * (i + 1))
        st = decode.DecodeStep(decode.build_inputs(c, h, dev), c, h, dev)
        sts.append(st)
    launches = decode.stack_launches(sts)
    torch.cuda.synchronize()
    ms, _ = run_timed(launches, steps, 5)
    br = run_breakdown(launches, 20)
    # the whole stack as one HIP graph (the launches have run eagerly above)
    g = decode.capture_launches(launches)
    ms_g = run_timed_replays([g], steps, 5)
    B, L = CSA_1M.B, 2 * pairs
    t_csa = sum(v for k, v in br.items() if k.split("_", 1)[1] in CSA_LAYER) / pairs
    t_hca = sum(v for k, v in br.items() if k.split("_", 1)[1] in HCA_LAYER) / pairs
    return {
        "workload": f"decode_stack_1m: B={B} sequences at T=2^20 through {L} alternating layers "
                    f"(CSA m=4 k=1024, HCA m'=128; W=128, H=64, D=512), each with its own caches",
        "stack_us": round(ms * 1e3, 2),
        "query_token_layers_per_s": round(B * L / (ms * 1e-3), 1),
        "hip_graph_replay_stack_us": round(ms_g * 1e3, 2),
        "hip_graph_query_token_layers_per_s": round(B * L / (ms_g * 1e-3), 1),
        "csa_layer_us": round(t_csa, 2),
        "hca_layer_us": round(t_hca, 2),
    }



def _oracle_decode_queries(inp, budget_s, max_pairs):
    """Whole CSA-layer and HCA-layer queries of the decode workloads through
    the float64 oracle, alternating, until the budget: (seconds per CSA
    query, seconds per HCA query, counts)."""
    import numpy as np
    import torch
    from long_context_sparse_csa_amd.configs import CSA_1M as c, HCA_1M as h
    from oracle import attend as oa, codecs, compress as oc, indexer as oi

    def f64(t):
        return codecs.bf16_decode(t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16))

    a, b = inp["csa"], inp["hca"]
    t_csa, t_hca, n_csa, n_hca = 0.0, 0.0, 0, 0
    t0 = time.perf_counter()
    s = 0
    while s < max_pairs and (s == 0 or time.perf_counter() - t0 < budget_s):
        bb = s % c.B
        # host copies of the sequence's bytes (not timed: the oracle's input)
        kI = a["k_idx"][bb].cpu()
        ent = a["entries"][bb].cpu().numpy()
        win = a["win"][bb].cpu().numpy()
        raw = a["raw"][bb]
        q, qI, w = a["q"][bb], a["q_idx"][bb], a["w_idx"][bb].cpu().double().numpy()
        x0 = time.perf_counter()
        e = oc.compress_pool(f64(raw), a["score"][bb].cpu().double().numpy(), c.T - 2 * c.m, c.m,
                             a["bias"].cpu().double().numpy(), np.ones(c.D), c.eps, c.R,
                             c.rope_base, j0=a["N"] - 1, n=1)[1]
        ent[-1] = codecs.pack_rows(e, c.R)[0]
        tk, _ = oi.index_topk(f64(qI), w, f64(kI), a["N"], [a["t"]], c.m, c.k)
        rows = codecs.unpack_rows(ent[tk[0][tk[0] >= 0]], c.D, c.R)
        rows = np.concatenate([rows, codecs.unpack_rows(win, c.D, c.R)])
        oa.attend_rows(f64(q)[0], np.ones(c.D), a["t"], rows, a["sink"].cpu().double().numpy(),
                       c.scale, c.eps, c.R, c.rope_base)
        t_csa += time.perf_counter() - x0
        n_csa += 1
        hb = s % h.B
        ent = b["entries"][0][hb].cpu().numpy()
        win = b["win"][hb].cpu().numpy()
        q = b["q"][hb]
        x0 = time.perf_counter()
        rows = np.concatenate([codecs.unpack_rows(ent, h.D, h.R), codecs.unpack_rows(win, h.D, h.R)])
        oa.attend_rows(f64(q)[0], np.ones(h.D), b["t"], rows, b["sink"].cpu().double().numpy(),
                       h.scale, h.eps, h.R, h.rope_base)
        t_hca += time.perf_counter() - x0
        n_hca += 1
        s += 1
    return t_csa / n_csa, t_hca / n_hca, n_csa, n_hca


def _oracle_prefill_queries(dev, n_sample, budget_s):
    """Float64 oracle on a stratified sample of the prefill chunk's 4096
    queries (evenly spaced, first and last included): per query, the CSA
    layer (indexer over every visible entry, top-1024, attention over the
    selection and the causal window) and the HCA layer (attention over every
    visible entry and the window).  Seconds per query, extrapolated to the
    chunk by the caller."""
    import numpy as np
    import torch
    from long_context_sparse_csa_amd import synth
    from long_context_sparse_csa_amd.configs import PREFILL_1M as p
    from oracle import attend as oa, codecs, indexer as oi
    P, Tq, H, D, R, W, k, m, mh = p.T, p.Tq, p.H, p.D, p.R, p.W, p.k, p.m, p.extra["m_hca"]
    Nc, Nh = P // m + Tq // m, P // mh + Tq // mh

    def f64(t):
        return codecs.bf16_decode(t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16))
    kI = f64(synth.normal((1, Nc, p.dI), p.seed, "kI", dev, dtype=torch.bfloat16)[0])
    ent_c = synth.packed_rows((1, Nc), D, R, p.seed, "entries", dev, chunk_rows=1 << 18)[0] \
        .cpu().numpy()
    ent_h = codecs.unpack_rows(synth.packed_rows((1, Nh), D, R, p.seed, "entries_h", dev)[0]
                               .cpu().numpy(), D, R)
    win = codecs.unpack_rows(synth.packed_rows((1, Tq + W - 1), D, R, p.seed, "win", dev)[0]
                             .cpu().numpy(), D, R)
    qI = synth.normal((1, Tq, p.HI, p.dI), p.seed, "qI", dev, dtype=torch.bfloat16)[0]
    wI = synth.normal((1, Tq, p.HI), p.seed, "w", dev)[0]
    q = synth.normal((1, Tq, H, D), p.seed, "q", dev, dtype=torch.bfloat16)[0]
    sink = synth.normal((H,), p.seed, "sink", dev).cpu().double().numpy()
    gq = np.ones(D)
    t_csa = t_hca = 0.0
    n = 0
    t0 = time.perf_counter()
    for r in np.linspace(0, Tq - 1, n_sample).round().astype(int):
        if n and time.perf_counter() - t0 > budget_s:
            break
        t = P + int(r)
        qn, qIn, wn = f64(q[r]), f64(qI[r]), wI[r].cpu().double().numpy()
        x0 = time.perf_counter()
        V = oi.visible_entries(t, Nc, m)
        sel = oi.topk_select(oi.index_scores(qIn, wn, kI, V), k)
        rows = codecs.unpack_rows(ent_c[sel[sel >= 0]], D, R)
        oa.attend_rows(qn, gq, t, np.concatenate([rows, oa.window_rows(win, t, P, W)]), sink,
                       p.scale, p.eps, R, p.rope_base)
        t_csa += time.perf_counter() - x0
        x0 = time.perf_counter()
        Vh = min(Nh, (t + 1) // mh)
        oa.attend_rows(qn, gq, t, np.concatenate([ent_h[:Vh], oa.window_rows(win, t, P, W)]), sink,
                       p.scale, p.eps, R, p.rope_base)
        t_hca += time.perf_counter() - x0
        n += 1
    return t_csa / n, t_hca / n, n


def cpu_baseline(inp, dev, budget_s, prefill):
    """The float64 oracle (never tuned) on bounded samples of the same
    workloads: decode queries with the BLAS thread pool as it is and with
    one thread, and a stratified sample of the prefill chunk's queries
    extrapolated to the chunk."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from long_context_sparse_csa_amd.configs import CSA_1M as c, HCA_1M as h, PREFILL_1M as p
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    per_csa, per_hca, n_csa, n_hca = _oracle_decode_queries(inp, budget_s * 0.5, 64)
    step = c.B * per_csa + h.B * per_hca
    with threadpool_limits(limits=1):
        one_csa, one_hca, n1c, n1h = _oracle_decode_queries(inp, budget_s * 0.2, 2)
    res = {
        "value": (c.B + h.B) / step,
        "unit": "query-token-layers/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{n_csa} CSA-layer queries (compress of one entry, float64 indexer over "
                   f"262,144 entries, top-1024, attention over 1152 rows) and {n_hca} HCA-layer "
                   f"queries (attention over 8320 rows) at 1M context, extrapolated to one CSA "
                   f"layer of 8 sequences followed by one HCA layer of 32"),
        "csa_query_tokens_per_s": 1.0 / per_csa,
        "hca_query_tokens_per_s": 1.0 / per_hca,
        "one_thread": {"value": (c.B + h.B) / (c.B * one_csa + h.B * one_hca), "cores": 1,
                       "csa_query_tokens_per_s": 1.0 / one_csa,
                       "hca_query_tokens_per_s": 1.0 / one_hca,
                       "sample": f"{n1c} CSA-layer and {n1h} HCA-layer queries, one BLAS thread"},
    }
    if prefill:
        pc, ph, npf = _oracle_prefill_queries(dev, 16, budget_s * 0.4)
        res["prefill_extrapolated"] = {
            "csa_layer_tokens_per_s": 1.0 / pc, "hca_layer_tokens_per_s": 1.0 / ph,
            "chunk_s_extrapolated": {"csa": pc * p.Tq, "hca": ph * p.Tq},
            "cores": threads,
            "sample": f"{npf} of the 4096 prefill queries (evenly spaced, first and last "
                      f"included), timed one by one and extrapolated linearly to the chunk",
        }
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the two-stream and HIP-graph timings of the step (a profile of the "
                         "one-stream launches alone)")
    ap.add_argument("--no-extra-decode", action="store_true",
                    help="skip the 128K CSA layer and the alternating layer stack")
    ap.add_argument("--cpu-seconds", type=float, default=30.0)
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill chunk (prints its section as the JSON line)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 and MXFP4 indexer sections")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the 4096-token prefill section")
    ap.add_argument("--no-nsa", action="store_true",
                    help="skip the NSA-style variant section")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the ragged-batch decode section")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the CSA layer backward section")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the CSA layer backward (prints its section as the JSON line)")
    ap.add_argument("--nsa-only", action="store_true",
                    help="time only the NSA-style variant (prints its section as the JSON line)")
    ap.add_argument("--counters", action="store_true",
                    help="no timing: run a 1 GiB elementwise copy (known bytes) and a few "
                         "decode steps for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_sparse_csa_amd import ops
    from long_context_sparse_csa_amd.configs import CSA_1M as c, HCA_1M as h

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    ops.lib()
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_section(dev, 3)}), flush=True)
        return
    if args.nsa_only:
        print(json.dumps({"nsa_variant": nsa_section(dev, 20)}), flush=True)
        return
    if args.backward_only:
        print(json.dumps({"backward": backward_section(dev, 3)}), flush=True)
        return
    log("generating inputs")
    inp = build_inputs(dev, args.rotate)
    launches, st = make_step(inp, dev)
    torch.cuda.synchronize()
    if args.counters:
        # calibration: torch's elementwise kernel reads and writes COPY_BYTES each
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        for _ in range(3):
            for _, fn in launches:
                fn()
        torch.cuda.synchronize()
        log("counters pass done")
        return
    log("timing")
    # headline: the CSA layer's calls, then the HCA layer's, on one stream
    ms, wall = run_timed(launches, args.steps, args.warmup)
    sched = ("one stream: the CSA layer (compress step, indexer, top-k, attention), then the "
             "HCA layer (compress step, attention)")
    log(f"step {ms * 1e3:.1f} us ({sched})")
    br = run_breakdown(launches, max(10, min(args.steps, 50)))
    log("breakdown (us): " + ", ".join(f"{k} {v:.1f}" for k, v in br.items()))
    abytes, aflops = algorithmic_bytes()
    t_csa_us = sum(br[k] for k in CSA_LAYER)
    t_hca_us = sum(br[k] for k in HCA_LAYER)
    kernels = {}
    for k, us in br.items():
        ent = {"us": round(us, 2)}
        if k in abytes:
            ent["GBps"] = round(abytes[k] / (us * 1e-6) / 1e9, 1)
            ent["hbm_frac"] = round(abytes[k] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        if k in aflops:
            ent["TFLOPs"] = round(aflops[k] / (us * 1e-6) / 1e12, 2)
        kernels[k] = ent
    dom = "index_score"
    # the dominant kernel's average launch duration: 20 launches back to back
    # (the per-call pairs above also hold the dispatch gap after the call before)
    t_dom = run_back_to_back(dict(launches)[dom], 20)
    ach = abytes[dom] / (t_dom * 1e-6) / 1e9
    roofline = {"kernel": "index_score_kernel<128,4>", "bound": "hbm",
                "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "algorithmic_bytes_per_launch": abytes[dom],
                "launch_us": round(t_dom, 2),
                "timing": "20 launches back to back between two HIP events on the launching "
                          "stream"}

    def layer(nq, us, names):
        by = sum(abytes.get(n, 0) for n in names)
        gbs = by / (us * 1e-6) / 1e9
        return {"query_tokens_per_s": round(nq / (us * 1e-6), 1), "layer_us": round(us, 2),
                "algorithmic_bytes": by, "GBps": round(gbs, 1),
                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "roofline_query_tokens_per_s": round(nq * HBM_PEAK_GBS * 1e9 / by, 1)}
    res = {
        "metric": METRIC,
        "value": round((c.B + h.B) / (ms * 1e-3), 1),
        "unit": "query-token-layers/s",
        "per_layer": {
            "csa": layer(c.B, t_csa_us, CSA_LAYER),
            "hca": layer(h.B, t_hca_us, HCA_LAYER),
        },
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_schedule": sched,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode_1m_csa_hca",
            "csa": f"B={c.B} T=2^20 m={c.m} N={c.T // c.m} H={c.H} D={c.D} R={c.R} "
                   f"HI={c.HI} dI={c.dI} k={c.k} W={c.W}",
            "hca": f"B={h.B} T=2^20 m={h.m} N={h.T // h.m} H={h.H} D={h.D} R={h.R} W={h.W}",
            "storage": "entries E4M3 (448 dims) + bf16 (64 rotary dims) = 576 B/row; "
                       "indexer keys bf16",
            "value_is": "query-token-layers/s: (8 CSA + 32 HCA query tokens) / (CSA layer time "
                        "+ HCA layer time), the two layers one after the other",
            "hca_cache_copies": args.rotate,
        },
        "kernels": kernels,
        "roofline": roofline,
        "wall_s": round(wall, 3),
    }
    # the same one-stream step replayed from HIP graphs (one per HCA cache copy)
    ms_g = run_timed_replays(one_stream_graphs(st, args.rotate), args.steps, args.warmup)
    res["hip_graph_one_stream"] = {
        "what": "the headline step's calls (CSA layer, then HCA layer, one stream) replayed "
                "from HIP graphs, one per HCA cache copy",
        "step_us": round(ms_g * 1e3, 2),
        "query_token_layers_per_s": round((c.B + h.B) / (ms_g * 1e-3), 1),
    }
    log("per layer: " + json.dumps(res["per_layer"]))
    log("one-stream graph replay: " + json.dumps(res["hip_graph_one_stream"]))
    # the same calls with the two layers' independent batches overlapped: both
    # compress steps in one launch, the HCA attention on a second stream
    # beside the CSA indexer, top-k and attention (not open to a dependent
    # stack, where each layer waits for the previous one)
    if not args.no_overlap:
        ms2, _ = run_timed_concurrent(st, args.rotate, args.steps, args.warmup)
        msg, _ = run_timed_graphs(st, args.rotate, args.steps, args.warmup)
        res["two_stream_overlap"] = {
            "what": "independent CSA and HCA batches overlapped on two streams (both compress "
                    "steps in one launch, HCA attention beside the CSA chain)",
            "step_us": round(ms2 * 1e3, 2),
            "query_token_layers_per_s": round((c.B + h.B) / (ms2 * 1e-3), 1),
            "hip_graph_replay_step_us": round(msg * 1e3, 2),
        }
        log("two-stream overlap: " + json.dumps(res["two_stream_overlap"]))
    if not args.no_extra_decode:
        log("csa decode 128k")
        res["csa_decode_128k"] = csa_128k_section(dev, args.steps)
        log("csa decode 128k: " + json.dumps(res["csa_decode_128k"]))
        log("layer stack")
        res["decode_stack"] = stack_section(dev, max(10, args.steps // 2))
        log("layer stack: " + json.dumps(res["decode_stack"]))
    if not args.no_ragged:
        log("ragged decode")
        res["ragged_decode"] = ragged_section(dev, inp, args.steps)
        log("ragged decode: " + json.dumps(res["ragged_decode"]))
    if not args.no_prefill:
        log("prefill chunk")
        res["prefill"] = prefill_section(dev, 3)
        log("prefill (ms): " + ", ".join(f"{k} {v}" for k, v in res["prefill"]["ms"].items()))
    if not args.no_fp8:
        for fmt in ("fp8", "mxfp4"):
            log(f"{fmt} indexer")
            sec = low_precision_indexer_section(dev, st, launches, 3, fmt)
            res[f"{fmt}_indexer"] = sec
            log(f"{fmt} indexer: " + json.dumps(sec["decode"]) +
                f", prefill index_topk {sec['prefill_index_topk_ms']} ms")
    if not args.no_nsa:
        log("nsa variant")
        res["nsa_variant"] = nsa_section(dev, 20)
        log("nsa variant: " + json.dumps(res["nsa_variant"]))
    if not args.no_backward:
        log("csa layer backward")
        res["backward"] = backward_section(dev, 3)
        log("backward: " + json.dumps(res["backward"]))
    if not args.no_cpu_baseline:
        log("cpu baseline (float64 oracle)")
        res["cpu_baseline"] = cpu_baseline(inp, dev, args.cpu_seconds, not args.no_prefill)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
