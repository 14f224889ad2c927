#!/usr/bin/env python3
"""Throughput of the block-sparse attention paths on one MI355X.

Headline (the JSON line's `value`): tokens/s of the whole prefill path —
pooled block scores, top-k + window selection, block-sparse attention — on
the largest prefill workload that fits one GPU, the bf16 64K mixture
workload (B=1, 32 query / 8 KV heads, D=128, S=65536, block 128, top-32
blocks + 1024-token window, keys from an 8-cluster mixture), inputs resident
in HBM.  `roofline` is its attention kernel: effective FLOPs on selected
blocks over the kernel's average launch time (HIP events on the launch
stream) against the bf16 MFMA peak, with HBM traffic from committed counter
summaries while the kernel source is unchanged.  The line also carries the
16K prefill workload, the decode path's HBM rate on the 128K-page workload
(with its own roofline block and a plain read stream as the achievable
ceiling), the three-branch workload, the backward of the 16K attention, the
per-query-head selection and value-driven mask variants, decode over a
paged pool with variable lengths, and the CPU oracle timed on a bounded
sample of the headline workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--only prefill|prefill16k|decode|nsa|nsa_tokens|backward|per_head|dma|paged]
                    [--copy-calibration]
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6     # MI355X dense bf16 (no sparsity)
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E
METRIC = "sparse-attn prefill tokens/s + effective TFLOP/s; decode HBM GB/s (1 GPU)"


ATTN_KERNEL = "k_attn_bf16_d128_pipe"
CSRC = os.path.join(ROOT, "dynamic_block_sparse_head_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
ATTN_TRAFFIC = (os.path.join(PROFILES, "k_attn_bf16_d128_pipe_prefill64k_traffic.txt"),
                os.path.join(CSRC, "k_attn.hip"))
ATTN16K_TRAFFIC = (os.path.join(PROFILES, "k_attn_bf16_d128_pipe_prefill16k_traffic.txt"),
                   os.path.join(CSRC, "k_attn.hip"))
DECODE_TRAFFIC = (os.path.join(PROFILES, "k_decode_split_decode128k_traffic.txt"),
                  os.path.join(CSRC, "k_decode.hip"))


def _measured_traffic(spec, key="hbm_bytes_per_launch"):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by what the same counters read for a
    plain copy of known size), or None when the summary is missing or was
    taken on a different version of the kernel source."""
    import hashlib
    path, source = spec
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, val = line.split(":", 1)
                    kv[k.strip()] = val.strip().split()[0]
        with open(source, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if kv.get("source_sha256") != sha:
            return None
        return int(float(kv[key]))
    except (OSError, KeyError, ValueError, IndexError):
        return None


def _progress(msg):
    """One line per finished stage on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _timed(fn, iters, torch):
    """Average ms per call of fn over `iters` back-to-back calls on the
    current stream (HIP events recorded on that stream)."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def _timed_each(fn, iters, torch):
    """Per-call ms of `iters` calls, each bracketed by its own HIP events on
    the current stream: (median, min, max)."""
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for e0, e1 in ev:
        e0.record(s)
        fn()
        e1.record(s)
    ev[-1][1].synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return t[len(t) // 2], t[0], t[-1]


def bench_prefill(cfg, steps, warmup, torch):
    """One prefill workload: the whole step (scores + selection + attention)
    timed back to back over `steps` steps, the same step replayed as a HIP
    graph, and each kernel alone (back-to-back average and per-call median,
    min, max of the attention).  Effective FLOPs count every selected block
    as a full tile: 4 D block^2 per (query head, selected key block)."""
    from dynamic_block_sparse_head_amd import inputs
    from dynamic_block_sparse_head_amd.pipeline import GraphedStep, PrefillPlan

    c = cfg
    x = inputs.prefill_inputs(c, seed=0, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, q.dtype, "cuda")
    for _ in range(warmup):
        plan.run(q, k, v)
    torch.cuda.synchronize()
    ms_step = _timed(lambda: plan.run(q, k, v), steps, torch)
    torch.cuda.synchronize()
    step = GraphedStep(lambda: plan.run(q, k, v), warmup=max(1, warmup))
    ms_graph = _timed(step, steps, torch)
    torch.cuda.synchronize()
    reps = max(steps, 10)
    ms_scores = _timed(lambda: plan.score(q, k), reps, torch)
    ms_topk = _timed(plan.select, reps, torch)
    for _ in range(2):   # untimed: the first call after the other kernels finds colder caches
        plan.attend(q, k, v)
    ms_attn = _timed(lambda: plan.attend(q, k, v), reps, torch)
    attn_each = _timed_each(lambda: plan.attend(q, k, v), max(reps, 20), torch)
    sel = int(plan.count.to(torch.int64).sum().item())  # (group, query block, key block) triples
    flops = 4.0 * c.D * c.block * c.block * c.G * sel
    del x, q, k, v, plan, step
    torch.cuda.empty_cache()
    return {"cfg": c, "ms_step": ms_step, "ms_scores": ms_scores, "ms_topk": ms_topk,
            "ms_attn": ms_attn, "ms_graph": ms_graph, "selected_block_pairs": sel,
            "effective_flops": flops, "attn_each": attn_each, "tokens_per_step": c.B * c.S}


def _workload(c):
    keys = f", {c.n_clusters}-cluster keys" if c.keys == "mixture" else ""
    return (f"{c.name}: B={c.B} Hq={c.Hq} Hkv={c.Hkv} S={c.S} D={c.D} block={c.block} "
            f"top-{c.topk} + window {c.window}{keys} (scores + selection + attention)")


def _roofline(r, traffic_spec):
    tflops = r["effective_flops"] / (r["ms_attn"] * 1e-3) / 1e12
    med = r["attn_each"][0]
    return {"bound": "mfma", "kernel": ATTN_KERNEL,
            "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": _measured_traffic(traffic_spec),
            "flops_per_launch": r["effective_flops"],
            "avg_launch_ms": round(r["ms_attn"], 4),
            "per_call_ms_median_min_max": [round(x, 4) for x in r["attn_each"]],
            "frac_at_per_call_median": round(r["effective_flops"] / (med * 1e-3) / 1e12
                                             / MFMA_BF16_PEAK_TFLOPS, 4)}


def _prefill_detail(r):
    c = r["cfg"]
    tflops = r["effective_flops"] / (r["ms_attn"] * 1e-3) / 1e12
    return {"workload": _workload(c),
            "ms_per_step": round(r["ms_step"], 4),
            "tokens_per_s": round(r["tokens_per_step"] / (r["ms_step"] * 1e-3), 1),
            "step_ms_graph_replay": round(r["ms_graph"], 4),
            "scores_ms": round(r["ms_scores"], 4), "topk_ms": round(r["ms_topk"], 4),
            "attn_ms": round(r["ms_attn"], 4),
            "attn_ms_per_call_median_min_max": [round(x, 4) for x in r["attn_each"]],
            "attn_tokens_per_s": round(c.S / (r["ms_attn"] * 1e-3), 1),
            "selected_block_pairs": r["selected_block_pairs"],
            "attn_effective_tflops": round(tflops, 2),
            "attn_frac_of_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}


def bench_decode(torch, iters=20, n_query_sets=4):
    """Decode step on the 128K cache: page bounds -> top 1/20 pages ->
    attention.  Between timed iterations a 1 GiB buffer is read (not timed)
    so the last-level cache holds no selected pages; reading (not writing)
    leaves no dirty lines whose write-back would steal bandwidth from the
    timed step.  The query rotates among several sets with their own
    selections."""
    from dynamic_block_sparse_head_amd import configs, inputs
    from dynamic_block_sparse_head_amd.pipeline import DecodePlan, GraphedStep
    from dynamic_block_sparse_head_amd.metrics import decode_selected_bytes

    c = configs.DECODE_128K
    x = inputs.decode_inputs(c, seed=0, device="cuda")
    qs = [inputs.decode_inputs(c.__class__(**{**c.__dict__, "L": c.page}), seed=s, device="cuda")["q"]
          for s in range(1, n_query_sets + 1)]
    plan = DecodePlan(c.B, c.Hq, c.Hkv, c.L, c.D, c.page, c.topk, x["q"].dtype, "cuda")
    plan.build_metadata(x["k"])
    flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    s = torch.cuda.current_stream()
    t_step = t_attn = t_meta = t_graph = 0.0
    plan.run(qs[0], x["k"], x["v"])
    for it in range(iters):
        q = qs[it % n_query_sets]
        flush.max()   # read-only sweep of 1 GiB
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(s)
        plan.score(q)
        plan.select()
        e[1].record(s)
        plan.attend(q, x["k"], x["v"])
        e[2].record(s)
        e[2].synchronize()
        t_step += e[0].elapsed_time(e[2])
        t_attn += e[1].elapsed_time(e[2])
    # the whole step as one HIP graph; the query is copied into its input first
    q_in = qs[0].clone()
    step = GraphedStep(lambda: plan.run(q_in, x["k"], x["v"]))
    for it in range(iters):
        q_in.copy_(qs[it % n_query_sets])
        flush.max()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(s)
        step()
        e[1].record(s)
        e[1].synchronize()
        t_graph += e[0].elapsed_time(e[1])
    # yardsticks: the library's plain read stream over the 1 GiB buffer (the
    # achievable read rate), and a plain device copy of 512 MiB (read + write)
    from dynamic_block_sparse_head_amd import binding as L
    sink = torch.zeros(L.load().dsa_read_stream_sink_words(), dtype=torch.int32, device="cuda")
    L.dsa_read_stream(flush, sink)
    read_ms = _timed(lambda: L.dsa_read_stream(flush, sink), 5, torch)
    read_gbs = flush.numel() * 4 / (read_ms * 1e-3) / 1e9
    src = flush[: (1 << 27)]
    dst = torch.empty_like(src)
    dst.copy_(src)
    copy_ms = _timed(lambda: dst.copy_(src), 5, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    plan.build_metadata(x["k"])
    e1.record(s)
    e1.synchronize()
    t_meta = e0.elapsed_time(e1)
    ms_step, ms_attn = t_step / iters, t_attn / iters
    sel_bytes = decode_selected_bytes(c.B, c.Hkv, c.topk, c.page, c.D)
    meta_bytes = 2 * c.B * c.Hkv * c.n_pages * c.D * 2
    cache_bytes = 2 * c.B * c.Hkv * c.L * c.D * 2
    gbs = sel_bytes / (ms_attn * 1e-3) / 1e9
    copy_gbs = 2 * src.numel() * 4 / (copy_ms * 1e-3) / 1e9
    ms_graph = t_graph / iters
    del x, qs, plan, flush, src, dst, step, q_in, sink
    torch.cuda.empty_cache()
    return {"workload": f"{c.name}: B=16 L=131072 page=64 Hq=32 Hkv=8 D=128, top {c.topk} of "
                        f"{c.n_pages} pages; LLC swept by a 1 GiB read between steps",
            "roofline": {"bound": "hbm", "kernel": "k_decode_split + k_decode_merge",
                         "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": _measured_traffic(DECODE_TRAFFIC, "fetch_bytes_per_dispatch"),
                         "bytes_per_launch": sel_bytes, "avg_launch_ms": round(ms_attn, 4),
                         "frac_of_read_stream": round(gbs / read_gbs, 4)},
            "ms_per_step": round(ms_step, 4), "tokens_per_s": round(c.B / (ms_step * 1e-3), 1),
            "ms_per_step_graph_replay": round(ms_graph, 4),
            "attn_ms": round(ms_attn, 4), "selected_bytes": sel_bytes,
            "attn_hbm_gbs": round(gbs, 1), "attn_frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "step_gbs_incl_metadata": round((sel_bytes + meta_bytes) / (ms_step * 1e-3) / 1e9, 1),
            "full_cache_bytes": cache_bytes,
            "read_stream_gbs": round(read_gbs, 1),
            "device_copy_gbs": round(copy_gbs, 1),
            "page_metadata_build_ms": round(t_meta, 3)}


def bench_paged(torch, iters=20, n_query_sets=4):
    """Serving decode over a paged pool: 16 sequences whose lengths are drawn
    uniformly in [64K, 128K] tokens share one pool of 64-token pages placed in
    random order; per step: page bounds through the page table, top 102 pages
    per (sequence, KV head), attention over their written tokens.  The LLC is
    swept by a 1 GiB read between steps, as for the contiguous decode."""
    import numpy as np
    from dynamic_block_sparse_head_amd import binding as L
    from dynamic_block_sparse_head_amd import configs
    from dynamic_block_sparse_head_amd.pipeline import PagedDecodePlan

    c = configs.DECODE_128K
    rng = np.random.default_rng(2025)
    lens = rng.integers(c.L // 2, c.L + 1, size=c.B)
    npg = -(-lens // c.page)
    max_pages = int(npg.max())
    n_pool = int(npg.sum()) + 8
    perm = rng.permutation(n_pool)
    table = np.zeros((c.B, max_pages), dtype=np.int32)
    off = 0
    for b in range(c.B):
        table[b, :npg[b]] = perm[off:off + npg[b]]
        off += npg[b]
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    shape = (n_pool, c.Hkv, c.page, c.D)
    k_pool = torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16)
    v_pool = torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16)
    # page summaries of the whole pool: one sequence of n_pool * Hkv pages
    kmin = torch.empty((n_pool, c.Hkv, c.D), dtype=torch.bfloat16, device="cuda")
    kmax = torch.empty_like(kmin)
    L.dsa_page_minmax(k_pool.view(1, 1, -1, c.D), c.page, kmin.view(1, 1, -1, c.D),
                      kmax.view(1, 1, -1, c.D))
    table_d = torch.from_numpy(table).to("cuda")
    seq = torch.from_numpy(lens.astype(np.int32)).to("cuda")
    plan = PagedDecodePlan(c.B, c.Hq, c.Hkv, c.D, c.page, max_pages, c.topk, "cuda")
    qs = [torch.randn((c.B, c.Hq, c.D), generator=g, device="cuda", dtype=torch.bfloat16)
          for _ in range(n_query_sets)]
    flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    sel_bytes = []
    for q in qs:                       # bytes of the written tokens of the selected pages
        plan.run(q, k_pool, v_pool, kmin, kmax, table_d, seq)
        idx, cnt = plan.idx.cpu().numpy()[:, :, 0], plan.count.cpu().numpy()[:, :, 0]
        tot = 0
        for b in range(c.B):
            for h in range(c.Hkv):
                for p in idx[b, h, :cnt[b, h]]:
                    if 0 <= p < npg[b]:
                        tot += min(c.page, int(lens[b]) - int(p) * c.page)
        sel_bytes.append(tot * c.D * 2 * 2)
    t_step = t_attn = 0.0
    for it in range(iters):
        q = qs[it % n_query_sets]
        flush.max()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(s)
        plan.score(q, kmin, kmax, table_d, seq)
        plan.select()
        e[1].record(s)
        plan.attend(q, k_pool, v_pool, table_d, seq)
        e[2].record(s)
        e[2].synchronize()
        t_step += e[0].elapsed_time(e[2])
        t_attn += e[1].elapsed_time(e[2])
    # appending one token to every sequence (each call grows seq by one)
    kn = torch.randn((c.B, c.Hkv, c.D), generator=g, device="cuda", dtype=torch.bfloat16)
    ms_append = _timed(lambda: plan.append(kn, kn, table_d, seq, k_pool, v_pool, kmin, kmax), 8, torch)
    ms_step, ms_attn = t_step / iters, t_attn / iters
    nbytes = float(np.mean(sel_bytes))
    gbs = nbytes / (ms_attn * 1e-3) / 1e9
    del k_pool, v_pool, kmin, kmax, plan, flush, qs
    return {"workload": f"paged pool: B=16 lengths U[64K,128K] (total {int(lens.sum())} tokens), "
                        f"page=64 in random pool order, Hq=32 Hkv=8 D=128, top {c.topk} pages",
            "ms_per_step": round(ms_step, 4), "tokens_per_s": round(c.B / (ms_step * 1e-3), 1),
            "attn_ms": round(ms_attn, 4), "selected_bytes": int(nbytes),
            "attn_hbm_gbs": round(gbs, 1), "attn_frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "append_us": round(ms_append * 1e3, 2)}


def bench_per_head(torch, iters=10):
    """The 16K prefill path with per-query-head selection (every query head
    ranks blocks by its own pooled score and keeps its own list): scores,
    selection and attention; effective FLOPs count each head's own blocks."""
    from dynamic_block_sparse_head_amd import configs, inputs
    from dynamic_block_sparse_head_amd.pipeline import PrefillPlan

    c = configs.PREFILL_16K
    x = inputs.prefill_inputs(c, seed=0, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, q.dtype, "cuda",
                       per_head=True)
    plan.run(q, k, v)
    ms_step = _timed(lambda: plan.run(q, k, v), iters, torch)
    ms_attn = _timed(lambda: plan.attend(q, k, v), iters, torch)
    sel = int(plan.count.to(torch.int64).sum().item())   # (query head, q-block, k-block) triples
    flops = 4.0 * c.D * c.block * c.block * sel
    del x, q, k, v, plan
    return {"workload": f"{c.name}: per-query-head selection (32 lists per query block)",
            "ms_per_step": round(ms_step, 4), "tokens_per_s": round(c.S / (ms_step * 1e-3), 1),
            "attn_ms": round(ms_attn, 4),
            "attn_effective_tflops": round(flops / (ms_attn * 1e-3) / 1e12, 2),
            "attn_frac_of_mfma_peak": round(flops / (ms_attn * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def bench_dma(torch, iters=10):
    """The 16K workload shape with the value-driven dynamic mask: weights from
    the values, heaviest 16 blocks + 512-token window, attention with each
    kept key's weight added to its logit."""
    from dynamic_block_sparse_head_amd import configs, inputs
    from dynamic_block_sparse_head_amd.pipeline import DMAPlan

    c = configs.PREFILL_16K
    x = inputs.prefill_inputs(c, seed=0, device="cuda")
    proj, gain = inputs.dma_params(c, seed=0, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    plan = DMAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, q.dtype, "cuda")
    plan.run(q, k, v, proj, gain)
    ms_step = _timed(lambda: plan.run(q, k, v, proj, gain), iters, torch)
    ms_w = _timed(lambda: plan.score(v, proj, gain), iters, torch)
    ms_attn = _timed(lambda: plan.attend(q, k, v), iters, torch)
    sel = int(plan.count.to(torch.int64).sum().item())
    flops = 4.0 * c.D * c.block * c.block * c.G * sel
    del x, q, k, v, plan
    return {"workload": f"{c.name} shape, value-driven mask: weights exp(A softplus(v.Delta)), "
                        "top-16 blocks by largest weight + window 512, weights added to logits",
            "ms_per_step": round(ms_step, 4), "tokens_per_s": round(c.S / (ms_step * 1e-3), 1),
            "weights_ms": round(ms_w, 4), "attn_ms": round(ms_attn, 4),
            "attn_effective_tflops": round(flops / (ms_attn * 1e-3) / 1e12, 2),
            "attn_frac_of_mfma_peak": round(flops / (ms_attn * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def bench_backward(torch, iters=10, warmup=10):
    """Gradients of the 16K prefill's attention (dq, dk, dv) for an N(0,1)
    upstream gradient, the forward's selection held fixed.  Effective FLOPs
    count the five products of each selected (query block, key block, head)
    tile once: S = QK^T, dP = dO V^T, dQ, dK, dV, 2 D block^2 each."""
    from dynamic_block_sparse_head_amd import configs, inputs
    from dynamic_block_sparse_head_amd.pipeline import PrefillPlan

    c = configs.PREFILL_16K
    x = inputs.prefill_inputs(c, seed=0, device="cuda")
    dout = inputs.grad_output(c, seed=0, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, q.dtype, "cuda")
    plan.run(q, k, v)
    # untimed: like the three-branch step, the first calls of a series run
    # slower (~2.1 ms settling to ~1.8 ms over its first ten or so)
    for _ in range(warmup):
        plan.backward(q, k, v, dout)
    ms = _timed(lambda: plan.backward(q, k, v, dout), iters, torch)
    sel = int(plan.count.to(torch.int64).sum().item())
    flops = 10.0 * c.D * c.block * c.block * c.G * sel
    del x, q, k, v, plan, dout
    return {"workload": f"{c.name}: gradients of the attention step (selection held fixed)",
            "ms_per_call": round(ms, 4), "tokens_per_s": round(c.S / (ms * 1e-3), 1),
            "effective_flops": flops,
            "effective_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_of_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def bench_nsa(torch, iters=10, warmup=10):
    from dynamic_block_sparse_head_amd import configs, inputs
    from dynamic_block_sparse_head_amd.pipeline import NSAPlan

    c = configs.NSA_32K
    x = inputs.nsa_inputs(c, seed=0, device="cuda")
    p = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k, c.window,
                x["q"].dtype, "cuda")
    args = (x["q"], x["k"], x["v"], x["z"])
    # untimed: the first steps of a series run slower (on an MI355X the step
    # settles from ~5.6 to ~3.6 ms over its first ten runs)
    for _ in range(warmup):
        p.run(*args)
    ms = _timed(lambda: p.run(*args), iters, torch)
    step_each = _timed_each(lambda: p.run(*args), iters, torch)
    # the step's calls one by one (same inputs, outputs rewritten identically)
    from dynamic_block_sparse_head_amd import binding as L
    q, k, v, z = args
    calls = {
        "compress": lambda: L.dsa_nsa_compress(k, v, c.cmp_len, c.cmp_stride, p.ck, p.cv),
        "cmp_attn": lambda: L.dsa_nsa_cmp_attn(q, p.ck, p.cv, c.cmp_len, c.cmp_stride, c.sel_block,
                                               p.scale, p.o_cmp, p.lse_cmp),
        "cmp_attn_with_block_scores": lambda: L.dsa_nsa_cmp_attn(
            q, p.ck, p.cv, c.cmp_len, c.cmp_stride, c.sel_block, p.scale, p.o_cmp, p.lse_cmp,
            p.scores),
        "topk": lambda: L.dsa_topk_select(p.scores, c.sel_k, 0, True, p.idx, p.count),
        "selected_attn": lambda: L.dsa_sparse_attn_prefill(q, k, v, p.idx, p.count, c.sel_block, 0,
                                                           p.scale, p.o_sel),
        "window_attn": lambda: L.dsa_sparse_attn_prefill(q, k, v, None, None, c.sel_block,
                                                         c.window, p.scale, p.o_win),
        "combine": lambda: L.dsa_nsa_combine(p.o_cmp, p.o_sel, p.o_win, z, p.out),
        "window_attn_with_combine": lambda: L.dsa_nsa_window_combine(
            q, k, v, c.window, p.scale, p.o_cmp, p.o_sel, z, p.out),
        "selected_window_combine_one_pass": lambda: L.dsa_nsa_select_window_combine(
            q, k, v, p.idx, p.count, c.sel_block, c.window, p.scale, p.o_cmp, z, p.out),
    }
    per_call = {}
    for name, fn in calls.items():
        fn()   # one untimed call first: each call's first launch in a series is not timed
        per_call[name] = round(_timed(fn, iters, torch), 4)
    # exact-pair FLOPs of branches 1 and 3, selected-block FLOPs of branch 2
    S, G, D = c.S, c.G, c.D
    f1 = sum(max(0, (t - (c.cmp_len - 1)) // c.cmp_stride + 1) if t >= c.cmp_len - 1 else 0
             for t in range(S)) * 4.0 * D * c.Hq
    f2 = 4.0 * D * c.sel_block * c.sel_block * G * int(p.count.to(torch.int64).sum().item())
    f3 = sum(min(t + 1, c.window) for t in range(S)) * 4.0 * D * c.Hq
    del x, p
    return {"workload": f"{c.name}: S=32768 Hq=64 Hkv=4 D=128; summaries 32/16, top-16 of 64-token "
                        "blocks, window 512, sigmoid gates",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(S / (ms * 1e-3), 1),
            "step_ms_per_call_median_min_max": [round(t, 4) for t in step_each],
            "branch_flops": f1 + f2 + f3,
            "effective_tflops_whole_step": round((f1 + f2 + f3) / (ms * 1e-3) / 1e12, 2),
            "per_call_ms": per_call,
            "cmp_attn_tflops": round(f1 / (per_call["cmp_attn"] * 1e-3) / 1e12, 2),
            "selected_attn_tflops": round(f2 / (per_call["selected_attn"] * 1e-3) / 1e12, 2),
            "window_attn_tflops": round(f3 / (per_call["window_attn"] * 1e-3) / 1e12, 2)}


def bench_nsa_tokens(torch, iters=5):
    """The 32K three-branch step with per-token selection (every query token
    ranks the blocks of its group from its own compressed-branch attention):
    per-kernel times and the selected branch's rate.  Its FLOPs count each
    (token, listed block) pair as 4 D x block x G, as the block-level figure
    counts each (query block, key block) pair."""
    from dynamic_block_sparse_head_amd import binding as L
    from dynamic_block_sparse_head_amd import configs, inputs
    from dynamic_block_sparse_head_amd.pipeline import NSAPlan

    c = configs.NSA_32K
    x = inputs.nsa_inputs(c, seed=0, device="cuda")
    p = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k, c.window,
                x["q"].dtype, "cuda", per_token=True)
    q, k, v, z = x["q"], x["k"], x["v"], x["z"]
    for _ in range(5):   # untimed warm-up steps
        p.run(q, k, v, z)
    ms = _timed(lambda: p.run(q, k, v, z), iters, torch)
    ms_scores = _timed(lambda: L.dsa_nsa_cmp_token_scores(q, p.ck, p.lse_cmp, c.cmp_len,
                                                          c.cmp_stride, c.sel_block, p.scale,
                                                          p.scores), iters, torch)
    ms_topk = _timed(lambda: L.dsa_topk_select_tokens(p.scores, c.sel_k, 0, c.sel_block, p.idx,
                                                      p.count), iters, torch)
    ms_attn = _timed(lambda: L.dsa_sparse_attn_tokens(q, k, v, p.idx, p.count, c.sel_block,
                                                      p.scale, p.o_sel), iters, torch)
    pairs = int(p.count.to(torch.int64).sum().item())      # (token, group, block) triples
    flops = 4.0 * c.D * c.sel_block * c.G * pairs
    # K/V bytes the selected branch would read with no sharing between tokens
    kv_unshared = pairs * c.sel_block * c.D * 2 * 2
    del x, p, q, k, v, z
    return {"workload": f"{c.name}: per-token selection, S=32768 Hq=64 Hkv=4 D=128; summaries "
                        "32/16, top-16 of 64-token blocks per token, window 512, sigmoid gates",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(c.S / (ms * 1e-3), 1),
            "token_scores_ms": round(ms_scores, 4), "topk_ms": round(ms_topk, 4),
            "selected_attn_ms": round(ms_attn, 4),
            "selected_attn_effective_tflops": round(flops / (ms_attn * 1e-3) / 1e12, 2),
            "selected_attn_frac_of_mfma_peak": round(flops / (ms_attn * 1e-3) / 1e12
                                                     / MFMA_BF16_PEAK_TFLOPS, 4),
            "selected_attn_unshared_kv_gb": round(kv_unshared / 1e9, 2)}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s=20.0):
    """The oracle, untouched, on a bounded sample of the headline workload:
    pooled scores and selection for every query block, then attention (all
    32 heads) for query blocks spread over the sequence until the time
    budget is used; the whole workload's time is extrapolated per block."""
    import torch

    from dynamic_block_sparse_head_amd import configs, inputs
    from oracle import prefill as Op

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    c = configs.PREFILL_64K
    x = inputs.prefill_inputs(c, seed=0, device="cpu")
    t0 = time.perf_counter()
    q = x["q"].to(torch.float64).numpy()
    k = x["k"].to(torch.float64).numpy()
    v = x["v"].to(torch.float64).numpy()
    s = Op.block_scores_pooled(q, k, c.block)
    idx, cnt = Op.select_blocks(s, c.topk, c.n_local, causal=True)
    t_sel = time.perf_counter() - t0
    order = list(range(c.n_blocks - 1, -1, -13)) + list(range(c.n_blocks - 7, -1, -13))
    done, flops = 0, 0.0
    t1 = time.perf_counter()
    for i in order:
        Op.sparse_attention(q, k, v, idx, cnt, c.block, c.scale, q_blocks=[i])
        done += 1
        flops += 4.0 * c.D * c.block * c.block * c.G * float(cnt[0, :, i].sum())
        if time.perf_counter() - t1 > budget_s:
            break
    t_attn = time.perf_counter() - t1
    per_block = t_attn / done
    est_total = t_sel + per_block * c.n_blocks          # the whole workload at this rate
    return {"value": round(c.S / est_total, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "cpu_model": _cpu_model(),
            "oracle_attn_gflops": round(flops / t_attn / 1e9, 2),
            "sample": (f"{c.name}: float64 numpy oracle; scores + selection for all {c.n_blocks} "
                       f"query blocks ({t_sel:.1f} s), attention for {done} of {c.n_blocks} query "
                       f"blocks spread over the sequence (all 32 heads, {t_attn:.1f} s, "
                       f"{flops / 1e12:.2f} effective TFLOP); tokens/s = S / (selection time + "
                       f"per-block attention time x {c.n_blocks}); BLAS threads {threads}, "
                       f"host cpus {len(os.sched_getaffinity(0))}")}


def copy_calibration(torch, nbytes=1 << 30, reps=3):
    """A plain device copy of known size, for scaling HBM byte counters."""
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "prefill16k", "decode", "nsa", "nsa_tokens",
                                       "backward", "per_head", "dma", "paged"], default=None)
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): this library's "
              "paths run on a single MI355X; multi-GPU sharding is a design note, not a run.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    from dynamic_block_sparse_head_amd import binding
    binding.load()
    # no garbage-collection pauses inside timed regions: a pause between two
    # event records leaves the GPU idle and counts against a short kernel
    # (one such 39 ms pause once showed up as a 2 ms decode average); each
    # leg collects before it starts
    gc.collect()
    gc.disable()

    if args.copy_calibration:
        copy_calibration(torch)
        return

    extra = {}
    if args.only in (None, "prefill"):
        from dynamic_block_sparse_head_amd import configs
        r = bench_prefill(configs.PREFILL_64K, args.steps, args.warmup, torch)
        c = r["cfg"]
        line = {
            "metric": METRIC,
            "value": round(r["tokens_per_step"] / (r["ms_step"] * 1e-3), 1),
            "unit": "tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(r["ms_step"], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": _workload(c), "global_batch": c.B, "seq_len": c.S,
                       "parallelism": "single GPU"},
            "roofline": _roofline(r, ATTN_TRAFFIC),
            "prefill_64k": _prefill_detail(r),
        }
    else:
        line = {"metric": METRIC, "n_gpus": 1}
    if args.only in (None, "prefill16k"):
        from dynamic_block_sparse_head_amd import configs
        gc.collect()
        r16 = bench_prefill(configs.PREFILL_16K, args.steps, args.warmup, torch)
        extra["prefill_16k"] = {**_prefill_detail(r16), "roofline": _roofline(r16, ATTN16K_TRAFFIC)}
    legs = [("decode", "decode", bench_decode), ("nsa", "nsa", bench_nsa),
            ("nsa_tokens", "nsa_per_token", bench_nsa_tokens),
            ("backward", "backward", bench_backward),
            ("per_head", "per_head_selection", bench_per_head), ("dma", "dma_mask", bench_dma),
            ("paged", "paged_decode", bench_paged)]
    _progress("prefill legs done")
    for only, key, fn in legs:
        if args.only in (None, only):
            gc.collect()
            extra[key] = fn(torch)
            _progress(f"{key} done")
    line.update(extra)
    gc.enable()
    if not args.no_cpu_baseline and args.only in (None, "prefill"):
        line["cpu_baseline"] = cpu_baseline()
        _progress("cpu baseline done")
    print(json.dumps(line))


if __name__ == "__main__":
    main()
