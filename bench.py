#!/usr/bin/env python
"""Benchmark of the HiLS attention forward hot path on one MI355X.

One step = one prefill pass over the 128K-token workload (landmark summary ->
score/select -> fused sparse attention, inputs resident in HBM), timed with
HIP events on the stream the kernels run on.  The same run times one decode
step over the 512K-token paged-cache workload (16 sequences), the dense
causal attention baselines of both (the full attention that the pages quote
HiLS's speedups against), and the fp64 CPU oracle on a bounded sample of the
prefill workload.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 / fp16 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector
METRIC = "HiLS prefill tokens/s @128K + decode μs/step @512K; % MFMA/HBM peak"
CSRC = os.path.join(ROOT, "long_context_chunk_landmark_amd", "csrc")


# ---------------------------------------------------------------- algorithmic work

def _chunks(cfg, q0=0):
    """Per query chunk of positions q0 .. q0 + N - 1 (q0 % S == 0): (first
    query, #queries, #candidates, #selected)."""
    S, w = cfg.S, cfg.W // cfg.S
    out = []
    end = q0 + cfg.N
    for qc in range(q0 // S, (end + S - 1) // S):
        n_q = min(S, end - qc * S)
        n_c = max(0, qc - w)
        out.append((qc * S, n_q, n_c, min(cfg.K, n_c)))
    return out


def attend_flops(cfg, q0=0):
    """4 d H_q sum_i (selected keys + window keys): QK^T and PV, 2 flops/MAC."""
    S = cfg.S
    keys = 0
    for i0, n_q, n_c, k in _chunks(cfg, q0):
        ws = max(0, i0 - cfg.W)
        # window of query i: keys [ws, i]; sum over the chunk's queries
        win = n_q * (i0 - ws) + n_q * (n_q + 1) // 2
        keys += n_q * k * S + win
    return 4.0 * cfg.d * cfg.H_q * keys * cfg.B


def score_flops(cfg, q0=0):
    return 2.0 * cfg.d * cfg.H_q * cfg.B * sum(n_q * n_c for _, n_q, n_c, _ in _chunks(cfg, q0))


def summary_bytes(cfg, io_bytes, sum_bytes):
    C = cfg.N // cfg.S
    return cfg.B * (cfg.H_kv * C * cfg.S * cfg.d * io_bytes + cfg.H_lm * C * cfg.d * io_bytes +
                    cfg.H_lm * C * cfg.d * sum_bytes + cfg.H_lm * C * 4)


def decode_bytes(cfg, seq_lens, io_bytes, sum_bytes):
    """Summaries of every candidate + K/V of the selected chunks and window
    tokens + block-table entries + q and out."""
    S, w = cfg.S, cfg.W // cfg.S
    total = 0
    for L in seq_lens:
        t = L - 1
        n_c = max(0, t // S - w)
        k = min(cfg.K, n_c)
        win = t - max(0, (t // S) * S - cfg.W) + 1
        total += cfg.H_lm * n_c * (cfg.d * sum_bytes + 4)
        total += cfg.H_kv * (k * S + win) * cfg.d * io_bytes * 2
        total += ((t // S) + 1) * 4
        total += 2 * cfg.H_q * cfg.d * io_bytes
    return total


# ---------------------------------------------------------------- rocprof counters

def _source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_file, workload, sources):
    """HBM bytes per launch from the committed counter summary, or None when
    missing or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel_file}_{workload}.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"source_sha:\s*(\w+)", txt)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not b or m.group(1) != _source_sha(sources):
        return None
    return float(b.group(1))


# ---------------------------------------------------------------- timing

def _timed(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = []
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        evs.append(fn())
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    per = {}
    for step_evs in evs:
        for name, (a, b) in step_evs.items():
            per.setdefault(name, []).append(a.elapsed_time(b))
    return total_ms, {k: sum(v) / len(v) for k, v in per.items()}


def bench_prefill(args, torch, hb, W, workload=None, steps=None, warmup=None):
    dev = torch.device("cuda:0")
    inp = W.make_prefill(workload or args.workload, device=dev)
    cfg = inp["cfg"]
    qcal = inp.get("qcal")
    q, k, v, q_lm = inp["q"], inp["k"], inp["v"], inp["q_lm"]
    C = cfg.C
    k_sum = torch.empty((cfg.B, cfg.H_lm, C, cfg.d), dtype=cfg.summary_dtype, device=dev)
    b_sum = torch.empty((cfg.B, cfg.H_lm, C), dtype=torch.float32, device=dev)
    sel = torch.empty((cfg.B, cfg.H_kv, cfg.N, cfg.K), dtype=torch.int32, device=dev)
    ss = torch.empty((cfg.B, cfg.H_q, cfg.N, cfg.K), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((cfg.B, cfg.H_q, cfg.N), dtype=torch.float32, device=dev)
    ws_s = torch.empty(hb.workspace_size(cfg, hb.WS_SCORE_QCAL if qcal else hb.WS_SCORE), dtype=torch.uint8,
                       device=dev)
    ws_f = torch.empty(max(1, hb.workspace_size(cfg, hb.WS_FUSED)), dtype=torch.uint8, device=dev)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step():
        e = [E() for _ in range(4)]
        e[0].record()
        hb.landmark_summarize(cfg, k, q_lm, k_sum, b_sum)
        e[1].record()
        hb.score_select(cfg, q, k_sum, b_sum, qcal=qcal, sel_idx=sel, sel_score=ss, workspace=ws_s)
        e[2].record()
        hb.sparse_attend_fused(cfg, q, k, v, sel, ss, out=out, lse=lse, workspace=ws_f)
        e[3].record()
        return {"summary": (e[0], e[1]), "score_select": (e[1], e[2]), "fused": (e[2], e[3])}

    steps = steps or args.steps
    total_ms, per = _timed(step, steps, args.warmup if warmup is None else warmup, torch)
    res = dict(cfg=cfg, inp=inp, ms_per_step=total_ms / steps, per_call_ms=per, sel=sel, ss=ss, out=out, lse=lse,
               fused_workspace_bytes=ws_f.numel())
    del ws_f
    return res


def attend_form(hb, cfg):
    """The selected-chunk form hils_sparse_attend_fused takes for cfg (auto:
    chunk-major for bf16 I/O with selections, the walk otherwise)."""
    m = cfg.attend_mode
    if m == hb.ATTEND_AUTO:
        import torch
        m = hb.ATTEND_CHUNK_MAJOR if cfg.io_dtype == torch.bfloat16 and cfg.K > 0 else hb.ATTEND_WALK
    return "chunk-major" if m == hb.ATTEND_CHUNK_MAJOR else "walk"


def fused_other_form(torch, hb, pre, reps=2):
    """hils_sparse_attend_fused in the form auto does not take, on the same
    inputs and selection (one untimed call, then reps timed calls): ms per call."""
    import dataclasses

    dev = torch.device("cuda:0")
    cfg, inp = pre["cfg"], pre["inp"]
    other = hb.ATTEND_WALK if attend_form(hb, cfg) == "chunk-major" else hb.ATTEND_CHUNK_MAJOR
    c = dataclasses.replace(cfg, attend_mode=other)
    ws = torch.empty(max(1, hb.workspace_size(c, hb.WS_FUSED)), dtype=torch.uint8, device=dev)
    out, lse = torch.empty_like(pre["out"]), torch.empty_like(pre["lse"])
    hb.sparse_attend_fused(c, inp["q"], inp["k"], inp["v"], pre["sel"], pre["ss"], out=out, lse=lse, workspace=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        hb.sparse_attend_fused(c, inp["q"], inp["k"], inp["v"], pre["sel"], pre["ss"], out=out, lse=lse,
                               workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    nb = ws.numel()
    del ws, out, lse
    torch.cuda.empty_cache()
    return {"form": attend_form(hb, c), "ms": e0.elapsed_time(e1) / reps, "workspace_bytes": nb}


def bench_decode(args, torch, hb, W):
    """The decode workload's step over a summary cache built by kernel 1 from
    the K cache and seeded landmark queries, then secondary summary layouts
    over the same K/V cache: one landmark head per kv head (H_lm = H_kv, bf16
    k'), fp32 k' (H_lm = H_q), and the normalised aggregation."""
    import dataclasses

    dev = torch.device("cuda:0")
    inp = W.make_decode(args.decode_workload, device=dev)
    cfg = inp["cfg"]
    B = inp["q"].shape[0]
    out = torch.empty((B, cfg.H_q, cfg.d), dtype=cfg.io_dtype, device=dev)
    lse = torch.empty((B, cfg.H_q), dtype=torch.float32, device=dev)
    sel = torch.empty((B, cfg.H_kv, cfg.K), dtype=torch.int32, device=dev)
    max_pages = inp["block_table"].shape[1]
    P = inp["k_cache"].shape[0]

    def run(c, ksum, bsum, steps, warmup):
        ws = torch.empty(hb.workspace_size(c, hb.WS_DECODE, B, max_pages), dtype=torch.uint8, device=dev)

        def step():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            hb.decode(c, inp["q"], inp["k_cache"], inp["v_cache"], ksum, bsum, inp["block_table"], inp["seq_lens"],
                      out=out, lse=lse, sel_idx=sel, workspace=ws)
            e1.record()
            return {"decode": (e0, e1)}

        total_ms, per = _timed(step, steps, warmup, torch)
        return 1000.0 * total_ms / steps, 1000.0 * per["decode"]

    def built_summaries(c, seed):
        """The summary cache as serving builds it: kernel 1 (hils_summarize_pages)
        over every page of the K cache, with seeded N(0, 1) landmark queries."""
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        q_lm = torch.randn((P, c.H_lm, c.d), generator=g, device=dev).to(c.io_dtype)
        ks = torch.empty((P, c.H_lm, c.d), dtype=c.summary_dtype, device=dev)
        bs = torch.empty((P, c.H_lm), dtype=torch.float32, device=dev)
        hb.summarize_pages(c, inp["k_cache"], q_lm, torch.arange(P, dtype=torch.int32, device=dev), ks, bs)
        torch.cuda.synchronize()
        del q_lm
        return ks, bs

    del inp["ksum_cache"], inp["bsum_cache"]
    ksum, bsum = built_summaries(cfg, 41)
    us, call_us = run(cfg, ksum, bsum, args.steps, args.warmup)
    del ksum, bsum
    seq_lens = inp["seq_lens"].cpu().tolist()
    dense_us = None
    if not args.no_dense:
        # the full-attention baseline: every key of each sequence
        wsd = torch.empty(hb.workspace_size(cfg, hb.WS_DENSE_DECODE, B, max_pages), dtype=torch.uint8, device=dev)

        def dstep():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            hb.dense_decode(cfg, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["seq_lens"],
                            out=out, lse=lse, workspace=wsd)
            e1.record()
            return {"dense": (e0, e1)}

        _, dper = _timed(dstep, max(2, args.steps // 2), 1, torch)
        dense_us = 1000.0 * dper["dense"]
        del wsd
    secondary = {}
    for name, c in (("H_lm=H_kv, bf16 k'", dataclasses.replace(cfg, H_lm=cfg.H_kv)),
                    ("H_lm=H_q, fp32 k'", dataclasses.replace(cfg, summary_dtype=torch.float32)),
                    ("H_lm=H_q, bf16 k', normalised aggregation", dataclasses.replace(cfg, agg_mode=hb.AGG_NORMALIZED))):
        ks, bs = built_summaries(c, 43)
        _, cu = run(c, ks, bs, max(2, args.steps // 2), 1)
        secondary[name] = (c, cu)
        del ks, bs
    return dict(cfg=cfg, us_per_step=us, call_us=call_us, seq_lens=seq_lens, secondary=secondary, dense_us=dense_us)


def bench_serving(args, torch, hb, W, pre):
    """Serving continuity on the prefill workload laid out in a paged cache:
    (a) summaries of every completed chunk written page by page
    (hils_summarize_pages); (b) the last args.chunk tokens prefilled as one
    chunk over the paged cache (hils_prefill_paged)."""
    dev = torch.device("cuda:0")
    inp = pre["inp"]
    cfg = pre["cfg"]
    kc, vc, bt = W.paged_layout(inp["k"], inp["v"], cfg.S, seed=17)
    P, C = kc.shape[0], cfg.C
    ks = torch.empty((P, cfg.H_lm, cfg.d), dtype=cfg.summary_dtype, device=dev)
    bs = torch.empty((P, cfg.H_lm), dtype=torch.float32, device=dev)
    bb = torch.arange(cfg.B, device=dev).repeat_interleave(C)
    cc = torch.arange(C, device=dev).repeat(cfg.B)
    pages = bt[bb, cc].contiguous()
    q_items = inp["q_lm"][bb, :, cc].contiguous()
    n = min(args.chunk, cfg.N)
    q_start = (cfg.N - n) // cfg.S * cfg.S
    n = cfg.N - q_start
    import dataclasses

    ccfg = dataclasses.replace(cfg, N=n)
    q = inp["q"][:, :, q_start:].contiguous()
    qcal = inp.get("qcal")
    if qcal is not None:
        qcal = (qcal[0][:, q_start:].contiguous(), qcal[1], qcal[2])
    out = torch.empty_like(q)
    lse = torch.empty((cfg.B, cfg.H_q, n), dtype=torch.float32, device=dev)
    sel = torch.empty((cfg.B, cfg.H_kv, n, cfg.K), dtype=torch.int32, device=dev)
    ss = torch.empty((cfg.B, cfg.H_q, n, cfg.K), dtype=torch.float32, device=dev)
    ws = torch.empty(hb.prefill_paged_workspace_size(ccfg, q_start, bt.shape[1], qcal is not None),
                     dtype=torch.uint8, device=dev)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step():
        e = [E() for _ in range(3)]
        e[0].record()
        hb.summarize_pages(cfg, kc, q_items, pages, ks, bs)
        e[1].record()
        hb.prefill_paged(ccfg, q_start, q, kc, vc, ks, bs, bt, qcal=qcal, out=out, lse=lse, sel_idx=sel,
                         sel_score=ss, workspace=ws)
        e[2].record()
        return {"summarize_pages": (e[0], e[1]), "prefill_paged": (e[1], e[2])}

    _, per = _timed(step, args.steps, args.warmup, torch)
    io_b = 2 if cfg.io_dtype == torch.bfloat16 else 4
    sum_b = 2 if cfg.summary_dtype == torch.bfloat16 else 4
    # the page-by-page summaries move the bytes of the contiguous summary
    # plus the page ids
    by = summary_bytes(cfg, io_b, sum_b) + 4 * cfg.B * C
    ms_s, ms_p = per["summarize_pages"], per["prefill_paged"]
    fl = attend_flops(ccfg, q_start) + score_flops(ccfg, q_start)
    del kc, vc, ks, bs, ws
    return {"workload": f"{args.workload} in a paged cache ({P} pages, random placement)",
            "summarize_pages": {"items": cfg.B * C, "ms": ms_s, "bound": "hbm", "gbs": by / (ms_s * 1e-3) / 1e9,
                                "frac": by / (ms_s * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": by},
            "prefill_paged": {"q_start": q_start, "n": n, "ms": ms_p, "tokens_per_s": cfg.B * n / (ms_p * 1e-3),
                              "tflops": fl / (ms_p * 1e-3) / 1e12, "flops": fl}}


def bench_variants(args, torch, hb, W, pre):
    """The method's variants on the prefill workload: summaries with one
    shared landmark query per head and with mean pooling (q' = 0),
    score/select with the normalised-weight group aggregation, and the
    streaming form of score/select (O(N K) workspace)."""
    import dataclasses

    dev = torch.device("cuda:0")
    inp = pre["inp"]
    cfg = pre["cfg"]
    C = cfg.C
    k_sum = torch.empty((cfg.B, cfg.H_lm, C, cfg.d), dtype=cfg.summary_dtype, device=dev)
    b_sum = torch.empty((cfg.B, cfg.H_lm, C), dtype=torch.float32, device=dev)
    shared_q = inp["q_lm"][0, :, 0].contiguous() if inp["q_lm"] is not None else None
    c_shared = dataclasses.replace(cfg, landmark_mode=hb.LM_SHARED)
    c_mean = dataclasses.replace(cfg, landmark_mode=hb.LM_MEAN)
    c_norm = dataclasses.replace(cfg, agg_mode=hb.AGG_NORMALIZED)
    c_stream = dataclasses.replace(cfg, score_mode=hb.SCORE_STREAMING)
    qcal = inp.get("qcal")
    sel = torch.empty((cfg.B, cfg.H_kv, cfg.N, cfg.K), dtype=torch.int32, device=dev)
    ss = torch.empty((cfg.B, cfg.H_q, cfg.N, cfg.K), dtype=torch.float32, device=dev)
    wk = hb.WS_SCORE_QCAL if qcal else hb.WS_SCORE
    ws = torch.empty(hb.workspace_size(c_norm, wk), dtype=torch.uint8, device=dev)
    ws_stream = torch.empty(hb.workspace_size(c_stream, wk), dtype=torch.uint8, device=dev)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step():
        e = [E() for _ in range(5)]
        e[0].record()
        hb.landmark_summarize(c_shared, inp["k"], shared_q, k_sum, b_sum)
        e[1].record()
        hb.landmark_summarize(c_mean, inp["k"], None, k_sum, b_sum)
        e[2].record()
        hb.score_select(c_norm, inp["q"], k_sum, b_sum, qcal=qcal, sel_idx=sel, sel_score=ss, workspace=ws)
        e[3].record()
        hb.score_select(c_stream, inp["q"], k_sum, b_sum, qcal=qcal, sel_idx=sel, sel_score=ss, workspace=ws_stream)
        e[4].record()
        return {"summary_shared": (e[0], e[1]), "summary_mean": (e[1], e[2]), "score_select_normalized": (e[2], e[3]),
                "score_select_streaming": (e[3], e[4])}

    _, per = _timed(step, max(1, args.steps // 2), 1, torch)
    io_b = 2 if cfg.io_dtype == torch.bfloat16 else 4
    sum_b = 2 if cfg.summary_dtype == torch.bfloat16 else 4
    # shared: the landmark queries shrink to one row per head; mean: none
    by_shared = summary_bytes(cfg, io_b, sum_b) - cfg.B * cfg.H_lm * C * cfg.d * io_b + cfg.H_lm * cfg.d * io_b
    by_mean = summary_bytes(cfg, io_b, sum_b) - cfg.B * cfg.H_lm * C * cfg.d * io_b
    fl = score_flops(cfg)
    out = {}
    for name, by in (("summary_shared", by_shared), ("summary_mean", by_mean)):
        ms = per[name]
        out[name] = {"ms": ms, "bound": "hbm", "gbs": by / (ms * 1e-3) / 1e9,
                     "frac": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": by}
    for name in ("score_select_normalized", "score_select_streaming"):
        ms = per[name]
        out[name] = {"ms": ms, "bound": "mfma", "tflops": fl / (ms * 1e-3) / 1e12,
                     "frac": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "flops": fl}
    out["score_select_streaming"]["workspace_bytes"] = ws_stream.numel()
    out["score_select_streaming"]["two_pass_workspace_bytes"] = hb.workspace_size(
        dataclasses.replace(cfg, score_mode=hb.SCORE_TWO_PASS), wk)
    del ws, ws_stream
    return out


def bench_backward(args, torch, hb, pre):
    """hils_sparse_attend_backward on the prefill workload (gradients of a
    random output / log-partition gradient, the forward's selection)."""
    dev = torch.device("cuda:0")
    inp = pre["inp"]
    cfg = pre["cfg"]
    fw = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    g = torch.Generator(device=dev)
    g.manual_seed(23)
    dout = torch.randn(fw["out"].shape, generator=g, device=dev).to(cfg.io_dtype)
    dlse = torch.randn(fw["lse"].shape, generator=g, device=dev)
    ws = torch.empty(hb.workspace_size(cfg, hb.WS_BACKWARD), dtype=torch.uint8, device=dev)

    def step():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        hb.sparse_attend_backward(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"], fw["k_sum"], fw["sel_idx"],
                                  fw["sel_score"], fw["lse"], dout, dlse, workspace=ws)
        e1.record()
        return {"backward": (e0, e1)}

    _, per = _timed(step, args.backward_steps, 1, torch)
    ms = per["backward"]
    # QK^T recompute, dO V^T, dV, dQ, dK: 2.5x the forward's attention FLOPs.
    # bf16 I/O runs them on bf16 MFMA (fp32 I/O: fp32 VALU)
    fl = 2.5 * attend_flops(cfg)
    mfma = cfg.io_dtype == torch.bfloat16
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_FP32_VALU_TFLOPS
    del fw, dout, dlse, ws
    return {"ms": ms, "bound": "mfma" if mfma else "alu", "tflops": fl / (ms * 1e-3) / 1e12, "peak": peak,
            "unit": "TFLOP/s", "frac": fl / (ms * 1e-3) / 1e12 / peak, "flops": fl,
            "tokens_per_s": cfg.B * cfg.N / (ms * 1e-3)}


def dense_flops(cfg):
    """Dense causal attention: 4 d FLOPs per (query head, query, visible key)."""
    return 4.0 * cfg.d * cfg.H_q * cfg.B * (cfg.N * (cfg.N + 1) / 2)


def bench_dense(torch, hb, pre, steps, hils_ms):
    """hils_dense_causal_attend on the prefill workload's inputs: the
    full-attention baseline of the pages' prefill speed comparison."""
    dev = torch.device("cuda:0")
    inp = pre["inp"]
    cfg = pre["cfg"]
    ws = torch.empty(hb.workspace_size(cfg, hb.WS_DENSE), dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp["q"])
    lse = torch.empty((cfg.B, cfg.H_q, cfg.N), dtype=torch.float32, device=dev)

    def step():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        hb.dense_causal_attend(cfg, inp["q"], inp["k"], inp["v"], out=out, lse=lse, workspace=ws)
        e1.record()
        return {"dense": (e0, e1)}

    _, per = _timed(step, steps, 1, torch)
    ms = per["dense"]
    fl = dense_flops(cfg)
    tfl = fl / (ms * 1e-3) / 1e12
    del ws, out, lse
    return {"kernel": "dense_attend_kernel (hils_dense_causal_attend)", "steps": steps, "ms": ms, "bound": "mfma",
            "tflops": tfl, "frac": tfl / PEAK_BF16_TFLOPS, "flops": fl,
            "tokens_per_s": cfg.B * cfg.N / (ms * 1e-3), "hils_speedup": ms / hils_ms}


def union_overlap(sel, M, sample=4096, seed=0):
    """Mean |union of the selections of M adjacent queries| / K over a sample
    of groups (1 = identical selections, M = disjoint)."""
    import numpy as np

    s = sel[0].cpu().numpy()  # [H_kv, N, K]
    H_kv, N, K = s.shape
    rng = np.random.default_rng(seed)
    vals = []
    for _ in range(sample):
        g = int(rng.integers(H_kv))
        i0 = int(rng.integers(N // M)) * M
        blk = s[g, i0:i0 + M]
        if (blk[:, 0] < 0).any() or (blk[:, -1] < 0).any():
            continue
        vals.append(len(np.unique(blk)) / K)
    return float(np.mean(vals)) if vals else None


def probes(torch):
    """Practical ceilings measured on this device, for context: a 1 GiB
    device-to-device copy (HBM read + write) and a bf16 8192^3 matrix product
    through torch (the vendor GEMM library)."""
    dev = torch.device("cuda:0")
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    out = {}
    for name, fn, work in (("copy", lambda: dst.copy_(src), 2.0 * src.numel() * 4),
                           ("gemm_bf16", lambda: torch.matmul(a, b), 2.0 * 8192 ** 3)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / 5
        out[name] = work / sec / 1e9
    del src, dst, a, b
    return {"copy_gbs": out["copy"], "copy_frac": out["copy"] / PEAK_HBM_GBS,
            "gemm_bf16_tflops": out["gemm_bf16"] / 1e3, "gemm_bf16_frac": out["gemm_bf16"] / 1e3 / PEAK_BF16_TFLOPS}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(pre, budget_s, max_rows=None):
    """The fp64 oracle on the host cores: summaries of every chunk plus a
    seeded stratified sample of query rows, extrapolated to tokens/s."""
    import numpy as np

    import oracle

    cfg = pre["cfg"]
    inp = pre["inp"]
    oc = cfg.oracle_dict()
    q, k, v, q_lm = (inp[n].detach().to("cpu", dtype=__import__("torch").float32).numpy() for n in
                     ("q", "k", "v", "q_lm"))
    qcal = None
    if inp.get("qcal") is not None:
        qcal = tuple(x.detach().to("cpu", dtype=__import__("torch").float32).numpy() for x in inp["qcal"])
    t0 = time.perf_counter()
    ks, bs = oracle.summarize(oc, k, q_lm)
    t_sum = time.perf_counter() - t0
    rng = np.random.default_rng(11)
    probe = np.sort(rng.choice(cfg.N, size=32, replace=False))
    t0 = time.perf_counter()
    oracle.forward_rows(oc, q, k, v, ks, bs, rows=probe, qcal=qcal)
    t_probe = time.perf_counter() - t0
    R = int(max(32, min(cfg.N, 32 * max(0.0, budget_s - t_sum - t_probe) / max(t_probe, 1e-6))))
    if max_rows:
        R = min(R, max_rows)
    rows = np.sort(rng.choice(cfg.N, size=R, replace=False))
    t0 = time.perf_counter()
    ref = oracle.forward_rows(oc, q, k, v, ks, bs, rows=rows, qcal=qcal)
    t_rows = time.perf_counter() - t0
    per_row = t_rows / R
    total = t_sum + cfg.N * per_row
    return {"value": cfg.N / total, "unit": "tokens/s", "cores": oracle.num_threads(), "cpu_model": _cpu_model(),
            "kind": "oracle",
            "sample": f"fp64 oracle: summaries of all {cfg.N // cfg.S} chunks x {cfg.H_lm} landmark heads "
                      f"({t_sum:.2f} s) + {R} uniformly sampled query rows, all {cfg.H_q} heads "
                      f"({t_rows:.2f} s); tokens/s extrapolated to {cfg.N} rows",
            "parity": _sample_parity(pre, ref, rows)}


def _sample_parity(pre, ref, rows):
    """The timed GPU step's outputs against the oracle on the sampled rows:
    selections identical or a near-tie (the oracle's K-th and (K+1)-th group
    scores within 1e-5), and out / lse within 2e-3 + 1e-2 |ref| (bf16) or
    1e-5 + 1e-5 |ref| (fp32) on the rows whose selection is identical."""
    import numpy as np
    import torch

    cfg = pre["cfg"]
    gsel = pre["sel"][:, :, rows].cpu().numpy()
    same = np.all(gsel == ref["sel_idx"], axis=-1)  # [B, H_kv, R]
    kth = ref["kth"]
    tie = (~same) & np.isfinite(kth[..., 0]) & np.isfinite(kth[..., 1]) & (kth[..., 0] - kth[..., 1] < 1e-5)
    atol, rtol = (2e-3, 1e-2) if cfg.io_dtype == torch.bfloat16 else (1e-5, 1e-5)
    gout = pre["out"][:, :, rows].float().cpu().numpy()
    glse = pre["lse"][:, :, rows].cpu().numpy()
    ok_rows = np.repeat(same, cfg.G, axis=1)  # [B, H_q, R]
    frac_out = np.abs(gout - ref["out"]) / (atol + rtol * np.abs(ref["out"])) * ok_rows[..., None]
    frac_lse = np.abs(glse - ref["lse"]) / (atol + rtol * np.abs(ref["lse"])) * ok_rows
    return {"rows": int(len(rows)), "selections": int(same.size), "identical": int(same.sum()),
            "near_tie": int(tie.sum()), "other_differences": int((~same & ~tie).sum()),
            "out_rows_outside_tolerance": int((frac_out > 1).any(-1).sum()),
            "lse_outside_tolerance": int((frac_lse > 1).sum()),
            "out_max_abs_err": float(np.max(np.abs(gout - ref["out"]) * ok_rows[..., None])),
            # worst |gpu - ref| / (atol + rtol |ref|): 1.0 is the edge of the tolerance
            "out_max_err_frac": float(frac_out.max()), "lse_max_err_frac": float(frac_lse.max()),
            "tolerance": {"atol": atol, "rtol": rtol}}


def bench_stress(args, torch, hb, W):
    """The 512K-token stress prefill with Q-Cal scoring (S = 128, K = 64):
    one step = summary -> score/select (Q-Cal pre-pass included) -> fused
    attention, timed like the headline workload; its fused kernel against
    the bf16 MFMA peak; the oracle on a sample of rows as a full-size parity
    check of the timed step."""
    steps = max(2, args.steps // 4)
    pre = bench_prefill(args, torch, hb, W, workload=args.stress_workload, steps=steps, warmup=1)
    cfg = pre["cfg"]
    io_b = 2 if cfg.io_dtype == torch.bfloat16 else 4
    sum_b = 2 if cfg.summary_dtype == torch.bfloat16 else 4
    per = pre["per_call_ms"]
    fl_att, fl_score, by_sum = attend_flops(cfg), score_flops(cfg), summary_bytes(cfg, io_b, sum_b)
    tfl = fl_att / (per["fused"] * 1e-3) / 1e12
    out = {"workload": args.stress_workload, "steps": steps, "warmup": 1, "ms_per_step": pre["ms_per_step"],
           "tokens_per_s": cfg.N * cfg.B / (pre["ms_per_step"] * 1e-3),
           "config": {"B": cfg.B, "N": cfg.N, "H_q": cfg.H_q, "H_kv": cfg.H_kv, "H_lm": cfg.H_lm, "d": cfg.d,
                      "S": cfg.S, "W": cfg.W, "K": cfg.K, "qcal_d_model": 2048, "qcal_r": 32},
           "kernels": {
               "summary": {"ms": per["summary"], "bound": "hbm", "gbs": by_sum / (per["summary"] * 1e-3) / 1e9,
                           "frac": by_sum / (per["summary"] * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": by_sum},
               "score_select_with_qcal": {"ms": per["score_select"], "bound": "mfma",
                                          "tflops": fl_score / (per["score_select"] * 1e-3) / 1e12,
                                          "frac": fl_score / (per["score_select"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                          "flops": fl_score},
               "fused": {"ms": per["fused"], "bound": "mfma", "tflops": tfl, "frac": tfl / PEAK_BF16_TFLOPS,
                         "flops": fl_att, "form": attend_form(hb, cfg),
                         "workspace_bytes": pre["fused_workspace_bytes"]}}}
    print("[bench] stress: fused attention in the other form", file=sys.stderr, flush=True)
    out["kernels"]["fused_other_form"] = fused_other_form(torch, hb, pre, reps=1)
    if not args.no_dense:
        print("[bench] stress: dense causal attention baseline", file=sys.stderr, flush=True)
        out["dense"] = bench_dense(torch, hb, pre, 1, pre["ms_per_step"])
    if not args.no_cpu_baseline:
        print("[bench] stress: oracle parity sample", file=sys.stderr, flush=True)
        cb = cpu_baseline(pre, min(args.cpu_seconds, 10.0), max_rows=256)
        out["parity"] = cb["parity"]
        out["parity"]["sample"] = cb["sample"]
    del pre
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_128k")
    ap.add_argument("--decode-workload", default="decode_512k")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-serving", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-probes", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-attention baselines")
    ap.add_argument("--stress-workload", default="prefill_512k_qcal")
    ap.add_argument("--no-stress", action="store_true", help="skip the 512K Q-Cal stress prefill leg")
    ap.add_argument("--backward-steps", type=int, default=2)
    ap.add_argument("--chunk", type=int, default=8192, help="tokens of the chunked-prefill leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, copy a MIB-MiB buffer twice (a device-to-device copy and an "
                         "elementwise negation), the known-size reference for hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_chunk_landmark_amd import _binding as hb
    from long_context_chunk_landmark_amd import workloads as W

    hb.load_library()
    print(f"[bench] prefill {args.workload}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    pre = bench_prefill(args, torch, hb, W)
    cfg = pre["cfg"]
    io_b = 2 if cfg.io_dtype == torch.bfloat16 else 4
    sum_b = 2 if cfg.summary_dtype == torch.bfloat16 else 4
    fl_att = attend_flops(cfg)
    fl_score = score_flops(cfg)
    by_sum = summary_bytes(cfg, io_b, sum_b)
    ms_f = pre["per_call_ms"]["fused"]
    ms_s = pre["per_call_ms"]["score_select"]
    ms_m = pre["per_call_ms"]["summary"]
    achieved = fl_att / (ms_f * 1e-3) / 1e12
    form = attend_form(hb, cfg)
    # the fused call's HBM bytes (all its kernels), from the committed counter summary
    traffic = traffic_from_profile("sparse_attend_fused", args.workload,
                                   ["attend.hip", "attend_cm.hip", "hils_device.hpp"])
    result = {
        "metric": METRIC,
        "value": cfg.N * cfg.B / (pre["ms_per_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.io_dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": cfg.B, "N": cfg.N, "H_q": cfg.H_q, "H_kv": cfg.H_kv,
                   "H_lm": cfg.H_lm, "d": cfg.d, "S": cfg.S, "W": cfg.W, "K": cfg.K, "M": cfg.M,
                   "summary_dtype": "bf16" if sum_b == 2 else "f32"},
        "roofline": {"kernel": ("hils_sparse_attend_fused, chunk-major: v_transpose, list build, cm_attend_kernel, "
                                "window pass" if form == "chunk-major" else
                                "hils_sparse_attend_fused, walk: v_transpose, sparse_attend_kernel"), "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "algorithmic_tflop_per_launch": fl_att / 1e12},
        "kernels": {
            "summary": {"ms": ms_m, "bound": "hbm", "gbs": by_sum / (ms_m * 1e-3) / 1e9,
                        "frac": by_sum / (ms_m * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": by_sum},
            "score_select": {"ms": ms_s, "bound": "mfma", "tflops": fl_score / (ms_s * 1e-3) / 1e12,
                             "frac": fl_score / (ms_s * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "flops": fl_score},
            "fused": {"ms": ms_f, "tflops": achieved, "flops": fl_att, "form": form,
                      "workspace_bytes": pre["fused_workspace_bytes"]},
        },
        "union_overlap_M": union_overlap(pre["sel"], cfg.M),
    }
    print("[bench] fused attention in the other form", file=sys.stderr, flush=True)
    result["kernels"]["fused_other_form"] = fused_other_form(torch, hb, pre)
    if not args.no_dense:
        print("[bench] dense causal attention baseline", file=sys.stderr, flush=True)
        result["dense"] = bench_dense(torch, hb, pre, max(2, args.steps // 3), pre["ms_per_step"])
    if not args.no_backward:
        print("[bench] backward", file=sys.stderr, flush=True)
        result["backward"] = bench_backward(args, torch, hb, pre)
    if not args.no_variants:
        print("[bench] variants: shared / mean landmarks, normalised aggregation", file=sys.stderr, flush=True)
        result["variants"] = bench_variants(args, torch, hb, W, pre)
    if not args.no_serving:
        print(f"[bench] serving: paged summaries + chunked prefill of {args.chunk} tokens", file=sys.stderr,
              flush=True)
        result["serving"] = bench_serving(args, torch, hb, W, pre)
    if not args.no_decode:
        print(f"[bench] decode {args.decode_workload}", file=sys.stderr, flush=True)
        dec = bench_decode(args, torch, hb, W)
        dcfg = dec["cfg"]
        dio = 2 if dcfg.io_dtype == torch.bfloat16 else 4
        dsum = 2 if dcfg.summary_dtype == torch.bfloat16 else 4
        by = decode_bytes(dcfg, dec["seq_lens"], dio, dsum)
        gbs = by / (dec["call_us"] * 1e-6) / 1e9
        result["decode"] = {"workload": args.decode_workload, "us_per_step": dec["us_per_step"],
                            "num_seqs": len(dec["seq_lens"]), "seq_len": dec["seq_lens"][0],
                            "roofline": {"kernel": "hils_decode (all phases)", "bound": "hbm", "achieved": gbs,
                                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                         "algorithmic_bytes": by}}
        if dec["dense_us"] is not None:
            # K and V of every token of every sequence, the queries and the outputs
            dby = sum(dcfg.H_kv * n * dcfg.d * dio * 2 for n in dec["seq_lens"])
            dby += 2 * len(dec["seq_lens"]) * dcfg.H_q * dcfg.d * dio
            dg = dby / (dec["dense_us"] * 1e-6) / 1e9
            result["decode"]["dense"] = {"kernel": "dense_decode_kernel (hils_dense_decode)",
                                         "us_per_call": dec["dense_us"], "bound": "hbm", "gbs": dg,
                                         "frac": dg / PEAK_HBM_GBS, "algorithmic_bytes": dby,
                                         "hils_speedup": dec["dense_us"] / dec["us_per_step"]}
        for name, (c2, cu) in dec["secondary"].items():
            b2 = decode_bytes(c2, dec["seq_lens"], dio, 2 if c2.summary_dtype == torch.bfloat16 else 4)
            g2 = b2 / (cu * 1e-6) / 1e9
            result["decode"].setdefault("secondary", {})[name] = {
                "us_per_call": cu, "gbs": g2, "frac": g2 / PEAK_HBM_GBS, "algorithmic_bytes": b2}
    if not args.no_probes:
        print("[bench] probes: copy and bf16 GEMM ceilings", file=sys.stderr, flush=True)
        result["probes"] = probes(torch)
    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        result["copy_calibration"] = {"bytes_read": nbytes, "bytes_written": nbytes,
                                      "kernels": ["device-to-device copy", "elementwise neg"]}
        del src, dst
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(pre, args.cpu_seconds)
    if not args.no_stress:
        del pre
        torch.cuda.empty_cache()
        print(f"[bench] stress prefill {args.stress_workload}", file=sys.stderr, flush=True)
        result["stress_prefill"] = bench_stress(args, torch, hb, W)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
