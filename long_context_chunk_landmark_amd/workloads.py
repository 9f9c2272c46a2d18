"""Seeded synthetic workloads for the tests, the smoke check and the benchmark.

This module only draws random inputs; it contains none of the HiLS
arithmetic.  The pages measure on NIAH / RULER / LongBench-style suites and
perplexity corpora that are not available here; these synthetic inputs stand
in for them with the shapes of the benchmark configurations:

  tiny_fp32          fp32, B=1, H_q=H_kv=1, d=64, N=1024, S=64, W=64, K=4
  gqa_8k             bf16, B=1, H_q=8, H_kv=2, d=128, N=8192, S=64, W=512, K=16,
                     8 planted needle keys (see ``_plant_needles``)
  prefill_128k       bf16, B=1, H_q=32, H_kv=8, d=128, N=131072, S=64, W=1024,
                     K=32, N(0,1) plus a slowly drifting per-position mean
  decode_512k        bf16, 16 sequences x 524288 tokens, H_q=32, H_kv=8, d=128,
                     S=64, W=1024, K=32, paged cache of 131072 pages
  prefill_512k_qcal  bf16, B=1, H_q=16, H_kv=4, d=128, N=524288, S=128,
                     W=2048, K=64, Q-Cal with d_model=2048, r=32

Tensors are drawn in a fixed order from one seeded generator per workload,
as float32 N(0,1) and then rounded to bf16 (round-to-nearest-even) where the
workload is bf16.  Small workloads are drawn on the CPU (bit-identical on
every machine), large ones on the target device.
"""
from __future__ import annotations

import math

import torch

from ._binding import Config

PRESETS = {
    "tiny_fp32": dict(seed=1, io=torch.float32, B=1, H_q=1, H_kv=1, d=64, N=1024, S=64, W=64, K=4, M=16),
    "gqa_8k": dict(seed=2, io=torch.bfloat16, B=1, H_q=8, H_kv=2, d=128, N=8192, S=64, W=512, K=16, M=4, needles=8),
    "prefill_128k": dict(seed=3, io=torch.bfloat16, B=1, H_q=32, H_kv=8, d=128, N=131072, S=64, W=1024, K=32, M=4,
                         drift=True),
    "decode_512k": dict(seed=4, io=torch.bfloat16, num_seqs=16, seq_len=524288, H_q=32, H_kv=8, d=128, S=64, W=1024,
                        K=32, pages=131072, summary=torch.bfloat16),
    "prefill_512k_qcal": dict(seed=5, io=torch.bfloat16, B=1, H_q=16, H_kv=4, d=128, N=524288, S=128, W=2048, K=64,
                              M=4, d_model=2048, r=32),
}

# Summary cache of the decode workload: the decode step reads (k', b') as
# inputs, so they are drawn directly: k' ~ N(0, 0.35^2) per component (the
# spread of a weighted mean of ~8 unit-variance keys) and b' ~ U(1.5, 3.5)
# (entropies inside [0, log 64]).
DECODE_KSUM_STD = 0.35
DECODE_BSUM_RANGE = (1.5, 3.5)


def config(name_or_params, **overrides) -> Config:
    p = dict(PRESETS[name_or_params]) if isinstance(name_or_params, str) else dict(name_or_params)
    p.update(overrides)
    return Config(H_q=p["H_q"], H_kv=p["H_kv"], d=p["d"], S=p["S"], W=p["W"], K=p["K"], B=p.get("B", 1),
                  N=p.get("N", 0), H_lm=p.get("H_lm"), M=p.get("M", 4), io_dtype=p.get("io", torch.bfloat16),
                  summary_dtype=p.get("summary", torch.float32), landmark_mode=p.get("landmark_mode", 0),
                  agg_mode=p.get("agg_mode", 0))


def _randn(gen, shape, device, dtype, std=1.0):
    x = torch.randn(shape, generator=gen, device=gen.device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(device=device, dtype=dtype)


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _drift(seed: int, N: int, d: int) -> torch.Tensor:
    """AR(1) per-position mean: mu_0 ~ N(0, I), mu_t = rho mu_{t-1} + 0.1 xi_t,
    rho = sqrt(1 - 0.01) (stationary unit variance, correlation length ~200
    tokens).  float64 on the CPU, evaluated block-wise."""
    g = _generator(seed + 1000, "cpu")
    rho = math.sqrt(1.0 - 0.01)
    xi = torch.randn((N, d), generator=g, dtype=torch.float64) * 0.1
    mu = torch.empty((N, d), dtype=torch.float64)
    mu[0] = torch.randn((d,), generator=g, dtype=torch.float64)
    BL = 512
    pw = rho ** torch.arange(1, BL + 1, dtype=torch.float64)  # rho^1 .. rho^BL
    for s in range(1, N, BL):
        blk = xi[s:s + BL]
        n = blk.shape[0]
        # mu_{s+t} = rho^{t+1} mu_{s-1} + sum_{u<=t} rho^{t-u} xi_{s+u}
        acc = torch.cumsum(blk / pw[:n, None], dim=0) * pw[:n, None]
        mu[s:s + n] = pw[:n, None] * mu[s - 1][None, :] + acc
    return mu


def _plant_needles(gen, q, k, S, W, count):
    """Pick a query position i* in the last 1024 positions and, for each kv
    head g, set one key in each of `count` distinct chunks lying before the
    window of i* to 4 * q[i*, h0] / ||q[i*, h0]|| (h0 = first query head of
    the group), so that those chunks stand out for that query."""
    B, H_q, N, d = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    istar = N - 1024 + int(torch.randint(1024, (1,), generator=gen))
    n_far = istar // S - W // S  # chunks wholly before the window of i*
    chunks = torch.randperm(n_far, generator=gen)[:count].tolist()
    for g in range(H_kv):
        qv = q[0, g * G, istar].float()
        needle = (4.0 * qv / qv.norm()).to(k.dtype)
        for c in chunks:
            j = c * S + int(torch.randint(S, (1,), generator=gen))
            k[:, g, j] = needle
    return istar, chunks


def make_prefill(name_or_params, device="cuda", **overrides):
    """Inputs of a prefill workload: dict(cfg, q, k, v, q_lm[, qcal]) on `device`."""
    p = dict(PRESETS[name_or_params]) if isinstance(name_or_params, str) else dict(name_or_params)
    p.update(overrides)
    cfg = config(p)
    small = cfg.B * cfg.H_q * cfg.N * cfg.d <= (1 << 24)
    gdev = "cpu" if small or not torch.cuda.is_available() else device
    gen = _generator(p["seed"], gdev)
    dt = cfg.io_dtype
    q = _randn(gen, (cfg.B, cfg.H_q, cfg.N, cfg.d), gdev, torch.float32)
    k = _randn(gen, (cfg.B, cfg.H_kv, cfg.N, cfg.d), gdev, torch.float32)
    v = _randn(gen, (cfg.B, cfg.H_kv, cfg.N, cfg.d), gdev, torch.float32)
    q_lm = _randn(gen, (cfg.B, cfg.H_lm, cfg.C, cfg.d), gdev, dt)
    if p.get("drift"):
        mu = _drift(p["seed"], cfg.N, cfg.d).to(device=gdev, dtype=torch.float32)
        q += mu
        k += mu
        v += mu
        del mu
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    out = dict(cfg=cfg)
    if p.get("needles"):
        out["needle"] = _plant_needles(gen, q, k, cfg.S, cfg.W, p["needles"])
    if p.get("d_model"):
        dm, r = p["d_model"], p["r"]
        h = _randn(gen, (cfg.B, cfg.N, dm), gdev, dt)
        w_down = _randn(gen, (r, dm), gdev, dt, std=1.0 / math.sqrt(dm))
        w_up = _randn(gen, (cfg.H_q * cfg.d, r), gdev, dt, std=1.0 / math.sqrt(dm))
        out["qcal"] = tuple(x.to(device) for x in (h, w_down, w_up))
    # landmark-free variant: one query per landmark head (the first chunk's
    # draw); mean pooling: none
    if cfg.landmark_mode == 1:
        q_lm = q_lm[0, :, 0].contiguous()
    elif cfg.landmark_mode == 2:
        q_lm = None
    out.update(q=q.to(device), k=k.to(device), v=v.to(device), q_lm=None if q_lm is None else q_lm.to(device))
    return out


def make_decode(name_or_params="decode_512k", device="cuda", **overrides):
    """Inputs of a decode workload over a paged cache.

    Returns dict(cfg, q [B,H_q,d], k_cache, v_cache [P,H_kv,S,d],
    ksum_cache [P,H_lm,d], bsum_cache [P,H_lm], block_table [B,max_pages],
    seq_lens [B]).  The block table is a seeded random permutation of the
    pages; sequences own disjoint pages.
    """
    p = dict(PRESETS[name_or_params]) if isinstance(name_or_params, str) else dict(name_or_params)
    p.update(overrides)
    cfg = config(p, N=0)
    B, L, P = p["num_seqs"], p["seq_len"], p["pages"]
    max_pages = (L + cfg.S - 1) // cfg.S
    if B * max_pages > P:
        raise ValueError("not enough pages for the sequences")
    small = P * cfg.H_kv * cfg.S * cfg.d <= (1 << 24)
    gdev = "cpu" if small or not torch.cuda.is_available() else device
    gen = _generator(p["seed"], gdev)
    cpu_gen = _generator(p["seed"] + 2000, "cpu")
    dt = cfg.io_dtype
    shape = (P, cfg.H_kv, cfg.S, cfg.d)
    k_cache = torch.empty(shape, dtype=dt, device=device)
    v_cache = torch.empty(shape, dtype=dt, device=device)
    step = max(1, (1 << 28) // (cfg.H_kv * cfg.S * cfg.d))  # pages per fp32 slice (~1 GiB)
    for cache in (k_cache, v_cache):
        for s in range(0, P, step):
            n = min(step, P - s)
            cache[s:s + n] = _randn(gen, (n,) + shape[1:], gdev, torch.float32).to(device=device, dtype=dt)
    q = _randn(gen, (B, cfg.H_q, cfg.d), gdev, dt).to(device)
    ksum = _randn(gen, (P, cfg.H_lm, cfg.d), gdev, torch.float32, std=DECODE_KSUM_STD).to(cfg.summary_dtype)
    lo, hi = DECODE_BSUM_RANGE
    bsum = torch.rand((P, cfg.H_lm), generator=gen, device=gen.device, dtype=torch.float32) * (hi - lo) + lo
    perm = torch.randperm(P, generator=cpu_gen)[:B * max_pages].view(B, max_pages).to(torch.int32)
    seq_lens = torch.full((B,), L, dtype=torch.int32)
    if "seq_lens" in p:
        seq_lens = torch.tensor(p["seq_lens"], dtype=torch.int32)
    out = dict(cfg=cfg, q=q, k_cache=k_cache, v_cache=v_cache, ksum_cache=ksum.to(device),
               bsum_cache=bsum.to(device), block_table=perm.to(device), seq_lens=seq_lens.to(device))
    if p.get("d_model"):
        dm, r = p["d_model"], p["r"]
        h = _randn(gen, (B, dm), gdev, dt)
        w_down = _randn(gen, (r, dm), gdev, dt, std=1.0 / math.sqrt(dm))
        w_up = _randn(gen, (cfg.H_q * cfg.d, r), gdev, dt, std=1.0 / math.sqrt(dm))
        out["qcal"] = tuple(x.to(device) for x in (h, w_down, w_up))
    return out


def paged_layout(k, v, S, seed, extra_pages=7):
    """Scatter contiguous [B, H_kv, N, d] keys and values into paged caches
    [P, H_kv, S, d] at a seeded random page placement: P = B * ceil(N/S) +
    extra_pages, sequences own disjoint pages, unused pages and the tail of a
    partial last page are zero.  Returns (k_cache, v_cache, block_table
    [B, ceil(N/S)] int32) on the device of k."""
    B, H_kv, N, d = k.shape
    CA = (N + S - 1) // S
    P = B * CA + extra_pages
    bt = torch.randperm(P, generator=_generator(seed, "cpu"))[:B * CA].view(B, CA).to(torch.int32)
    idx = bt.view(-1).long().to(k.device)

    def scatter(x):
        xp = torch.zeros((B, H_kv, CA * S, d), dtype=x.dtype, device=x.device)
        xp[:, :, :N] = x
        cache = torch.zeros((P, H_kv, S, d), dtype=x.dtype, device=x.device)
        cache[idx] = xp.view(B, H_kv, CA, S, d).permute(0, 2, 1, 3, 4).reshape(B * CA, H_kv, S, d)
        return cache

    return scatter(k), scatter(v), bt.to(k.device)


def decode_summary_cache(cfg, P, seed, device="cuda"):
    """A summary cache of P pages for the configuration's landmark heads and
    summary dtype, drawn like the decode workload's (k' ~ N(0, 0.35^2) per
    component, b' ~ U(1.5, 3.5)).  Returns (ksum_cache [P, H_lm, d],
    bsum_cache [P, H_lm] fp32)."""
    gdev = device if torch.cuda.is_available() else "cpu"
    gen = _generator(seed, gdev)
    ksum = _randn(gen, (P, cfg.H_lm, cfg.d), gdev, torch.float32, std=DECODE_KSUM_STD).to(cfg.summary_dtype)
    lo, hi = DECODE_BSUM_RANGE
    bsum = torch.rand((P, cfg.H_lm), generator=gen, device=gen.device, dtype=torch.float32) * (hi - lo) + lo
    return ksum.to(device), bsum.to(device)
