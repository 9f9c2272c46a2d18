"""How much of the bf16 path's tolerance each of its roundings uses.

The fused kernel (bf16 I/O) computes the HiLS output (hyper.ai HiLS summary,
section 方法: per-chunk exact softmax, chunk-aligned window, fusion by
exp(s^_c) / Z^) with four roundings beyond fp32 arithmetic:
  * the output is stored as bf16;
  * the probabilities of a selected chunk, times the chunk's fusion factor,
    and the window's probabilities enter the PV product as fp16;
  * the per-chunk fusion weights exp(s^_c - m^) are held as fp16 (the
    running mass keeps them in fp32);
  * v enters the PV product as fp16.
This CPU test rebuilds the output in fp64 from the oracle's selection and
scores, checks that rebuild against the oracle's own output, then applies
each rounding alone (numpy's fp16 and a round-to-nearest-even bf16) and
measures the largest error as a fraction of the tolerance
2e-3 + 1e-2 |ref| on rows of the 128K workload's distribution (drifting
mean) at N = 16384.  The window's probabilities are rounded relative to the
row's final running max (the kernel rounds them relative to the max reached
so far; fp16's relative precision is the same either way above 2^-14).
"""
import numpy as np
import pytest
import torch

import oracle
from long_context_chunk_landmark_amd import workloads as W

ATOL, RTOL = 2e-3, 1e-2


def _f16(x):
    return x.astype(np.float16).astype(np.float64)


def _bf16(x):
    """Round-to-nearest-even to bfloat16 (finite values)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _row_outputs(cfg, q, k, v, sel, shat, i, h):
    """Exact fp64 output of row i, head h and its variants with one rounding each."""
    G = cfg.H_q // cfg.H_kv
    g, S, W_, scale = h // G, cfg.S, cfg.W, cfg.scale or 1.0 / np.sqrt(cfg.d)
    qv = q[0, h, i]
    ok = sel >= 0
    chunks, sc = sel[ok], shat[ok]
    mh = sc.max() if len(sc) else -np.inf
    # selected chunks: normalised output o_c, weight e^(s^_c - m^)
    parts = []
    for c, s_c in zip(chunks, sc):
        kc, vc = k[0, g, c * S:(c + 1) * S], v[0, g, c * S:(c + 1) * S]
        x = kc @ qv * scale
        e = np.exp(x - x.max())
        parts.append((e / e.sum(), vc, np.exp(s_c - mh)))
    # window: keys max(0, floor(i/S) S - W) .. i
    w0 = max(0, (i // S) * S - W_)
    kw, vw = k[0, g, w0:i + 1], v[0, g, w0:i + 1]
    xw = kw @ qv * scale
    M = max(mh, xw.max())
    alpha = np.exp(mh - M) if len(sc) else 0.0
    pw = np.exp(xw - M)
    lrun = alpha * sum(w for _, _, w in parts) + pw.sum()

    def combine(rp=lambda a: a, rw=lambda a: a, rv=lambda a: a):
        sel_part = np.zeros(cfg.d)
        for p, vc, w in parts:
            sel_part += rp(p * rw(np.float64(w))) @ rv(vc)
        return (alpha * sel_part + rp(pw) @ rv(vw)) / lrun

    exact = combine()
    return dict(exact=exact, out_bf16=_bf16(exact), p_fp16=combine(rp=_f16), w_fp16=combine(rw=_f16),
                v_fp16=combine(rv=_f16), all=_bf16(combine(rp=_f16, rw=_f16, rv=_f16)))


@pytest.fixture(scope="module")
def budget():
    inp = W.make_prefill("prefill_128k", device="cpu", N=16384)
    cfg = inp["cfg"]
    cd = cfg.oracle_dict()
    ks, bs = oracle.summarize(cd, inp["k"], inp["q_lm"])
    rows = np.sort(np.random.default_rng(0).choice(np.arange(cfg.S * 20, cfg.N), 24, replace=False))
    res = oracle.forward_rows(cd, inp["q"], inp["k"], inp["v"], ks, bs, rows=rows)
    q, k, v = (inp[n].double().numpy() for n in ("q", "k", "v"))
    G = cfg.H_q // cfg.H_kv
    worst = {}
    rebuild = 0.0
    for r, i in enumerate(rows):
        for h in range(cfg.H_q):
            outs = _row_outputs(cfg, q, k, v, res["sel_idx"][0, h // G, r], res["sel_score"][0, h, r], int(i), h)
            ref = res["out"][0, h, r]
            rebuild = max(rebuild, float(np.abs(outs["exact"] - ref).max()))
            tol = ATOL + RTOL * np.abs(ref)
            for name, o in outs.items():
                if name != "exact":
                    worst[name] = max(worst.get(name, 0.0), float((np.abs(o - ref) / tol).max()))
    return rebuild, worst


def test_rebuild_matches_oracle(budget):
    rebuild, _ = budget
    assert rebuild < 1e-9


def test_each_rounding_share_of_tolerance(budget):
    """Measured on these rows: bf16 output 0.353 (bound 2^-8 / 1e-2 = 0.39),
    fp16 P 0.097, fp16 fusion weights 0.006, fp16 v below 1e-6, all four
    together 0.354."""
    _, worst = budget
    print({k: round(v, 4) for k, v in worst.items()})
    # bf16 keeps 8 significant bits: rounding moves a value by at most 2^-8 of it
    assert worst["out_bf16"] <= 2.0 ** -8 / RTOL + 1e-9
    assert worst["p_fp16"] < 0.15
    assert worst["w_fp16"] < 0.03
    assert worst["v_fp16"] < 1e-3
    assert worst["all"] < 0.45
