"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Stage tests feed the GPU and the oracle the same inputs (the oracle's own
summaries / selection rounded to the GPU input dtype); end-to-end tests run
both pipelines independently and compare selections with the near-tie rule
and outputs to the output tolerance of tests/parity.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_chunk_landmark_amd import _binding as hb
from long_context_chunk_landmark_amd import workloads as W
from tests.parity import (agg_lookup, assert_close, check_selection, host, oracle_prefill, round_to,
                          stratified_rows, tol_for)

pytestmark = pytest.mark.gpu

BF = torch.bfloat16
F32 = torch.float32

# Small prefill cases: several tiles, a ragged tail, every supported shape
# family.  (name, params)
CASES = {
    "tiny_fp32": W.PRESETS["tiny_fp32"],
    "tiny_fp32_allK": dict(W.PRESETS["tiny_fp32"], K=16),
    "gqa_8k": W.PRESETS["gqa_8k"],
    "gqa_lmkv": dict(seed=21, io=BF, B=1, H_q=8, H_kv=2, H_lm=2, d=128, N=4096, S=64, W=256, K=8),
    "ragged_d64_g2": dict(seed=22, io=BF, B=2, H_q=4, H_kv=2, d=64, N=3000, S=64, W=128, K=8),
    "s128_ragged": dict(seed=23, io=BF, B=1, H_q=8, H_kv=2, d=128, N=4100, S=128, W=256, K=8),
    "g8_w0_bf16sum": dict(seed=24, io=BF, B=1, H_q=8, H_kv=1, d=64, N=2048, S=64, W=0, K=5, summary=BF),
    "g1_bf16": dict(seed=25, io=BF, B=1, H_q=2, H_kv=2, d=128, N=2048, S=64, W=64, K=3),
    "k0": dict(seed=26, io=BF, B=1, H_q=4, H_kv=1, d=128, N=1024, S=64, W=128, K=0),
    "fp32_g4_s128": dict(seed=27, io=F32, B=1, H_q=4, H_kv=1, d=128, N=1500, S=128, W=128, K=3),
    "qcal_small": dict(seed=28, io=BF, B=1, H_q=4, H_kv=1, d=128, N=2048, S=128, W=256, K=4, d_model=256, r=16),
    # Q-Cal on MFMA with rank 32 / 64 and a ragged token tail; VALU Q-Cal for other shapes
    "qcal_r32_b2": dict(seed=35, io=BF, B=2, H_q=8, H_kv=2, d=64, N=1300, S=64, W=128, K=8, d_model=512, r=32),
    "qcal_r64": dict(seed=36, io=BF, B=1, H_q=4, H_kv=1, d=128, N=2500, S=128, W=256, K=8, d_model=384, r=64),
    "qcal_valu_r12": dict(seed=37, io=BF, B=1, H_q=4, H_kv=2, d=64, N=1100, S=64, W=64, K=4, d_model=200, r=12),
    "qcal_fp32": dict(seed=38, io=F32, B=1, H_q=2, H_kv=1, d=64, N=700, S=64, W=64, K=3, d_model=96, r=8),
    "few_candidates": dict(seed=29, io=BF, B=1, H_q=4, H_kv=2, d=128, N=1024, S=64, W=512, K=16),
    # block shapes picked by LDS capacity: 8-wave blocks at S=128 with K=64 / G=2, and
    # 2-wave blocks (fewer waves than ring stages at S=64) with G=1, K=128
    "s128_k64": dict(seed=33, io=BF, B=1, H_q=8, H_kv=2, d=128, N=9000, S=128, W=256, K=64),
    "s128_g2": dict(seed=34, io=BF, B=1, H_q=4, H_kv=2, d=128, N=6000, S=128, W=128, K=32),
    "g1_k128_s64": dict(seed=39, io=BF, B=1, H_q=2, H_kv=2, d=128, N=9000, S=64, W=128, K=128),
    "g1_k128_s128": dict(seed=40, io=BF, B=1, H_q=1, H_kv=1, d=128, N=20000, S=128, W=256, K=128),
    # variants: one shared landmark query per head (landmark-free), mean pooling (q' = 0),
    # normalised-weight group aggregation (both select paths, Q-Cal, fp32, bf16 summaries)
    "lm_shared_b2": dict(seed=81, io=BF, B=2, H_q=8, H_kv=2, d=128, N=3000, S=64, W=256, K=8, landmark_mode=1),
    "lm_mean_s128_d64": dict(seed=82, io=BF, B=1, H_q=4, H_kv=2, d=64, N=2600, S=128, W=256, K=6, landmark_mode=2),
    "lm_shared_fp32": dict(seed=83, io=F32, B=1, H_q=2, H_kv=1, d=64, N=1000, S=64, W=64, K=3, landmark_mode=1),
    "aggnorm_g4": dict(seed=84, io=BF, B=1, H_q=8, H_kv=2, d=128, N=4096, S=64, W=256, K=8, agg_mode=1),
    "aggnorm_g8_bf16sum": dict(seed=85, io=BF, B=1, H_q=8, H_kv=1, d=64, N=3000, S=64, W=128, K=6, summary=BF,
                               agg_mode=1),
    "aggnorm_lmkv": dict(seed=86, io=BF, B=1, H_q=8, H_kv=2, H_lm=2, d=128, N=3000, S=64, W=128, K=8, agg_mode=1),
    "aggnorm_qcal": dict(seed=87, io=BF, B=1, H_q=4, H_kv=1, d=128, N=2500, S=128, W=256, K=4, d_model=256, r=16,
                         agg_mode=1),
    "aggnorm_fp32": dict(seed=88, io=F32, B=1, H_q=4, H_kv=2, d=64, N=1500, S=64, W=128, K=4, agg_mode=1),
}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hb.load_library()
    return torch.device("cuda:0")


_cache = {}


def _inputs(name, dev):
    if name not in _cache:
        _cache[name] = W.make_prefill(CASES[name], device=dev)
    return _cache[name]


def _oracle_full(name, dev):
    key = ("oracle", name)
    if key not in _cache:
        inp = _inputs(name, dev)
        _cache[key] = oracle_prefill(inp["cfg"], inp)
    return _cache[key]


@pytest.mark.parametrize("name", list(CASES))
def test_summary_matches_oracle(name, dev):
    inp = _inputs(name, dev)
    cfg = inp["cfg"]
    print(f"[summary] {name}", flush=True)
    k_sum, b_sum = hb.landmark_summarize(cfg, inp["k"], inp["q_lm"])
    torch.cuda.synchronize()
    ref = _oracle_full(name, dev)
    if cfg.summary_dtype == BF:
        # bf16 storage: within one bf16 rounding of the exact value
        assert_close(host(k_sum).float().numpy(), ref["k_sum_exact"], 1e-5, 2 ** -8, "k_sum")
    else:
        assert_close(host(k_sum).numpy(), ref["k_sum_exact"], 1e-5, 1e-5, "k_sum")
    assert_close(host(b_sum).numpy(), ref["b_sum"], 1e-5, 1e-5, "b_sum")


@pytest.mark.parametrize("name", list(CASES))
def test_score_select_stage(name, dev):
    """Same summaries on both sides (the oracle's, stored in the GPU's
    summary dtype); selection bit-exact up to near-ties, scores to 1e-5."""
    inp = _inputs(name, dev)
    cfg = inp["cfg"]
    print(f"[score_select] {name}", flush=True)
    ref0 = _oracle_full(name, dev)
    ks_t = round_to(ref0["k_sum_exact"], cfg.summary_dtype)
    bs_t = round_to(ref0["b_sum"], F32)
    ks64 = ks_t.to(torch.float64).numpy()
    bs64 = bs_t.to(torch.float64).numpy()
    sel, ss = hb.score_select(cfg, inp["q"], ks_t.to(dev), bs_t.to(dev), qcal=inp.get("qcal"))
    torch.cuda.synchronize()
    ref = oracle_prefill(cfg, inp, k_sum=ks64, b_sum=bs64)
    exempt = check_selection(host(sel).numpy(), ref["sel_idx"], ref["kth"], agg_lookup(cfg, inp, ks64, bs64, None),
                             cfg.K)
    ss_h = host(ss).numpy()
    mask = np.ones(ss_h.shape, bool)
    G = cfg.G
    for b, g, r in exempt:
        mask[b, g * G:(g + 1) * G, r, :] = False
    assert_close(np.where(mask, ss_h, 0), np.where(mask, ref["sel_score"], 0), 2e-5, 1e-5, "sel_score")
    assert len(exempt) <= max(2, ref["sel_idx"].size // max(1, cfg.K) // 200), f"{len(exempt)} near-tie rows"


@pytest.mark.parametrize("name", list(CASES))
def test_attend_stage(name, dev):
    """Same selection and scores on both sides (the oracle's)."""
    inp = _inputs(name, dev)
    cfg = inp["cfg"]
    print(f"[attend] {name}", flush=True)
    ref = _oracle_full(name, dev)
    sel_t = torch.from_numpy(ref["sel_idx"]).to(dev)
    ss_t = round_to(ref["sel_score"], F32).to(dev)
    out, lse = hb.sparse_attend_fused(cfg, inp["q"], inp["k"], inp["v"], sel_t, ss_t)
    torch.cuda.synchronize()
    atol, rtol = tol_for(cfg.io_dtype)
    # oracle with the fp32-rounded scores it handed over
    oc = cfg.oracle_dict()
    ref2 = oracle.forward_rows(oc, host(inp["q"]), host(inp["k"]), host(inp["v"]), ref["k_sum"], ref["b_sum"],
                               given_sel=ref["sel_idx"], qcal=None if inp.get("qcal") is None else tuple(
                                   host(x) for x in inp["qcal"]))
    # given_sel keeps the oracle's own s^ (fp64); the GPU saw them rounded
    # to fp32 -- a 1e-7 relative perturbation, far inside the tolerance
    assert_close(host(out).float().numpy(), ref2["out"], atol, rtol, "out")
    assert_close(host(lse).numpy(), ref2["lse"], atol, rtol, "lse")


@pytest.mark.parametrize("name", list(CASES))
def test_end_to_end(name, dev):
    inp = _inputs(name, dev)
    cfg = inp["cfg"]
    print(f"[end_to_end] {name}", flush=True)
    res = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"], qcal=inp.get("qcal"))
    torch.cuda.synchronize()
    ref = _oracle_full(name, dev)
    gsel = host(res["sel_idx"]).numpy()
    exempt = check_selection(gsel, ref["sel_idx"], ref["kth"], agg_lookup(cfg, inp, ref["k_sum"], ref["b_sum"], None),
                             cfg.K)
    refo, refl = ref["out"], ref["lse"]
    if exempt:
        # rows where a near-tie let the GPU pick differently: compare with
        # the oracle run on the GPU's selection
        alt = oracle_prefill(cfg, inp, k_sum=ref["k_sum"], b_sum=ref["b_sum"], given_sel=gsel)
        refo, refl = refo.copy(), refl.copy()
        G = cfg.G
        for b, g, r in exempt:
            refo[b, g * G:(g + 1) * G, r] = alt["out"][b, g * G:(g + 1) * G, r]
            refl[b, g * G:(g + 1) * G, r] = alt["lse"][b, g * G:(g + 1) * G, r]
    atol, rtol = tol_for(cfg.io_dtype)
    assert_close(host(res["out"]).float().numpy(), refo, atol, rtol, "out")
    assert_close(host(res["lse"]).numpy(), refl, atol, rtol, "lse")


def test_needles_are_selected(dev):
    """gqa_8k plants needle keys aligned with one query: its group selects
    every needle chunk (a property of the workload, checked on both sides)."""
    inp = _inputs("gqa_8k", dev)
    cfg = inp["cfg"]
    res = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    istar, chunks = inp["needle"]
    sel = host(res["sel_idx"])[0, :, istar].numpy()
    ref = _oracle_full("gqa_8k", dev)["sel_idx"][0, :, istar]
    np.testing.assert_array_equal(sel, ref)


def test_schedule_hint_and_determinism(dev):
    """Results do not depend on the M hint and are bitwise reproducible."""
    inp = _inputs("gqa_8k", dev)
    cfg = inp["cfg"]
    a = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    b = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    import dataclasses
    c = hb.prefill(dataclasses.replace(cfg, M=1), inp["q"], inp["k"], inp["v"], inp["q_lm"])
    torch.cuda.synchronize()
    for key in ("k_sum", "b_sum", "sel_idx", "sel_score", "out", "lse"):
        assert torch.equal(a[key], b[key]), key
        assert torch.equal(a[key], c[key]), key


def test_empty_and_degenerate_shapes(dev):
    """N = 0 and B = 0 are no-ops; N < S (no completed chunk) works."""
    for params in (dict(seed=30, io=BF, B=1, H_q=4, H_kv=1, d=64, N=0, S=64, W=64, K=4),
                   dict(seed=31, io=BF, B=0, H_q=4, H_kv=1, d=64, N=128, S=64, W=64, K=4)):
        cfg = W.config(params)
        q = torch.zeros((cfg.B, cfg.H_q, cfg.N, cfg.d), dtype=BF, device=dev)
        k = torch.zeros((cfg.B, cfg.H_kv, cfg.N, cfg.d), dtype=BF, device=dev)
        ql = torch.zeros((cfg.B, cfg.H_lm, cfg.C, cfg.d), dtype=BF, device=dev)
        hb.prefill(cfg, q, k, k, ql)
    p = dict(seed=32, io=BF, B=1, H_q=4, H_kv=2, d=128, N=40, S=64, W=64, K=4)
    inp = W.make_prefill(p, device=dev)
    cfg = inp["cfg"]
    res = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    ref = oracle_prefill(cfg, inp)
    assert np.all(host(res["sel_idx"]).numpy() == -1)
    assert_close(host(res["out"]).float().numpy(), ref["out"], 2e-3, 1e-2, "out")


# ---------------------------------------------------------------- decode


def _decode_case(dev, **kw):
    p = dict(seed=41, io=BF, num_seqs=3, seq_len=0, H_q=8, H_kv=2, d=128, S=64, W=256, K=8, pages=200,
             summary=BF)
    p.update(kw)
    return p


def _qcal_host(inp):
    return None if inp.get("qcal") is None else tuple(host(x) for x in inp["qcal"])


def _oracle_decode(cfg, inp, seq_lens, given_sel=None):
    oc = cfg.oracle_dict()
    return oracle.decode(oc, host(inp["q"]), host(inp["k_cache"]), host(inp["v_cache"]), host(inp["ksum_cache"]),
                         host(inp["bsum_cache"]), host(inp["block_table"]), seq_lens, given_sel=given_sel,
                         qcal=_qcal_host(inp))


@pytest.mark.parametrize("variant", ["bf16_hq", "bf16_hkv", "fp32sum", "fp32io", "ragged", "g8_s128", "qcal",
                                     "qcal_fp32io", "aggnorm_hq", "aggnorm_hkv_fp32io"])
def test_decode_matches_oracle(variant, dev):
    kw = {
        "bf16_hq": dict(seq_len=3000, seq_lens=[3000, 2113, 64]),
        "bf16_hkv": dict(seq_len=3000, H_lm=2, seq_lens=[3000, 1999, 700]),
        "fp32sum": dict(seq_len=2500, summary=F32, seq_lens=[2500, 2500, 1]),
        "fp32io": dict(seq_len=2000, io=F32, summary=F32, d=64, seq_lens=[2000, 1500, 333]),
        "ragged": dict(seq_len=4000, seq_lens=[3999, 257, 1280], K=40, W=128),
        "g8_s128": dict(seq_len=6000, H_q=8, H_kv=1, S=128, pages=160, seq_lens=[6000, 4097, 129]),
        # Q-Cal calibrates the scoring query only; attention uses the raw q
        "qcal": dict(seq_len=3000, seq_lens=[3000, 1500, 900], d_model=256, r=16),
        "qcal_fp32io": dict(seq_len=2000, io=F32, summary=F32, d=64, seq_lens=[2000, 1111, 700], d_model=128, r=8),
        # normalised-weight aggregation (two scoring passes)
        "aggnorm_hq": dict(seq_len=3000, seq_lens=[3000, 2113, 900], agg_mode=1),
        "aggnorm_hkv_fp32io": dict(seq_len=2500, io=F32, summary=F32, H_lm=2, d=64, seq_lens=[2500, 1700, 64],
                                   agg_mode=1),
    }[variant]
    inp = W.make_decode(_decode_case(dev, **kw), device=dev)
    cfg = inp["cfg"]
    print(f"[decode] {variant}", flush=True)
    out, lse, sel = hb.decode(cfg, inp["q"], inp["k_cache"], inp["v_cache"], inp["ksum_cache"], inp["bsum_cache"],
                              inp["block_table"], inp["seq_lens"], qcal=inp.get("qcal"))
    torch.cuda.synchronize()
    sl = host(inp["seq_lens"]).numpy()
    ref = _oracle_decode(cfg, inp, sl)
    gsel = host(sel).numpy()
    oc = cfg.oracle_dict()

    def agg_of(b, g, r):
        res = oracle.decode(oc, host(inp["q"]), None, None, host(inp["ksum_cache"]), host(inp["bsum_cache"]),
                            host(inp["block_table"]), sl, attend=False, want_agg=True, qcal=_qcal_host(inp))
        return res["agg"][b, g]

    exempt = check_selection(gsel[:, :, None, :], ref["sel_idx"][:, :, None, :], ref["kth"][:, :, None, :],
                             lambda b, g, r: agg_of(b, g, r), cfg.K)
    refo, refl = ref["out"], ref["lse"]
    if exempt:
        alt = _oracle_decode(cfg, inp, sl, given_sel=gsel)
        refo, refl = alt["out"], alt["lse"]
    atol, rtol = tol_for(cfg.io_dtype)
    assert_close(host(out).float().numpy(), refo, atol, rtol, "out")
    assert_close(host(lse).numpy(), refl, atol, rtol, "lse")


def test_decode_page_permutation_invariance(dev):
    """Moving pages to other physical slots (and the block table with them)
    leaves the result bitwise unchanged."""
    inp = W.make_decode(_decode_case(dev, seq_len=3000, seq_lens=[3000, 2000, 1000]), device=dev)
    cfg = inp["cfg"]
    a = hb.decode(cfg, inp["q"], inp["k_cache"], inp["v_cache"], inp["ksum_cache"], inp["bsum_cache"],
                  inp["block_table"], inp["seq_lens"])
    P = inp["k_cache"].shape[0]
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(5)).to(dev)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(P, device=dev)
    # new slot perm[p] holds old page p
    kc = torch.empty_like(inp["k_cache"]); kc[perm] = inp["k_cache"]
    vc = torch.empty_like(inp["v_cache"]); vc[perm] = inp["v_cache"]
    ks = torch.empty_like(inp["ksum_cache"]); ks[perm] = inp["ksum_cache"]
    bs = torch.empty_like(inp["bsum_cache"]); bs[perm] = inp["bsum_cache"]
    bt = perm[inp["block_table"].long()].to(torch.int32)
    b = hb.decode(cfg, inp["q"], kc, vc, ks, bs, bt, inp["seq_lens"])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_decode_equals_prefill_row(dev):
    """A decode step at t over the paged layout of a prefill workload equals
    prefill row t (same keys, values and summaries)."""
    p = dict(seed=51, io=BF, B=1, H_q=8, H_kv=2, d=128, N=2560, S=64, W=256, K=8, summary=BF)
    inp = W.make_prefill(p, device=dev)
    cfg = inp["cfg"]
    res = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    C = cfg.C
    kc = inp["k"][0].view(cfg.H_kv, C, cfg.S, cfg.d).permute(1, 0, 2, 3).contiguous()
    vc = inp["v"][0].view(cfg.H_kv, C, cfg.S, cfg.d).permute(1, 0, 2, 3).contiguous()
    ks = res["k_sum"][0].permute(1, 0, 2).contiguous()
    bs = res["b_sum"][0].permute(1, 0).contiguous()
    ts = [cfg.N - 1, 2000, 1300, 100]
    q = torch.stack([inp["q"][0, :, t] for t in ts])
    bt = torch.arange(C, dtype=torch.int32, device=dev)[None].repeat(len(ts), 1)
    sl = torch.tensor([t + 1 for t in ts], dtype=torch.int32, device=dev)
    out, lse, sel = hb.decode(cfg, q, kc, vc, ks, bs, bt, sl)
    torch.cuda.synchronize()
    for n, t in enumerate(ts):
        assert torch.equal(sel[n], res["sel_idx"][0, :, t])
        assert_close(host(out[n]).float().numpy(), host(res["out"][0, :, t]).float().numpy(), 2e-3, 1e-2, "out")
        assert_close(host(lse[n]).numpy(), host(res["lse"][0, :, t]).numpy(), 1e-4, 1e-4, "lse")


def test_summary_on_paged_cache(dev):
    """The summary kernel applied to a paged cache ([P, H_kv, S, d] viewed as
    B = P sequences of one chunk) matches the oracle."""
    p = _decode_case(dev, seq_len=640, pages=40, summary=F32)
    inp = W.make_decode(p, device=dev)
    cfg = inp["cfg"]
    P = inp["k_cache"].shape[0]
    import dataclasses
    pc = dataclasses.replace(cfg, B=P, N=cfg.S)
    q_lm = torch.randn((P, cfg.H_lm, 1, cfg.d), generator=torch.Generator().manual_seed(3)).to(BF).to(dev)
    ks, bs = hb.landmark_summarize(pc, inp["k_cache"], q_lm)
    torch.cuda.synchronize()
    rk, rb = oracle.summarize(pc.oracle_dict(), host(inp["k_cache"]), host(q_lm))
    assert_close(host(ks).numpy(), rk, 1e-5, 1e-5, "k_sum")
    assert_close(host(bs).numpy(), rb, 1e-5, 1e-5, "b_sum")
