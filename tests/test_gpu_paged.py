"""GPU parity of the serving-continuity entry points through the C ABI:
summaries of pages that complete during serving (hils_summarize_pages) and
chunked prefill over the paged KV / summary cache (hils_prefill_paged).

Each case draws a whole-sequence prefill workload, scatters its keys and
values into a paged cache at a seeded random page placement, and compares
against the fp64 oracle's paged functions (end to end: the GPU and the
oracle compute their own summaries).  Equivalence tests check that the paged
path reproduces the whole-sequence prefill bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from long_context_chunk_landmark_amd import _binding as hb
from long_context_chunk_landmark_amd import workloads as W
from tests.parity import assert_close, check_selection, host, round_to, tol_for

pytestmark = pytest.mark.gpu

BF = torch.bfloat16
F32 = torch.float32


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hb.load_library()
    return torch.device("cuda:0")


def _paged_inputs(params, q_start, n, dev):
    """Whole-sequence workload of q_start + n tokens and its paged layout."""
    inp = W.make_prefill(dict(params, N=q_start + n), device=dev)
    kc, vc, bt = W.paged_layout(inp["k"], inp["v"], inp["cfg"].S, seed=params["seed"] + 500)
    inp.update(k_cache=kc, v_cache=vc, block_table=bt)
    return inp


def _empty_summary_cache(cfg, P, dev, fill=0.0):
    ks = torch.full((P, cfg.H_lm, cfg.d), fill, dtype=cfg.summary_dtype, device=dev)
    bs = torch.full((P, cfg.H_lm), fill, dtype=F32, device=dev)
    return ks, bs


def _item_queries(cfg, q_lm, bb, cc):
    """Landmark queries of the items (b, c) for the configured landmark mode."""
    if cfg.landmark_mode == hb.LM_CHUNK:
        return q_lm[bb, :, cc].contiguous()
    return q_lm  # one shared query per head, or none (mean pooling)


def _summarize_all(cfg, inp, dev):
    """GPU summaries of every completed chunk, written at their pages."""
    C = cfg.C
    P = inp["k_cache"].shape[0]
    ks, bs = _empty_summary_cache(cfg, P, dev)
    if C:
        bb = torch.arange(cfg.B, device=dev).repeat_interleave(C)
        cc = torch.arange(C, device=dev).repeat(cfg.B)
        pages = inp["block_table"][bb, cc].contiguous()
        hb.summarize_pages(cfg, inp["k_cache"], _item_queries(cfg, inp["q_lm"], bb, cc), pages, ks, bs)
    return ks, bs


# ---------------------------------------------------------------- paged summaries

SUMMARY_CASES = {
    "d128_s64_f32sum": dict(seed=61, io=BF, B=2, H_q=8, H_kv=2, d=128, N=1024, S=64, W=0, K=0),
    "d128_s128_bf16sum": dict(seed=62, io=BF, B=1, H_q=8, H_kv=2, d=128, N=2048, S=128, W=0, K=0, summary=BF),
    "d64_lmkv": dict(seed=63, io=BF, B=2, H_q=8, H_kv=2, H_lm=2, d=64, N=1024, S=64, W=0, K=0),
    "fp32io_s128": dict(seed=64, io=F32, B=1, H_q=4, H_kv=2, d=64, N=1024, S=128, W=0, K=0),
    "shared_d128": dict(seed=65, io=BF, B=2, H_q=8, H_kv=2, d=128, N=1024, S=64, W=0, K=0, landmark_mode=1),
    "mean_d64_s128": dict(seed=66, io=BF, B=1, H_q=4, H_kv=2, d=64, N=1024, S=128, W=0, K=0, landmark_mode=2),
}


@pytest.mark.parametrize("name", list(SUMMARY_CASES))
def test_summarize_pages_matches_oracle(name, dev):
    """Shuffled items (every completed chunk) plus two ids outside [0, P):
    summaries match the oracle; skipped ids and pages no item names keep
    their previous contents."""
    p = SUMMARY_CASES[name]
    print(f"[summarize_pages] {name}", flush=True)
    inp = W.make_prefill(p, device=dev)
    cfg = inp["cfg"]
    kc, _, bt = W.paged_layout(inp["k"], inp["v"], cfg.S, seed=p["seed"] + 500)
    P, C = kc.shape[0], cfg.C
    order = torch.randperm(cfg.B * C, generator=torch.Generator().manual_seed(p["seed"]))
    bb, cc = order // C, order % C
    pages = torch.cat([bt.cpu()[bb, cc], torch.tensor([-1, P], dtype=torch.int32)]).to(torch.int32)
    q_items = inp["q_lm"]
    if cfg.landmark_mode == hb.LM_CHUNK:
        q_items = inp["q_lm"][bb.to(dev), :, cc.to(dev)]
        q_items = torch.cat([q_items, q_items[:2]]).contiguous()
    ks, bs = _empty_summary_cache(cfg, P, dev, fill=7.0)
    hb.summarize_pages(cfg, kc, q_items, pages.to(dev), ks, bs)
    torch.cuda.synchronize()
    rk, rb = oracle.summarize_pages(cfg.oracle_dict(), host(kc), None if q_items is None else host(q_items),
                                    pages.numpy(), landmark=oracle.LANDMARK_MODES[cfg.landmark_mode])
    n = len(order)
    assert np.isnan(rk[n:]).all()
    idx = pages[:n].long()
    got_k = host(ks)[idx].float().numpy()
    got_b = host(bs)[idx].numpy()
    if cfg.summary_dtype == BF:
        assert_close(got_k, rk[:n], 1e-5, 2 ** -8, "k_sum")  # within one bf16 rounding
    else:
        assert_close(got_k, rk[:n], 1e-5, 1e-5, "k_sum")
    assert_close(got_b, rb[:n], 1e-5, 1e-5, "b_sum")
    untouched = torch.ones(P, dtype=torch.bool)
    untouched[idx] = False
    assert torch.all(host(ks)[untouched].float() == 7.0)
    assert torch.all(host(bs)[untouched] == 7.0)


def test_summarize_pages_equals_landmark_summarize(dev):
    """Page-by-page summaries are bitwise those of the whole-sequence kernel."""
    p = SUMMARY_CASES["d128_s64_f32sum"]
    inp = _paged_inputs(p, 0, p["N"], dev)
    cfg = inp["cfg"]
    ks_ref, bs_ref = hb.landmark_summarize(cfg, inp["k"], inp["q_lm"])
    ks, bs = _summarize_all(cfg, inp, dev)
    torch.cuda.synchronize()
    for b in range(cfg.B):
        pg = inp["block_table"][b, :cfg.C].long()
        assert torch.equal(ks[pg], ks_ref[b].permute(1, 0, 2))
        assert torch.equal(bs[pg], bs_ref[b].permute(1, 0))


# ---------------------------------------------------------------- chunked prefill

# (params, q_start, n): new rows at positions q_start .. q_start + n - 1
PAGED_CASES = {
    "mid_ragged_b2": (dict(seed=71, io=BF, B=2, H_q=8, H_kv=2, d=128, S=64, W=256, K=8), 1536, 1300),
    "start0": (dict(seed=72, io=BF, B=1, H_q=8, H_kv=2, d=128, S=64, W=256, K=8), 0, 1000),
    "s128_qcal": (dict(seed=73, io=BF, B=1, H_q=4, H_kv=1, d=128, S=128, W=256, K=4, d_model=256, r=16), 1024, 1500),
    "g8_bf16sum_d64": (dict(seed=74, io=BF, B=1, H_q=8, H_kv=1, d=64, S=64, W=128, K=6, summary=BF), 2048, 700),
    "fp32io": (dict(seed=75, io=F32, B=1, H_q=4, H_kv=2, d=64, S=64, W=128, K=4), 640, 500),
    "lmkv": (dict(seed=76, io=BF, B=1, H_q=8, H_kv=2, H_lm=2, d=128, S=64, W=128, K=8), 4096, 333),
    "k0": (dict(seed=77, io=BF, B=1, H_q=4, H_kv=1, d=128, S=64, W=128, K=0), 512, 400),
    "aggnorm_lmshared": (dict(seed=79, io=BF, B=1, H_q=8, H_kv=2, d=128, S=64, W=256, K=8, agg_mode=1,
                              landmark_mode=1), 1024, 900),
}


def _new_rows(cfg_new, inp, q_start):
    q = inp["q"][:, :, q_start:].contiguous()
    qcal = None
    if inp.get("qcal") is not None:
        h, wd, wu = inp["qcal"]
        qcal = (h[:, q_start:].contiguous(), wd, wu)
    return q, qcal


@pytest.mark.parametrize("name", list(PAGED_CASES))
def test_prefill_paged_matches_oracle(name, dev):
    params, q_start, n = PAGED_CASES[name]
    print(f"[prefill_paged] {name} q_start={q_start} n={n}", flush=True)
    inp = _paged_inputs(params, q_start, n, dev)
    cfg_full = inp["cfg"]
    cfg = W.config(params, N=n)
    ks, bs = _summarize_all(cfg_full, inp, dev)
    q, qcal = _new_rows(cfg, inp, q_start)
    out, lse, sel, ssc = hb.prefill_paged(cfg, q_start, q, inp["k_cache"], inp["v_cache"], ks, bs,
                                          inp["block_table"], qcal=qcal)
    torch.cuda.synchronize()

    # oracle: its own summaries of the contiguous sequence, stored in the
    # summary dtype at the same pages
    oc_full = cfg_full.oracle_dict()
    rk, rb = oracle.summarize(oc_full, host(inp["k"]), None if inp["q_lm"] is None else host(inp["q_lm"]),
                              landmark=oracle.LANDMARK_MODES[cfg.landmark_mode])
    P = inp["k_cache"].shape[0]
    ksc = np.zeros((P, cfg.H_lm, cfg.d), np.float32)
    bsc = np.zeros((P, cfg.H_lm), np.float32)
    rk_s = round_to(rk, cfg.summary_dtype).float().numpy()
    bt = host(inp["block_table"]).numpy()
    for b in range(cfg.B):
        ksc[bt[b, :cfg_full.C]] = rk_s[b].transpose(1, 0, 2)
        bsc[bt[b, :cfg_full.C]] = rb[b].T
    hq = None if qcal is None else tuple(host(x) for x in qcal)
    args = (cfg.oracle_dict(), q_start, host(q), host(inp["k_cache"]), host(inp["v_cache"]), ksc, bsc, bt)
    ref = oracle.prefill_paged(*args, qcal=hq)
    gsel = host(sel).numpy()
    refo, refl = ref["out"], ref["lse"]
    if cfg.K > 0:
        agg = {}

        def agg_of(b, g, r):
            if "a" not in agg:
                agg["a"] = oracle.prefill_paged(*args, qcal=hq, attend=False, want_agg=True)["agg"]
            return agg["a"][b, g, r]

        exempt = check_selection(gsel, ref["sel_idx"], ref["kth"], agg_of, cfg.K)
        if exempt:
            alt = oracle.prefill_paged(*args, qcal=hq, given_sel=gsel)
            refo, refl = alt["out"], alt["lse"]
        else:
            atol, rtol = tol_for(cfg.io_dtype)
            assert_close(host(ssc).numpy(), ref["sel_score"], atol, rtol, "sel_score")
    atol, rtol = tol_for(cfg.io_dtype)
    assert_close(host(out).float().numpy(), refo, atol, rtol, "out")
    assert_close(host(lse).numpy(), refl, atol, rtol, "lse")


@pytest.mark.parametrize("mode", [hb.ATTEND_AUTO, hb.ATTEND_WALK])
@pytest.mark.parametrize("name", ["mid_ragged_b2", "s128_qcal", "g8_bf16sum_d64", "aggnorm_lmshared"])
def test_prefill_paged_equals_prefill_rows(name, mode, dev):
    """Chunked prefill over the paged cache reproduces rows q_start.. of the
    whole-sequence prefill bitwise (same summaries, selections, outputs), in
    each attention form (auto: chunk-major; the walk)."""
    params, q_start, n = PAGED_CASES[name]
    print(f"[prefill_paged == prefill] {name} mode={mode}", flush=True)
    inp = _paged_inputs(params, q_start, n, dev)
    cfg_full = dataclasses.replace(inp["cfg"], attend_mode=mode)
    full = hb.prefill(cfg_full, inp["q"], inp["k"], inp["v"], inp["q_lm"], qcal=inp.get("qcal"))
    cfg = dataclasses.replace(W.config(params, N=n), attend_mode=mode)
    ks, bs = _summarize_all(cfg_full, inp, dev)
    q, qcal = _new_rows(cfg, inp, q_start)
    out, lse, sel, ssc = hb.prefill_paged(cfg, q_start, q, inp["k_cache"], inp["v_cache"], ks, bs,
                                          inp["block_table"], qcal=qcal)
    torch.cuda.synchronize()
    assert torch.equal(sel, full["sel_idx"][:, :, q_start:])
    assert torch.equal(ssc, full["sel_score"][:, :, q_start:])
    assert torch.equal(out, full["out"][:, :, q_start:])
    assert torch.equal(lse, full["lse"][:, :, q_start:])


def test_serving_in_chunks_equals_whole_prefill(dev):
    """A sequence served in three prefill chunks -- each appending its keys and
    values to freshly allocated pages, summarising the chunks it completes
    with hils_summarize_pages, then running hils_prefill_paged -- yields the
    whole-sequence prefill bitwise."""
    params = dict(seed=78, io=BF, B=2, H_q=8, H_kv=2, d=128, S=64, W=256, K=8)
    splits = [0, 1024, 2048, 2600]
    inp = _paged_inputs(params, 0, splits[-1], dev)
    cfg_full = inp["cfg"]
    full = hb.prefill(cfg_full, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    S = cfg_full.S
    P = inp["k_cache"].shape[0]
    bt = inp["block_table"]
    kc = torch.zeros_like(inp["k_cache"])
    vc = torch.zeros_like(inp["v_cache"])
    ks, bs = _empty_summary_cache(cfg_full, P, dev)
    outs = []
    for a, e in zip(splits[:-1], splits[1:]):
        # append tokens a .. e-1 (page by page)
        for c in range(a // S, (e + S - 1) // S):
            lo, hi = max(a, c * S), min(e, c * S + S)
            for b in range(cfg_full.B):
                pg = int(bt[b, c])
                kc[pg, :, lo - c * S:hi - c * S] = inp["k"][b, :, lo:hi]
                vc[pg, :, lo - c * S:hi - c * S] = inp["v"][b, :, lo:hi]
        # summaries of the chunks completed by this step
        done = list(range(a // S, e // S))
        if done:
            cc = torch.tensor(done, device=dev).repeat(cfg_full.B)
            bb = torch.arange(cfg_full.B, device=dev).repeat_interleave(len(done))
            hb.summarize_pages(cfg_full, kc, inp["q_lm"][bb, :, cc].contiguous(), bt[bb, cc].contiguous(), ks, bs)
        cfg = W.config(params, N=e - a)
        o, l, s, _ = hb.prefill_paged(cfg, a, inp["q"][:, :, a:e].contiguous(), kc, vc, ks, bs, bt)
        outs.append((o, l, s))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([x[2] for x in outs], dim=2), full["sel_idx"])
    assert torch.equal(torch.cat([x[0] for x in outs], dim=2), full["out"])
    assert torch.equal(torch.cat([x[1] for x in outs], dim=2), full["lse"])
