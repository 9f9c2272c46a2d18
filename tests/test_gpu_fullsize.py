"""Parity at the benchmark's full sizes, in the launch configuration bench.py
times: the whole prefill at 128K and 512K (with Q-Cal) and the batched decode
step at 512K.  The GPU computes every output; the fp64 oracle checks all
summaries and a seeded stratified sample of query rows (chunk starts and
ends, rows without candidates, the final rows), one by one."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from long_context_chunk_landmark_amd import _binding as hb
from long_context_chunk_landmark_amd import workloads as W

from parity import (agg_lookup, assert_close, check_selection, host, oracle_prefill, round_to, stratified_rows,
                    tol_for)

pytestmark = pytest.mark.gpu

ROWS = {"prefill_128k": 2048, "prefill_512k_qcal": 1024}
# (workload, selected-chunk form): each workload in the form auto takes
# (chunk-major) and in the walk
CASES = [("prefill_128k", hb.ATTEND_AUTO), ("prefill_512k_qcal", hb.ATTEND_AUTO),
         ("prefill_128k", hb.ATTEND_WALK), ("prefill_512k_qcal", hb.ATTEND_WALK)]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hb.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("name,mode", CASES)
def test_prefill_full_size(name, mode, dev):
    print(f"[fullsize] {name} attend_mode={mode}: inputs", flush=True)
    inp = W.make_prefill(name, device=dev)
    cfg = dataclasses.replace(inp["cfg"], attend_mode=mode)
    qcal = inp.get("qcal")
    print(f"[fullsize] {name}: GPU prefill N={cfg.N}", flush=True)
    res = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"], qcal=qcal)
    torch.cuda.synchronize()
    rows = stratified_rows(cfg.N, cfg.S, cfg.W, ROWS[name], seed=7)
    gsel = host(res["sel_idx"][:, :, rows]).numpy()
    gout = host(res["out"][:, :, rows]).float().numpy()
    glse = host(res["lse"][:, :, rows]).numpy()
    gks, gbs = host(res["k_sum"]).float().numpy(), host(res["b_sum"]).numpy()
    del res
    # host copies for the oracle (the device inputs are no longer needed)
    hinp = {n: host(inp[n]) for n in ("q", "k", "v", "q_lm")}
    if qcal is not None:
        hinp["qcal"] = tuple(host(x) for x in qcal)
    del inp
    torch.cuda.empty_cache()
    print(f"[fullsize] {name}: oracle, {len(rows)} rows", flush=True)
    ref = oracle_prefill(cfg, hinp, rows=rows)
    # every summary of the sequence
    assert_close(gks, ref["k_sum_exact"], 1e-5, 1e-5, "k_sum")
    assert_close(gbs, ref["b_sum"], 1e-5, 1e-5, "b_sum")
    exempt = check_selection(gsel, ref["sel_idx"], ref["kth"], agg_lookup(cfg, hinp, ref["k_sum"], ref["b_sum"], rows),
                             cfg.K)
    refo, refl = ref["out"], ref["lse"]
    if exempt:
        alt = oracle_prefill(cfg, hinp, rows=rows, k_sum=ref["k_sum"], b_sum=ref["b_sum"], given_sel=gsel)
        refo, refl = refo.copy(), refl.copy()
        G = cfg.G
        for b, g, r in exempt:
            refo[b, g * G:(g + 1) * G, r] = alt["out"][b, g * G:(g + 1) * G, r]
            refl[b, g * G:(g + 1) * G, r] = alt["lse"][b, g * G:(g + 1) * G, r]
    atol, rtol = tol_for(cfg.io_dtype)
    assert_close(gout, refo, atol, rtol, "out")
    assert_close(glse, refl, atol, rtol, "lse")
    assert len(exempt) <= max(2, len(rows) * cfg.H_kv // 50), f"{len(exempt)} near-tie rows"


def test_decode_full_size(dev):
    """decode_512k: 16 sequences x 524288 tokens over 131072 pages.  The oracle
    selects from the host copy of the summary cache, then reads the K/V pages
    of its own selection, the GPU's and the window, gathered from the device
    into a compact cache."""
    print("[fullsize] decode_512k: inputs", flush=True)
    inp = W.make_decode("decode_512k", device=dev)
    cfg = inp["cfg"]
    print("[fullsize] decode_512k: GPU step", flush=True)
    out, lse, sel = hb.decode(cfg, inp["q"], inp["k_cache"], inp["v_cache"], inp["ksum_cache"], inp["bsum_cache"],
                              inp["block_table"], inp["seq_lens"])
    torch.cuda.synchronize()
    oc = cfg.oracle_dict()
    q_h, ks_h, bs_h = host(inp["q"]), host(inp["ksum_cache"]), host(inp["bsum_cache"])
    bt = host(inp["block_table"]).numpy()
    sl = host(inp["seq_lens"]).numpy()
    gsel = host(sel).numpy()
    print("[fullsize] decode_512k: oracle selection", flush=True)
    pre = oracle.decode(oc, q_h, None, None, ks_h, bs_h, bt, sl, attend=False, want_agg=True)
    # compact K/V cache: the chunks either side selects plus the window
    B, max_pages = bt.shape
    S, w = cfg.S, cfg.W // cfg.S
    need = []
    for b in range(B):
        t = int(sl[b]) - 1
        lo = max(0, t // S - w)
        chunks = set(range(lo, t // S + 1))
        chunks |= set(int(c) for c in pre["sel_idx"][b].ravel() if c >= 0)
        chunks |= set(int(c) for c in gsel[b].ravel() if c >= 0)
        need.append(sorted(chunks))
    logical = [(b, c) for b in range(B) for c in need[b]]
    pages = torch.tensor([int(bt[b, c]) for b, c in logical], dtype=torch.long, device=dev)
    kc = host(inp["k_cache"].index_select(0, pages))
    vc = host(inp["v_cache"].index_select(0, pages))
    kvbt = np.zeros_like(bt)
    for j, (b, c) in enumerate(logical):
        kvbt[b, c] = j
    print(f"[fullsize] decode_512k: oracle attention over {len(logical)} gathered pages", flush=True)
    ref = oracle.decode(oc, q_h, kc, vc, ks_h, bs_h, bt, sl, kv_block_table=kvbt)

    def agg_of(b, g, r):
        return pre["agg"][b, g]

    exempt = check_selection(gsel[:, :, None, :], ref["sel_idx"][:, :, None, :], ref["kth"][:, :, None, :], agg_of,
                             cfg.K)
    refo, refl = ref["out"], ref["lse"]
    if exempt:
        alt = oracle.decode(oc, q_h, kc, vc, ks_h, bs_h, bt, sl, kv_block_table=kvbt, given_sel=gsel)
        refo, refl = alt["out"], alt["lse"]
    atol, rtol = tol_for(cfg.io_dtype)
    assert_close(host(out).float().numpy(), refo, atol, rtol, "out")
    assert_close(host(lse).numpy(), refl, atol, rtol, "lse")


def test_paged_prefill_full_size(dev):
    """prefill_128k laid out in a paged cache at a random page placement:
    page-by-page summaries equal the whole-sequence summaries, and the last
    8192 tokens prefilled as one chunk over the paged cache (the bench's
    serving call) equal the whole-sequence prefill's rows, bit for bit."""
    inp = W.make_prefill("prefill_128k", device=dev)
    cfg = inp["cfg"]
    print(f"[fullsize] paged prefill: whole-sequence prefill N={cfg.N}", flush=True)
    full = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    kc, vc, bt = W.paged_layout(inp["k"], inp["v"], cfg.S, seed=17)
    P, C = kc.shape[0], cfg.C
    ks = torch.empty((P, cfg.H_lm, cfg.d), dtype=cfg.summary_dtype, device=dev)
    bs = torch.empty((P, cfg.H_lm), dtype=torch.float32, device=dev)
    bb = torch.arange(cfg.B, device=dev).repeat_interleave(C)
    cc = torch.arange(C, device=dev).repeat(cfg.B)
    hb.summarize_pages(cfg, kc, inp["q_lm"][bb, :, cc].contiguous(), bt[bb, cc].contiguous(), ks, bs)
    n = 8192
    q_start = cfg.N - n
    print(f"[fullsize] paged prefill: rows {q_start}..{cfg.N - 1}", flush=True)
    out, lse, sel, ssc = hb.prefill_paged(dataclasses.replace(cfg, N=n), q_start,
                                          inp["q"][:, :, q_start:].contiguous(), kc, vc, ks, bs, bt)
    torch.cuda.synchronize()
    pg = bt[0, :C].long()
    assert torch.equal(ks[pg], full["k_sum"][0].permute(1, 0, 2))
    assert torch.equal(bs[pg], full["b_sum"][0].permute(1, 0))
    assert torch.equal(sel, full["sel_idx"][:, :, q_start:])
    assert torch.equal(ssc, full["sel_score"][:, :, q_start:])
    assert torch.equal(out, full["out"][:, :, q_start:])
    assert torch.equal(lse, full["lse"][:, :, q_start:])
