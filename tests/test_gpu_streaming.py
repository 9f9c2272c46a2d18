"""The streaming form of score/select (hils_config_t.score_mode =
HILS_SCORE_STREAMING) against the oracle: the same criteria as the two-pass
form's stage test (selection bit-exact up to near-ties, scores to 1e-5), the
exact-tie cases end to end, and the chunked prefill over a paged cache.
Shapes the streaming kernel does not cover must be refused."""
import dataclasses

import numpy as np
import pytest
import torch

from long_context_chunk_landmark_amd import _binding as hb
from long_context_chunk_landmark_amd import workloads as W
from tests.parity import (agg_lookup, assert_close, check_selection, host, oracle_prefill, round_to, tol_for)
from tests.test_gpu_parity import CASES
from tests.test_gpu_ties import PREFILL_TIES, _tie_rows, _twin_chunks

pytestmark = pytest.mark.gpu

BF = torch.bfloat16
F32 = torch.float32


def _covered(p):
    """Every shape but d = 128 with G = 8, fp32 summaries and K > 32."""
    fp32_sum = p.get("summary", F32) == F32
    return not (p["d"] == 128 and p["H_q"] // p["H_kv"] == 8 and fp32_sum and p["K"] > 32)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hb.load_library()
    return torch.device("cuda:0")


STREAM_CASES = [n for n, p in CASES.items() if _covered(p)]


@pytest.mark.parametrize("name", STREAM_CASES)
def test_streaming_score_select_matches_oracle(name, dev):
    inp = W.make_prefill(CASES[name], device=dev)
    cfg = dataclasses.replace(inp["cfg"], score_mode=hb.SCORE_STREAMING)
    print(f"[streaming score_select] {name}", flush=True)
    ref0 = oracle_prefill(inp["cfg"], inp)
    ks_t = round_to(ref0["k_sum_exact"], cfg.summary_dtype)
    bs_t = round_to(ref0["b_sum"], F32)
    ks64 = ks_t.to(torch.float64).numpy()
    bs64 = bs_t.to(torch.float64).numpy()
    sel, ss = hb.score_select(cfg, inp["q"], ks_t.to(dev), bs_t.to(dev), qcal=inp.get("qcal"))
    torch.cuda.synchronize()
    ref = oracle_prefill(inp["cfg"], inp, k_sum=ks64, b_sum=bs64)
    exempt = check_selection(host(sel).numpy(), ref["sel_idx"], ref["kth"], agg_lookup(cfg, inp, ks64, bs64, None),
                             cfg.K)
    ss_h = host(ss).numpy()
    mask = np.ones(ss_h.shape, bool)
    G = cfg.G
    for b, g, r in exempt:
        mask[b, g * G:(g + 1) * G, r, :] = False
    assert_close(np.where(mask, ss_h, 0), np.where(mask, ref["sel_score"], 0), 2e-5, 1e-5, "sel_score")
    assert len(exempt) <= max(2, ref["sel_idx"].size // max(1, cfg.K) // 200), f"{len(exempt)} near-tie rows"


@pytest.mark.parametrize("name", [n for n, p in PREFILL_TIES.items() if _covered(p)])
def test_streaming_exact_ties_take_lower_index(name, dev):
    p = PREFILL_TIES[name]
    inp = W.make_prefill(p, device=dev)
    cfg = dataclasses.replace(inp["cfg"], score_mode=hb.SCORE_STREAMING)
    _twin_chunks(inp, cfg.S)
    print(f"[streaming ties] {name}", flush=True)
    res = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"], qcal=inp.get("qcal"))
    torch.cuda.synchronize()
    ref = oracle_prefill(inp["cfg"], inp)
    gsel = host(res["sel_idx"]).numpy()
    assert _tie_rows(ref, cfg.K).sum() > 0
    bad = np.argwhere(np.any(gsel != ref["sel_idx"], axis=-1))
    assert len(bad) == 0, f"{len(bad)} rows differ from the oracle, e.g. {bad[:3].tolist()}"
    atol, rtol = tol_for(cfg.io_dtype)
    assert_close(host(res["out"]).float().numpy(), ref["out"], atol, rtol, "out")


def test_streaming_paged_prefill_equals_contiguous(dev):
    p = dict(seed=77, io=BF, B=1, H_q=8, H_kv=2, d=128, N=6144, S=64, W=256, K=8)
    inp = W.make_prefill(p, device=dev)
    # the paged prefill walks the selected chunks: the contiguous one walks too
    cfg = dataclasses.replace(inp["cfg"], score_mode=hb.SCORE_STREAMING, attend_mode=hb.ATTEND_WALK)
    print("[streaming paged]", flush=True)
    res = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    kc, vc, bt = W.paged_layout(inp["k"], inp["v"], cfg.S, seed=5)
    P = kc.shape[0]
    ks = torch.zeros((P, cfg.H_lm, cfg.d), dtype=cfg.summary_dtype, device=dev)
    bs = torch.zeros((P, cfg.H_lm), dtype=torch.float32, device=dev)
    pages = bt[0, :cfg.C].long()
    ks[pages] = res["k_sum"][0].permute(1, 0, 2)
    bs[pages] = res["b_sum"][0].permute(1, 0)
    q_start = 4096
    cc = dataclasses.replace(cfg, N=cfg.N - q_start)
    out, lse, sel, _ = hb.prefill_paged(cc, q_start, inp["q"][:, :, q_start:].contiguous(), kc, vc, ks, bs, bt)
    torch.cuda.synchronize()
    assert torch.equal(sel, res["sel_idx"][:, :, q_start:])
    assert torch.equal(out, res["out"][:, :, q_start:])


def test_streaming_refused_where_not_covered(dev):
    p = dict(seed=78, io=BF, B=1, H_q=8, H_kv=1, d=128, N=4096, S=64, W=128, K=40)  # G = 8, d = 128, K > 32
    inp = W.make_prefill(p, device=dev)
    cfg = dataclasses.replace(inp["cfg"], score_mode=hb.SCORE_STREAMING)
    ks, bs = hb.landmark_summarize(inp["cfg"], inp["k"], inp["q_lm"])
    with pytest.raises(hb.HilsError) as e:
        hb.score_select(cfg, inp["q"], ks, bs)
    assert e.value.status == hb.HILS_ERR_UNSUPPORTED
