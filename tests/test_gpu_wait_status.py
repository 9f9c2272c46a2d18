"""The fused kernel's bounded waits report when they give up.

Its ring protocol waits for each chunk's data with a bounded number of
pauses (include/hils.h, hils_config_t.wait_spins).  A wait that runs out
gives up; the call then sets word 0 of its workspace and writes NaN to the
rows of the waves that gave up, instead of returning stale results with no
sign.  The test forces the give-up path from the host with a bound of one
pause (every kernel still runs to its end: the protocol's counters stay
exact), then checks that a call with the default bound clears the word and
reproduces the normal result bitwise.
"""
import dataclasses

import pytest
import torch

from long_context_chunk_landmark_amd import _binding as hb
from long_context_chunk_landmark_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hb.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("mode", [hb.ATTEND_WALK, hb.ATTEND_CHUNK_MAJOR])
def test_wait_expiry_sets_status_and_marks_rows(mode, dev):
    """Both forms: the walk's ring waits, and the chunk-major form's window
    pass (the same kernel walking the window only)."""
    inp = W.make_prefill(W.PRESETS["gqa_8k"], device=dev)
    cfg = dataclasses.replace(inp["cfg"], attend_mode=mode)
    ref = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    ws = torch.empty(hb.workspace_size(cfg, hb.WS_FUSED), dtype=torch.uint8, device=dev)
    print("[wait status] default bound", flush=True)
    out, lse = hb.sparse_attend_fused(cfg, inp["q"], inp["k"], inp["v"], ref["sel_idx"], ref["sel_score"],
                                      workspace=ws)
    assert hb.status_word(ws) == 0
    assert torch.equal(out, ref["out"]) and torch.equal(lse, ref["lse"])
    print("[wait status] bound of one pause", flush=True)
    c1 = dataclasses.replace(cfg, wait_spins=1)
    out1, lse1 = hb.sparse_attend_fused(c1, inp["q"], inp["k"], inp["v"], ref["sel_idx"], ref["sel_score"],
                                        workspace=ws)
    assert hb.status_word(ws) != 0
    assert torch.isnan(lse1).any() and torch.isnan(out1.float()).any()
    print("[wait status] default bound again", flush=True)
    out2, lse2 = hb.sparse_attend_fused(cfg, inp["q"], inp["k"], inp["v"], ref["sel_idx"], ref["sel_score"],
                                        workspace=ws)
    assert hb.status_word(ws) == 0
    assert torch.equal(out2, ref["out"]) and torch.equal(lse2, ref["lse"])


def test_paged_prefill_status_word_is_clear(dev):
    """The chunked prefill's workspace carries the same status word at offset 0."""
    p = dict(seed=71, io=torch.bfloat16, B=1, H_q=8, H_kv=2, d=128, N=4096, S=64, W=256, K=8)
    inp = W.make_prefill(p, device=dev)
    cfg = dataclasses.replace(inp["cfg"], attend_mode=hb.ATTEND_WALK)  # the paged prefill walks
    res = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    kc, vc, bt = W.paged_layout(inp["k"], inp["v"], cfg.S, seed=3)
    P = kc.shape[0]
    ks = torch.zeros((P, cfg.H_lm, cfg.d), dtype=cfg.summary_dtype, device=dev)
    bs = torch.zeros((P, cfg.H_lm), dtype=torch.float32, device=dev)
    pages = bt[0, :cfg.C].long()
    ks[pages] = res["k_sum"][0].permute(1, 0, 2)
    bs[pages] = res["b_sum"][0].permute(1, 0)
    q_start = 2048
    cc = dataclasses.replace(cfg, N=cfg.N - q_start)
    ws = torch.empty(hb.prefill_paged_workspace_size(cc, q_start, bt.shape[1]), dtype=torch.uint8, device=dev)
    ws.fill_(0xFF)
    out, lse, sel, _ = hb.prefill_paged(cc, q_start, inp["q"][:, :, q_start:].contiguous(), kc, vc, ks, bs, bt,
                                        workspace=ws)
    assert hb.status_word(ws) == 0
    assert torch.equal(out, res["out"][:, :, q_start:])


def test_v_beyond_fp16_range_sets_status_bit(dev):
    """v enters the probability-weighted sum as fp16: a value fp16 cannot hold
    (|v| >= 65520) sets bit 1 of the status word, and a normal call clears it."""
    inp = W.make_prefill(dict(seed=72, io=torch.bfloat16, B=1, H_q=4, H_kv=1, d=128, N=1024, S=64, W=128, K=4),
                         device=dev)
    cfg = inp["cfg"]
    ref = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    ws = torch.empty(hb.workspace_size(cfg, hb.WS_FUSED), dtype=torch.uint8, device=dev)
    ws.fill_(0xFF)
    v_big = inp["v"].clone()
    v_big[0, 0, 517, 3] = 1.0e5  # bf16 99840
    print("[status] v beyond fp16 range", flush=True)
    hb.sparse_attend_fused(cfg, inp["q"], inp["k"], v_big, ref["sel_idx"], ref["sel_score"], workspace=ws)
    assert hb.status_word(ws) & 2
    v_edge = inp["v"].clone()
    v_edge[0, 0, 517, 3] = 65280.0  # the largest bf16 value fp16 holds: no report
    print("[status] v at the edge of fp16 range", flush=True)
    hb.sparse_attend_fused(cfg, inp["q"], inp["k"], v_edge, ref["sel_idx"], ref["sel_score"], workspace=ws)
    assert hb.status_word(ws) == 0
    print("[status] normal v", flush=True)
    out, lse = hb.sparse_attend_fused(cfg, inp["q"], inp["k"], inp["v"], ref["sel_idx"], ref["sel_score"],
                                      workspace=ws)
    assert hb.status_word(ws) == 0
    assert torch.equal(out, ref["out"]) and torch.equal(lse, ref["lse"])
