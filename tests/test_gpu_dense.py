"""Dense causal attention (hils_dense_causal_attend), the full-attention
baseline that the pages measure HiLS's prefill speed against (wmrh.cn article
on HiLS-Attention, results table; hyper.ai summary, experiments paragraph on
inference efficiency).  Every output row and log-sum-exp is compared with the
oracle's textbook dense rows (pinned against numpy/scipy attention in
tests/test_oracle_pins.py) at small shapes over every G, both head dims, one
and several 64-key tiles and ragged tails; at the 128K benchmark shape on a
seeded sample of rows."""
import numpy as np
import pytest
import torch

import oracle
from long_context_chunk_landmark_amd import _binding as hb
from long_context_chunk_landmark_amd import workloads as W
from tests.parity import assert_close, host, stratified_rows, tol_for

pytestmark = pytest.mark.gpu

BF = torch.bfloat16

# S, W, K are validated by the call and otherwise unused
SMALL = {
    "g4_d128_ragged": dict(seed=201, io=BF, B=1, H_q=8, H_kv=2, d=128, N=700, S=64, W=128, K=4),
    "g1_d64_b2": dict(seed=202, io=BF, B=2, H_q=3, H_kv=3, d=64, N=300, S=64, W=64, K=2),
    "g8_d128": dict(seed=203, io=BF, B=1, H_q=8, H_kv=1, d=128, N=513, S=64, W=64, K=2),
    "g2_d64": dict(seed=204, io=BF, B=1, H_q=4, H_kv=2, d=64, N=1000, S=128, W=128, K=2),
    "g2_d128_one_row": dict(seed=205, io=BF, B=1, H_q=4, H_kv=2, d=128, N=1, S=64, W=64, K=2),
    "g4_d128_one_tile": dict(seed=206, io=BF, B=1, H_q=4, H_kv=1, d=128, N=64, S=64, W=64, K=2),
    "g1_d128_tile_plus_one": dict(seed=207, io=BF, B=1, H_q=2, H_kv=2, d=128, N=65, S=64, W=64, K=2),
    "g8_d64_b2": dict(seed=208, io=BF, B=2, H_q=16, H_kv=2, d=64, N=777, S=64, W=64, K=2),
    "g4_d128_drift": dict(seed=209, io=BF, B=1, H_q=8, H_kv=2, d=128, N=2048, S=64, W=256, K=8, drift=True),
}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hb.load_library()
    return torch.device("cuda:0")


def _check(cfg, out, lse, ref_o, ref_l, what):
    atol, rtol = tol_for(cfg.io_dtype)
    assert_close(out, ref_o, atol, rtol, f"{what} out")
    # fp32 log-sum-exp of exact bf16 products
    assert_close(lse, ref_l, 1e-4, 1e-5, f"{what} lse")
    frac = np.max(np.abs(out - ref_o) / (atol + rtol * np.abs(ref_o)))
    print(f"[dense] {what}: worst out error = {frac:.3f} of the bound", flush=True)


@pytest.mark.parametrize("name", list(SMALL))
def test_dense_matches_oracle(name, dev):
    inp = W.make_prefill(SMALL[name], device=dev)
    cfg = inp["cfg"]
    print(f"[dense] {name} N={cfg.N}", flush=True)
    ws = torch.empty(hb.workspace_size(cfg, hb.WS_DENSE), dtype=torch.uint8, device=dev)
    out, lse = hb.dense_causal_attend(cfg, inp["q"], inp["k"], inp["v"], workspace=ws)
    assert hb.status_word(ws) == 0
    ref_o, ref_l = oracle.dense_causal_rows(cfg.oracle_dict(), host(inp["q"]), host(inp["k"]), host(inp["v"]))
    _check(cfg, host(out).float().numpy(), host(lse).numpy(), ref_o, ref_l, name)


def test_dense_without_lse_and_repeatable(dev):
    inp = W.make_prefill(SMALL["g4_d128_ragged"], device=dev)
    cfg = inp["cfg"]
    out1, lse1 = hb.dense_causal_attend(cfg, inp["q"], inp["k"], inp["v"])
    out2, lse2 = hb.dense_causal_attend(cfg, inp["q"], inp["k"], inp["v"], want_lse=False)
    torch.cuda.synchronize()
    assert lse2 is None
    assert torch.equal(out1, out2)


def test_dense_full_size_128k_sampled_rows(dev):
    """The 128K benchmark shape (B=1, H_q=32, H_kv=8, d=128, N=131072), as
    bench.py times it: every row on the GPU, a seeded sample checked."""
    print("[dense] 128K: inputs", flush=True)
    inp = W.make_prefill("prefill_128k", device=dev)
    cfg = inp["cfg"]
    print("[dense] 128K: GPU", flush=True)
    out, lse = hb.dense_causal_attend(cfg, inp["q"], inp["k"], inp["v"])
    torch.cuda.synchronize()
    rows = stratified_rows(cfg.N, 64, 0, 24, seed=11)
    gout = host(out[:, :, rows]).float().numpy()
    glse = host(lse[:, :, rows]).numpy()
    del out, lse
    hq, hk, hv = host(inp["q"]), host(inp["k"]), host(inp["v"])
    del inp
    torch.cuda.empty_cache()
    print(f"[dense] 128K: oracle, {len(rows)} rows", flush=True)
    ref_o, ref_l = oracle.dense_causal_rows(cfg.oracle_dict(), hq, hk, hv, rows=rows)
    _check(cfg, gout, glse, ref_o, ref_l, "128K")
