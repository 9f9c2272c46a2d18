"""Dense causal attention (hils_dense_causal_attend) and the dense decode
step (hils_dense_decode): the full-attention baselines that the pages measure
HiLS's prefill and decode speed against (wmrh.cn article on HiLS-Attention,
results table; hyper.ai summary, experiments paragraph on inference
efficiency).  Every output row and log-sum-exp is compared with the oracle's
textbook dense rows (pinned against numpy/scipy attention in
tests/test_oracle_pins.py): prefill at small shapes over every G, both head
dims, one and several 64-key tiles and ragged tails, and at the 128K benchmark
shape on a seeded sample of rows; decode at ragged sequence lengths over every
G, a sequence split over many blocks, and two sequences of the 16 x 512K
benchmark step."""
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


# decode: sequences of mixed lengths (one token, one page, partial pages)
DECODE = {
    "g4_ragged": dict(seed=301, io=BF, num_seqs=3, seq_len=700, H_q=8, H_kv=2, d=128, S=64, W=128, K=4, pages=40,
                      summary=BF, seq_lens=[700, 1, 257]),
    "g1": dict(seed=302, io=BF, num_seqs=2, seq_len=2000, H_q=4, H_kv=4, d=128, S=64, W=128, K=4, pages=70,
               summary=BF, seq_lens=[2000, 64]),
    "g8": dict(seed=303, io=BF, num_seqs=2, seq_len=1500, H_q=16, H_kv=2, d=128, S=64, W=128, K=4, pages=50,
               summary=BF, seq_lens=[1500, 65]),
    "g2_many_splits": dict(seed=304, io=BF, num_seqs=1, seq_len=20000, H_q=4, H_kv=2, d=128, S=64, W=128, K=4,
                           pages=320, summary=BF),
}


def _dense_decode_ref(cfg, inp, seqs):
    """Oracle rows for the last position of each listed sequence, from the
    sequence's pages gathered into a contiguous layout, one kv group at a time
    (the oracle reads the query only at the requested row)."""
    bt = host(inp["block_table"]).long()
    lens = host(inp["seq_lens"]).long()
    q = host(inp["q"]).float()
    G = cfg.H_q // cfg.H_kv
    outs, lses = [], []
    for b in seqs:
        L = int(lens[b])
        npg = (L + cfg.S - 1) // cfg.S
        pages = bt[b, :npg].to(inp["k_cache"].device)
        o_b = np.zeros((cfg.H_q, cfg.d))
        l_b = np.zeros(cfg.H_q)
        for g in range(cfg.H_kv):
            k = host(inp["k_cache"][pages, g].reshape(1, 1, npg * cfg.S, cfg.d)[:, :, :L]).float()
            v = host(inp["v_cache"][pages, g].reshape(1, 1, npg * cfg.S, cfg.d)[:, :, :L]).float()
            qf = torch.zeros((1, G, L, cfg.d), dtype=torch.float32)
            qf[0, :, L - 1] = q[b, g * G:(g + 1) * G]
            oc = dict(cfg.oracle_dict(), B=1, N=L, H_q=G, H_kv=1, H_lm=G)
            o, l = oracle.dense_causal_rows(oc, qf, k, v, rows=np.array([L - 1]))
            o_b[g * G:(g + 1) * G] = o[0, :, 0]
            l_b[g * G:(g + 1) * G] = l[0, :, 0]
        outs.append(o_b)
        lses.append(l_b)
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("name", list(DECODE))
def test_dense_decode_matches_oracle(name, dev):
    inp = W.make_decode(DECODE[name], device=dev)
    cfg = inp["cfg"]
    print(f"[dense decode] {name}", flush=True)
    out, lse = hb.dense_decode(cfg, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["seq_lens"])
    torch.cuda.synchronize()
    seqs = list(range(inp["q"].shape[0]))
    ref_o, ref_l = _dense_decode_ref(cfg, inp, seqs)
    _check(cfg, host(out).float().numpy(), host(lse).numpy(), ref_o, ref_l, f"decode {name}")


def test_dense_decode_full_size_512k(dev):
    """The 16 x 512K decode step as bench.py times it: every sequence on the
    GPU, the first and the last checked against the oracle."""
    print("[dense decode] 512K: inputs", flush=True)
    inp = W.make_decode("decode_512k", device=dev)
    cfg = inp["cfg"]
    print("[dense decode] 512K: GPU", flush=True)
    out, lse = hb.dense_decode(cfg, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["seq_lens"])
    torch.cuda.synchronize()
    seqs = [0, inp["q"].shape[0] - 1]
    print("[dense decode] 512K: oracle", flush=True)
    ref_o, ref_l = _dense_decode_ref(cfg, inp, seqs)
    _check(cfg, host(out[seqs]).float().numpy(), host(lse[seqs]).numpy(), ref_o, ref_l, "decode 512K")
