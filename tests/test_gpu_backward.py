"""GPU parity of hils_sparse_attend_backward against the fp64 backward
oracle (oracle/backward.py), through the C ABI.

Each case runs the GPU forward (summaries, score/select, fused attention),
draws an output gradient and a log-partition gradient, and compares the
GPU's dq, dk, dv and dq_lm with the oracle's on the same inputs and the
GPU's selection (the backward holds the selection fixed).

Tolerance: both sides take the same inputs (bf16 values promoted exactly);
the GPU sums in fp32 over up to a few thousand terms per gradient element,
and its fusion weights come from the forward's fp32 log-partition and chunk
scores.  |gpu - ref| <= 1e-4 max|ref| + 1e-3 |ref| (bf16 inputs) and
1e-5 max|ref| + 1e-4 |ref| (fp32 inputs).
"""
import numpy as np
import pytest
import torch

from long_context_chunk_landmark_amd import _binding as hb
from long_context_chunk_landmark_amd import workloads as W
from oracle.backward import backward as oracle_backward
from tests.parity import host

pytestmark = pytest.mark.gpu

BF = torch.bfloat16
F32 = torch.float32

CASES = {
    "bf16_g2_ragged": dict(seed=91, io=BF, B=1, H_q=4, H_kv=2, d=128, N=1100, S=64, W=128, K=4),
    "fp32_d64_s128_g1": dict(seed=92, io=F32, B=1, H_q=2, H_kv=2, d=64, N=1500, S=128, W=256, K=3),
    "lmkv_g4_d64": dict(seed=93, io=BF, B=1, H_q=4, H_kv=1, H_lm=1, d=64, N=900, S=64, W=64, K=5),
    "mean_g8": dict(seed=94, io=BF, B=1, H_q=8, H_kv=1, d=128, N=800, S=64, W=128, K=3, landmark_mode=2),
    "k0_window_only": dict(seed=95, io=BF, B=1, H_q=2, H_kv=1, d=64, N=700, S=64, W=128, K=0),
    "b2_s128_d128": dict(seed=96, io=BF, B=2, H_q=4, H_kv=2, d=128, N=1000, S=128, W=128, K=2),
    "shared_b2_g2": dict(seed=97, io=BF, B=2, H_q=4, H_kv=2, d=128, N=900, S=64, W=128, K=4, landmark_mode=1),
}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hb.load_library()
    return torch.device("cuda:0")


def _run(name, dev):
    p = CASES[name]
    inp = W.make_prefill(p, device=dev)
    cfg = inp["cfg"]
    fw = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    g = torch.Generator().manual_seed(p["seed"] + 7)
    dout = torch.randn(fw["out"].shape, generator=g).to(cfg.io_dtype).to(dev)
    dlse = torch.randn(fw["lse"].shape, generator=g).to(dev)
    grads = hb.sparse_attend_backward(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"], fw["k_sum"], fw["sel_idx"],
                                      fw["sel_score"], fw["lse"], dout, dlse)
    torch.cuda.synchronize()
    return cfg, inp, fw, dout, dlse, grads


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name, dev):
    print(f"[backward] {name}", flush=True)
    cfg, inp, fw, dout, dlse, (dq, dk, dv, dq_lm) = _run(name, dev)
    lm = {hb.LM_CHUNK: "chunk", hb.LM_SHARED: "shared", hb.LM_MEAN: "mean"}[cfg.landmark_mode]
    ref = oracle_backward(cfg.oracle_dict(), host(inp["q"]), host(inp["k"]), host(inp["v"]),
                          None if inp["q_lm"] is None else host(inp["q_lm"]), host(fw["sel_idx"]), host(dout),
                          host(dlse), landmark=lm)
    a, r = (1e-4, 1e-3) if cfg.io_dtype == BF else (1e-5, 1e-4)
    pairs = [("dq", dq), ("dk", dk), ("dv", dv)] + ([("dq_lm", dq_lm)] if lm != "mean" else [])
    for key, got in pairs:
        got = host(got).numpy().astype(np.float64)
        want = ref[key]
        bound = a * np.abs(want).max() + r * np.abs(want)
        bad = np.abs(got - want) > bound
        print(f"  {key}: max err {np.abs(got - want).max():.3g} (max |ref| {np.abs(want).max():.3g})", flush=True)
        assert not bad.any(), (f"{key}: {bad.sum()} of {bad.size} outside; max err "
                               f"{np.abs(got - want).max():.3g}, max |ref| {np.abs(want).max():.3g}")
    if lm == "mean":
        assert dq_lm is None


def test_backward_is_deterministic(dev):
    cfg, inp, fw, dout, dlse, first = _run("bf16_g2_ragged", dev)
    again = hb.sparse_attend_backward(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"], fw["k_sum"], fw["sel_idx"],
                                      fw["sel_score"], fw["lse"], dout, dlse)
    torch.cuda.synchronize()
    for x, y in zip(first, again):
        assert torch.equal(x, y)


def _sampled_rows_backward(dev, p, rows, seed):
    """GPU backward against the oracle with the output gradient nonzero on
    the given rows only: the oracle visits just those rows (the gradients
    are linear in dout and dlse; its row-subset pin).  dq of every other row
    must be exactly zero."""
    inp = W.make_prefill(p, device=dev)
    cfg = inp["cfg"]
    fw = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"])
    g = torch.Generator().manual_seed(seed)
    dout = torch.zeros(fw["out"].shape, dtype=torch.float32)
    dlse = torch.zeros(fw["lse"].shape, dtype=torch.float32)
    dout[:, :, rows] = torch.randn((cfg.B, cfg.H_q, len(rows), cfg.d), generator=g)
    dlse[:, :, rows] = torch.randn((cfg.B, cfg.H_q, len(rows)), generator=g)
    dout = dout.to(cfg.io_dtype).to(dev)
    dlse = dlse.to(dev)
    dq, dk, dv, dq_lm = hb.sparse_attend_backward(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"], fw["k_sum"],
                                                  fw["sel_idx"], fw["sel_score"], fw["lse"], dout, dlse)
    torch.cuda.synchronize()
    print("[backward] oracle on the sampled rows", flush=True)
    ref = oracle_backward(cfg.oracle_dict(), host(inp["q"]), host(inp["k"]), host(inp["v"]), host(inp["q_lm"]),
                          host(fw["sel_idx"]), host(dout), host(dlse), landmark="chunk", rows=rows)
    others = np.ones(cfg.N, bool)
    others[rows] = False
    got_dq = host(dq).numpy()
    assert np.all(got_dq[:, :, others] == 0.0)
    del got_dq
    for key, got in (("dq", dq), ("dk", dk), ("dv", dv), ("dq_lm", dq_lm)):
        got = host(got).numpy().astype(np.float64)
        want = ref[key]
        bound = 1e-4 * np.abs(want).max() + 1e-3 * np.abs(want)
        bad = np.abs(got - want) > bound
        print(f"  {key}: max err {np.abs(got - want).max():.3g} (max |ref| {np.abs(want).max():.3g})", flush=True)
        assert not bad.any(), (f"{key}: {bad.sum()} of {bad.size} outside; max err "
                               f"{np.abs(got - want).max():.3g}, max |ref| {np.abs(want).max():.3g}")


def test_backward_8k_k16_sampled_rows(dev):
    """The 8K GQA workload (N = 8192, K = 16, G = 4, d = 128, S = 64: the MFMA
    row and key passes, several walk tiles and bitmap batches per block), the
    output gradient on 96 sampled rows."""
    p = dict(W.PRESETS["gqa_8k"])
    print("[backward] gqa_8k sampled rows", flush=True)
    N = p["N"]
    rng = np.random.default_rng(123)
    rows = np.sort(np.concatenate([rng.choice(np.arange(0, 2048), 24, replace=False),
                                   rng.choice(np.arange(2048, N - 1024), 40, replace=False),
                                   rng.choice(np.arange(N - 1024, N), 32, replace=False)]))
    _sampled_rows_backward(dev, p, rows, 321)


def test_backward_128k_k32_sampled_rows(dev):
    """The 128K prefill workload the bench times (N = 131072, H_q = 32,
    H_kv = 8, d = 128, S = 64, W = 1024, K = 32, drifting inputs), the output
    gradient on 32 sampled rows: early rows with fewer candidates than K,
    rows across the sequence and the last rows (the longest walks)."""
    p = dict(W.PRESETS["prefill_128k"])
    print("[backward] prefill_128k sampled rows", flush=True)
    N = p["N"]
    rng = np.random.default_rng(124)
    rows = np.sort(np.concatenate([rng.choice(np.arange(0, 4096), 8, replace=False),
                                   rng.choice(np.arange(4096, N - 2048), 16, replace=False),
                                   rng.choice(np.arange(N - 2048, N), 8, replace=False)]))
    _sampled_rows_backward(dev, p, rows, 322)