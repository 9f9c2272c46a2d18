"""The landmark summary (hyper.ai HiLS summary, section 方法: p = softmax of
the scaled landmark-query logits over the chunk's keys, k' = sum_j p_j k_j,
b' = the entropy of p) on the d = 128, bf16-key shapes that the end-to-end
cases leave out: eight landmark heads per kv head, bf16 summaries, mean-pooled
and shared landmark queries at both chunk sizes, two sequences.  Summaries
only, against the oracle's, with the tolerances of the summary stage test."""
import pytest
import torch

import oracle
from long_context_chunk_landmark_amd import _binding as hb
from long_context_chunk_landmark_amd import workloads as W
from tests.parity import assert_close, host

pytestmark = pytest.mark.gpu

BF, F32 = torch.bfloat16, torch.float32
LANDMARK = {0: "chunk", 1: "shared", 2: "mean"}

SHAPES = {
    "s64_glm8_f32": dict(seed=91, io=BF, B=1, H_q=16, H_kv=2, d=128, N=1000, S=64, W=128, K=4),
    "s128_glm8_bf16sum": dict(seed=92, io=BF, B=1, H_q=8, H_kv=1, d=128, N=1100, S=128, W=256, K=4, summary=BF),
    "s64_glm4_mean": dict(seed=93, io=BF, B=1, H_q=8, H_kv=2, d=128, N=900, S=64, W=128, K=4, landmark_mode=2),
    "s128_glm4_shared_bf16sum": dict(seed=94, io=BF, B=1, H_q=8, H_kv=2, d=128, N=1300, S=128, W=256, K=4,
                                     summary=BF, landmark_mode=1),
    "s128_glm2_mean": dict(seed=95, io=BF, B=1, H_q=4, H_kv=2, d=128, N=800, S=128, W=128, K=2, landmark_mode=2),
    "s64_glm1_shared_bf16sum": dict(seed=96, io=BF, B=1, H_q=4, H_kv=4, d=128, N=700, S=64, W=64, K=2,
                                    summary=BF, landmark_mode=1),
    "s64_glm4_b2": dict(seed=97, io=BF, B=2, H_q=8, H_kv=2, d=128, N=640, S=64, W=128, K=4),
}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hb.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("name", list(SHAPES))
def test_summary_shape_matches_oracle(name, dev):
    p = SHAPES[name]
    inp = W.make_prefill(p, device=dev)
    cfg = inp["cfg"]
    print(f"[summary shape] {name}", flush=True)
    k_sum, b_sum = hb.landmark_summarize(cfg, inp["k"], inp["q_lm"])
    torch.cuda.synchronize()
    q_lm = None if inp["q_lm"] is None else host(inp["q_lm"])
    ks, bs = oracle.summarize(cfg.oracle_dict(), host(inp["k"]), q_lm, landmark=LANDMARK[cfg.landmark_mode])
    if cfg.summary_dtype == BF:
        # bf16 storage: within one bf16 rounding of the exact value
        assert_close(host(k_sum).float().numpy(), ks, 1e-5, 2 ** -8, "k_sum")
    else:
        assert_close(host(k_sum).numpy(), ks, 1e-5, 1e-5, "k_sum")
    assert_close(host(b_sum).numpy(), bs, 1e-5, 1e-5, "b_sum")
