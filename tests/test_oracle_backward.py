"""Pins of the fp64 backward oracle (oracle/backward.py).

The gradients are checked against things other than themselves: central
finite differences of the forward (fp64, every input, random directions), a
textbook dense causal attention differentiated by torch autograd (fp64, the
limit with no selected chunks and a window covering the prefix), and the C
oracle's forward (the backward's recomputed outputs, log-partitions and
chunk scores must equal it for the same selection).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.backward import backward


def _case(seed, B=1, H_q=4, H_kv=2, H_lm=None, N=96, d=8, S=8, W=16, K=3):
    rng = np.random.default_rng(seed)
    H_lm = H_lm or H_q
    cfg = dict(B=B, N=N, H_q=H_q, H_kv=H_kv, H_lm=H_lm, d=d, S=S, W=W, K=K)
    q = rng.standard_normal((B, H_q, N, d))
    k = rng.standard_normal((B, H_kv, N, d))
    v = rng.standard_normal((B, H_kv, N, d))
    ql = rng.standard_normal((B, H_lm, N // S, d))
    dout = rng.standard_normal((B, H_q, N, d))
    dlse = rng.standard_normal((B, H_q, N))
    # the oracle's own selection (it stays fixed under the perturbations)
    ks, bs = oracle.summarize(cfg, k, ql)
    sel = oracle.forward_rows(cfg, q, k, v, ks, bs, attend=False)["sel_idx"]
    return cfg, q, k, v, ql, dout, dlse, sel


def _loss(cfg, q, k, v, ql, sel, dout, dlse, landmark="chunk"):
    r = backward(cfg, q, k, v, ql, sel, dout, dlse, landmark=landmark)
    return float((r["out"] * dout).sum() + (r["lse"] * dlse).sum())


@pytest.mark.parametrize("H_lm", [None, 2])
def test_gradients_match_finite_differences(H_lm):
    cfg, q, k, v, ql, dout, dlse, sel = _case(3, H_lm=H_lm)
    g = backward(cfg, q, k, v, ql, sel, dout, dlse)
    rng = np.random.default_rng(9)
    eps = 1e-6
    args = {"q": q, "k": k, "v": v, "ql": ql}
    grads = {"q": g["dq"], "k": g["dk"], "v": g["dv"], "ql": g["dq_lm"]}
    for name, x in args.items():
        for _ in range(2):
            u = rng.standard_normal(x.shape)
            plus = dict(args, **{name: x + eps * u})
            minus = dict(args, **{name: x - eps * u})
            fd = (_loss(cfg, plus["q"], plus["k"], plus["v"], plus["ql"], sel, dout, dlse) -
                  _loss(cfg, minus["q"], minus["k"], minus["v"], minus["ql"], sel, dout, dlse)) / (2 * eps)
            an = float((grads[name] * u).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_mean_pooling_gradients_match_finite_differences():
    cfg, q, k, v, _, dout, dlse, _ = _case(4)
    ks, bs = oracle.summarize(cfg, k, None, landmark="mean")
    sel = oracle.forward_rows(cfg, q, k, v, ks, bs, attend=False)["sel_idx"]
    g = backward(cfg, q, k, v, None, sel, dout, dlse, landmark="mean")
    assert g["dq_lm"] is None
    u = np.random.default_rng(5).standard_normal(k.shape)
    eps = 1e-6
    fd = (_loss(cfg, q, k + eps * u, v, None, sel, dout, dlse, "mean") -
          _loss(cfg, q, k - eps * u, v, None, sel, dout, dlse, "mean")) / (2 * eps)
    assert abs(fd - float((g["dk"] * u).sum())) <= 1e-6 * max(1.0, abs(fd))


def test_forward_recompute_equals_c_oracle():
    cfg, q, k, v, ql, dout, dlse, sel = _case(6, B=2, N=80)
    g = backward(cfg, q, k, v, ql, sel, dout, dlse)
    ks, bs = oracle.summarize(cfg, k, ql)
    f = oracle.forward_rows(cfg, q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), ks, bs)
    # the C oracle takes float32 data: compare on float32-rounded inputs
    g32 = backward(cfg, q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), ql.astype(np.float32), sel,
                   dout, dlse)
    np.testing.assert_array_equal(f["sel_idx"], sel)
    np.testing.assert_allclose(g32["out"], f["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g32["lse"], f["lse"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g32["sel_score"], f["sel_score"], rtol=0, atol=1e-12)
    assert np.isfinite(g["dq"]).all()


def test_dense_limit_matches_autograd():
    """No candidates (W covers the prefix): the gradients are those of plain
    causal softmax attention, here from torch autograd in fp64."""
    rng = np.random.default_rng(7)
    B, H_q, H_kv, N, d, S = 1, 4, 2, 40, 8, 8
    cfg = dict(B=B, N=N, H_q=H_q, H_kv=H_kv, d=d, S=S, W=N, K=2)
    q, k, v = (rng.standard_normal(s) for s in ((B, H_q, N, d), (B, H_kv, N, d), (B, H_kv, N, d)))
    ql = rng.standard_normal((B, H_q, N // S, d))
    dout, dlse = rng.standard_normal((B, H_q, N, d)), rng.standard_normal((B, H_q, N))
    sel = np.full((B, H_kv, N, 2), -1, np.int32)
    g = backward(cfg, q, k, v, ql, sel, dout, dlse)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(H_q // H_kv, dim=1)
    vv = tv.repeat_interleave(H_q // H_kv, dim=1)
    s = tq @ kk.transpose(-1, -2) / math.sqrt(d)
    s = s.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    lse = torch.logsumexp(s, -1)
    out = torch.softmax(s, -1) @ vv
    ((out * torch.tensor(dout)).sum() + (lse * torch.tensor(dlse)).sum()).backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=0, atol=1e-10, err_msg=name)
    assert np.all(g["dq_lm"] == 0)


def test_shared_landmark_gradients_match_finite_differences():
    cfg, q, k, v, _, dout, dlse, _ = _case(8, B=2, N=64)
    qs = np.random.default_rng(2).standard_normal((cfg["H_lm"], cfg["d"]))
    ks, bs = oracle.summarize(cfg, k, qs, landmark="shared")
    sel = oracle.forward_rows(cfg, q, k, v, ks, bs, attend=False)["sel_idx"]
    g = backward(cfg, q, k, v, qs, sel, dout, dlse, landmark="shared")
    assert g["dq_lm"].shape == qs.shape
    eps = 1e-6
    for name, x in (("q_lm", qs), ("k", k)):
        u = np.random.default_rng(3).standard_normal(x.shape)
        if name == "q_lm":
            fd = (_loss(cfg, q, k, v, qs + eps * u, sel, dout, dlse, "shared") -
                  _loss(cfg, q, k, v, qs - eps * u, sel, dout, dlse, "shared")) / (2 * eps)
            an = float((g["dq_lm"] * u).sum())
        else:
            fd = (_loss(cfg, q, k + eps * u, v, qs, sel, dout, dlse, "shared") -
                  _loss(cfg, q, k - eps * u, v, qs, sel, dout, dlse, "shared")) / (2 * eps)
            an = float((g["dk"] * u).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_row_subset_is_the_full_loop_when_other_rows_carry_no_gradient():
    """The loss is linear in dout and dlse: zeroing them outside a row set and
    visiting only those rows gives the full loop's gradients."""
    cfg, q, k, v, ql, dout, dlse, sel = _case(31)
    rows = np.array([5, 40, 41, 77, 95])
    mask = np.zeros(cfg["N"], bool)
    mask[rows] = True
    dout0 = np.where(mask[None, None, :, None], dout, 0.0)
    dlse0 = np.where(mask[None, None, :], dlse, 0.0)
    full = backward(cfg, q, k, v, ql, sel, dout0, dlse0)
    part = backward(cfg, q, k, v, ql, sel, dout0, dlse0, rows=rows)
    for key in ("dq", "dk", "dv", "dq_lm"):
        np.testing.assert_allclose(part[key], full[key], rtol=0, atol=1e-12)
    assert np.abs(full["dk"]).max() > 0 and np.abs(full["dq"][:, :, ~mask]).max() == 0
