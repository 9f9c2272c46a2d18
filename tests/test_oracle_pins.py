"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the
hand-derived worked examples in tests/golden/, closed forms (the Taylor
identity at the landmark point, the mean and one-hot limits), textbook
routines (dense causal softmax attention via scipy/numpy), brute-force
selection, and invariants (bounds, permutation invariance, linearity).
Sources: hyper.ai HiLS summary, section 方法 (surrogate-score equation,
entropy-calibrated compressed key, partition estimate, hierarchical
factorisation, Q-Cal and GQA paragraphs) and its 引言 (first-order Taylor
expansion of the chunk mass); wmrh.cn news page, "解决一" paragraph (the
expansion keeps mean and max logits as its extreme cases).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _num(x):
    if isinstance(x, (int, float)):
        return float(x)
    env = {"ln2": math.log(2), "ln3": math.log(3), "ln4": math.log(4), "ln5": math.log(5), "ln6": math.log(6),
           "ln8": math.log(8), "ln10": math.log(10)}
    return float(eval(x, {"__builtins__": {}}, env))


def _cfg(**kw):
    c = dict(B=1, H_q=1, H_kv=1, W=0, K=1)
    c.update(kw)
    c.setdefault("H_lm", c["H_q"])
    return c


def _rng(seed):
    return np.random.default_rng(seed)


def _dense_textbook(q, k, v, scale):
    """Causal softmax attention with scipy, [B,H_q,N,d] x [B,H_kv,N,d]."""
    B, H_q, N, d = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    kk = np.repeat(k.astype(np.float64), G, axis=1)
    vv = np.repeat(v.astype(np.float64), G, axis=1)
    s = scale * np.einsum("bhid,bhjd->bhij", q.astype(np.float64), kk)
    mask = np.tril(np.ones((N, N), bool))
    s = np.where(mask, s, -np.inf)
    lse = logsumexp(s, axis=-1)
    p = np.exp(s - lse[..., None])
    return np.einsum("bhij,bhjd->bhid", p, vv), lse


# ---------------------------------------------------------------- worked examples


def test_worked_summary_two_keys():
    g = json.load(open(GOLDEN))["summary_two_keys"]
    cfg = _cfg(N=2, S=2, d=1)
    k = np.array([[[[_num(x[0])] for x in g["keys"]]]], np.float32)
    ql = np.array([[[[g["q_lm"][0]]]]], np.float32)
    # the oracle sees the float32 rounding L of ln 3; the closed forms with
    # that L are p = [1, e^L] / (1 + e^L), k' = p_2 L, b' = -sum p log p
    L = float(k[0, 0, 1, 0])
    p2 = math.exp(L) / (1 + math.exp(L))
    p1 = 1 - p2
    k_sum, b_sum = oracle.summarize(cfg, k, ql)
    assert k_sum[0, 0, 0, 0] == pytest.approx(p2 * L, abs=1e-15)
    assert b_sum[0, 0, 0] == pytest.approx(-(p1 * math.log(p1) + p2 * math.log(p2)), abs=1e-15)
    # and the exact-ln3 closed forms of the fixture, within the float32 rounding of ln 3
    assert k_sum[0, 0, 0, 0] == pytest.approx(_num(g["k_sum"][0]), abs=1e-7)
    assert b_sum[0, 0, 0] == pytest.approx(_num(g["b_sum"][0]), abs=1e-7)
    # surrogate score of q = 1 and q = 2 against the closed forms
    for qv, key in ((1.0, "score_q1"), (2.0, "score_q2")):
        s = qv * k_sum[0, 0, 0, 0] + b_sum[0, 0, 0]
        assert s == pytest.approx(_num(g[key]), abs=1e-7)
    assert 2.0 * k_sum[0, 0, 0, 0] + b_sum[0, 0, 0] < _num(g["log_mass_q2"])


def test_worked_prefill_s1():
    g = json.load(open(GOLDEN))["prefill_s1"]
    cfg = _cfg(N=g["N"], S=g["S"], W=g["W"], K=g["K"], d=g["d"])
    q = np.array(g["q"], np.float32).reshape(1, 1, -1, 1)
    k = np.array([_num(x) for x in g["k"]], np.float32).reshape(1, 1, -1, 1)
    v = np.array(g["v"], np.float32).reshape(1, 1, -1, 1)
    ql = np.array(g["q_lm"], np.float32).reshape(1, 1, -1, 1)
    ks, bs = oracle.summarize(cfg, k, ql)
    res = oracle.forward_rows(cfg, q, k, v, ks, bs)
    assert res["sel_idx"][0, 0, :, :].tolist() == g["sel"]
    np.testing.assert_allclose(res["out"][0, 0, :, 0], g["out"], atol=1e-6)
    np.testing.assert_allclose(res["lse"][0, 0], [_num(x) for x in g["lse"]], atol=1e-6)


@pytest.mark.parametrize("K", [1, 2])
def test_worked_prefill_s2(K):
    g = json.load(open(GOLDEN))["prefill_s2"]
    cfg = _cfg(N=g["N"], S=g["S"], W=g["W"], K=K, d=g["d"])
    q = np.array(g["q"], np.float32).reshape(1, 1, -1, 1)
    k = np.array([_num(x) for x in g["k"]], np.float32).reshape(1, 1, -1, 1)
    v = np.array(g["v"], np.float32).reshape(1, 1, -1, 1)
    ql = np.array(g["q_lm"], np.float32).reshape(1, 1, -1, 1)
    ks, bs = oracle.summarize(cfg, k, ql)
    res = oracle.forward_rows(cfg, q, k, v, ks, bs, rows=[g["row"]])
    exp = g["K%d" % K]
    assert res["sel_idx"][0, 0, 0, :].tolist() == exp["sel"]
    assert res["out"][0, 0, 0, 0] == pytest.approx(exp["out"], abs=1e-6)
    assert res["lse"][0, 0, 0] == pytest.approx(_num(exp["lse"]), abs=1e-6)


# ---------------------------------------------------------------- summary pins


def test_taylor_identity_landmark_equals_query():
    """Invariant (a): with q'_c = q_i, s^_ic = log sum_{j in c} exp(s_ij)."""
    rng = _rng(11)
    S, d, N = 16, 32, 256
    C = N // S
    cfg = _cfg(N=N, S=S, d=d, W=S, K=4)
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    i = N - 1
    ql = np.broadcast_to(q[:, :, i:i + 1, :], (1, 1, C, d)).copy()
    ks, bs = oracle.summarize(cfg, k, ql)
    res = oracle.forward_rows(cfg, q, k, v, ks, bs, rows=[i], want_agg=True, attend=False)
    scale = 1 / math.sqrt(d)
    s = scale * (k[0, 0].astype(np.float64) @ q[0, 0, i].astype(np.float64))
    n_cand = i // S - 1
    want = [logsumexp(s[c * S:(c + 1) * S]) for c in range(n_cand)]
    np.testing.assert_allclose(res["agg"][0, 0, 0, :n_cand], want, rtol=0, atol=1e-11)


def test_self_landmark_mode_matches_log_mass():
    rng = _rng(12)
    S, d, N, G = 8, 16, 128, 2
    cfg = _cfg(N=N, S=S, d=d, W=2 * S, K=3, H_q=G, H_kv=1, H_lm=G)
    q = rng.standard_normal((1, G, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    rows = [50, 77, 127]
    a = oracle.forward_rows(cfg, q, k, v, rows=rows, mode="self_landmark", want_agg=True, attend=False)
    b = oracle.forward_rows(cfg, q, k, v, rows=rows, mode="exact_mass", want_agg=True, attend=False)
    scale = 1 / math.sqrt(d)
    for ri, i in enumerate(rows):
        n_cand = max(0, i // S - 2)
        s = scale * np.einsum("hd,jd->hj", q[0, :, i].astype(np.float64), k[0, 0].astype(np.float64))
        lm = np.array([[logsumexp(s[h, c * S:(c + 1) * S]) for c in range(n_cand)] for h in range(G)])
        np.testing.assert_allclose(b["agg"][0, 0, ri, :n_cand], lm.max(0), atol=1e-11)
        np.testing.assert_allclose(a["agg"][0, 0, ri, :n_cand], lm.max(0), atol=1e-11)


def test_mean_limit_zero_landmark():
    """q' = 0: p uniform, k' = mean key, b' = log S (mean-logit extreme)."""
    rng = _rng(13)
    S, d, N = 16, 24, 64
    cfg = _cfg(N=N, S=S, d=d)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    ql = np.zeros((1, 1, N // S, d), np.float32)
    ks, bs = oracle.summarize(cfg, k, ql)
    np.testing.assert_allclose(ks[0, 0], k[0, 0].astype(np.float64).reshape(-1, S, d).mean(1), atol=1e-12)
    np.testing.assert_allclose(bs[0, 0], math.log(S), atol=1e-12)


def test_one_hot_limit_dominant_key():
    """A landmark query aligned with one key, scaled up: p -> one-hot,
    k' -> that key, b' -> 0 (max-logit extreme)."""
    rng = _rng(14)
    S, d, N = 8, 16, 32
    cfg = _cfg(N=N, S=S, d=d)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    jstar = [3, 0, 7, 5]
    ql = np.stack([400.0 * k[0, 0, c * S + j] for c, j in enumerate(jstar)])[None, None].astype(np.float32)
    ks, bs = oracle.summarize(cfg, k, ql)
    for c, j in enumerate(jstar):
        np.testing.assert_allclose(ks[0, 0, c], k[0, 0, c * S + j], atol=1e-6)
        assert 0.0 <= bs[0, 0, c] < 1e-5


def test_equal_keys_give_exact_mass_for_any_landmark():
    rng = _rng(15)
    S, d, N = 8, 16, 64
    cfg = _cfg(N=N, S=S, d=d, W=S, K=2)
    base = rng.standard_normal((N // S, d)).astype(np.float32)
    k = np.repeat(base, S, axis=0)[None, None]
    ql = rng.standard_normal((1, 1, N // S, d)).astype(np.float32) * 3
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    ks, bs = oracle.summarize(cfg, k, ql)
    i = N - 1
    res = oracle.forward_rows(cfg, q, k, v, ks, bs, rows=[i], want_agg=True, attend=False)
    s = (k[0, 0].astype(np.float64) @ q[0, 0, i].astype(np.float64)) / math.sqrt(d)
    n_cand = i // S - 1
    want = [logsumexp(s[c * S:(c + 1) * S]) for c in range(n_cand)]
    np.testing.assert_allclose(res["agg"][0, 0, 0, :n_cand], want, atol=1e-11)


def test_summary_bounds_and_permutation_invariance():
    rng = _rng(16)
    S, d, N, H_kv, H_lm = 16, 32, 256, 2, 4
    cfg = _cfg(N=N, S=S, d=d, H_q=4, H_kv=H_kv, H_lm=H_lm)
    k = (rng.standard_normal((1, H_kv, N, d)) * 2).astype(np.float32)
    ql = (rng.standard_normal((1, H_lm, N // S, d)) * 2).astype(np.float32)
    ks, bs = oracle.summarize(cfg, k, ql)
    assert np.all(bs >= -1e-12) and np.all(bs <= math.log(S) + 1e-12)
    kc = k.astype(np.float64).reshape(1, H_kv, N // S, S, d)
    for l in range(H_lm):
        g = l * H_kv // H_lm
        assert np.all(ks[0, l] <= kc[0, g].max(1) + 1e-12)
        assert np.all(ks[0, l] >= kc[0, g].min(1) - 1e-12)
    perm = np.concatenate([c * S + rng.permutation(S) for c in range(N // S)])
    ks2, bs2 = oracle.summarize(cfg, k[:, :, perm], ql)
    np.testing.assert_allclose(ks2, ks, atol=1e-12)
    np.testing.assert_allclose(bs2, bs, atol=1e-12)


def test_surrogate_never_exceeds_log_mass():
    """The tangent of the convex log-sum-exp lies below it: s^ <= log Z."""
    rng = _rng(17)
    S, d, N = 16, 32, 512
    cfg = _cfg(N=N, S=S, d=d, W=S, K=2)
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    ql = rng.standard_normal((1, 1, N // S, d)).astype(np.float32)
    ks, bs = oracle.summarize(cfg, k, ql)
    rows = np.arange(2 * S, N, 7)
    a = oracle.forward_rows(cfg, q, k, v, ks, bs, rows=rows, want_agg=True, attend=False)["agg"]
    scale = 1 / math.sqrt(d)
    for ri, i in enumerate(rows):
        n = i // S - 1
        s = scale * (k[0, 0].astype(np.float64) @ q[0, 0, i].astype(np.float64))
        lz = np.array([logsumexp(s[c * S:(c + 1) * S]) for c in range(n)])
        assert np.all(a[0, 0, ri, :n] <= lz + 1e-12)


# ---------------------------------------------------------------- selection pins


def _random_case(seed, S=8, d=16, N=256, G=2, H_kv=2, H_lm=None, W_chunks=1, K=3):
    rng = _rng(seed)
    H_q = G * H_kv
    H_lm = H_lm or H_q
    cfg = _cfg(N=N, S=S, d=d, W=W_chunks * S, K=K, H_q=H_q, H_kv=H_kv, H_lm=H_lm)
    q = rng.standard_normal((1, H_q, N, d)).astype(np.float32)
    k = rng.standard_normal((1, H_kv, N, d)).astype(np.float32)
    v = rng.standard_normal((1, H_kv, N, d)).astype(np.float32)
    ql = rng.standard_normal((1, H_lm, N // S, d)).astype(np.float32)
    return cfg, q, k, v, ql


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_k1_selection_is_brute_force_argmax(seed):
    """Invariant (c): K = 1 selects the argmax of the group score."""
    cfg, q, k, v, ql = _random_case(seed, K=1)
    ks, bs = oracle.summarize(cfg, k, ql)
    rows = np.arange(cfg["N"])
    res = oracle.forward_rows(cfg, q, k, v, ks, bs, rows=rows, want_agg=True, attend=False)
    S, W = cfg["S"], cfg["W"]
    for g in range(cfg["H_kv"]):
        for i in rows:
            n = max(0, i // S - W // S)
            sel = res["sel_idx"][0, g, i, 0]
            if n == 0:
                assert sel == -1
                continue
            agg = res["agg"][0, g, i, :n]
            best = int(np.flatnonzero(agg == agg.max())[0])
            assert sel == best


@pytest.mark.parametrize("K", [0, 1, 2, 5, 40])
def test_topk_selection_is_brute_force_sort(K):
    cfg, q, k, v, ql = _random_case(31 + K, K=K)
    ks, bs = oracle.summarize(cfg, k, ql)
    res = oracle.forward_rows(cfg, q, k, v, ks, bs, want_agg=True, attend=False)
    S, W = cfg["S"], cfg["W"]
    for g in range(cfg["H_kv"]):
        for i in range(cfg["N"]):
            n = max(0, i // S - W // S)
            agg = res["agg"][0, g, i, :n]
            order = sorted(range(n), key=lambda c: (-agg[c], c))[:K]
            want = sorted(order) + [-1] * (K - len(order))
            assert res["sel_idx"][0, g, i].tolist() == want


def test_group_score_is_max_over_heads():
    """GQA: the group score of a chunk is the max of its per-head scores."""
    cfg, q, k, v, ql = _random_case(41, G=4, H_kv=1, K=2)
    ks, bs = oracle.summarize(cfg, k, ql)
    rows = np.arange(100, 256, 5)
    full = oracle.forward_rows(cfg, q, k, v, ks, bs, rows=rows, want_agg=True, attend=False)["agg"]
    per_head = []
    for h in range(4):
        c1 = dict(cfg, H_q=1, H_kv=1, H_lm=1)
        r = oracle.forward_rows(c1, q[:, h:h + 1], k, v, ks[:, h:h + 1], bs[:, h:h + 1], rows=rows, want_agg=True,
                                attend=False)
        per_head.append(r["agg"][0, 0])
    np.testing.assert_array_equal(np.nan_to_num(full[0, 0], nan=-7.0),
                                  np.nan_to_num(np.max(per_head, axis=0), nan=-7.0))


def test_identical_heads_equal_one_head():
    cfg, q, k, v, ql = _random_case(42, G=4, H_kv=1, K=3)
    q[:, 1:] = q[:, :1]
    ql[:, 1:] = ql[:, :1]
    ks, bs = oracle.summarize(cfg, k, ql)
    full = oracle.forward_rows(cfg, q, k, v, ks, bs)
    c1 = dict(cfg, H_q=1, H_kv=1, H_lm=1)
    one = oracle.forward_rows(c1, q[:, :1], k, v, ks[:, :1], bs[:, :1])
    np.testing.assert_array_equal(full["sel_idx"], one["sel_idx"])
    for h in range(4):
        np.testing.assert_allclose(full["out"][0, h], one["out"][0, 0], atol=1e-13)


def test_exact_tie_resolves_to_lower_index():
    """A duplicated chunk with an identical landmark query ties exactly; the
    lower chunk index must win."""
    rng = _rng(51)
    S, d, N = 8, 16, 128
    cfg = _cfg(N=N, S=S, d=d, W=S, K=1)
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32) * 0.1
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    ql = rng.standard_normal((1, 1, N // S, d)).astype(np.float32)
    i = N - 1
    # chunks 3 and 9 get identical keys aligned with q_i (top scores)
    blk = (np.outer(np.ones(S), q[0, 0, i]) + 0.01 * rng.standard_normal((S, d))).astype(np.float32)
    k[0, 0, 3 * S:4 * S] = blk
    k[0, 0, 9 * S:10 * S] = blk
    ql[0, 0, 9] = ql[0, 0, 3]
    ks, bs = oracle.summarize(cfg, k, ql)
    res = oracle.forward_rows(cfg, q, k, v, ks, bs, rows=[i], want_agg=True, attend=False)
    agg = res["agg"][0, 0, 0]
    assert agg[3] == agg[9] and agg[3] == np.nanmax(agg)
    assert res["sel_idx"][0, 0, 0, 0] == 3
    cfg2 = dict(cfg, K=2)
    res2 = oracle.forward_rows(cfg2, q, k, v, ks, bs, rows=[i], attend=False)
    assert res2["sel_idx"][0, 0, 0].tolist() == [3, 9]


def test_candidates_and_window_partition_the_prefix():
    """Window keys and candidate chunks are disjoint and cover [0, i]: with
    S = 1, every key is its own chunk, s^ equals the logit, and HiLS with
    K >= n_cand is dense causal attention."""
    rng = _rng(61)
    for W in (0, 1, 3):
        N, d = 40, 8
        cfg = _cfg(N=N, S=1, d=d, W=W, K=N)
        q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
        k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
        v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
        ql = rng.standard_normal((1, 1, N, d)).astype(np.float32)
        ks, bs = oracle.summarize(cfg, k, ql)
        res = oracle.forward_rows(cfg, q, k, v, ks, bs)
        o, l = _dense_textbook(q, k, v, 1 / math.sqrt(d))
        np.testing.assert_allclose(res["out"], o, atol=1e-12)
        np.testing.assert_allclose(res["lse"], l, atol=1e-12)


def test_s1_topk_tokens_plus_window():
    """S = 1: chunk = one key, so HiLS is exact softmax attention restricted to
    the window plus the K highest-logit earlier keys (ties to the lower index)."""
    rng = _rng(62)
    N, d, W, K = 64, 8, 4, 5
    cfg = _cfg(N=N, S=1, d=d, W=W, K=K)
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    ql = np.zeros((1, 1, N, d), np.float32)
    ks, bs = oracle.summarize(cfg, k, ql)
    res = oracle.forward_rows(cfg, q, k, v, ks, bs)
    scale = 1 / math.sqrt(d)
    for i in range(N):
        s = scale * (k[0, 0].astype(np.float64) @ q[0, 0, i].astype(np.float64))
        n = max(0, i - W)
        top = sorted(range(n), key=lambda c: (-s[c], c))[:K]
        keys = sorted(top) + list(range(n, i + 1))
        p = np.exp(s[keys] - logsumexp(s[keys]))
        np.testing.assert_allclose(res["out"][0, 0, i], p @ v[0, 0, keys].astype(np.float64), atol=1e-12)
        assert res["lse"][0, 0, i] == pytest.approx(logsumexp(s[keys]), abs=1e-12)
        assert res["sel_idx"][0, 0, i].tolist() == sorted(top) + [-1] * (K - len(top))


# ---------------------------------------------------------------- fused output pins


@pytest.mark.parametrize("G,H_kv", [(1, 1), (2, 2), (4, 1)])
def test_self_landmark_all_chunks_is_dense(G, H_kv):
    """Invariant (b): landmark = query and K >= n_cand give dense
    causal attention."""
    rng = _rng(71 + G)
    S, d, N = 8, 16, 96
    H_q = G * H_kv
    cfg = _cfg(N=N, S=S, d=d, W=2 * S, K=N // S, H_q=H_q, H_kv=H_kv)
    q = rng.standard_normal((1, H_q, N, d)).astype(np.float32)
    k = rng.standard_normal((1, H_kv, N, d)).astype(np.float32)
    v = rng.standard_normal((1, H_kv, N, d)).astype(np.float32)
    res = oracle.forward_rows(cfg, q, k, v, mode="self_landmark")
    o, l = _dense_textbook(q, k, v, 1 / math.sqrt(d))
    np.testing.assert_allclose(res["out"], o, atol=1e-11)
    np.testing.assert_allclose(res["lse"], l, atol=1e-11)


def test_chunk_constant_keys_all_chunks_is_dense():
    """Keys constant inside each chunk make s^ the exact log-mass for any
    landmark query; with K >= n_cand the result is dense causal attention."""
    rng = _rng(81)
    S, d, N, G = 8, 16, 128, 2
    cfg = _cfg(N=N, S=S, d=d, W=S, K=N // S, H_q=G, H_kv=1, H_lm=G)
    base = rng.standard_normal((1, 1, N // S, d)).astype(np.float32)
    k = np.repeat(base, S, axis=2)
    q = rng.standard_normal((1, G, N, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    ql = (rng.standard_normal((1, G, N // S, d)) * 5).astype(np.float32)
    ks, bs = oracle.summarize(cfg, k, ql)
    res = oracle.forward_rows(cfg, q, k, v, ks, bs)
    o, l = _dense_textbook(q, k, v, 1 / math.sqrt(d))
    np.testing.assert_allclose(res["out"], o, atol=1e-11)
    np.testing.assert_allclose(res["lse"], l, atol=1e-11)


def test_rows_without_candidates_are_dense():
    cfg, q, k, v, ql = _random_case(91, S=8, N=128, W_chunks=3, K=2)
    ks, bs = oracle.summarize(cfg, k, ql)
    rows = np.arange(0, 4 * 8)  # floor(i/S) - W/S <= 0
    res = oracle.forward_rows(cfg, q, k, v, ks, bs, rows=rows)
    o, l = _dense_textbook(q, k, v, 1 / math.sqrt(cfg["d"]))
    np.testing.assert_allclose(res["out"], o[:, :, rows], atol=1e-12)
    np.testing.assert_allclose(res["lse"], l[:, :, rows], atol=1e-12)


def test_dense_causal_rows_is_textbook_attention():
    """The oracle's dense causal attention equals the numpy/scipy textbook
    softmax attention under GQA (query head h reads kv head h // G), on all
    rows and on a row subset; with every key equal, each row's output is the
    mean of the values 0..i and its log-mass is s + log(i + 1)."""
    rng = _rng(97)
    B, H_q, H_kv, N, d = 2, 4, 2, 40, 16
    cfg = _cfg(B=B, H_q=H_q, H_kv=H_kv, N=N, S=8, d=d)
    q = rng.standard_normal((B, H_q, N, d)).astype(np.float32)
    k = rng.standard_normal((B, H_kv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, H_kv, N, d)).astype(np.float32)
    o_ref, l_ref = _dense_textbook(q, k, v, 1 / math.sqrt(d))
    o, l = oracle.dense_causal_rows(cfg, q, k, v)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, atol=1e-12)
    rows = np.array([0, 7, 8, 39])
    o2, l2 = oracle.dense_causal_rows(cfg, q, k, v, rows=rows)
    np.testing.assert_allclose(o2, o_ref[:, :, rows], atol=1e-12)
    np.testing.assert_allclose(l2, l_ref[:, :, rows], atol=1e-12)
    ke = np.broadcast_to(k[:, :, :1], k.shape).copy()
    o3, l3 = oracle.dense_causal_rows(cfg, q, ke, v)
    cnt = np.arange(1, N + 1, dtype=np.float64)
    mean_v = np.cumsum(v.astype(np.float64), axis=2) / cnt[None, None, :, None]
    s = np.einsum("bhid,bhd->bhi", q.astype(np.float64), np.repeat(ke[:, :, 0].astype(np.float64), 2, axis=1))
    np.testing.assert_allclose(o3, np.repeat(mean_v, 2, axis=1), atol=1e-12)
    np.testing.assert_allclose(l3, s / math.sqrt(d) + np.log(cnt)[None, None, :], atol=1e-12)


def test_fusion_weights_are_convex_and_output_linear_in_v():
    cfg, q, k, v, ql = _random_case(92, K=2)
    ks, bs = oracle.summarize(cfg, k, ql)
    const = np.full_like(v, 0.37)
    r = oracle.forward_rows(cfg, q, k, const, ks, bs)
    np.testing.assert_allclose(r["out"], 0.37, atol=1e-13)
    v2 = _rng(93).standard_normal(v.shape).astype(np.float32)
    a = oracle.forward_rows(cfg, q, k, v, ks, bs)
    b = oracle.forward_rows(cfg, q, k, v2, ks, bs)
    both = oracle.forward_rows(cfg, q, k, (v.astype(np.float64) + 2 * v2.astype(np.float64)).astype(np.float32), ks,
                               bs)
    # v + 2 v2 is rounded to float32 once; compare within that rounding
    np.testing.assert_allclose(both["out"], a["out"] + 2 * b["out"], atol=2e-6)
    np.testing.assert_array_equal(a["sel_idx"], b["sel_idx"])


def test_fusion_equals_bias_form_softmax():
    """Bias form: the fused output is softmax attention over selected and
    window keys with logits s_ij + (s^_ic - log Z_ic) on selected keys."""
    cfg, q, k, v, ql = _random_case(94, S=8, N=160, G=2, H_kv=1, K=3)
    ks, bs = oracle.summarize(cfg, k, ql)
    res = oracle.forward_rows(cfg, q, k, v, ks, bs)
    S, W, d = cfg["S"], cfg["W"], cfg["d"]
    scale = 1 / math.sqrt(d)
    for h in range(2):
        for i in range(0, 160, 3):
            s = scale * (k[0, 0].astype(np.float64) @ q[0, h, i].astype(np.float64))
            logits, keys = [], []
            for kk, c in enumerate(res["sel_idx"][0, 0, i]):
                if c < 0:
                    continue
                blk = s[c * S:(c + 1) * S]
                delta = res["sel_score"][0, h, i, kk] - logsumexp(blk)
                logits += list(blk + delta)
                keys += list(range(c * S, (c + 1) * S))
            w0 = max(0, (i // S) * S - W)
            logits += list(s[w0:i + 1])
            keys += list(range(w0, i + 1))
            logits = np.array(logits)
            p = np.exp(logits - logsumexp(logits))
            np.testing.assert_allclose(res["out"][0, h, i], p @ v[0, 0, keys].astype(np.float64), atol=1e-12)
            assert res["lse"][0, h, i] == pytest.approx(logsumexp(logits), abs=1e-12)


# ---------------------------------------------------------------- Q-Cal pins


def _qcal_inputs(seed, N, H_q, d, d_model=24, r=3):
    rng = _rng(seed)
    h = rng.standard_normal((1, N, d_model)).astype(np.float32)
    wd = (rng.standard_normal((r, d_model)) / math.sqrt(d_model)).astype(np.float32)
    wu = (rng.standard_normal((H_q * d, r)) / math.sqrt(d_model)).astype(np.float32)
    return h, wd, wu


def test_qcal_rows_match_matmul():
    cfg, q, k, v, ql = _random_case(101, G=2, H_kv=2)
    h, wd, wu = _qcal_inputs(102, cfg["N"], cfg["H_q"], cfg["d"])
    rows = np.array([0, 5, 99, 255])
    got = oracle.qcal_rows(cfg, q, h, wd, wu, rows)
    hd = h[0, rows].astype(np.float64)
    delta = (hd @ wd.astype(np.float64).T) @ wu.astype(np.float64).T  # [R, H_q*d]
    want = q[0][:, rows].astype(np.float64) + delta.reshape(len(rows), cfg["H_q"], cfg["d"]).transpose(1, 0, 2)
    np.testing.assert_allclose(got[0], want, atol=1e-12)


def test_qcal_zero_up_projection_is_identity():
    cfg, q, k, v, ql = _random_case(103)
    h, wd, wu = _qcal_inputs(104, cfg["N"], cfg["H_q"], cfg["d"])
    ks, bs = oracle.summarize(cfg, k, ql)
    a = oracle.forward_rows(cfg, q, k, v, ks, bs)
    b = oracle.forward_rows(cfg, q, k, v, ks, bs, qcal=(h, wd, np.zeros_like(wu)))
    for key in ("sel_idx", "sel_score", "out", "lse"):
        np.testing.assert_array_equal(a[key], b[key])


def test_qcal_only_changes_scoring():
    """Q-Cal moves the scoring query only: scores equal those of the plain
    path run with q + dq, while the intra-chunk attention still uses raw q."""
    cfg, q, k, v, ql = _random_case(105, G=2, H_kv=1, K=2)
    h, wd, wu = _qcal_inputs(106, cfg["N"], cfg["H_q"], cfg["d"])
    ks, bs = oracle.summarize(cfg, k, ql)
    qs = oracle.qcal_rows(cfg, q, h, wd, wu)  # float64
    a = oracle.forward_rows(cfg, q, k, v, ks, bs, qcal=(h, wd, wu), want_agg=True)
    b = oracle.forward_rows(cfg, qs.astype(np.float32), k, v, ks, bs, want_agg=True)
    np.testing.assert_allclose(np.nan_to_num(a["agg"]), np.nan_to_num(b["agg"]), atol=1e-5)
    # fixed selection: raw-q attention inside chunks, Q-Cal scores as weights
    c = oracle.forward_rows(cfg, q, k, v, ks, bs, given_sel=a["sel_idx"])
    S, W = cfg["S"], cfg["W"]
    scale = 1 / math.sqrt(cfg["d"])
    i, hh = 200, 1
    s = scale * (k[0, 0].astype(np.float64) @ q[0, hh, i].astype(np.float64))
    terms, outs = [], []
    for kk, ch in enumerate(a["sel_idx"][0, 0, i]):
        blk = s[ch * S:(ch + 1) * S]
        p = np.exp(blk - logsumexp(blk))
        outs.append(p @ v[0, 0, ch * S:(ch + 1) * S].astype(np.float64))
        terms.append(a["sel_score"][0, hh, i, kk])
    w0 = (i // S) * S - W
    sw = s[w0:i + 1]
    outs.append(np.exp(sw - logsumexp(sw)) @ v[0, 0, w0:i + 1].astype(np.float64))
    terms.append(logsumexp(sw))
    wts = np.exp(np.array(terms) - logsumexp(terms))
    np.testing.assert_allclose(a["out"][0, hh, i], wts @ np.array(outs), atol=1e-12)
    assert not np.allclose(a["sel_score"], c["sel_score"])


# ---------------------------------------------------------------- decode pins


def test_decode_equals_prefill_row():
    """A decode step at position t over a paged cache equals prefill row t."""
    rng = _rng(111)
    S, d, G, H_kv = 8, 16, 2, 2
    H_q = G * H_kv
    N = 200  # ragged: the last chunk is partial
    cfg = _cfg(N=N, S=S, d=d, W=2 * S, K=3, H_q=H_q, H_kv=H_kv)
    q = rng.standard_normal((1, H_q, N, d)).astype(np.float32)
    k = rng.standard_normal((1, H_kv, N, d)).astype(np.float32)
    v = rng.standard_normal((1, H_kv, N, d)).astype(np.float32)
    ql = rng.standard_normal((1, H_q, N // S, d)).astype(np.float32)
    ks, bs = oracle.summarize(cfg, k, ql)
    ks32, bs32 = ks.astype(np.float32), bs.astype(np.float32)
    n_pages = (N + S - 1) // S
    P = n_pages + 5
    perm = rng.permutation(P)[:n_pages].astype(np.int32)
    kc = np.zeros((P, H_kv, S, d), np.float32)
    vc = np.zeros((P, H_kv, S, d), np.float32)
    ksc = np.zeros((P, H_q, d), np.float32)
    bsc = np.zeros((P, H_q), np.float32)
    for c in range(n_pages):
        n = min(S, N - c * S)
        kc[perm[c], :, :n] = k[0, :, c * S:c * S + n]
        vc[perm[c], :, :n] = v[0, :, c * S:c * S + n]
        if c < N // S:
            ksc[perm[c]] = ks32[0, :, c]
            bsc[perm[c]] = bs32[0, :, c]
    ts = [N - 1, 150, 63, 10]
    for t in ts:
        dec = oracle.decode(cfg, q[0, :, t][None], kc, vc, ksc, bsc, perm[None], np.array([t + 1], np.int32))
        pre = oracle.forward_rows(cfg, q, k, v, ks32.astype(np.float64), bs32.astype(np.float64), rows=[t])
        np.testing.assert_array_equal(dec["sel_idx"][0], pre["sel_idx"][0, :, 0])
        np.testing.assert_allclose(dec["out"][0], pre["out"][0, :, 0], atol=1e-13)
        np.testing.assert_allclose(dec["lse"][0], pre["lse"][0, :, 0], atol=1e-13)
        np.testing.assert_allclose(dec["sel_score"][0], pre["sel_score"][0, :, 0], atol=1e-13)


# ---------------------------------------------------------------- paged serving pins


def _paged_layout(rng, k, v, ks32, bs32, S, extra=5):
    """Scatter contiguous [B, H, N, d] keys/values (and [B, H_lm, C, ...]
    summaries) into a paged cache at a random page placement."""
    B, H_kv, N, d = k.shape
    H_lm = ks32.shape[1]
    n_pages = (N + S - 1) // S
    P = B * n_pages + extra
    bt = rng.permutation(P)[:B * n_pages].reshape(B, n_pages).astype(np.int32)
    kc = np.zeros((P, H_kv, S, d), np.float32)
    vc = np.zeros((P, H_kv, S, d), np.float32)
    ksc = np.zeros((P, H_lm, d), np.float32)
    bsc = np.zeros((P, H_lm), np.float32)
    for b in range(B):
        for c in range(n_pages):
            n = min(S, N - c * S)
            kc[bt[b, c], :, :n] = k[b, :, c * S:c * S + n]
            vc[bt[b, c], :, :n] = v[b, :, c * S:c * S + n]
            if c < N // S:
                ksc[bt[b, c]] = ks32[b, :, c]
                bsc[bt[b, c]] = bs32[b, :, c]
    return kc, vc, ksc, bsc, bt


def test_summarize_pages_equals_contiguous_summaries():
    """Summaries computed page by page, at any page placement, are those of
    the contiguous sequence (placement independence); ids outside [0, P)
    are skipped."""
    rng = _rng(131)
    S, d, H_kv, H_lm, B = 8, 16, 2, 4, 2
    N = 6 * S
    k = rng.standard_normal((B, H_kv, N, d)).astype(np.float32)
    ql = rng.standard_normal((B, H_lm, N // S, d)).astype(np.float32)
    cfg = _cfg(B=B, N=N, S=S, d=d, H_q=H_lm, H_kv=H_kv, H_lm=H_lm)
    ks, bs = oracle.summarize(cfg, k, ql)
    kc, _, _, _, bt = _paged_layout(rng, k, k, ks.astype(np.float32), bs.astype(np.float32), S)
    P = kc.shape[0]
    items = [(b, c) for b in range(B) for c in range(N // S)]
    order = rng.permutation(len(items))
    pages = np.array([bt[items[i]] for i in order] + [-1, P], np.int32)
    q_items = np.stack([ql[items[i][0], :, items[i][1]] for i in order] + [ql[0, :, 0]] * 2)
    got_k, got_b = oracle.summarize_pages(cfg, kc, q_items, pages)
    for j, i in enumerate(order):
        b, c = items[i]
        np.testing.assert_allclose(got_k[j], ks[b, :, c], rtol=0, atol=1e-14)
        np.testing.assert_allclose(got_b[j], bs[b, :, c], rtol=0, atol=1e-14)
    assert np.isnan(got_k[-2:]).all() and np.isnan(got_b[-2:]).all()


@pytest.mark.parametrize("q_start,n,qcal", [(0, 70, False), (48, 100, False), (96, 61, True)])
def test_prefill_paged_equals_prefill_rows(q_start, n, qcal):
    """Chunked prefill of rows q_start .. q_start + n - 1 over a paged cache
    (random page placement) equals those rows of the whole-sequence prefill:
    selection, selected scores, output and log-partition."""
    rng = _rng(141 + q_start)
    S, d, G, H_kv, B = 8, 16, 2, 2, 2
    H_q = G * H_kv
    N = q_start + n
    cfg = _cfg(B=B, N=N, S=S, d=d, W=2 * S, K=3, H_q=H_q, H_kv=H_kv)
    q = rng.standard_normal((B, H_q, N, d)).astype(np.float32)
    k = rng.standard_normal((B, H_kv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, H_kv, N, d)).astype(np.float32)
    ql = rng.standard_normal((B, H_q, N // S, d)).astype(np.float32)
    ks, bs = oracle.summarize(cfg, k, ql)
    ks32, bs32 = ks.astype(np.float32), bs.astype(np.float32)
    kc, vc, ksc, bsc, bt = _paged_layout(rng, k, v, ks32, bs32, S)
    qc_full = qc_new = None
    if qcal:
        h, wd, wu = _qcal_inputs(7, N, H_q, d)
        h = np.concatenate([h, rng.standard_normal(h.shape).astype(np.float32)])  # B = 2
        qc_full = (h, wd, wu)
        qc_new = (h[:, q_start:], wd, wu)
    rows = np.arange(q_start, N)
    pre = oracle.forward_rows(cfg, q, k, v, ks32.astype(np.float64), bs32.astype(np.float64), rows=rows,
                              qcal=qc_full)
    got = oracle.prefill_paged(cfg, q_start, q[:, :, q_start:], kc, vc, ksc, bsc, bt, qcal=qc_new)
    np.testing.assert_array_equal(got["sel_idx"], pre["sel_idx"])
    assert (got["sel_idx"] >= 0).any()  # some rows have candidates
    for key in ("sel_score", "out", "lse", "kth"):
        np.testing.assert_allclose(got[key], pre[key], rtol=0, atol=1e-12, err_msg=key)


# ---------------------------------------------------------------- variants


def test_mean_landmark_mode_is_mean_pooling():
    """Landmark mode "mean" (q' = 0): k' is the chunk's mean key and b' = log S."""
    rng = _rng(151)
    S, d, N, B = 8, 16, 48, 2
    cfg = _cfg(B=B, N=N, S=S, d=d, H_q=2, H_kv=1)
    k = rng.standard_normal((B, 1, N, d)).astype(np.float32)
    ks, bs = oracle.summarize(cfg, k, None, landmark="mean")
    mean = k.astype(np.float64).reshape(B, 1, N // S, S, d).mean(3)
    for l in range(2):  # both landmark heads read kv head 0
        np.testing.assert_allclose(ks[:, l], mean[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(bs, math.log(S), rtol=0, atol=1e-12)


def test_shared_landmark_mode_uses_one_query_per_head():
    """Landmark-free variant: one landmark query per landmark head, the same
    for every chunk and sequence; equals per-chunk queries all set to it."""
    rng = _rng(152)
    S, d, N, B, H_lm = 8, 16, 40, 2, 4
    cfg = _cfg(B=B, N=N, S=S, d=d, H_q=H_lm, H_kv=2)
    k = rng.standard_normal((B, 2, N, d)).astype(np.float32)
    qs = rng.standard_normal((H_lm, d)).astype(np.float32)
    ks, bs = oracle.summarize(cfg, k, qs, landmark="shared")
    tiled = np.tile(qs[None, :, None, :], (B, 1, N // S, 1))
    ks2, bs2 = oracle.summarize(cfg, k, tiled)
    np.testing.assert_array_equal(ks, ks2)
    np.testing.assert_array_equal(bs, bs2)
    # and a chunk whose keys are all equal to one key gets that key for any query
    k[:, :, :S] = k[:, :, :1]
    ks3, _ = oracle.summarize(cfg, k, qs, landmark="shared")
    np.testing.assert_allclose(ks3[:, :2, 0], k[:, :1, 0].repeat(2, axis=1), rtol=0, atol=1e-12)


def _per_head_scores(cfg, q, k, v, ks, bs, rows):
    """ŝ of each query head separately (a one-head configuration per head)."""
    out = []
    for h in range(cfg["H_q"]):
        c1 = dict(cfg, H_q=1, H_kv=1, H_lm=1, agg_mode=0)
        g = h // (cfg["H_q"] // cfg["H_kv"])
        r = oracle.forward_rows(c1, q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], ks[:, h:h + 1], bs[:, h:h + 1],
                                rows=rows, want_agg=True, attend=False)
        out.append(r["agg"][0, 0])  # [R, C]
    return np.stack(out)  # [H_q, R, C]


@pytest.mark.parametrize("K", [1, 3])
def test_normalized_aggregation_is_max_of_log_softmax(K):
    """agg_mode 1: the group score of chunk c is max over the group's heads of
    ŝ[h,c] - log Σ_c' exp(ŝ[h,c']) over the row's candidates (numpy
    log-softmax of the per-head scores); the top-K follows that score by
    brute-force sort; the fusion still weighs by the raw ŝ."""
    cfg, q, k, v, ql = _random_case(161 + K, G=4, H_kv=2, K=K)
    q[:, 1] *= 3.0  # heads with different score spreads: the modes disagree
    ks, bs = oracle.summarize(cfg, k, ql)
    rows = np.arange(40, 256, 3)
    per = _per_head_scores(cfg, q, k, v, ks, bs, rows)
    cn = dict(cfg, agg_mode=1)
    res = oracle.forward_rows(cn, q, k, v, ks, bs, rows=rows, want_agg=True)
    raw = oracle.forward_rows(cfg, q, k, v, ks, bs, rows=rows, want_agg=True)
    S, W, G = cfg["S"], cfg["W"], 4
    differ = 0
    for g in range(cfg["H_kv"]):
        for r, i in enumerate(rows):
            n = max(0, i // S - W // S)
            if n == 0:
                continue
            hs = per[g * G:(g + 1) * G, r, :n]
            want = (hs - logsumexp(hs, axis=1, keepdims=True)).max(0)
            np.testing.assert_allclose(res["agg"][0, g, r, :n], want, rtol=0, atol=1e-12)
            order = sorted(range(n), key=lambda c: (-want[c], c))[:K]
            assert res["sel_idx"][0, g, r].tolist() == sorted(order) + [-1] * (K - len(order))
            sel = [c for c in res["sel_idx"][0, g, r] if c >= 0]
            for e in range(G):
                np.testing.assert_allclose(res["sel_score"][0, g * G + e, r, :len(sel)],
                                           per[g * G + e, r, sel], rtol=0, atol=1e-12)
            differ += res["sel_idx"][0, g, r].tolist() != raw["sel_idx"][0, g, r].tolist()
    assert differ > 0


def test_normalized_aggregation_with_one_head_changes_nothing():
    """With G = 1 the normalisation shifts a row's scores by a constant."""
    cfg, q, k, v, ql = _random_case(171, G=1, H_kv=2, K=3)
    ks, bs = oracle.summarize(cfg, k, ql)
    a = oracle.forward_rows(cfg, q, k, v, ks, bs)
    b = oracle.forward_rows(dict(cfg, agg_mode=1), q, k, v, ks, bs)
    np.testing.assert_array_equal(a["sel_idx"], b["sel_idx"])
    np.testing.assert_array_equal(a["out"], b["out"])
