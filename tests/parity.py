"""Comparison helpers shared by the GPU parity tests and the smoke check.

Tolerances (the parity bar of the benchmark workloads):
  * bf16 inputs: |gpu - ref| <= 2e-3 + 1e-2 * |ref| elementwise;
  * fp32 inputs: |gpu - ref| <= 1e-5 + 1e-5 * |ref|;
  * selected chunk ids: identical sets, except rows where the oracle's K-th
    and (K+1)-th group scores differ by less than 1e-5 and every chunk in the
    symmetric difference scores within 1e-5 of the oracle's K-th score.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

TIE_TOL = 1e-5


def tol_for(dtype):
    if dtype == torch.float32:
        return 1e-5, 1e-5
    return 2e-3, 1e-2


def assert_close(got, ref, atol, rtol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    with np.errstate(invalid="ignore"):
        bad = ~(np.abs(got - ref) <= atol + rtol * np.abs(ref))
    # identical infinities (e.g. -inf padding) are equal
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    bad &= ~both_inf
    if bad.any():
        idx = np.argwhere(bad)[:5]
        ex = [(tuple(i), got[tuple(i)], ref[tuple(i)]) for i in idx]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside atol={atol} rtol={rtol}; e.g. {ex}; "
                             f"max abs err {np.nanmax(np.abs(np.where(both_inf, 0, got - ref))):.3g}")


def host(t):
    return t.detach().to("cpu")


def check_selection(gpu_sel, ora_sel, ora_kth, agg_of_row, K):
    """gpu_sel / ora_sel: [B, H_kv, R, K]; ora_kth: [B, H_kv, R, 2];
    agg_of_row(b, g, r) -> oracle group scores of that row (NaN past the
    candidates).  Returns the (b, g, r) rows exempted as near-ties."""
    gpu_sel = np.asarray(gpu_sel)
    ora_sel = np.asarray(ora_sel)
    # layout: ascending ids then -1 padding
    for arr, name in ((gpu_sel, "gpu"), (ora_sel, "oracle")):
        valid = arr >= 0
        n = valid.sum(-1)
        assert np.all(valid == (np.arange(K)[None, None, None, :] < n[..., None])), f"{name} selection padding"
        d = np.diff(arr, axis=-1)
        both = valid[..., 1:] & valid[..., :-1]
        assert np.all(d[both] > 0), f"{name} selection not strictly ascending"
    exempt = []
    diff_rows = np.argwhere(np.any(gpu_sel != ora_sel, axis=-1))
    for b, g, r in diff_rows:
        gs = set(int(x) for x in gpu_sel[b, g, r] if x >= 0)
        os_ = set(int(x) for x in ora_sel[b, g, r] if x >= 0)
        assert len(gs) == len(os_), f"row {(b, g, r)}: {len(gs)} vs {len(os_)} chunks"
        kth, kth1 = ora_kth[b, g, r]
        assert np.isfinite(kth) and np.isfinite(kth1) and kth - kth1 < TIE_TOL, (
            f"row {(b, g, r)}: selections differ {sorted(gs ^ os_)} but K-th/(K+1)-th gap is {kth - kth1}")
        agg = agg_of_row(b, g, r)
        for c in gs ^ os_:
            assert abs(agg[c] - kth) < TIE_TOL, f"row {(b, g, r)}: chunk {c} scores {agg[c]} vs K-th {kth}"
        exempt.append((int(b), int(g), int(r)))
    return exempt


def stratified_rows(N, S, W, count, seed):
    """Seeded row sample: chunk starts/ends, rows without candidates, the last
    rows, and uniform fill."""
    rng = np.random.default_rng(seed)
    C = N // S
    must = {0, 1, N - 1, N - 2, min(N - 1, W + S - 1), min(N - 1, W + S)}
    for c in rng.choice(max(C, 1), size=min(C, count // 8), replace=False):
        must.add(int(c) * S)
        must.add(min(N - 1, int(c) * S + S - 1))
    rows = set(r for r in must if 0 <= r < N)
    while len(rows) < min(count, N):
        rows.add(int(rng.integers(N)))
    return np.array(sorted(rows), dtype=np.int64)


def oracle_prefill(cfg, inputs, rows=None, k_sum=None, b_sum=None, given_sel=None, want_agg=False):
    """Run the oracle on a prefill workload's host copies.

    When the configuration stores summaries in bf16, the oracle scores from
    its summaries as stored (fp64 values rounded to bf16), like the decode
    step reads its cache; res["k_sum_exact"] keeps the unrounded values."""
    oc = cfg.oracle_dict()
    q, k, v = (host(inputs[n]) for n in ("q", "k", "v"))
    q_lm = None if inputs.get("q_lm") is None else host(inputs["q_lm"])
    exact = None
    if k_sum is None:
        k_sum, b_sum = oracle.summarize(oc, k, q_lm, landmark=oracle.LANDMARK_MODES[cfg.landmark_mode])
        exact = k_sum
        if cfg.summary_dtype == torch.bfloat16:
            k_sum = round_to(k_sum, torch.bfloat16).to(torch.float64).numpy()
    qcal = None
    if inputs.get("qcal") is not None:
        qcal = tuple(host(x) for x in inputs["qcal"])
    res = oracle.forward_rows(oc, q, k, v, k_sum, b_sum, rows=rows, qcal=qcal, given_sel=given_sel,
                              want_agg=want_agg)
    res["k_sum"], res["b_sum"] = k_sum, b_sum
    res["k_sum_exact"] = exact if exact is not None else k_sum
    return res


def agg_lookup(cfg, inputs, k_sum, b_sum, rows):
    """Lazy per-row oracle group scores for the tie exemption."""
    cache = {}
    oc = cfg.oracle_dict()
    q, k, v = (host(inputs[n]) for n in ("q", "k", "v"))
    qcal = None if inputs.get("qcal") is None else tuple(host(x) for x in inputs["qcal"])

    def f(b, g, r):
        i = int(rows[r]) if rows is not None else int(r)
        if i not in cache:
            res = oracle.forward_rows(oc, q, k, v, k_sum, b_sum, rows=[i], qcal=qcal, want_agg=True, attend=False)
            cache[i] = res["agg"][:, :, 0, :]
        return cache[i][b, g]

    return f


def round_to(x64, dtype):
    """Round oracle float64 values to the dtype a GPU input is stored in."""
    return torch.from_numpy(np.asarray(x64)).to(torch.float32).to(dtype)


def sci(x):
    return "%.3g" % x if isinstance(x, float) and math.isfinite(x) else str(x)
