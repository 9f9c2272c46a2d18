"""The chunk-major form of the selected-chunk attention
(hils_config_t.attend_mode = HILS_ATTEND_CHUNK_MAJOR) against the fp64 oracle,
through the C ABI.

Each chunk's weighted exact output is computed for every query that selected
it and summed per row before the window pass (hyper.ai HiLS summary, 方法:
partition estimate and the hierarchical factorisation; the per-chunk terms
are independent).  Checked here: every bf16 prefill shape of the parity
suite at the stage level (the oracle's own selection) and end to end, slabs
of a few chunks (bitwise equal to one slab: a row's result does not depend on
which rows share its tiles or slab), and closeness to the query-major walk.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from long_context_chunk_landmark_amd import _binding as hb
from long_context_chunk_landmark_amd import workloads as W
from tests.parity import agg_lookup, assert_close, check_selection, host, oracle_prefill, round_to, tol_for
from tests.test_gpu_parity import CASES

pytestmark = pytest.mark.gpu

BF = torch.bfloat16
F32 = torch.float32
CM = hb.ATTEND_CHUNK_MAJOR

# bf16 I/O shapes with selections (the form applies to those)
BF_CASES = [n for n, p in CASES.items() if p["io"] == BF and p["K"] > 0]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hb.load_library()
    return torch.device("cuda:0")


_cache = {}


def _inputs(name, dev):
    if name not in _cache:
        _cache[name] = W.make_prefill(CASES[name], device=dev)
    return _cache[name]


def _oracle(name, dev):
    key = ("oracle", name)
    if key not in _cache:
        inp = _inputs(name, dev)
        _cache[key] = oracle_prefill(inp["cfg"], inp)
    return _cache[key]


def _attend(cfg, inp, sel_t, ss_t, **kw):
    c = dataclasses.replace(cfg, **kw)
    out, lse = hb.sparse_attend_fused(c, inp["q"], inp["k"], inp["v"], sel_t, ss_t)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("name", BF_CASES)
def test_chunk_major_attend_stage(name, dev):
    """Same selection and scores on both sides (the oracle's)."""
    inp = _inputs(name, dev)
    cfg = inp["cfg"]
    print(f"[cm attend] {name}", flush=True)
    ref = _oracle(name, dev)
    sel_t = torch.from_numpy(ref["sel_idx"]).to(dev)
    ss_t = round_to(ref["sel_score"], F32).to(dev)
    out, lse = _attend(cfg, inp, sel_t, ss_t, attend_mode=CM)
    oc = cfg.oracle_dict()
    ref2 = oracle.forward_rows(oc, host(inp["q"]), host(inp["k"]), host(inp["v"]), ref["k_sum"], ref["b_sum"],
                               given_sel=ref["sel_idx"], qcal=None if inp.get("qcal") is None else tuple(
                                   host(x) for x in inp["qcal"]))
    atol, rtol = tol_for(cfg.io_dtype)
    assert_close(host(out).float().numpy(), ref2["out"], atol, rtol, "out")
    assert_close(host(lse).numpy(), ref2["lse"], atol, rtol, "lse")
    # the walk computes the same definition: both within the tolerance of
    # each other as well
    out_w, lse_w = _attend(cfg, inp, sel_t, ss_t, attend_mode=hb.ATTEND_WALK)
    assert_close(host(out).float().numpy(), host(out_w).float().numpy(), atol, rtol, "out vs walk")


@pytest.mark.parametrize("name", ["gqa_8k", "s128_k64", "ragged_d64_g2", "g1_k128_s64", "aggnorm_lmkv"])
def test_chunk_major_slabs_bitwise(name, dev):
    """Slabs of one or a few chunks give bit-identical outputs to one slab."""
    inp = _inputs(name, dev)
    cfg = inp["cfg"]
    ref = _oracle(name, dev)
    sel_t = torch.from_numpy(ref["sel_idx"]).to(dev)
    ss_t = round_to(ref["sel_score"], F32).to(dev)
    out1, lse1 = _attend(cfg, inp, sel_t, ss_t, attend_mode=CM)
    for slab in (cfg.S, 3 * cfg.S, cfg.N - 1):
        print(f"[cm slabs] {name} slab={slab}", flush=True)
        out2, lse2 = _attend(cfg, inp, sel_t, ss_t, attend_mode=CM, attend_slab=slab)
        assert torch.equal(out1, out2), f"out differs with slab={slab}"
        assert torch.equal(lse1, lse2), f"lse differs with slab={slab}"


@pytest.mark.parametrize("name", ["gqa_8k", "s128_k64", "qcal_r32_b2", "lm_shared_b2", "aggnorm_qcal"])
def test_chunk_major_end_to_end(name, dev):
    inp = _inputs(name, dev)
    cfg = dataclasses.replace(inp["cfg"], attend_mode=CM)
    print(f"[cm end_to_end] {name}", flush=True)
    res = hb.prefill(cfg, inp["q"], inp["k"], inp["v"], inp["q_lm"], qcal=inp.get("qcal"))
    torch.cuda.synchronize()
    ref = _oracle(name, dev)
    gsel = host(res["sel_idx"]).numpy()
    exempt = check_selection(gsel, ref["sel_idx"], ref["kth"], agg_lookup(cfg, inp, ref["k_sum"], ref["b_sum"], None),
                             cfg.K)
    refo, refl = ref["out"], ref["lse"]
    if exempt:
        alt = oracle_prefill(cfg, inp, k_sum=ref["k_sum"], b_sum=ref["b_sum"], given_sel=gsel)
        refo, refl = refo.copy(), refl.copy()
        G = cfg.G
        for b, g, r in exempt:
            refo[b, g * G:(g + 1) * G, r] = alt["out"][b, g * G:(g + 1) * G, r]
            refl[b, g * G:(g + 1) * G, r] = alt["lse"][b, g * G:(g + 1) * G, r]
    atol, rtol = tol_for(cfg.io_dtype)
    assert_close(host(res["out"]).float().numpy(), refo, atol, rtol, "out")
    assert_close(host(res["lse"]).numpy(), refl, atol, rtol, "lse")


def test_chunk_major_empty_selections(dev):
    """Rows without candidates, chunks no row selected, padded selections
    (-1) and a selection list that is all padding."""
    p = dict(seed=91, io=BF, B=1, H_q=4, H_kv=1, d=128, N=1500, S=64, W=256, K=8)
    inp = W.make_prefill(p, device=dev)
    cfg = inp["cfg"]
    ref = oracle_prefill(cfg, inp)
    sel = ref["sel_idx"].copy()
    # pad out the tail of every third row's selection, and all of row 900's
    sel[:, :, ::3, 5:] = -1
    sel[:, :, 900, :] = -1
    sc = ref["sel_score"].copy()
    G = cfg.G
    for g in range(cfg.H_kv):
        pad = sel[0, g] < 0
        for e in range(G):
            sc[0, g * G + e][pad] = -np.inf
    sel_t = torch.from_numpy(sel).to(dev)
    ss_t = round_to(sc, F32).to(dev)
    out, lse = _attend(cfg, inp, sel_t, ss_t, attend_mode=CM)
    ref2 = oracle.forward_rows(cfg.oracle_dict(), host(inp["q"]), host(inp["k"]), host(inp["v"]), ref["k_sum"],
                               ref["b_sum"], given_sel=sel)
    atol, rtol = tol_for(cfg.io_dtype)
    assert_close(host(out).float().numpy(), ref2["out"], atol, rtol, "out")
    assert_close(host(lse).numpy(), ref2["lse"], atol, rtol, "lse")
