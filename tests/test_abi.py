"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import long_context_chunk_landmark_amd as hils
from long_context_chunk_landmark_amd import _binding as hb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hils.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hb.LIB_PATH):
        from long_context_chunk_landmark_amd import build

        build.build()
    return hb.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hils_[a-z_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(hb.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", hb.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (hils_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert hils.version() == 10100


def _cfg(**kw):
    c = dict(H_q=8, H_kv=2, d=128, S=64, W=256, K=16, B=1, N=4096)
    c.update(kw)
    return hb.Config(**c).to_c()


A = ctypes.c_void_p(0x10000)      # aligned stand-in pointers: validation never dereferences
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10001)    # misaligned


def _summ(lib, cfg, k=A, q_lm=A, ks=A, bs=A):
    return lib.hils_landmark_summarize(ctypes.byref(cfg) if cfg is not None else None, k, q_lm, ks, bs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), hb.HILS_ERR_UNSUPPORTED),
    (dict(S=32), hb.HILS_ERR_UNSUPPORTED),
    (dict(H_q=6, H_kv=4), hb.HILS_ERR_INVALID_ARG),
    (dict(H_q=16, H_kv=1), hb.HILS_ERR_UNSUPPORTED),
    (dict(W=100), hb.HILS_ERR_INVALID_ARG),
    (dict(K=129), hb.HILS_ERR_UNSUPPORTED),
    (dict(K=-1), hb.HILS_ERR_INVALID_ARG),
    (dict(H_lm=3), hb.HILS_ERR_INVALID_ARG),
    (dict(N=-5), hb.HILS_ERR_INVALID_ARG),
    (dict(N=64 * 8193), hb.HILS_ERR_UNSUPPORTED),
])
def test_bad_config_is_rejected(lib, kw, status):
    cfg = _cfg(**kw)
    assert _summ(lib, cfg) == status
    assert hb.last_error()


def test_null_config_and_pointers(lib):
    assert _summ(lib, None) == hb.HILS_ERR_INVALID_ARG
    cfg = _cfg()
    assert _summ(lib, cfg, k=None) == hb.HILS_ERR_INVALID_ARG
    assert "k is NULL" in hb.last_error()
    assert _summ(lib, cfg, q_lm=MIS) == hb.HILS_ERR_INVALID_ARG
    assert "aligned" in hb.last_error()


def test_bad_dtype_code(lib):
    cfg = _cfg()
    cfg.io_dtype = 7
    assert _summ(lib, cfg) == hb.HILS_ERR_INVALID_ARG


def test_empty_problem_is_ok_without_pointers(lib):
    cfg = _cfg(N=0)
    assert lib.hils_landmark_summarize(ctypes.byref(cfg), None, None, None, None, None) == hb.HILS_OK
    assert lib.hils_score_select(ctypes.byref(cfg), None, None, None, None, None, None, 0, 0, None, None, None, 0,
                                 None) == hb.HILS_OK
    assert lib.hils_sparse_attend_fused(ctypes.byref(cfg), None, None, None, None, None, None, None, None, 0,
                                        None) == hb.HILS_OK
    assert lib.hils_decode(ctypes.byref(cfg), 0, None, None, None, None, None, None, 1, None, None, None, None, 0, 0,
                           None, None, None, None, 0, None) == hb.HILS_OK


def test_workspace_is_checked(lib):
    cfg = _cfg()
    need = lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_SCORE, 0, 0)
    assert need > 0
    st = lib.hils_score_select(ctypes.byref(cfg), A, A, A, None, None, None, 0, 0, A, A, A2, need - 1, None)
    assert st == hb.HILS_ERR_WORKSPACE
    st = lib.hils_score_select(ctypes.byref(cfg), A, A, A, None, None, None, 0, 0, A, A, None, 0, None)
    assert st == hb.HILS_ERR_WORKSPACE
    need_f = lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_FUSED, 0, 0)
    assert need_f > 0
    st = lib.hils_sparse_attend_fused(ctypes.byref(cfg), A, A, A, A, A, A, None, A2, need_f - 16, None)
    assert st == hb.HILS_ERR_WORKSPACE
    need_d = lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_DECODE, 4, 100)
    st = lib.hils_decode(ctypes.byref(cfg), 4, A, A, A, A, A, A, 100, A, None, None, None, 0, 0, A, None, None, A2,
                         need_d - 1, None)
    assert st == hb.HILS_ERR_WORKSPACE


def test_workspace_sizes_scale_with_problem(lib):
    small, big = _cfg(N=4096), _cfg(N=8192)
    for which in (hb.WS_SCORE, hb.WS_SCORE_QCAL, hb.WS_FUSED):
        a = lib.hils_workspace_size(ctypes.byref(small), which, 0, 0)
        b = lib.hils_workspace_size(ctypes.byref(big), which, 0, 0)
        assert 0 < a < b
    qc = lib.hils_workspace_size(ctypes.byref(small), hb.WS_SCORE_QCAL, 0, 0)
    assert qc > lib.hils_workspace_size(ctypes.byref(small), hb.WS_SCORE, 0, 0)
    f32 = _cfg()
    f32.io_dtype = hb.HILS_F32
    assert lib.hils_workspace_size(ctypes.byref(f32), hb.WS_FUSED, 0, 0) == 0  # fp32 path needs none
    assert lib.hils_workspace_size(ctypes.byref(_cfg(d=96)), hb.WS_SCORE, 0, 0) == 0
    assert "d=96" in hb.last_error()


def test_qcal_arguments_are_checked(lib):
    cfg = _cfg()
    need = lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_SCORE_QCAL, 0, 0)
    st = lib.hils_score_select(ctypes.byref(cfg), A, A, A, A, None, A, 256, 16, A, A, A2, need, None)
    assert st == hb.HILS_ERR_INVALID_ARG and "w_down" in hb.last_error()
    st = lib.hils_score_select(ctypes.byref(cfg), A, A, A, A, A, A, 256, 65, A, A, A2, need, None)
    assert st == hb.HILS_ERR_UNSUPPORTED


def test_decode_argument_checks(lib):
    cfg = _cfg()
    need = lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_DECODE, 2, 10)
    st = lib.hils_decode(ctypes.byref(cfg), 2, A, A, A, A, A, A, 0, A, None, None, None, 0, 0, A, None, None, A2,
                         need, None)
    assert st == hb.HILS_ERR_INVALID_ARG
    st = lib.hils_decode(ctypes.byref(cfg), 2, A, A, A, A, A, None, 10, A, None, None, None, 0, 0, A, None, None, A2,
                         need, None)
    assert st == hb.HILS_ERR_INVALID_ARG and "block_table" in hb.last_error()
    st = lib.hils_decode(ctypes.byref(cfg), 2, A, A, A, A, A, A, 70000, A, None, None, None, 0, 0, A, None, None, A2,
                         need, None)
    assert st == hb.HILS_ERR_UNSUPPORTED


def test_fused_shape_beyond_lds_is_unsupported(lib):
    """G = 1 at S = 128, d = 128 with K = 128 and 4096 chunks: the walk has no
    block shape whose LDS fits (its union list), so the walk rejects it before
    launch; the chunk-major form (no union list, auto for this shape) takes it."""
    cfg = _cfg(H_q=2, H_kv=2, S=128, W=256, K=128, N=128 * 4096, attend_mode=hb.ATTEND_WALK)
    need = lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_FUSED, 0, 0)
    st = lib.hils_sparse_attend_fused(ctypes.byref(cfg), A, A, A, A, A, A, None, A2, need, None)
    assert st == hb.HILS_ERR_UNSUPPORTED and "LDS" in hb.last_error()
    for mode in (hb.ATTEND_AUTO, hb.ATTEND_CHUNK_MAJOR):
        cfg = _cfg(H_q=2, H_kv=2, S=128, W=256, K=128, N=128 * 4096, attend_mode=mode)
        need_cm = lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_FUSED, 0, 0)
        assert need_cm > need
        st = lib.hils_sparse_attend_fused(ctypes.byref(cfg), A, A, A, A, A, A, None, A2, need_cm - 1, None)
        assert st == hb.HILS_ERR_WORKSPACE


def test_attend_mode_and_workspace(lib):
    """attend_mode / attend_slab validation; the chunk-major workspace holds
    the V^T copy plus a slab's lists and fp16 partials, bounded by the slab."""
    bad = _cfg(attend_mode=3)
    assert lib.hils_sparse_attend_fused(ctypes.byref(bad), A, A, A, A, A, A, None, A2, 1 << 40, None) == \
        hb.HILS_ERR_INVALID_ARG and "attend_mode" in hb.last_error()
    bad = _cfg(attend_slab=-1)
    assert lib.hils_sparse_attend_fused(ctypes.byref(bad), A, A, A, A, A, A, None, A2, 1 << 40, None) == \
        hb.HILS_ERR_INVALID_ARG and "attend_slab" in hb.last_error()
    N, B, H_q, H_kv, d, S, K = 4096, 1, 8, 2, 128, 64, 16
    ws = lambda **kw: lib.hils_workspace_size(ctypes.byref(_cfg(N=N, **kw)), hb.WS_FUSED, 0, 0)  # noqa: E731
    walk = ws(attend_mode=hb.ATTEND_WALK)
    cm = ws(attend_mode=hb.ATTEND_CHUNK_MAJOR)
    assert ws() == cm  # auto takes the chunk-major form
    part = B * H_q * N * K * d * 2
    qt = B * H_q * N * d * 2  # q regrouped per query
    # the partials (and a trash region of G d values), the regrouped q, the lists with their weights,
    # row maxima and per-chunk counters and offsets, each region 256-byte aligned
    assert part + qt < cm - walk < (part + qt + B * H_q * N * K * 8 + B * H_kv * (3 * (N // S) + 3) * 4
                                    + 9 * 256 + 2 * d * (H_q // H_kv))
    # a slab of 1024 rows: a quarter of the partials
    cm_slab = ws(attend_mode=hb.ATTEND_CHUNK_MAJOR, attend_slab=1000)  # rounded up to a multiple of S
    assert part // 4 < cm_slab - walk < cm - walk
    # fp32 I/O walks whatever the mode (no workspace)
    assert lib.hils_workspace_size(ctypes.byref(hb.Config(H_q=8, H_kv=2, d=128, S=64, W=256, K=16, N=N,
                                                          io_dtype=__import__("torch").float32,
                                                          attend_mode=hb.ATTEND_CHUNK_MAJOR).to_c()),
                                   hb.WS_FUSED, 0, 0) == 0


def _paged(lib, cfg, q_start=1024, num_pages=200, max_pages=100, bt=A, ws=A2, nbytes=None, h=None, wd=None,
           wu=None, d_model=0, r=0):
    if nbytes is None:
        nbytes = lib.hils_prefill_paged_workspace_size(ctypes.byref(cfg), q_start, max_pages, int(h is not None))
    return lib.hils_prefill_paged(ctypes.byref(cfg), q_start, A, A, A, A, A, num_pages, bt, max_pages, h, wd, wu,
                                  d_model, r, A, A, A, None, ws, nbytes, None)


def test_prefill_paged_argument_checks(lib):
    cfg = _cfg(N=512)
    assert _paged(lib, cfg, q_start=1000) == hb.HILS_ERR_INVALID_ARG and "multiple of S" in hb.last_error()
    assert _paged(lib, cfg, q_start=-64) == hb.HILS_ERR_INVALID_ARG
    # keys 0 .. q_start + N - 1 need more pages than the block table has
    assert _paged(lib, cfg, q_start=64 * 95, max_pages=100) == hb.HILS_ERR_INVALID_ARG
    assert "pages" in hb.last_error()
    assert _paged(lib, cfg, num_pages=0) == hb.HILS_ERR_INVALID_ARG
    assert _paged(lib, cfg, num_pages=(1 << 18) + 1) == hb.HILS_ERR_UNSUPPORTED
    assert _paged(lib, cfg, bt=None) == hb.HILS_ERR_INVALID_ARG and "block_table" in hb.last_error()
    assert _paged(lib, cfg, ws=None) == hb.HILS_ERR_WORKSPACE
    need = lib.hils_prefill_paged_workspace_size(ctypes.byref(cfg), 1024, 100, 0)
    assert _paged(lib, cfg, nbytes=need - 1) == hb.HILS_ERR_WORKSPACE
    assert _paged(lib, cfg, h=A, wd=None, wu=A, d_model=256, r=16) == hb.HILS_ERR_INVALID_ARG
    assert lib.hils_prefill_paged(ctypes.byref(_cfg(N=0)), 0, None, None, None, None, None, 1, None, 1, None, None,
                                  None, 0, 0, None, None, None, None, None, 0, None) == hb.HILS_OK


def test_prefill_paged_workspace_grows_with_position(lib):
    cfg = _cfg(N=512)
    a = lib.hils_prefill_paged_workspace_size(ctypes.byref(cfg), 0, 400, 0)
    b = lib.hils_prefill_paged_workspace_size(ctypes.byref(cfg), 64 * 300, 400, 0)
    c = lib.hils_prefill_paged_workspace_size(ctypes.byref(cfg), 64 * 300, 400, 1)
    assert 0 < a < b < c
    assert lib.hils_prefill_paged_workspace_size(ctypes.byref(cfg), 64 * 399, 400, 0) == 0  # too few pages
    assert "pages" in hb.last_error()


def test_summarize_pages_argument_checks(lib):
    cfg = _cfg()
    f = lib.hils_summarize_pages
    assert f(ctypes.byref(cfg), -1, A, 100, A, A, A, A, None) == hb.HILS_ERR_INVALID_ARG
    assert f(ctypes.byref(cfg), 4, A, 100, A, None, A, A, None) == hb.HILS_ERR_INVALID_ARG
    assert "pages" in hb.last_error()
    assert f(ctypes.byref(cfg), 4, A, 100, MIS, A, A, A, None) == hb.HILS_ERR_INVALID_ARG
    assert f(ctypes.byref(_cfg(d=96)), 4, A, 100, A, A, A, A, None) == hb.HILS_ERR_UNSUPPORTED
    assert f(ctypes.byref(cfg), 0, None, 100, None, None, None, None, None) == hb.HILS_OK


def test_variant_modes_are_validated(lib):
    for field, bad in (("landmark_mode", 3), ("landmark_mode", -1), ("agg_mode", 2)):
        cfg = _cfg()
        setattr(cfg, field, bad)
        assert _summ(lib, cfg) == hb.HILS_ERR_INVALID_ARG and field in hb.last_error()
    # per-chunk and shared landmark queries need q_lm; mean pooling does not
    for mode in (hb.LM_CHUNK, hb.LM_SHARED):
        cfg = _cfg(landmark_mode=mode)
        assert _summ(lib, cfg, q_lm=None) == hb.HILS_ERR_INVALID_ARG and "q_lm" in hb.last_error()
    # the decode step keeps each head's partial log-sum-exp per split for the normalised mode
    d0 = lib.hils_workspace_size(ctypes.byref(_cfg()), hb.WS_DECODE, 4, 100)
    d1 = lib.hils_workspace_size(ctypes.byref(_cfg(agg_mode=hb.AGG_NORMALIZED)), hb.WS_DECODE, 4, 100)
    assert d1 > d0
    # the normalised aggregation keeps a per-head log-sum-exp in the score workspace
    a = lib.hils_workspace_size(ctypes.byref(_cfg()), hb.WS_SCORE, 0, 0)
    b = lib.hils_workspace_size(ctypes.byref(_cfg(agg_mode=hb.AGG_NORMALIZED)), hb.WS_SCORE, 0, 0)
    assert b == a + 8 * 4096 * 4


def _bwd(lib, cfg, ws=A2, nbytes=None, **ptr):
    p = dict(q=A, k=A, v=A, q_lm=A, k_sum=A, sel_idx=A, sel_score=A, lse=A, dout=A, dlse=None, dq=A, dk=A, dv=A,
             dq_lm=A)
    p.update(ptr)
    if nbytes is None:
        nbytes = lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_BACKWARD, 0, 0)
    return lib.hils_sparse_attend_backward(ctypes.byref(cfg), p["q"], p["k"], p["v"], p["q_lm"], p["k_sum"],
                                           p["sel_idx"], p["sel_score"], p["lse"], p["dout"], p["dlse"], p["dq"],
                                           p["dk"], p["dv"], p["dq_lm"], ws, nbytes, None)


def test_backward_argument_checks(lib):
    cfg = _cfg()
    need = lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_BACKWARD, 0, 0)
    assert need > 0
    bf16sum = _cfg()
    bf16sum.summary_dtype = hb.HILS_BF16
    assert _bwd(lib, bf16sum) == hb.HILS_ERR_UNSUPPORTED and "summary_dtype" in hb.last_error()
    for name in ("q", "k", "v", "lse", "dout", "dq", "dk", "dv", "sel_idx", "sel_score", "k_sum", "q_lm", "dq_lm"):
        assert _bwd(lib, cfg, **{name: None}) == hb.HILS_ERR_INVALID_ARG, name
        assert f"{name} is NULL" in hb.last_error()
    # K = 0 reads no selection; mean pooling has no landmark query and no gradient for one
    assert _bwd(lib, _cfg(K=0), sel_idx=None, sel_score=None, ws=None, nbytes=0) == hb.HILS_ERR_WORKSPACE
    mean = _cfg(landmark_mode=hb.LM_MEAN)
    assert _bwd(lib, mean, q_lm=None, dq_lm=None, ws=None, nbytes=0) == hb.HILS_ERR_WORKSPACE
    assert _bwd(lib, cfg, dlse=MIS) == hb.HILS_ERR_INVALID_ARG and "dlse" in hb.last_error()
    assert _bwd(lib, cfg, nbytes=need - 1) == hb.HILS_ERR_WORKSPACE
    assert _bwd(lib, cfg, ws=MIS, nbytes=need) == hb.HILS_ERR_INVALID_ARG and "workspace" in hb.last_error()
    empty = _cfg(N=0)
    assert lib.hils_sparse_attend_backward(ctypes.byref(empty), *([None] * 15), 0, None) == hb.HILS_OK


def test_score_modes_and_their_workspaces(lib):
    """Two-pass form: workspace grows with N^2 / S (the ragged score array);
    streaming form: with N K.  Auto keeps the two-pass form while its score
    array stays within 32 GiB and streams beyond.  An unknown mode is refused."""
    def ws(mode, N, B=1):
        c = hb.Config(H_q=32, H_kv=8, d=128, S=64, W=1024, K=32, B=B, N=N, score_mode=mode).to_c()
        return lib.hils_workspace_size(ctypes.byref(c), hb.WS_SCORE, 0, 0)
    two_small, two_big = ws(hb.SCORE_TWO_PASS, 65536), ws(hb.SCORE_TWO_PASS, 131072)
    st_small, st_big = ws(hb.SCORE_STREAMING, 65536), ws(hb.SCORE_STREAMING, 131072)
    assert two_big > 3.5 * two_small  # quadratic term dominates
    assert 1.9 * st_small < st_big < 2.1 * st_small  # linear in N
    assert st_big < two_big / 4
    assert ws(hb.SCORE_AUTO, 131072) == two_big  # 4.3 GB of scores: the two-pass form
    big2 = ws(hb.SCORE_AUTO, 524288, B=2)  # 137 GB of scores: streaming
    assert big2 == ws(hb.SCORE_STREAMING, 524288, B=2) < ws(hb.SCORE_TWO_PASS, 524288, B=2) / 10
    c = hb.Config(H_q=8, H_kv=2, d=128, S=64, W=128, K=4, N=1024, score_mode=3).to_c()
    assert lib.hils_score_select(ctypes.byref(c), None, None, None, None, None, None, 0, 0, None, None, None, 0,
                                 None) == hb.HILS_ERR_INVALID_ARG


def test_streaming_coverage_is_checked_before_pointers(lib):
    """The streaming form is refused for d = 128, G = 8, fp32 summaries and
    K > 32 (its per-block working set exceeds the LDS) and accepted otherwise:
    an accepted shape gets as far as the pointer checks."""
    def st(**kw):
        c = hb.Config(**dict(dict(H_q=8, H_kv=1, d=128, S=64, W=128, K=40, N=4096,
                                  score_mode=hb.SCORE_STREAMING), **kw)).to_c()
        return lib.hils_score_select(ctypes.byref(c), None, None, None, None, None, None, 0, 0, None, None, None, 0,
                                     None)
    assert st() == hb.HILS_ERR_UNSUPPORTED
    assert st(K=32) == hb.HILS_ERR_INVALID_ARG  # covered: fails on the NULL q
    assert st(summary_dtype=torch.bfloat16) == hb.HILS_ERR_INVALID_ARG
    assert st(H_q=4) == hb.HILS_ERR_INVALID_ARG
    assert st(score_mode=hb.SCORE_TWO_PASS) == hb.HILS_ERR_INVALID_ARG


def test_dense_attention_arguments_are_checked(lib):
    """The dense causal attention entry: empty problems need no pointers,
    the workspace is sized and checked, and fp32 I/O is refused."""
    assert lib.hils_dense_causal_attend(ctypes.byref(_cfg(N=0)), None, None, None, None, None, None, 0,
                                        None) == hb.HILS_OK
    cfg = _cfg()
    need = lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_DENSE, 0, 0)
    assert need > lib.hils_workspace_size(ctypes.byref(_cfg(N=cfg.N // 2)), hb.WS_DENSE, 0, 0) > 0
    st = lib.hils_dense_causal_attend(ctypes.byref(cfg), A, A, A, A, None, A2, need - 16, None)
    assert st == hb.HILS_ERR_WORKSPACE
    st = lib.hils_dense_causal_attend(ctypes.byref(cfg), A, None, A, A, None, A2, need, None)
    assert st == hb.HILS_ERR_INVALID_ARG
    f32 = _cfg()
    f32.io_dtype = hb.HILS_F32
    assert lib.hils_dense_causal_attend(ctypes.byref(f32), A, A, A, A, None, A2, need, None) == hb.HILS_ERR_UNSUPPORTED
    assert lib.hils_workspace_size(ctypes.byref(f32), hb.WS_DENSE, 0, 0) == 0


def test_dense_decode_arguments_are_checked(lib):
    cfg = _cfg()
    assert lib.hils_dense_decode(ctypes.byref(cfg), 0, None, None, None, None, 1, None, None, None, None, 0,
                                 None) == hb.HILS_OK
    need = lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_DENSE_DECODE, 4, 100)
    assert need > lib.hils_workspace_size(ctypes.byref(cfg), hb.WS_DENSE_DECODE, 2, 100) > 0
    st = lib.hils_dense_decode(ctypes.byref(cfg), 4, A, A, A, A, 100, A, A, None, A2, need - 1, None)
    assert st == hb.HILS_ERR_WORKSPACE
    st = lib.hils_dense_decode(ctypes.byref(cfg), 4, A, A, A, A, 0, A, A, None, A2, need, None)
    assert st == hb.HILS_ERR_INVALID_ARG
    s128 = _cfg(S=128, W=128)
    assert lib.hils_dense_decode(ctypes.byref(s128), 4, A, A, A, A, 100, A, A, None, A2, need,
                                 None) == hb.HILS_ERR_UNSUPPORTED
