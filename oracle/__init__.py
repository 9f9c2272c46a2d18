"""fp64 CPU oracle of the HiLS attention forward pass -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``hils_oracle.c`` (plain C,
double precision, OpenMP over query rows) with ctypes.  It shares no code
with the GPU library and never imports it.

Method: "HiLS: Hierarchical Landmark Sparse Attention" (hyper.ai paper
summary, section 方法): landmark summaries (k'_c, b'_c), surrogate chunk
scores, GQA max-aggregation, top-K chunk selection, exact attention inside
each selected chunk and a chunk-aligned causal window, fusion by
exp(s^)/Z^.  Readings of points the pages leave open are documented in
``hils_oracle.c`` next to the code that takes them.

Array arguments may be torch tensors or numpy arrays.  Data arrays (q, k, v,
landmark queries, hidden states, weights, caches) are promoted to float32
(exact for bf16/fp32 data) and then to double inside the C code; computed
summaries are passed as float64.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hils_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libhils_oracle.so")
_lib = None

SCORE_MODES = {"landmark": 0, "self_landmark": 1, "exact_mass": 2}


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "N", "H_q", "H_kv", "H_lm", "d", "S", "W", "K")] + [
        ("scale", ctypes.c_double), ("agg_mode", ctypes.c_int64)
    ]


def build(force: bool = True) -> str:
    """Compile hils_oracle.c into libhils_oracle.so (gcc, -O2, OpenMP)."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_SRC[:-2] + ".h"))
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"],
            cwd=_HERE,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build(force=False)  # (re)builds when missing or older than its sources
        _lib = ctypes.CDLL(_LIB_PATH)
        for fn in ("hils_ref_summarize", "hils_ref_qcal_rows", "hils_ref_forward_rows", "hils_ref_decode",
                   "hils_ref_dense_causal_rows"):
            getattr(_lib, fn).restype = ctypes.c_int
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS, else all cores)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return os.cpu_count() or 1


def _f32(x):
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _f64(x):
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x):
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.int32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a, ctype=ctypes.c_float):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _cfg(cfg: dict) -> _Cfg:
    d = int(cfg["d"])
    scale = cfg.get("scale") or 0.0
    if not scale:
        scale = 1.0 / math.sqrt(d)
    H_q = int(cfg["H_q"])
    return _Cfg(
        int(cfg.get("B", 1)), int(cfg.get("N", 0)), H_q, int(cfg["H_kv"]), int(cfg.get("H_lm", H_q)), d,
        int(cfg["S"]), int(cfg["W"]), int(cfg["K"]), float(scale), int(cfg.get("agg_mode", 0)),
    )


LANDMARK_MODES = ("chunk", "shared", "mean")


def landmark_queries(cfg: dict, q_lm, lead, landmark: str = "chunk"):
    """The landmark query of every chunk, [*lead, H_lm, d] with lead = (B, C)
    or (items,).  "chunk": q_lm holds them.  "shared" (the landmark-free
    variant: one query per landmark head for every chunk): q_lm [H_lm, d]
    repeated.  "mean": q' = 0 (mean-pooled keys)."""
    c = _cfg(cfg)
    if landmark == "chunk":
        return _f32(q_lm)
    if landmark == "shared":
        ql = _f32(q_lm)
        assert ql.shape == (c.H_lm, c.d), ql.shape
        return np.ascontiguousarray(np.broadcast_to(ql, tuple(lead) + (c.H_lm, c.d)))
    assert landmark == "mean", landmark
    return np.zeros(tuple(lead) + (c.H_lm, c.d), np.float32)


def summarize(cfg: dict, k, q_lm, landmark: str = "chunk"):
    """Landmark summaries of every completed chunk.

    k: [B, H_kv, N, d]; q_lm: [B, H_lm, C, d] with C = N // S (see
    ``landmark_queries`` for the other landmark modes).
    Returns (k_sum [B, H_lm, C, d] float64, b_sum [B, H_lm, C] float64).
    """
    c = _cfg(cfg)
    C = c.N // c.S
    k32 = _f32(k)
    if landmark == "chunk":
        ql32 = _f32(q_lm)
    else:  # [B, C, H_lm, d] -> [B, H_lm, C, d]
        ql32 = np.ascontiguousarray(landmark_queries(cfg, q_lm, (c.B, C), landmark).transpose(0, 2, 1, 3))
    assert k32.shape == (c.B, c.H_kv, c.N, c.d), k32.shape
    assert ql32.shape == (c.B, c.H_lm, C, c.d), ql32.shape
    k_sum = np.zeros((c.B, c.H_lm, C, c.d), np.float64)
    b_sum = np.zeros((c.B, c.H_lm, C), np.float64)
    rc = _load().hils_ref_summarize(ctypes.byref(c), _ptr(k32), _ptr(ql32), _ptr(k_sum, ctypes.c_double),
                                    _ptr(b_sum, ctypes.c_double))
    if rc:
        raise ValueError("oracle summarize rejected the configuration")
    return k_sum, b_sum


def qcal_rows(cfg: dict, q, h, w_down, w_up, rows=None):
    """Scoring queries q + W_up (W_down h_i) for the given rows: [B, H_q, R, d]."""
    c = _cfg(cfg)
    rows = np.arange(c.N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    q32, h32, wd32, wu32 = _f32(q), _f32(h), _f32(w_down), _f32(w_up)
    r, d_model = wd32.shape
    out = np.zeros((c.B, c.H_q, len(rows), c.d), np.float64)
    _load().hils_ref_qcal_rows(ctypes.byref(c), ctypes.c_int64(d_model), ctypes.c_int64(r), _ptr(q32), _ptr(h32),
                               _ptr(wd32), _ptr(wu32), ctypes.c_int64(len(rows)), _ptr(rows, ctypes.c_int64),
                               _ptr(out, ctypes.c_double))
    return out


def forward_rows(cfg: dict, q, k, v, k_sum=None, b_sum=None, rows=None, mode: str = "landmark", qcal=None,
                 given_sel=None, want_agg: bool = False, attend: bool = True):
    """Score -> select -> attend -> fuse for the query positions in ``rows``.

    qcal: optional (h [B,N,d_model], w_down [r,d_model], w_up [H_q*d, r]).
    given_sel: optional [B, H_kv, R, K] int32 selection to use instead of the
    oracle's own top-K (the surrogate scores are still the oracle's).
    Returns a dict: sel_idx [B,H_kv,R,K] int32, sel_score [B,H_q,R,K],
    kth [B,H_kv,R,2] (K-th and (K+1)-th group scores, NaN if absent),
    out [B,H_q,R,d], lse [B,H_q,R], and agg [B,H_kv,R,C] when want_agg.
    """
    c = _cfg(cfg)
    rows = np.arange(c.N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = len(rows)
    C = c.N // c.S
    q32, k32, v32 = _f32(q), _f32(k), _f32(v)
    assert q32.shape == (c.B, c.H_q, c.N, c.d)
    assert k32.shape == (c.B, c.H_kv, c.N, c.d) and v32.shape == k32.shape
    ks = _f64(k_sum)
    bs = _f64(b_sum)
    if mode == "landmark":
        assert ks is not None and ks.shape == (c.B, c.H_lm, C, c.d)
        assert bs is not None and bs.shape == (c.B, c.H_lm, C)
    h32 = wd32 = wu32 = None
    d_model = r = 0
    if qcal is not None:
        h32, wd32, wu32 = (_f32(x) for x in qcal)
        r, d_model = wd32.shape
    gs = _i32(given_sel)
    if gs is not None:
        assert gs.shape == (c.B, c.H_kv, R, c.K)
    res = {
        "sel_idx": np.zeros((c.B, c.H_kv, R, c.K), np.int32),
        "sel_score": np.zeros((c.B, c.H_q, R, c.K), np.float64),
        "kth": np.zeros((c.B, c.H_kv, R, 2), np.float64),
    }
    if attend:
        res["out"] = np.zeros((c.B, c.H_q, R, c.d), np.float64)
        res["lse"] = np.zeros((c.B, c.H_q, R), np.float64)
    if want_agg:
        res["agg"] = np.zeros((c.B, c.H_kv, R, C), np.float64)
    dp = ctypes.c_double
    rc = _load().hils_ref_forward_rows(
        ctypes.byref(c), ctypes.c_int(SCORE_MODES[mode]), _ptr(q32), _ptr(k32), _ptr(v32), _ptr(ks, dp),
        _ptr(bs, dp), ctypes.c_int64(d_model), ctypes.c_int64(r), _ptr(h32), _ptr(wd32), _ptr(wu32),
        ctypes.c_int64(R), _ptr(rows, ctypes.c_int64), _ptr(gs, ctypes.c_int32), _ptr(res["sel_idx"], ctypes.c_int32),
        _ptr(res["sel_score"], dp), _ptr(res["kth"], dp), _ptr(res.get("out"), dp), _ptr(res.get("lse"), dp),
        _ptr(res.get("agg"), dp))
    if rc:
        raise ValueError("oracle forward rejected the configuration")
    return res


def decode(cfg: dict, q, k_cache, v_cache, ksum_cache, bsum_cache, block_table, seq_lens, qcal=None,
           kv_block_table=None, given_sel=None, attend: bool = True, want_agg: bool = False):
    """One decode step per sequence at position seq_len-1 over a paged cache.

    q [B, H_q, d]; k_cache / v_cache [P', H_kv, S, d] (None when attend is
    False); ksum_cache [P, H_lm, d]; bsum_cache [P, H_lm]; block_table
    [B, max_pages] (pages of the summary cache; also of the K/V caches unless
    kv_block_table is given); seq_lens [B] including the new token.
    """
    c = _cfg(cfg)
    q32 = _f32(q)
    B = q32.shape[0]
    bt = _i32(block_table)
    sl = _i32(seq_lens)
    max_pages = bt.shape[1]
    kc, vc = _f32(k_cache), _f32(v_cache)
    ksc, bsc = _f32(ksum_cache), _f32(bsum_cache)
    kvbt = _i32(kv_block_table)
    gs = _i32(given_sel)
    h32 = wd32 = wu32 = None
    d_model = r = 0
    if qcal is not None:
        h32, wd32, wu32 = (_f32(x) for x in qcal)
        r, d_model = wd32.shape
    res = {
        "sel_idx": np.zeros((B, c.H_kv, c.K), np.int32),
        "sel_score": np.zeros((B, c.H_q, c.K), np.float64),
        "kth": np.zeros((B, c.H_kv, 2), np.float64),
    }
    if attend:
        res["out"] = np.zeros((B, c.H_q, c.d), np.float64)
        res["lse"] = np.zeros((B, c.H_q), np.float64)
    agg_stride = 0
    if want_agg:
        agg_stride = max_pages
        res["agg"] = np.zeros((B, c.H_kv, agg_stride), np.float64)
    dp = ctypes.c_double
    rc = _load().hils_ref_decode(
        ctypes.byref(c), ctypes.c_int64(B), _ptr(q32), _ptr(kc), _ptr(vc), _ptr(ksc), _ptr(bsc),
        _ptr(bt, ctypes.c_int32), ctypes.c_int64(max_pages), _ptr(sl, ctypes.c_int32), ctypes.c_int64(d_model),
        ctypes.c_int64(r), _ptr(h32), _ptr(wd32), _ptr(wu32), _ptr(kvbt, ctypes.c_int32), _ptr(gs, ctypes.c_int32),
        _ptr(res["sel_idx"], ctypes.c_int32), _ptr(res["sel_score"], dp), _ptr(res["kth"], dp),
        _ptr(res.get("out"), dp), _ptr(res.get("lse"), dp), _ptr(res.get("agg"), dp), ctypes.c_int64(agg_stride))
    if rc:
        raise ValueError("oracle decode rejected the configuration")
    return res


def summarize_pages(cfg: dict, k_cache, q_lm, pages, landmark: str = "chunk"):
    """Summaries of the chunks held by pages of a paged key cache.

    Item i summarises page pages[i] of k_cache [P, H_kv, S, d] (one completed
    chunk) with the landmark queries q_lm[i] [H_lm, d]: the summary of
    ``summarize`` for a one-chunk sequence made of that page.  Items whose id
    lies outside [0, P) are skipped; their rows are NaN.
    Returns (k_sum [n, H_lm, d], b_sum [n, H_lm]) float64.
    """
    c = _cfg(cfg)
    kc = _f32(k_cache)
    pg = np.asarray(pages, dtype=np.int64).reshape(-1)
    P = kc.shape[0]
    n = len(pg)
    ql = landmark_queries(cfg, q_lm, (n,), landmark)
    assert kc.shape == (P, c.H_kv, c.S, c.d), kc.shape
    assert ql.shape == (n, c.H_lm, c.d), ql.shape
    k_sum = np.full((n, c.H_lm, c.d), np.nan)
    b_sum = np.full((n, c.H_lm), np.nan)
    ok = np.nonzero((pg >= 0) & (pg < P))[0]
    if len(ok):
        one = dict(cfg, B=len(ok), N=c.S)
        ks, bs = summarize(one, kc[pg[ok]], ql[ok][:, :, None, :])
        k_sum[ok], b_sum[ok] = ks[:, :, 0, :], bs[:, :, 0]
    return k_sum, b_sum


def prefill_paged(cfg: dict, q_start: int, q, k_cache, v_cache, ksum_cache, bsum_cache, block_table, qcal=None,
                  given_sel=None, attend: bool = True, want_agg: bool = False):
    """Chunked prefill over a paged cache: the new tokens at positions
    q_start .. q_start + n - 1 of each sequence.

    Row t of sequence b is, by definition, the decode step of that sequence
    at position q_start + t: the same keys (those up to and including its
    own), the same summaries read from the cache, its own query (and Q-Cal
    hidden state).  q [B, H_q, n, d]; block_table [B, max_pages]; qcal =
    (h [B, n, d_model], w_down, w_up) or None; given_sel [B, H_kv, n, K].
    Returns sel_idx [B,H_kv,n,K], sel_score [B,H_q,n,K], kth [B,H_kv,n,2],
    out [B,H_q,n,d], lse [B,H_q,n] (and agg [B,H_kv,n,max_pages]).
    """
    q32 = _f32(q)
    B, H_q, n, d = q32.shape
    bt = _i32(block_table)
    # one decode query per (sequence, new token), b-major
    qd = np.ascontiguousarray(q32.transpose(0, 2, 1, 3).reshape(B * n, H_q, d))
    btd = np.ascontiguousarray(np.repeat(bt, n, axis=0))
    seq_lens = (q_start + 1 + np.tile(np.arange(n), B)).astype(np.int32)
    qc = None
    if qcal is not None:
        h, wd, wu = (_f32(x) for x in qcal)
        qc = (np.ascontiguousarray(h.reshape(B * n, h.shape[-1])), wd, wu)
    gs = None
    if given_sel is not None:
        g = _i32(given_sel)
        gs = np.ascontiguousarray(g.transpose(0, 2, 1, 3).reshape(B * n, g.shape[1], g.shape[3]))
    r = decode(cfg, qd, k_cache, v_cache, ksum_cache, bsum_cache, btd, seq_lens, qcal=qc, given_sel=gs,
               attend=attend, want_agg=want_agg)

    def back(x):  # [B*n, H, ...] -> [B, H, n, ...]
        x = x.reshape((B, n) + x.shape[1:])
        return np.ascontiguousarray(np.moveaxis(x, 1, 2))

    return {key: back(val) for key, val in r.items()}


def dense_causal_rows(cfg: dict, q, k, v, rows=None):
    """Textbook causal softmax attention (keys 0..i) for the given rows."""
    c = _cfg(cfg)
    rows = np.arange(c.N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    q32, k32, v32 = _f32(q), _f32(k), _f32(v)
    out = np.zeros((c.B, c.H_q, len(rows), c.d), np.float64)
    lse = np.zeros((c.B, c.H_q, len(rows)), np.float64)
    _load().hils_ref_dense_causal_rows(ctypes.byref(c), _ptr(q32), _ptr(k32), _ptr(v32), ctypes.c_int64(len(rows)),
                                       _ptr(rows, ctypes.c_int64), _ptr(out, ctypes.c_double),
                                       _ptr(lse, ctypes.c_double))
    return out, lse
