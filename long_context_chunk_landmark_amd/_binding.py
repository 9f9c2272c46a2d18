"""ctypes binding of libhils.so (include/hils.h).

Argument marshalling only: shape/dtype/device checks, output and workspace
allocation through torch (device memory), and the current HIP stream.  Every
step of the HiLS computation runs in the library's HIP kernels; there is no
fallback path -- a missing library raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhils.so")

HILS_OK, HILS_ERR_INVALID_ARG, HILS_ERR_UNSUPPORTED, HILS_ERR_WORKSPACE, HILS_ERR_HIP = range(5)
HILS_F32, HILS_BF16 = 0, 1
LM_CHUNK, LM_SHARED, LM_MEAN = 0, 1, 2   # hils_landmark_mode_t
AGG_MAX, AGG_NORMALIZED = 0, 1           # hils_agg_mode_t
SCORE_AUTO, SCORE_TWO_PASS, SCORE_STREAMING = 0, 1, 2  # hils_score_mode_t
ATTEND_AUTO, ATTEND_WALK, ATTEND_CHUNK_MAJOR = 0, 1, 2  # hils_attend_mode_t
WS_SCORE, WS_SCORE_QCAL, WS_FUSED, WS_DECODE, WS_BACKWARD, WS_DENSE, WS_DENSE_DECODE = range(7)

# Every symbol include/hils.h declares.
EXPORTED_SYMBOLS = (
    "hils_landmark_summarize",
    "hils_score_select",
    "hils_sparse_attend_fused",
    "hils_dense_causal_attend",
    "hils_dense_decode",
    "hils_decode",
    "hils_decode_noalloc",
    "hils_summarize_pages",
    "hils_prefill_paged",
    "hils_prefill_paged_workspace_size",
    "hils_sparse_attend_backward",
    "hils_workspace_size",
    "hils_last_error",
    "hils_version",
)


class HilsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hils status {status}: {message}")
        self.status = status


class _CConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "N", "H_q", "H_kv", "H_lm", "d", "S", "W", "K", "M", "io_dtype", "summary_dtype")] + [
                   ("scale", ctypes.c_float), ("landmark_mode", ctypes.c_int32), ("agg_mode", ctypes.c_int32),
                   ("wait_spins", ctypes.c_int32), ("score_mode", ctypes.c_int32),
                   ("attend_mode", ctypes.c_int32), ("attend_slab", ctypes.c_int32)]


@dataclasses.dataclass
class Config:
    """Mirror of hils_config_t.  ``io_dtype``/``summary_dtype`` are torch dtypes."""
    H_q: int
    H_kv: int
    d: int
    S: int
    W: int
    K: int
    B: int = 1
    N: int = 0
    H_lm: Optional[int] = None
    M: int = 4
    io_dtype: torch.dtype = torch.bfloat16
    summary_dtype: torch.dtype = torch.float32
    scale: float = 0.0
    landmark_mode: int = LM_CHUNK
    agg_mode: int = AGG_MAX
    wait_spins: int = 0
    score_mode: int = 0
    attend_mode: int = 0
    attend_slab: int = 0

    def __post_init__(self):
        if self.H_lm is None:
            self.H_lm = self.H_q

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def C(self) -> int:
        return self.N // self.S

    def to_c(self) -> _CConfig:
        def code(dt):
            if dt == torch.float32:
                return HILS_F32
            if dt == torch.bfloat16:
                return HILS_BF16
            raise ValueError(f"unsupported dtype {dt}")

        return _CConfig(self.B, self.N, self.H_q, self.H_kv, self.H_lm, self.d, self.S, self.W, self.K, self.M,
                        code(self.io_dtype), code(self.summary_dtype), float(self.scale), int(self.landmark_mode),
                        int(self.agg_mode), int(self.wait_spins), int(self.score_mode), int(self.attend_mode),
                        int(self.attend_slab))

    def oracle_dict(self) -> dict:
        return dict(B=self.B, N=self.N, H_q=self.H_q, H_kv=self.H_kv, H_lm=self.H_lm, d=self.d, S=self.S, W=self.W,
                    K=self.K, scale=self.scale or 1.0 / math.sqrt(self.d), agg_mode=self.agg_mode)

    def q_lm_shape(self, items=None):
        """Shape of the landmark queries for the landmark mode (None: unused).
        items: per-item queries of hils_summarize_pages instead of [B, H_lm, C, d]."""
        if self.landmark_mode == LM_MEAN:
            return None
        if self.landmark_mode == LM_SHARED:
            return (self.H_lm, self.d)
        return (items, self.H_lm, self.d) if items is not None else (self.B, self.H_lm, self.C, self.d)


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libhils.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m long_context_chunk_landmark_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(_CConfig)
    lib.hils_landmark_summarize.argtypes = [cfgp, vp, vp, vp, vp, vp]
    lib.hils_score_select.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.hils_sparse_attend_fused.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hils_decode.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, sz,
                                vp]
    lib.hils_decode_noalloc.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp,
                                        vp]
    lib.hils_summarize_pages.argtypes = [cfgp, i32, vp, i32, vp, vp, vp, vp, vp]
    lib.hils_prefill_paged.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp, i32, i32, vp, vp, vp,
                                       vp, vp, sz, vp]
    lib.hils_prefill_paged_workspace_size.argtypes = [cfgp, i32, i32, i32]
    lib.hils_prefill_paged_workspace_size.restype = sz
    lib.hils_sparse_attend_backward.argtypes = [cfgp] + [vp] * 15 + [sz, vp]
    lib.hils_dense_causal_attend.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hils_dense_decode.argtypes = [cfgp, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.hils_workspace_size.argtypes = [cfgp, ctypes.c_int, i32, i32]
    lib.hils_workspace_size.restype = sz
    lib.hils_last_error.restype = ctypes.c_char_p
    lib.hils_version.restype = ctypes.c_int
    for fn in ("hils_landmark_summarize", "hils_score_select", "hils_sparse_attend_fused", "hils_decode",
               "hils_decode_noalloc",
               "hils_summarize_pages", "hils_prefill_paged", "hils_sparse_attend_backward", "hils_dense_causal_attend",
               "hils_dense_decode"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def version() -> int:
    return load_library().hils_version()


def last_error() -> str:
    return load_library().hils_last_error().decode()


def _check(status: int):
    if status != HILS_OK:
        raise HilsError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _want(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: device {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_size(cfg: Config, which: int, num_seqs: int = 0, max_pages: int = 0) -> int:
    c = cfg.to_c()
    n = load_library().hils_workspace_size(ctypes.byref(c), which, num_seqs, max_pages)
    if n == 0 and last_error():
        raise HilsError(HILS_ERR_INVALID_ARG, last_error())
    return n


def _workspace(cfg: Config, which: int, device, ws: Optional[torch.Tensor], num_seqs=0, max_pages=0):
    need = workspace_size(cfg, which, num_seqs, max_pages)
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    if need == 0:
        return None, 0
    return torch.empty(need, dtype=torch.uint8, device=device), need


def _want_q_lm(cfg: Config, q_lm, dev, items=None):
    shape = cfg.q_lm_shape(items)
    if shape is None:
        return None  # mean pooling: no landmark queries
    _want(q_lm, "q_lm", shape, cfg.io_dtype, dev)
    return q_lm


def status_word(workspace: torch.Tensor) -> int:
    """Word 0 of a fused-attention (or chunked-prefill) workspace after the
    call: 0 when the call completed normally; bit 0 when a bounded wait of
    the kernel gave up, bit 1 when a value of v is beyond fp16's range.
    Synchronises the current stream."""
    torch.cuda.current_stream().synchronize()
    return int(workspace[:4].view(torch.int32).item())


def landmark_summarize(cfg: Config, k: torch.Tensor, q_lm: Optional[torch.Tensor], k_sum=None, b_sum=None):
    """k [B,H_kv,N,d], q_lm per ``cfg.q_lm_shape()`` -> (k_sum [B,H_lm,C,d], b_sum [B,H_lm,C] fp32)."""
    dev = k.device
    _want(k, "k", (cfg.B, cfg.H_kv, cfg.N, cfg.d), cfg.io_dtype, dev)
    q_lm = _want_q_lm(cfg, q_lm, dev)
    if k_sum is None:
        k_sum = torch.empty((cfg.B, cfg.H_lm, cfg.C, cfg.d), dtype=cfg.summary_dtype, device=dev)
    if b_sum is None:
        b_sum = torch.empty((cfg.B, cfg.H_lm, cfg.C), dtype=torch.float32, device=dev)
    _want(k_sum, "k_sum", (cfg.B, cfg.H_lm, cfg.C, cfg.d), cfg.summary_dtype, dev)
    _want(b_sum, "b_sum", (cfg.B, cfg.H_lm, cfg.C), torch.float32, dev)
    c = cfg.to_c()
    _check(load_library().hils_landmark_summarize(ctypes.byref(c), _ptr(k), _ptr(q_lm), _ptr(k_sum), _ptr(b_sum),
                                                  _stream()))
    return k_sum, b_sum


def score_select(cfg: Config, q, k_sum, b_sum, qcal=None, sel_idx=None, sel_score=None, workspace=None):
    """Surrogate scores, GQA max and top-K.

    qcal: optional (h [B,N,d_model], w_down [r,d_model], w_up [H_q*d, r]).
    Returns (sel_idx [B,H_kv,N,K] int32, sel_score [B,H_q,N,K] fp32).
    """
    dev = q.device
    _want(q, "q", (cfg.B, cfg.H_q, cfg.N, cfg.d), cfg.io_dtype, dev)
    _want(k_sum, "k_sum", (cfg.B, cfg.H_lm, cfg.C, cfg.d), cfg.summary_dtype, dev)
    _want(b_sum, "b_sum", (cfg.B, cfg.H_lm, cfg.C), torch.float32, dev)
    h = wd = wu = None
    d_model = r = 0
    if qcal is not None:
        h, wd, wu = qcal
        r, d_model = wd.shape
        _want(h, "h", (cfg.B, cfg.N, d_model), cfg.io_dtype, dev)
        _want(wd, "w_down", (r, d_model), cfg.io_dtype, dev)
        _want(wu, "w_up", (cfg.H_q * cfg.d, r), cfg.io_dtype, dev)
    if sel_idx is None:
        sel_idx = torch.empty((cfg.B, cfg.H_kv, cfg.N, cfg.K), dtype=torch.int32, device=dev)
    if sel_score is None:
        sel_score = torch.empty((cfg.B, cfg.H_q, cfg.N, cfg.K), dtype=torch.float32, device=dev)
    _want(sel_idx, "sel_idx", (cfg.B, cfg.H_kv, cfg.N, cfg.K), torch.int32, dev)
    _want(sel_score, "sel_score", (cfg.B, cfg.H_q, cfg.N, cfg.K), torch.float32, dev)
    ws, nbytes = _workspace(cfg, WS_SCORE_QCAL if qcal is not None else WS_SCORE, dev, workspace)
    c = cfg.to_c()
    _check(load_library().hils_score_select(ctypes.byref(c), _ptr(q), _ptr(k_sum), _ptr(b_sum), _ptr(h), _ptr(wd),
                                            _ptr(wu), d_model, r, _ptr(sel_idx), _ptr(sel_score), _ptr(ws), nbytes,
                                            _stream()))
    return sel_idx, sel_score


def sparse_attend_fused(cfg: Config, q, k, v, sel_idx, sel_score, out=None, lse=None, workspace=None,
                        want_lse: bool = True):
    """Exact per-chunk + window attention fused by exp(s^)/Z^ -> (out, lse)."""
    dev = q.device
    _want(q, "q", (cfg.B, cfg.H_q, cfg.N, cfg.d), cfg.io_dtype, dev)
    _want(k, "k", (cfg.B, cfg.H_kv, cfg.N, cfg.d), cfg.io_dtype, dev)
    _want(v, "v", (cfg.B, cfg.H_kv, cfg.N, cfg.d), cfg.io_dtype, dev)
    _want(sel_idx, "sel_idx", (cfg.B, cfg.H_kv, cfg.N, cfg.K), torch.int32, dev)
    _want(sel_score, "sel_score", (cfg.B, cfg.H_q, cfg.N, cfg.K), torch.float32, dev)
    if out is None:
        out = torch.empty((cfg.B, cfg.H_q, cfg.N, cfg.d), dtype=cfg.io_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((cfg.B, cfg.H_q, cfg.N), dtype=torch.float32, device=dev)
    _want(out, "out", (cfg.B, cfg.H_q, cfg.N, cfg.d), cfg.io_dtype, dev)
    if lse is not None:
        _want(lse, "lse", (cfg.B, cfg.H_q, cfg.N), torch.float32, dev)
    ws, nbytes = _workspace(cfg, WS_FUSED, dev, workspace)
    c = cfg.to_c()
    _check(load_library().hils_sparse_attend_fused(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(sel_idx),
                                                   _ptr(sel_score), _ptr(out), _ptr(lse), _ptr(ws), nbytes,
                                                   _stream()))
    return out, lse


def dense_causal_attend(cfg: Config, q, k, v, out=None, lse=None, workspace=None, want_lse: bool = True):
    """Dense causal attention over every key (the full-attention baseline) -> (out, lse)."""
    dev = q.device
    _want(q, "q", (cfg.B, cfg.H_q, cfg.N, cfg.d), cfg.io_dtype, dev)
    _want(k, "k", (cfg.B, cfg.H_kv, cfg.N, cfg.d), cfg.io_dtype, dev)
    _want(v, "v", (cfg.B, cfg.H_kv, cfg.N, cfg.d), cfg.io_dtype, dev)
    if out is None:
        out = torch.empty((cfg.B, cfg.H_q, cfg.N, cfg.d), dtype=cfg.io_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((cfg.B, cfg.H_q, cfg.N), dtype=torch.float32, device=dev)
    _want(out, "out", (cfg.B, cfg.H_q, cfg.N, cfg.d), cfg.io_dtype, dev)
    if lse is not None:
        _want(lse, "lse", (cfg.B, cfg.H_q, cfg.N), torch.float32, dev)
    ws, nbytes = _workspace(cfg, WS_DENSE, dev, workspace)
    c = cfg.to_c()
    _check(load_library().hils_dense_causal_attend(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                                   _ptr(ws), nbytes, _stream()))
    return out, lse


def dense_decode(cfg: Config, q, k_cache, v_cache, block_table, seq_lens, out=None, lse=None, workspace=None,
                 want_lse: bool = True):
    """One dense decode step over the paged cache (every key of each sequence) -> (out, lse)."""
    dev = q.device
    num_seqs = q.shape[0]
    max_pages = block_table.shape[1]
    P = k_cache.shape[0]
    _want(q, "q", (num_seqs, cfg.H_q, cfg.d), cfg.io_dtype, dev)
    _want(k_cache, "k_cache", (P, cfg.H_kv, cfg.S, cfg.d), cfg.io_dtype, dev)
    _want(v_cache, "v_cache", (P, cfg.H_kv, cfg.S, cfg.d), cfg.io_dtype, dev)
    _want(block_table, "block_table", (num_seqs, max_pages), torch.int32, dev)
    _want(seq_lens, "seq_lens", (num_seqs,), torch.int32, dev)
    if out is None:
        out = torch.empty((num_seqs, cfg.H_q, cfg.d), dtype=cfg.io_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((num_seqs, cfg.H_q), dtype=torch.float32, device=dev)
    ws, nbytes = _workspace(cfg, WS_DENSE_DECODE, dev, workspace, num_seqs, max_pages)
    c = cfg.to_c()
    _check(load_library().hils_dense_decode(ctypes.byref(c), num_seqs, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(block_table), max_pages, _ptr(seq_lens), _ptr(out), _ptr(lse),
                                            _ptr(ws), nbytes, _stream()))
    return out, lse


def decode(cfg: Config, q, k_cache, v_cache, ksum_cache, bsum_cache, block_table, seq_lens, qcal=None, out=None,
           lse=None, sel_idx=None, workspace=None, want_sel: bool = True):
    """One decode step per sequence over a paged KV / summary cache -> (out, lse, sel_idx)."""
    dev = q.device
    num_seqs = q.shape[0]
    P = k_cache.shape[0]
    max_pages = block_table.shape[1]
    _want(q, "q", (num_seqs, cfg.H_q, cfg.d), cfg.io_dtype, dev)
    _want(k_cache, "k_cache", (P, cfg.H_kv, cfg.S, cfg.d), cfg.io_dtype, dev)
    _want(v_cache, "v_cache", (P, cfg.H_kv, cfg.S, cfg.d), cfg.io_dtype, dev)
    _want(ksum_cache, "ksum_cache", (ksum_cache.shape[0], cfg.H_lm, cfg.d), cfg.summary_dtype, dev)
    _want(bsum_cache, "bsum_cache", (ksum_cache.shape[0], cfg.H_lm), torch.float32, dev)
    _want(block_table, "block_table", (num_seqs, max_pages), torch.int32, dev)
    _want(seq_lens, "seq_lens", (num_seqs,), torch.int32, dev)
    h = wd = wu = None
    d_model = r = 0
    if qcal is not None:
        h, wd, wu = qcal
        r, d_model = wd.shape
        _want(h, "h", (num_seqs, d_model), cfg.io_dtype, dev)
        _want(wd, "w_down", (r, d_model), cfg.io_dtype, dev)
        _want(wu, "w_up", (cfg.H_q * cfg.d, r), cfg.io_dtype, dev)
    if out is None:
        out = torch.empty((num_seqs, cfg.H_q, cfg.d), dtype=cfg.io_dtype, device=dev)
    if lse is None:
        lse = torch.empty((num_seqs, cfg.H_q), dtype=torch.float32, device=dev)
    if sel_idx is None and want_sel:
        sel_idx = torch.empty((num_seqs, cfg.H_kv, cfg.K), dtype=torch.int32, device=dev)
    ws, nbytes = _workspace(cfg, WS_DECODE, dev, workspace, num_seqs, max_pages)
    c = cfg.to_c()
    _check(load_library().hils_decode(ctypes.byref(c), num_seqs, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(ksum_cache), _ptr(bsum_cache), _ptr(block_table), max_pages,
                                      _ptr(seq_lens), _ptr(h), _ptr(wd), _ptr(wu), d_model, r, _ptr(out), _ptr(lse),
                                      _ptr(sel_idx), _ptr(ws), nbytes, _stream()))
    return out, lse, sel_idx


def decode_noalloc(cfg: Config, q, k_cache, v_cache, ksum_cache, bsum_cache, block_table, seq_lens, out, lse,
                   sel_idx, qcal=None):
    """hils_decode_noalloc: the decode step with the library's static scratch
    instead of a workspace.  The outputs are the caller's (no tensor is
    created here)."""
    dev = q.device
    num_seqs = q.shape[0]
    P = k_cache.shape[0]
    max_pages = block_table.shape[1]
    _want(q, "q", (num_seqs, cfg.H_q, cfg.d), cfg.io_dtype, dev)
    _want(k_cache, "k_cache", (P, cfg.H_kv, cfg.S, cfg.d), cfg.io_dtype, dev)
    _want(v_cache, "v_cache", (P, cfg.H_kv, cfg.S, cfg.d), cfg.io_dtype, dev)
    _want(ksum_cache, "ksum_cache", (ksum_cache.shape[0], cfg.H_lm, cfg.d), cfg.summary_dtype, dev)
    _want(bsum_cache, "bsum_cache", (ksum_cache.shape[0], cfg.H_lm), torch.float32, dev)
    _want(block_table, "block_table", (num_seqs, max_pages), torch.int32, dev)
    _want(seq_lens, "seq_lens", (num_seqs,), torch.int32, dev)
    _want(out, "out", (num_seqs, cfg.H_q, cfg.d), cfg.io_dtype, dev)
    _want(lse, "lse", (num_seqs, cfg.H_q), torch.float32, dev)
    if sel_idx is not None:
        _want(sel_idx, "sel_idx", (num_seqs, cfg.H_kv, cfg.K), torch.int32, dev)
    h = wd = wu = None
    d_model = r = 0
    if qcal is not None:
        h, wd, wu = qcal
        r, d_model = wd.shape
    c = cfg.to_c()
    _check(load_library().hils_decode_noalloc(ctypes.byref(c), num_seqs, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                              _ptr(ksum_cache), _ptr(bsum_cache), _ptr(block_table), max_pages,
                                              _ptr(seq_lens), _ptr(h), _ptr(wd), _ptr(wu), d_model, r, _ptr(out),
                                              _ptr(lse), _ptr(sel_idx), _stream()))
    return out, lse, sel_idx


def summarize_pages(cfg: Config, k_cache, q_lm, pages, ksum_cache, bsum_cache):
    """Summaries of the pages ``pages`` (one completed chunk each) written into the summary caches in place."""
    dev = k_cache.device
    P = k_cache.shape[0]
    n = pages.shape[0]
    _want(k_cache, "k_cache", (P, cfg.H_kv, cfg.S, cfg.d), cfg.io_dtype, dev)
    q_lm = _want_q_lm(cfg, q_lm, dev, items=n)
    _want(pages, "pages", (n,), torch.int32, dev)
    _want(ksum_cache, "ksum_cache", (P, cfg.H_lm, cfg.d), cfg.summary_dtype, dev)
    _want(bsum_cache, "bsum_cache", (P, cfg.H_lm), torch.float32, dev)
    c = cfg.to_c()
    _check(load_library().hils_summarize_pages(ctypes.byref(c), n, _ptr(k_cache), P, _ptr(q_lm), _ptr(pages),
                                               _ptr(ksum_cache), _ptr(bsum_cache), _stream()))
    return ksum_cache, bsum_cache


def prefill_paged_workspace_size(cfg: Config, q_start: int, max_pages: int, qcal: bool = False) -> int:
    n = load_library().hils_prefill_paged_workspace_size(ctypes.byref(cfg.to_c()), q_start, max_pages, int(qcal))
    if n == 0 and last_error():
        raise HilsError(HILS_ERR_INVALID_ARG, last_error())
    return n


def prefill_paged(cfg: Config, q_start: int, q, k_cache, v_cache, ksum_cache, bsum_cache, block_table, qcal=None,
                  out=None, lse=None, sel_idx=None, sel_score=None, workspace=None):
    """Chunked prefill of cfg.N new tokens per sequence at positions q_start.. over the paged cache.

    Returns (out, lse, sel_idx, sel_score)."""
    dev = q.device
    P = k_cache.shape[0]
    max_pages = block_table.shape[1]
    _want(q, "q", (cfg.B, cfg.H_q, cfg.N, cfg.d), cfg.io_dtype, dev)
    _want(k_cache, "k_cache", (P, cfg.H_kv, cfg.S, cfg.d), cfg.io_dtype, dev)
    _want(v_cache, "v_cache", (P, cfg.H_kv, cfg.S, cfg.d), cfg.io_dtype, dev)
    _want(ksum_cache, "ksum_cache", (ksum_cache.shape[0], cfg.H_lm, cfg.d), cfg.summary_dtype, dev)
    _want(bsum_cache, "bsum_cache", (ksum_cache.shape[0], cfg.H_lm), torch.float32, dev)
    _want(block_table, "block_table", (cfg.B, max_pages), torch.int32, dev)
    h = wd = wu = None
    d_model = r = 0
    if qcal is not None:
        h, wd, wu = qcal
        r, d_model = wd.shape
        _want(h, "h", (cfg.B, cfg.N, d_model), cfg.io_dtype, dev)
        _want(wd, "w_down", (r, d_model), cfg.io_dtype, dev)
        _want(wu, "w_up", (cfg.H_q * cfg.d, r), cfg.io_dtype, dev)
    if out is None:
        out = torch.empty((cfg.B, cfg.H_q, cfg.N, cfg.d), dtype=cfg.io_dtype, device=dev)
    if lse is None:
        lse = torch.empty((cfg.B, cfg.H_q, cfg.N), dtype=torch.float32, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty((cfg.B, cfg.H_kv, cfg.N, cfg.K), dtype=torch.int32, device=dev)
    if sel_score is None:
        sel_score = torch.empty((cfg.B, cfg.H_q, cfg.N, cfg.K), dtype=torch.float32, device=dev)
    _want(out, "out", (cfg.B, cfg.H_q, cfg.N, cfg.d), cfg.io_dtype, dev)
    _want(lse, "lse", (cfg.B, cfg.H_q, cfg.N), torch.float32, dev)
    _want(sel_idx, "sel_idx", (cfg.B, cfg.H_kv, cfg.N, cfg.K), torch.int32, dev)
    _want(sel_score, "sel_score", (cfg.B, cfg.H_q, cfg.N, cfg.K), torch.float32, dev)
    nbytes = prefill_paged_workspace_size(cfg, q_start, max_pages, qcal is not None)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    c = cfg.to_c()
    _check(load_library().hils_prefill_paged(ctypes.byref(c), q_start, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                             _ptr(ksum_cache), _ptr(bsum_cache), P, _ptr(block_table), max_pages,
                                             _ptr(h), _ptr(wd), _ptr(wu), d_model, r, _ptr(sel_idx), _ptr(sel_score),
                                             _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))
    return out, lse, sel_idx, sel_score


def sparse_attend_backward(cfg: Config, q, k, v, q_lm, k_sum, sel_idx, sel_score, lse, dout, dlse=None,
                           workspace=None):
    """Gradients of sum(dout*out) + sum(dlse*lse) with the selection fixed -> (dq, dk, dv, dq_lm), fp32."""
    dev = q.device
    _want(q, "q", (cfg.B, cfg.H_q, cfg.N, cfg.d), cfg.io_dtype, dev)
    _want(k, "k", (cfg.B, cfg.H_kv, cfg.N, cfg.d), cfg.io_dtype, dev)
    _want(v, "v", (cfg.B, cfg.H_kv, cfg.N, cfg.d), cfg.io_dtype, dev)
    q_lm = _want_q_lm(cfg, q_lm, dev)
    _want(k_sum, "k_sum", (cfg.B, cfg.H_lm, cfg.C, cfg.d), torch.float32, dev)
    _want(sel_idx, "sel_idx", (cfg.B, cfg.H_kv, cfg.N, cfg.K), torch.int32, dev)
    _want(sel_score, "sel_score", (cfg.B, cfg.H_q, cfg.N, cfg.K), torch.float32, dev)
    _want(lse, "lse", (cfg.B, cfg.H_q, cfg.N), torch.float32, dev)
    _want(dout, "dout", (cfg.B, cfg.H_q, cfg.N, cfg.d), cfg.io_dtype, dev)
    if dlse is not None:
        _want(dlse, "dlse", (cfg.B, cfg.H_q, cfg.N), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((cfg.B, cfg.H_q, cfg.N, cfg.d), **f32)
    dk = torch.empty((cfg.B, cfg.H_kv, cfg.N, cfg.d), **f32)
    dv = torch.empty((cfg.B, cfg.H_kv, cfg.N, cfg.d), **f32)
    dq_lm = None
    if cfg.landmark_mode == LM_CHUNK:
        dq_lm = torch.empty((cfg.B, cfg.H_lm, cfg.C, cfg.d), **f32)
    elif cfg.landmark_mode == LM_SHARED:
        dq_lm = torch.empty((cfg.H_lm, cfg.d), **f32)
    ws, nbytes = _workspace(cfg, WS_BACKWARD, dev, workspace)
    c = cfg.to_c()
    _check(load_library().hils_sparse_attend_backward(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(q_lm), _ptr(k_sum), _ptr(sel_idx), _ptr(sel_score),
        _ptr(lse), _ptr(dout), _ptr(dlse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dq_lm), _ptr(ws), nbytes, _stream()))
    return dq, dk, dv, dq_lm


def prefill(cfg: Config, q, k, v, q_lm, qcal=None):
    """Whole forward: summaries -> score/select -> fused attention."""
    k_sum, b_sum = landmark_summarize(cfg, k, q_lm)
    sel_idx, sel_score = score_select(cfg, q, k_sum, b_sum, qcal=qcal)
    out, lse = sparse_attend_fused(cfg, q, k, v, sel_idx, sel_score)
    return dict(k_sum=k_sum, b_sum=b_sum, sel_idx=sel_idx, sel_score=sel_score, out=out, lse=lse)
