"""HiLS (Hierarchical Landmark Sparse) attention forward for AMD MI355X.

The computation lives in ``libhils.so`` (hand-written HIP kernels for gfx950
behind the C ABI of ``include/hils.h``); this package is the thin Python
binding used by the tests and the benchmark.
"""
from ._binding import (EXPORTED_SYMBOLS, HILS_BF16, HILS_F32, LIB_PATH, WS_DECODE, WS_FUSED, WS_SCORE,
                       WS_SCORE_QCAL, Config, HilsError, decode, landmark_summarize, last_error, load_library,
                       prefill, score_select, sparse_attend_fused, version, workspace_size)

__all__ = [
    "Config", "HilsError", "landmark_summarize", "score_select", "sparse_attend_fused", "decode", "prefill",
    "workspace_size", "load_library", "last_error", "version", "EXPORTED_SYMBOLS", "LIB_PATH", "HILS_F32",
    "HILS_BF16", "WS_SCORE", "WS_SCORE_QCAL", "WS_FUSED", "WS_DECODE",
]
