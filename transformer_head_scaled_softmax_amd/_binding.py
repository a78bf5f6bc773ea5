"""ctypes binding of libmha.so, the C ABI declared in include/mha.h.

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  If the
library has not been built, loading it raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import pathlib

PKG = pathlib.Path(__file__).resolve().parent
LIB_PATH = PKG / "libmha.so"

MASK_NONE = 0
MASK_CAUSAL = 1
PLAN_AUTO, PLAN_UNFUSED, PLAN_FUSED = 0, 1, 2
F32, BF16, F16 = 0, 1, 2

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE = -3
ERR_HIP = -4

# Every symbol include/mha.h declares.
EXPORTS = ("mha_forward", "mha_forward_timed", "mha_proj_workspace_bytes", "mha_proj_forward",
           "mha_proj_forward_timed", "mha_proj_fused", "mha_forward_block_queries", "mha_proj_ln_forward", "mha_proj_ln_forward_timed",
           "mha_proj_ln_workspace_bytes", "mha_decode_workspace_bytes", "mha_decode_forward",
           "mha_decode_forward_timed", "mha_decode_forward_noalloc", "mha_decode_split", "mha_forward_lse", "mha_forward_strided",
           "mha_forward_gqa", "mha_backward_workspace_bytes", "mha_backward", "mha_backward_timed",
           "mha_backward_gqa", "mha_backward_gqa_timed", "mha_backward_gqa_workspace_bytes", "mha_proj_forward_gqa",
           "mha_proj_forward_gqa_timed", "mha_proj_gqa_workspace_bytes", "mha_backward_single_launch",
           "mha_status_string", "mha_last_error_message", "mha_last_error", "mha_version")


class MhaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def load(path: pathlib.Path | str | None = None) -> ctypes.CDLL:
    """Load libmha.so (once) and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = pathlib.Path(path) if path else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} is not built; run `python -m transformer_head_scaled_softmax_amd.build`")
    lib = ctypes.CDLL(str(p))
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.mha_forward.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp, f, i, vp]
    lib.mha_forward.restype = i
    lib.mha_forward_timed.argtypes = lib.mha_forward.argtypes + [vp]
    lib.mha_forward_timed.restype = i
    lib.mha_proj_workspace_bytes.argtypes = [i] * 8
    lib.mha_proj_workspace_bytes.restype = ctypes.c_size_t
    lib.mha_proj_forward.argtypes = [vp] * 11 + [i] * 8 + [vp, f, i, vp, ctypes.c_size_t, vp]
    lib.mha_proj_forward.restype = i
    lib.mha_proj_forward_timed.argtypes = lib.mha_proj_forward.argtypes + [vp, i]
    lib.mha_proj_forward_timed.restype = i
    lib.mha_proj_fused.argtypes = [i] * 7
    lib.mha_proj_fused.restype = i
    lib.mha_forward_block_queries.argtypes = [i] * 5
    lib.mha_forward_block_queries.restype = i
    lib.mha_proj_ln_forward.argtypes = [vp] * 12 + [f, vp] + [i] * 8 + [vp, f, i, vp, ctypes.c_size_t, vp]
    lib.mha_proj_ln_forward.restype = i
    lib.mha_proj_ln_forward_timed.argtypes = lib.mha_proj_ln_forward.argtypes + [vp, i]
    lib.mha_proj_ln_forward_timed.restype = i
    lib.mha_proj_ln_workspace_bytes.argtypes = [i] * 8
    lib.mha_proj_ln_workspace_bytes.restype = ctypes.c_size_t
    lib.mha_decode_workspace_bytes.argtypes = [i] * 8
    lib.mha_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.mha_decode_forward.argtypes = [vp] * 4 + [i] * 8 + [vp, f, i, vp, ctypes.c_size_t, vp]
    lib.mha_decode_forward.restype = i
    lib.mha_decode_forward_timed.argtypes = lib.mha_decode_forward.argtypes + [vp]
    lib.mha_decode_forward_timed.restype = i
    lib.mha_decode_forward_noalloc.argtypes = [vp] * 4 + [i] * 8 + [vp, f, i, vp]
    lib.mha_decode_forward_noalloc.restype = i
    lib.mha_decode_split.argtypes = [i] * 8
    lib.mha_decode_split.restype = i
    lib.mha_forward_lse.argtypes = [vp] * 5 + [i] * 7 + [vp, f, i, vp]
    lib.mha_forward_lse.restype = i
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.mha_forward_strided.argtypes = [vp, i64p, vp, i64p, vp, i64p, vp, i64p, vp] + [i] * 7 + [vp, f, i, vp]
    lib.mha_forward_strided.restype = i
    lib.mha_backward_workspace_bytes.argtypes = [i] * 7
    lib.mha_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.mha_backward.argtypes = [vp] * 9 + [i] * 7 + [vp, f, i, vp, ctypes.c_size_t, vp]
    lib.mha_backward.restype = i
    lib.mha_backward_timed.argtypes = lib.mha_backward.argtypes + [vp]
    lib.mha_backward_timed.restype = i
    lib.mha_forward_gqa.argtypes = [vp] * 5 + [i] * 8 + [vp, f, i, vp]
    lib.mha_forward_gqa.restype = i
    lib.mha_backward_gqa.argtypes = [vp] * 9 + [i] * 8 + [vp, f, i, vp, ctypes.c_size_t, vp]
    lib.mha_backward_gqa.restype = i
    lib.mha_backward_gqa_timed.argtypes = lib.mha_backward_gqa.argtypes + [vp]
    lib.mha_backward_gqa_timed.restype = i
    lib.mha_backward_gqa_workspace_bytes.argtypes = [i] * 8
    lib.mha_backward_gqa_workspace_bytes.restype = ctypes.c_size_t
    lib.mha_proj_gqa_workspace_bytes.argtypes = [i] * 9
    lib.mha_proj_gqa_workspace_bytes.restype = ctypes.c_size_t
    lib.mha_backward_single_launch.argtypes = [i] * 8
    lib.mha_backward_single_launch.restype = i
    lib.mha_proj_forward_gqa.argtypes = [vp] * 11 + [i] * 9 + [vp, f, i, vp, ctypes.c_size_t, vp]
    lib.mha_proj_forward_gqa.restype = i
    lib.mha_proj_forward_gqa_timed.argtypes = lib.mha_proj_forward_gqa.argtypes + [vp]
    lib.mha_proj_forward_gqa_timed.restype = i
    lib.mha_status_string.argtypes = [i]
    lib.mha_status_string.restype = ctypes.c_char_p
    lib.mha_last_error_message.argtypes = []
    lib.mha_last_error_message.restype = ctypes.c_char_p
    lib.mha_last_error.argtypes = []
    lib.mha_last_error.restype = ctypes.c_char_p
    lib.mha_version.argtypes = []
    lib.mha_version.restype = i
    if path is None:
        _lib = lib
    return lib


def check(lib: ctypes.CDLL, status: int) -> None:
    if status != OK:
        detail = lib.mha_last_error_message().decode() or lib.mha_status_string(status).decode()
        raise MhaError(status, detail)
