"""ctypes binding of libkdkl.so: the C ABI declared in include/kd_fused_kl.h.

Argument marshalling only. If the library is not built, every call raises;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

from ._build import LIB_PATH

KD_OK, KD_ERR_INVALID_ARG, KD_ERR_UNSUPPORTED, KD_ERR_WORKSPACE, KD_ERR_HIP = range(5)
KD_F32, KD_BF16 = 0, 1
KD_PASS_FWD, KD_PASS_BWD, KD_PASS_TEACHER, KD_PASS_FWD_BWD = 0, 1, 2, 3
KD_REDUCE_SUM, KD_REDUCE_MEAN = 0, 1
KD_CHECK_ID_RANGE, KD_CHECK_DUPLICATE, KD_CHECK_LOGP = 1, 2, 4
KD_NOALLOC_SCRATCH_BYTES = 64 << 20  # the library-held scratch of kd_fused_kl_fwd_noalloc

# Every function the header declares, with (restype, argtypes).
_vp, _i64, _i, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "kd_status_str": (ctypes.c_char_p, [_i]),
    "kd_fused_kl_workspace_bytes": (_sz, [_i, _i64, _i64, _i64, _i64, _i64, _i]),
    "kd_fused_kl_fwd": (_i, [_vp, _vp, _i, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                             _vp, _vp, _vp, _vp, _sz, _vp]),
    "kd_fused_kl_bwd": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                             _vp, _vp, _vp, _i, _vp, _sz, _vp]),
    "kd_fused_kl_fwd_ex": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _i, _i64, _i64, _i64, _i64, _i64,
                                _vp, _vp, _vp, _vp, _sz, _vp]),
    "kd_fused_kl_bwd_ex": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _i, _vp, _i64, _i64, _i64, _i64,
                                _i64, _vp, _vp, _vp, _i, _vp, _sz, _vp]),
    "kd_fused_kl_fwd_noalloc": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _i, _i64, _i64, _i64, _i64,
                                     _i64, _vp, _vp, _vp, _vp]),
    "kd_fused_kl_fwd_bwd": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _i, _i64, _i64, _i64, _i64, _i64,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _sz, _vp]),
    "kd_teacher_topk": (_i, [_vp, _vp, _i, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz,
                             _vp]),
    "kd_fused_kl_check_inputs": (_i, [_vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "kd_cast_f32_to_bf16": (_i, [_vp, _vp, _i64, _vp]),
    "kd_scale": (_i, [_vp, _i, _i64, _vp, _vp]),
    "kd_timing_enable": (_i, [_i]),
    "kd_timing_read": (_i, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
}

KERNEL_CLASSES = ("prep", "fwd_logits", "bwd_dlogits", "bwd_dh", "bwd_dw", "other", "dl_stream")

_LIB = None


class KDError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m chunked_kl_loss_chunk_amd._build` "
                "(or __graft_entry__.build()); there is no non-HIP implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def status_str(status: int) -> str:
    return lib().kd_status_str(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != KD_OK:
        raise KDError(fn, status)
