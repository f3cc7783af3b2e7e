"""ctypes binding of libgtrscan (include/gtrscan.h).

Argument marshalling only: every step of the mixer runs in the library's HIP
kernels.  There is no fallback; if the shared library is missing or cannot be
loaded, loading raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgtrscan.so")

GTR_OK, GTR_ERR_ARG, GTR_ERR_UNSUPPORTED, GTR_ERR_HIP = 0, -1, -2, -3
GTR_F32, GTR_F16, GTR_BF16 = 0, 1, 2
PATH_AUTO, PATH_MFMA, PATH_FAST, PATH_SERIAL = 0, 1, 2, 3

EXPORTS = ("gtr_gla_fwd", "gtr_gla_fwd_noalloc", "gtr_gla_fwd_path", "gtr_gla_fwd_events", "gtr_gla_stack_fwd",
           "gtr_gla_lowrank_fwd", "gtr_gla_bwd", "gtr_gla_states_bytes", "gtr_gla_fwd_states",
           "gtr_gla_bwd_states", "gtr_sswiglu_mix", "gtr_gla_auto_path", "gtr_last_error",
           "gtr_version", "gtr_release_workspace", "gtr_set_segment_chunks", "gtr_set_wait_limit")

_lib = None


class GtrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libgtrscan status {status}: {message}")
        self.status = status


def load():
    """Load libgtrscan.so (built in-tree by the package's build step)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, i = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
    lib.gtr_gla_fwd.restype = i
    lib.gtr_gla_fwd.argtypes = [vp, vp, vp, fp, vp, fp, vp] + [i] * 9 + [vp]
    lib.gtr_gla_fwd_noalloc.restype = i
    lib.gtr_gla_fwd_noalloc.argtypes = [vp, vp, vp, fp, vp, fp, vp] + [i] * 9 + [vp]
    lib.gtr_gla_fwd_path.restype = i
    lib.gtr_gla_fwd_path.argtypes = [vp, vp, vp, fp, vp, fp, vp] + [i] * 10 + [vp]
    lib.gtr_gla_fwd_events.restype = i
    lib.gtr_gla_fwd_events.argtypes = ([vp, vp, vp, fp, vp, fp, vp] + [i] * 10 +
                                       [ctypes.POINTER(ctypes.c_void_p), i,
                                        ctypes.POINTER(ctypes.c_int), vp])
    lib.gtr_gla_stack_fwd.restype = i
    lib.gtr_gla_stack_fwd.argtypes = [vp, vp, vp, fp, vp, fp, vp] + [i] * 10 + [vp]
    lib.gtr_gla_lowrank_fwd.restype = i
    lib.gtr_gla_lowrank_fwd.argtypes = ([vp, vp, vp, vp, vp, fp, ctypes.c_float, i, vp, fp, vp] +
                                        [i] * 10 + [ctypes.POINTER(ctypes.c_void_p), i,
                                                    ctypes.POINTER(ctypes.c_int), vp])
    lib.gtr_gla_bwd.restype = i
    lib.gtr_gla_bwd.argtypes = ([vp, vp, vp, fp, vp, fp, vp, vp, vp, vp, fp, vp, fp] + [i] * 9 +
                                [ctypes.POINTER(ctypes.c_void_p), i, ctypes.POINTER(ctypes.c_int),
                                 vp])
    lib.gtr_gla_states_bytes.restype = ctypes.c_size_t
    lib.gtr_gla_states_bytes.argtypes = [i] * 8
    lib.gtr_gla_fwd_states.restype = i
    lib.gtr_gla_fwd_states.argtypes = ([vp, vp, vp, fp, vp, fp, vp] + [i] * 9 +
                                       [fp, ctypes.c_size_t, vp])
    lib.gtr_gla_bwd_states.restype = i
    lib.gtr_gla_bwd_states.argtypes = ([vp, vp, vp, fp, vp, fp, vp, vp, vp, vp, fp, vp, fp] +
                                       [i] * 9 + [fp, ctypes.c_size_t,
                                                  ctypes.POINTER(ctypes.c_void_p), i,
                                                  ctypes.POINTER(ctypes.c_int), vp])
    lib.gtr_sswiglu_mix.restype = i
    lib.gtr_sswiglu_mix.argtypes = [vp, fp, fp, vp] + [i] * 6 + [vp]
    lib.gtr_gla_auto_path.restype = i
    lib.gtr_gla_auto_path.argtypes = [i] * 8
    lib.gtr_last_error.restype = ctypes.c_char_p
    lib.gtr_last_error.argtypes = []
    lib.gtr_version.restype = i
    lib.gtr_version.argtypes = []
    lib.gtr_set_segment_chunks.restype = None
    lib.gtr_set_segment_chunks.argtypes = [i]
    lib.gtr_set_wait_limit.restype = None
    lib.gtr_set_wait_limit.argtypes = [ctypes.c_uint]
    lib.gtr_release_workspace.restype = None
    lib.gtr_release_workspace.argtypes = []
    _lib = lib
    return lib


def last_error() -> str:
    return load().gtr_last_error().decode()


def check(status: int) -> None:
    if status != GTR_OK:
        raise GtrError(status, last_error())
