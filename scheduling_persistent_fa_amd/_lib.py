"""ctypes binding of libdash_attn.so (declared in include/dash_attn.h).

Argument marshalling only: every step of the attention path runs in the
library's HIP kernels.  The library is loaded on first use; if it has not been
built the call fails loudly (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdash_attn.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_HIP = -3
ERR_INVALID_SCHEDULE = -4
ERR_TIMEOUT = -5
ERR_WORKSPACE = -6

MASK_FULL, MASK_CAUSAL = 0, 1
SERIAL, DESC_Q, SHIFT, SYM_SHIFT, ATOMIC, AUTO = 0, 1, 2, 3, 4, 5
SCHEDULE_NAMES = {SERIAL: "serial", DESC_Q: "desc_q", SHIFT: "shift", SYM_SHIFT: "sym_shift", ATOMIC: "atomic",
                  AUTO: "auto"}
FIRST_FLAG = 1 << 28
LAST_FLAG = 1 << 29
ORD_MASK = FIRST_FLAG - 1

# Every symbol include/dash_attn.h declares.
EXPORTS = (
    "dash_attn_fwd", "dash_attn_fwd_qk", "dash_attn_fwd_window", "dash_attn_bwd", "dash_attn_bwd_qk",
    "dash_attn_bwd_window", "dash_attn_bwd_workspace_bytes", "dash_schedule_build_band",
    "dash_attn_bwd_delta", "dash_schedule_build", "dash_schedule_build_qk", "dash_schedule_num_workgroups", "dash_schedule_num_steps", "dash_schedule_export",
    "dash_schedule_validate", "dash_schedule_simulate", "dash_schedule_free", "dash_schedule_choose",
    "dash_schedule_choose_qk", "dash_schedule_choose_band",
    "dash_status_string",
    "dash_last_error", "dash_device_info", "dash_check_async_error", "dash_attn_bwd_qk_noalloc",
)


class DashError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class BwdOpts(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_workgroups", ctypes.c_int),
        ("tile", ctypes.c_int),
        ("atomic_walk", ctypes.c_int),
        ("xcd_local", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stall_cycles_out", ctypes.c_void_p),
        ("spin_timeout_cycles", ctypes.c_ulonglong),
        ("sync_check", ctypes.c_int),
        ("event_start", ctypes.c_void_p),
        ("event_stop", ctypes.c_void_p),
        ("max_gang", ctypes.c_int),
        ("debug_delay_seed", ctypes.c_uint32),
        ("xcc_id_out", ctypes.c_void_p),
    ]


_lock = threading.Lock()
_lib = None


def _declare(lib):
    vp, i, f, i32p = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.POINTER(ctypes.c_int32)
    lib.dash_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.dash_attn_fwd_qk.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.dash_attn_bwd.argtypes = [vp] * 9 + [i, i, i, i, i, f, i, i, ctypes.POINTER(BwdOpts), vp]
    lib.dash_attn_bwd_qk.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, i, i, ctypes.POINTER(BwdOpts), vp]
    lib.dash_attn_bwd_qk_noalloc.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, i, i, ctypes.POINTER(BwdOpts), vp]
    lib.dash_attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.dash_attn_bwd_window.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, i, i, i, ctypes.POINTER(BwdOpts), vp]
    lib.dash_schedule_build_band.argtypes = [i, i, i, i, i, i, i, i, i, i, i, ctypes.POINTER(vp)]
    lib.dash_schedule_choose_band.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.dash_attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(ctypes.c_size_t)]
    lib.dash_attn_bwd_delta.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.dash_schedule_build.argtypes = [i, i, i, i, i, i, i, i, i, ctypes.POINTER(vp)]
    lib.dash_schedule_build_qk.argtypes = [i, i, i, i, i, i, i, i, i, i, ctypes.POINTER(vp)]
    lib.dash_schedule_num_workgroups.argtypes = [vp]
    lib.dash_schedule_num_steps.argtypes = [vp]
    lib.dash_schedule_num_steps.restype = ctypes.c_longlong
    lib.dash_schedule_export.argtypes = [vp, i32p, i32p]
    lib.dash_schedule_validate.argtypes = [vp]
    lib.dash_schedule_simulate.argtypes = [vp, ctypes.c_double, ctypes.c_double, ctypes.c_uint64,
                                           ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.dash_schedule_free.argtypes = [vp]
    lib.dash_schedule_free.restype = None
    lib.dash_schedule_choose.argtypes = [i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.dash_schedule_choose_qk.argtypes = [i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.dash_status_string.argtypes = [i]
    lib.dash_status_string.restype = ctypes.c_char_p
    lib.dash_last_error.argtypes = []
    lib.dash_last_error.restype = ctypes.c_char_p
    lib.dash_device_info.argtypes = [i, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.dash_check_async_error.argtypes = [vp]


def lib():
    """The loaded library; raises if it is missing (no fallback exists)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m scheduling_persistent_fa_amd.build` "
                    "(the attention path has no CPU fallback)")
            h = ctypes.CDLL(LIB_PATH)
            _declare(h)
            _lib = h
        return _lib


def check(status: int) -> None:
    if status != OK:
        msg = lib().dash_last_error().decode(errors="replace")
        raise DashError(status, msg or lib().dash_status_string(status).decode())
