"""Deterministic attention backward (DASH schedules) for AMD MI355X.

The compute path lives in libdash_attn.so (HIP kernels for gfx950 behind the C
ABI of include/dash_attn.h).  This package is its thin Python binding:
``attention`` (torch tensors in, torch tensors out) and ``schedule`` (the
host-side step lists).  Build the library with
``python -m scheduling_persistent_fa_amd.build``.
"""
from ._lib import ATOMIC, DESC_Q, MASK_CAUSAL, MASK_FULL, SCHEDULE_NAMES, SERIAL, SHIFT, SYM_SHIFT, DashError  # noqa: F401

__all__ = ["ATOMIC", "DESC_Q", "MASK_CAUSAL", "MASK_FULL", "SCHEDULE_NAMES", "SERIAL", "SHIFT", "SYM_SHIFT",
           "DashError"]
