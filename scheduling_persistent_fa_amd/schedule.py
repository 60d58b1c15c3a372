"""Python view of the library's host-side schedule generator (no GPU needed)."""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib


def choose(mask: int, N: int, D: int, g: int, P: int, Nk: int | None = None):
    """(schedule, max_gang) the library's adaptive rule picks for a shape (N query
    tiles, Nk key/value tiles, default N)."""
    kind, cap = ctypes.c_int(), ctypes.c_int()
    _lib.check(_lib.lib().dash_schedule_choose_qk(mask, N, N if Nk is None else Nk, D, g, P, ctypes.byref(kind),
                                                  ctypes.byref(cap)))
    return kind.value, cap.value


def choose_band(Nq: int, Nk: int, band, D: int, g: int, P: int):
    """(schedule, max_gang) the adaptive rule picks for a band mask with
    (left, right) tile extents (None = unbounded side)."""
    kind, cap = ctypes.c_int(), ctypes.c_int()
    bl, br = (-1 if x is None else int(x) for x in band)
    _lib.check(_lib.lib().dash_schedule_choose_band(Nq, Nk, bl, br, D, g, P, ctypes.byref(kind), ctypes.byref(cap)))
    return kind.value, cap.value


class Schedule:
    """Per-workgroup step lists built by ``dash_schedule_build``.

    ``offsets`` has P+1 entries; ``steps`` is [num_steps, 4] int32 with columns
    (head, qi, kj, ord | flags).
    """

    def __init__(self, mask: int, schedule: int, N: int, g: int, groups: int, P: int,
                 xcd_local: bool = True, atomic_walk: int = -1, max_gang: int = 0, Nk: int | None = None,
                 band=None):
        """``band`` = (left, right) tile extents (None = unbounded side) builds a
        band-mask schedule through ``dash_schedule_build_band``; ``mask`` is then
        ignored."""
        L = _lib.lib()
        h = ctypes.c_void_p()
        nk = N if Nk is None else Nk
        if band is None:
            _lib.check(L.dash_schedule_build_qk(mask, schedule, N, nk, g, groups, P, int(bool(xcd_local)),
                                                atomic_walk, max_gang, ctypes.byref(h)))
        else:
            bl, br = (-1 if x is None else int(x) for x in band)
            _lib.check(L.dash_schedule_build_band(schedule, N, nk, bl, br, g, groups, P, int(bool(xcd_local)),
                                                  atomic_walk, max_gang, ctypes.byref(h)))
        self._h = h
        self.P = L.dash_schedule_num_workgroups(h)
        self.num_steps = L.dash_schedule_num_steps(h)
        self.offsets = np.zeros(self.P + 1, dtype=np.int32)
        self.steps = np.zeros((max(1, self.num_steps), 4), dtype=np.int32)
        _lib.check(L.dash_schedule_export(h, self.offsets.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                          self.steps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        self.steps = self.steps[: self.num_steps]

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                _lib.lib().dash_schedule_free(h)
            except (TypeError, AttributeError):
                pass  # interpreter shutdown: module globals are already gone, and the process frees the memory
            self._h = None

    def validate(self) -> None:
        _lib.check(_lib.lib().dash_schedule_validate(self._h))

    def simulate(self, c: float, r: float, jitter_seed: int = 0):
        """(makespan, total wait) of the unit-cost DAG model; a non-zero
        ``jitter_seed`` scales each step's compute cost into [0.5, 1.5) c."""
        mk, wt = ctypes.c_double(), ctypes.c_double()
        _lib.check(_lib.lib().dash_schedule_simulate(self._h, c, r, jitter_seed, ctypes.byref(mk), ctypes.byref(wt)))
        return mk.value, wt.value

    def lists(self):
        """Per workgroup: list of (head, qi, kj, ord, first, last) tuples."""
        out = []
        for w in range(self.P):
            rows = self.steps[self.offsets[w]: self.offsets[w + 1]]
            out.append([(int(h), int(q), int(k), int(o & _lib.ORD_MASK), bool(o & _lib.FIRST_FLAG),
                         bool(o & _lib.LAST_FLAG)) for h, q, k, o in rows])
        return out
