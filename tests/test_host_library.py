"""CPU tests of libdash_attn.so: it loads, exports every declared symbol, and
its host-side schedule generator matches the schedule oracle exactly."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import schedules as Sch
from scheduling_persistent_fa_amd import _lib
from scheduling_persistent_fa_amd.schedule import Schedule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "dash_attn.h")).read()
    declared = set(re.findall(r"\b(dash_[a-z_]+)\s*\(", header))
    assert declared == set(_lib.EXPORTS)
    L = _lib.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings():
    L = _lib.lib()
    assert L.dash_status_string(0) == b"ok"
    assert L.dash_status_string(_lib.ERR_TIMEOUT) == b"semaphore wait timed out"


def _oracle_tuples(lists):
    return [[(s.head, s.qi, s.kj, s.ord, s.first, s.last) for s in l] for l in lists]


def _placement_free(lists):
    """The member lists of a schedule as a multiset: every list's steps in
    order (chains, walks, ordinals, chain flags), without the index of the
    workgroup that runs it.  Which compute unit runs a member list is a
    placement choice of the library; the schedule is the rest."""
    return sorted(tuple(l) for l in lists if l)


def _same_schedule(lib_s, ora, sched):
    """The library's lists equal the oracle's up to placement; SERIAL and
    DESC_Q also place each chain on the same workgroup (least-loaded list
    scheduling is part of their definition)."""
    got = lib_s.lists()
    want = _oracle_tuples(ora)
    assert len(got) == len(want)
    assert _placement_free(got) == _placement_free(want)
    if sched in (Sch.SERIAL, Sch.DESC_Q):
        assert got == want


CASES = [
    (Sch.FULL, Sch.SERIAL, 4, 1, 1, 4, 0), (Sch.FULL, Sch.SHIFT, 4, 1, 1, 4, 0), (Sch.CAUSAL, Sch.SYM_SHIFT, 4, 1, 1, 2, 0),
    (Sch.FULL, Sch.SERIAL, 16, 1, 8, 256, 0), (Sch.FULL, Sch.DESC_Q, 16, 2, 3, 20, 0),
    (Sch.CAUSAL, Sch.SERIAL, 16, 1, 64, 256, 0), (Sch.CAUSAL, Sch.DESC_Q, 16, 1, 64, 256, 0),
    (Sch.CAUSAL, Sch.SYM_SHIFT, 16, 1, 64, 256, 0), (Sch.FULL, Sch.SHIFT, 32, 1, 48, 256, 0),
    (Sch.CAUSAL, Sch.SYM_SHIFT, 64, 4, 8, 256, 0), (Sch.CAUSAL, Sch.DESC_Q, 64, 4, 8, 256, 0),
    (Sch.FULL, Sch.SHIFT, 6, 3, 5, 13, 0), (Sch.CAUSAL, Sch.SYM_SHIFT, 10, 2, 3, 11, 0),
    # capped gangs (rounds)
    (Sch.FULL, Sch.SHIFT, 128, 1, 16, 256, 32), (Sch.CAUSAL, Sch.SYM_SHIFT, 128, 1, 16, 256, 32),
    (Sch.FULL, Sch.SHIFT, 10, 2, 3, 12, 4), (Sch.CAUSAL, Sch.SYM_SHIFT, 14, 3, 2, 9, 3),
]


@pytest.mark.parametrize("mask,sched,N,g,groups,P,cap", CASES)
@pytest.mark.parametrize("xcd", [True, False])
def test_host_schedule_matches_oracle(mask, sched, N, g, groups, P, cap, xcd):
    lib_s = Schedule(mask, sched, N, g, groups, P, xcd_local=xcd, max_gang=cap)
    lib_s.validate()
    ora = Sch.build(mask, sched, N, g, groups, P, max_gang=cap)
    _same_schedule(lib_s, ora, sched)


@pytest.mark.parametrize("mask,sched,N,g,groups,P,cap", CASES[:8] + CASES[-2:])
def test_host_simulator_matches_oracle(mask, sched, N, g, groups, P, cap):
    lib_s = Schedule(mask, sched, N, g, groups, P, max_gang=cap)
    ora = Sch.build(mask, sched, N, g, groups, P, max_gang=cap)
    for c, r in ((1.0, 1.0), (2.5, 0.75)):
        assert lib_s.simulate(c, r) == pytest.approx(Sch.simulate(ora, c, r), rel=1e-12, abs=1e-9)


@pytest.mark.parametrize("mask,sched,N,g,groups,P,cap", CASES[:8] + CASES[-4:])
def test_jittered_simulation_matches_oracle(mask, sched, N, g, groups, P, cap):
    # Same seeded step costs on both sides (SplitMix64 per (seed, workgroup,
    # position)): same makespan and waiting time.  The lists are compared up
    # to placement, so each side simulates its own lists.
    lib_s = Schedule(mask, sched, N, g, groups, P, max_gang=cap, xcd_local=False)
    ora = Sch.build(mask, sched, N, g, groups, P, max_gang=cap)
    assert lib_s.lists() == _oracle_tuples(ora)  # contiguous placement on both sides
    for seed in (1, 12345, 2**63 + 5):
        assert lib_s.simulate(1.0, 0.5, seed) == pytest.approx(Sch.simulate(ora, 1.0, 0.5, seed), rel=1e-12, abs=1e-9)


@pytest.mark.parametrize("mask,sched,N,g,groups", [(1, 0, 16, 1, 64), (1, 1, 16, 1, 64), (1, 3, 16, 1, 64),
                                                   (0, 2, 32, 1, 48), (0, 2, 128, 1, 16), (1, 3, 128, 1, 16),
                                                   (1, 3, 64, 4, 8), (1, 0, 64, 4, 8), (0, 1, 128, 1, 16)])
def test_thousand_jittered_runs_never_deadlock(mask, sched, N, g, groups):
    # The workload shapes on 256 workgroups: under 1000 different seeded
    # timings every list still runs to completion (the order a schedule fixes
    # is acyclic whatever the step costs).
    s = Schedule(mask, sched, N, g, groups, 256)
    base, _ = s.simulate(1.0, 1.0)
    for seed in range(1, 1001):
        mk, wait = s.simulate(1.0, 1.0, seed)  # raises on deadlock
        assert mk > 0 and wait >= 0


def test_full_size_schedules_validate():
    # the workloads' shapes: (mask, schedule, N, g, groups) with 256 workgroups
    for mask, sched, N, g, groups in [(1, 0, 16, 1, 64), (1, 1, 16, 1, 64), (1, 3, 16, 1, 64),
                                      (0, 0, 32, 1, 48), (0, 2, 32, 1, 48), (0, 2, 128, 1, 16),
                                      (0, 1, 128, 1, 16), (1, 3, 128, 1, 16), (1, 1, 128, 1, 16),
                                      (1, 3, 64, 4, 8), (1, 0, 64, 4, 8)]:
        s = Schedule(mask, sched, N, g, groups, 256)
        s.validate()
        expect = g * groups * (N * N if mask == 0 else N * (N + 1) // 2)
        assert s.num_steps == expect


def test_atomic_walks_follow_their_base_schedule():
    for walk in (_lib.SERIAL, _lib.DESC_Q, _lib.SYM_SHIFT):
        a = Schedule(_lib.MASK_CAUSAL, _lib.ATOMIC, 8, 1, 4, 16, atomic_walk=walk)
        b = Schedule(_lib.MASK_CAUSAL, walk, 8, 1, 4, 16)
        assert np.array_equal(a.steps, b.steps)
    d = Schedule(_lib.MASK_FULL, _lib.ATOMIC, 8, 1, 4, 16)  # default full-mask walk: serial
    assert np.array_equal(d.steps, Schedule(_lib.MASK_FULL, _lib.SERIAL, 8, 1, 4, 16).steps)


def test_schedule_build_rejects_bad_input():
    for args, status in [((1, 2, 4, 1, 1, 4), _lib.ERR_UNSUPPORTED), ((0, 3, 4, 1, 1, 4), _lib.ERR_UNSUPPORTED),
                         ((1, 3, 5, 1, 1, 4), _lib.ERR_UNSUPPORTED), ((0, 2, 8, 1, 1, 4), _lib.ERR_UNSUPPORTED),
                         ((0, 0, 0, 1, 1, 4), _lib.ERR_INVALID_ARG), ((0, 9, 4, 1, 1, 4), _lib.ERR_INVALID_ARG)]:
        with pytest.raises(_lib.DashError) as ei:
            Schedule(*args)
        assert ei.value.status == status


def test_bwd_argument_errors_need_no_gpu():
    L = _lib.lib()
    vp = ctypes.c_void_p
    good = [vp(4096 * (i + 1)) for i in range(9)]
    # null pointer
    st = L.dash_attn_bwd(*([vp(0)] + good[1:]), 1, 1, 1, 128, 64, 0.0, 0, 0, None, None)
    assert st == _lib.ERR_INVALID_ARG
    # Hq not a multiple of Hkv
    assert L.dash_attn_bwd(*good, 1, 3, 2, 128, 64, 0.0, 0, 0, None, None) == _lib.ERR_INVALID_ARG
    # unsupported head dimension
    assert L.dash_attn_bwd(*good, 1, 1, 1, 128, 96, 0.0, 0, 0, None, None) == _lib.ERR_UNSUPPORTED
    # negative sizes; keys missing; causal with fewer keys than queries
    assert L.dash_attn_bwd(*good, 1, 1, 1, -1, 64, 0.0, 0, 0, None, None) == _lib.ERR_INVALID_ARG
    assert L.dash_attn_bwd_qk(*good, 1, 1, 1, 100, 0, 64, 0.0, 0, 0, None, None) == _lib.ERR_INVALID_ARG
    assert L.dash_attn_bwd_qk(*good, 1, 1, 1, 100, 99, 64, 0.0, 1, 0, None, None) == _lib.ERR_INVALID_ARG
    assert L.dash_attn_fwd_qk(*good[:5], 1, 1, 1, 7, 0, 64, 0.0, 0, None) == _lib.ERR_INVALID_ARG
    # misaligned pointer
    bad = list(good)
    bad[3] = vp(4096 + 8)
    assert L.dash_attn_bwd(*bad, 1, 1, 1, 128, 64, 0.0, 0, 0, None, None) == _lib.ERR_INVALID_ARG
    assert b"aligned" in L.dash_last_error()
    n = ctypes.c_size_t()
    assert L.dash_attn_bwd_workspace_bytes(2, 24, 24, 4096, 64, 0, _lib.SHIFT, ctypes.byref(n)) == 0
    assert n.value >= 2 * 24 * 4096 * 64 * 4
    # ragged lengths: room for up to one extra tile of virtual query rows per head
    assert L.dash_attn_bwd_workspace_bytes(1, 2, 1, 100, 64, 1, _lib.AUTO, ctypes.byref(n)) == 0
    assert n.value >= 2 * (128 + 128) * 64 * 4


def test_empty_problems_are_no_ops_without_touching_the_device():
    # No batch entries: every output is empty, nothing is launched, and null
    # pointers are accepted (an empty tensor may have none).
    L = _lib.lib()
    z = [ctypes.c_void_p(0)] * 9
    for mask in (0, 1):
        assert L.dash_attn_bwd_qk(*z, 0, 4, 2, 300, 500, 128, 0.0, mask, _lib.AUTO, None, None) == 0
        assert L.dash_attn_fwd_qk(*z[:5], 0, 4, 2, 300, 500, 128, 0.0, mask, None) == 0
    # No queries: the forward has nothing to write
    assert L.dash_attn_fwd_qk(*z[:5], 2, 4, 2, 0, 500, 128, 0.0, 1, None) == 0
    assert L.dash_attn_bwd_delta(*z[:3], 2, 4, 0, 64, None) == 0
    # No queries and no keys: nothing at all
    assert L.dash_attn_bwd_qk(*z, 2, 4, 2, 0, 0, 64, 0.0, 0, _lib.AUTO, None, None) == 0


# Fastest deterministic schedule per workload, measured on MI355X (every
# schedule of every workload timed on one device): the adaptive rule must
# reproduce these choices.
MEASURED_BEST = [  # (mask, N, D, g, P, schedule)
    (Sch.FULL, 4, 64, 1, 4, _lib.SHIFT),           # B1 H1 S256 D64, tile 64, 4 workgroups
    (Sch.CAUSAL, 16, 128, 1, 256, _lib.SYM_SHIFT),  # B4 H16 S2048 D128
    (Sch.FULL, 32, 64, 1, 256, _lib.SHIFT),         # B2 H24 S4096 D64
    (Sch.FULL, 128, 128, 1, 256, _lib.SHIFT),       # B1 H16 S16384 D128
    (Sch.CAUSAL, 128, 128, 1, 256, _lib.SYM_SHIFT),  # same, causal
    (Sch.CAUSAL, 64, 128, 4, 256, _lib.SYM_SHIFT),  # B1 Hq32 Hkv8 S8192 D128
]


@pytest.mark.parametrize("mask,N,D,g,P,best", MEASURED_BEST)
def test_adaptive_choice_matches_measured_best(mask, N, D, g, P, best):
    from scheduling_persistent_fa_amd.schedule import choose
    assert choose(mask, N, D, g, P) == (best, 0)


def test_adaptive_choice_rules():
    from scheduling_persistent_fa_amd.schedule import choose
    assert choose(Sch.CAUSAL, 5, 128, 1, 256) == (_lib.DESC_Q, 0)       # odd N: no symmetric shift
    assert choose(Sch.FULL, 512, 128, 1, 256) == (_lib.SHIFT, 256)      # gang of 512 capped to the grid
    assert choose(Sch.CAUSAL, 1024, 128, 1, 256) == (_lib.SYM_SHIFT, 256)
    assert choose(Sch.CAUSAL, 512, 128, 1, 256) == (_lib.SYM_SHIFT, 0)  # N/2 = 256 fits exactly
    assert choose(Sch.BAND, 8, 128, 1, 256) == (_lib.DESC_Q, 0)         # band masks: descending walk
    for bad in [(Sch.FULL, 0, 128, 1, 256), (3, 8, 128, 1, 256), (Sch.FULL, 8, 128, 1, 0)]:
        with pytest.raises(_lib.DashError) as ei:
            choose(*bad)
        assert ei.value.status == _lib.ERR_INVALID_ARG


@pytest.mark.parametrize("mask,N,g,groups,P", [(Sch.FULL, 512, 1, 2, 256), (Sch.CAUSAL, 1024, 1, 1, 256),
                                               (Sch.CAUSAL, 7, 4, 3, 16), (Sch.FULL, 24, 2, 5, 8)])
def test_adaptive_choice_builds_valid_schedules(mask, N, g, groups, P):
    from scheduling_persistent_fa_amd.schedule import choose
    kind, cap = choose(mask, N, 128, g, P)
    s = Schedule(mask, kind, N, g, groups, P, max_gang=cap)
    s.validate()
    lists = Sch.build(mask, kind, N, g, groups, P, max_gang=cap)
    assert sum(len(x) for x in lists) == s.num_steps


# ---- rectangular tile grids (Nq query tiles x Nk key/value tiles) ----

RECT_CASES = [  # mask, sched, Nq, Nk, g, groups, P, cap
    (Sch.FULL, Sch.SERIAL, 4, 6, 1, 2, 5, 0), (Sch.FULL, Sch.DESC_Q, 6, 3, 2, 3, 7, 0),
    (Sch.FULL, Sch.SHIFT, 4, 6, 1, 2, 12, 0), (Sch.FULL, Sch.SHIFT, 6, 4, 2, 3, 8, 0),
    (Sch.CAUSAL, Sch.SERIAL, 3, 7, 1, 2, 6, 0), (Sch.CAUSAL, Sch.DESC_Q, 4, 9, 2, 2, 5, 0),
    (Sch.FULL, Sch.SHIFT, 8, 32, 1, 16, 256, 0), (Sch.FULL, Sch.SHIFT, 16, 40, 1, 3, 64, 16),
    (Sch.CAUSAL, Sch.SYM_SHIFT, 4, 10, 2, 3, 8, 0), (Sch.CAUSAL, Sch.SYM_SHIFT, 8, 32, 1, 16, 256, 0),
    (Sch.CAUSAL, Sch.SYM_SHIFT, 6, 11, 1, 2, 5, 2), (Sch.FULL, Sch.SHIFT, 5, 13, 2, 2, 9, 0),
]


@pytest.mark.parametrize("mask,sched,Nq,Nk,g,groups,P,cap", RECT_CASES)
@pytest.mark.parametrize("xcd", [True, False])
def test_rectangular_schedules_match_oracle(mask, sched, Nq, Nk, g, groups, P, cap, xcd):
    lib_s = Schedule(mask, sched, Nq, g, groups, P, xcd_local=xcd, max_gang=cap, Nk=Nk)
    lib_s.validate()
    ora = Sch.build(mask, sched, Nq, g, groups, P, max_gang=cap, Nk=Nk)
    Sch.validate(ora, mask, Nq, g, groups, Nk=Nk)
    _same_schedule(lib_s, ora, sched)


def test_rectangular_rejections():
    for args in [(Sch.CAUSAL, Sch.SERIAL, 5, 4), (Sch.CAUSAL, Sch.SYM_SHIFT, 5, 6), (Sch.CAUSAL, Sch.SHIFT, 4, 6),
                 (Sch.CAUSAL, Sch.SYM_SHIFT, 6, 4)]:
        mask, sched, nq, nk = args
        with pytest.raises(_lib.DashError):
            Schedule(mask, sched, nq, 1, 1, 16, Nk=nk)


def test_adaptive_choice_on_rectangles():
    from scheduling_persistent_fa_amd.schedule import choose
    assert choose(Sch.FULL, 16, 128, 1, 256, Nk=64) == (_lib.SHIFT, 0)
    assert choose(Sch.FULL, 16, 128, 1, 256, Nk=300) == (_lib.SHIFT, 0)     # gang of min(Nq, Nk) = 16
    assert choose(Sch.FULL, 400, 128, 1, 256, Nk=300) == (_lib.SHIFT, 256)  # gang of 300 capped to the grid
    assert choose(Sch.CAUSAL, 16, 128, 1, 256, Nk=64) == (_lib.SYM_SHIFT, 0)
    assert choose(Sch.CAUSAL, 15, 128, 1, 256, Nk=64) == (_lib.DESC_Q, 0)   # odd Nq: no tile pairs
    assert choose(Sch.CAUSAL, 16, 128, 1, 256, Nk=16) == (_lib.SYM_SHIFT, 0)
    with pytest.raises(_lib.DashError):
        choose(Sch.CAUSAL, 16, 128, 1, 256, Nk=8)


# ---- band (sliding-window) masks ----

BAND_CASES = [  # sched, Nq, Nk, band, g, groups, P
    (Sch.SERIAL, 6, 6, (2, 0), 1, 2, 5), (Sch.DESC_Q, 6, 6, (2, 0), 2, 2, 7), (Sch.DESC_Q, 5, 9, (1, 1), 1, 3, 4),
    (Sch.SERIAL, 4, 11, (0, 2), 2, 2, 6), (Sch.DESC_Q, 32, 128, (8, 0), 1, 16, 256),
    (Sch.DESC_Q, 7, 7, (None, 2), 1, 1, 3), (Sch.SERIAL, 7, 10, (3, None), 1, 2, 4),
]


@pytest.mark.parametrize("sched,Nq,Nk,band,g,groups,P", BAND_CASES)
def test_band_schedules_match_oracle(sched, Nq, Nk, band, g, groups, P):
    lib_s = Schedule(0, sched, Nq, g, groups, P, Nk=Nk, band=band)
    lib_s.validate()
    ora = Sch.build(Sch.BAND, sched, Nq, g, groups, P, Nk=Nk, band=band)
    Sch.validate(ora, Sch.BAND, Nq, g, groups, Nk=Nk, band=band)
    _same_schedule(lib_s, ora, sched)
    # atomic default walk on a band: descending
    a = Schedule(0, _lib.ATOMIC, Nq, g, groups, P, Nk=Nk, band=band)
    assert np.array_equal(a.steps, Schedule(0, Sch.DESC_Q, Nq, g, groups, P, Nk=Nk, band=band).steps)


def test_band_schedule_rejections():
    for sched in (Sch.SHIFT, Sch.SYM_SHIFT):
        with pytest.raises(_lib.DashError) as ei:
            Schedule(0, sched, 4, 1, 1, 4, band=(1, 0))
        assert ei.value.status == _lib.ERR_UNSUPPORTED
    for args in [dict(N=5, Nk=4, band=(1, 0)), dict(N=4, Nk=4, band=(-2, 0))]:
        with pytest.raises(_lib.DashError) as ei:
            Schedule(0, Sch.SERIAL, args["N"], 1, 1, 4, Nk=args["Nk"], band=args["band"])
        assert ei.value.status == _lib.ERR_INVALID_ARG


def test_window_argument_errors_need_no_gpu():
    L = _lib.lib()
    vp = ctypes.c_void_p
    good = [vp(4096 * (i + 1)) for i in range(9)]
    # a bounded window side needs Sk >= Sq; extents below -1 are invalid
    assert L.dash_attn_bwd_window(*good, 1, 1, 1, 300, 200, 64, 0.0, 16, 0, _lib.AUTO, None, None) == _lib.ERR_INVALID_ARG
    assert L.dash_attn_bwd_window(*good, 1, 1, 1, 300, 300, 64, 0.0, -2, 0, _lib.AUTO, None, None) == _lib.ERR_INVALID_ARG
    assert L.dash_attn_fwd_window(*good[:5], 1, 1, 1, 300, 200, 64, 0.0, 16, -1, None) == _lib.ERR_INVALID_ARG
    # empty batch: nothing launched
    assert L.dash_attn_bwd_window(*([vp(0)] * 9), 0, 1, 1, 300, 300, 64, 0.0, 16, 0, _lib.AUTO, None, None) == 0


@pytest.mark.parametrize("N,Nk,dl,g,groups,P,xcd", [(12, 12, 4, 1, 1, 10, True), (16, 16, 6, 2, 3, 7, False),
                                                    (8, 20, 4, 1, 2, 5, True), (128, 128, 32, 1, 16, 256, True),
                                                    (32, 64, 8, 2, 3, 50, True), (64, 64, 16, 4, 8, 256, False)])
def test_band_shift_matches_oracle(N, Nk, dl, g, groups, P, xcd):
    lib_s = Schedule(0, Sch.SHIFT, N, g, groups, P, xcd_local=xcd, Nk=Nk, band=(dl, 0))
    lib_s.validate()
    ora = Sch.build(Sch.BAND, Sch.SHIFT, N, g, groups, P, Nk=Nk, band=(dl, 0))
    _same_schedule(lib_s, ora, Sch.SHIFT)


def test_band_choice_rule():
    from scheduling_persistent_fa_amd.schedule import choose_band
    assert choose_band(128, 128, (32, 0), 128, 1, 256) == (_lib.SHIFT, 0)   # sliding window 4096 / 16384
    assert choose_band(128, 128, (31, 0), 128, 1, 256) == (_lib.DESC_Q, 0)  # odd corner triangle
    assert choose_band(8, 20, (4, 0), 128, 1, 256) == (_lib.SHIFT, 0)       # clipped pairs
    assert choose_band(8, 10, (4, 0), 128, 1, 256) == (_lib.DESC_Q, 0)
    assert choose_band(8, 8, (2, 1), 128, 1, 256) == (_lib.DESC_Q, 0)       # two-sided band
    assert choose_band(8, 8, (None, 3), 128, 1, 256) == (_lib.DESC_Q, 0)
    with pytest.raises(_lib.DashError):
        choose_band(8, 4, (2, 0), 128, 1, 256)
    # the rule agrees with where the oracle's band shift applies
    for nq in range(1, 9):
        for nk in range(nq, 14):
            for dl in range(0, 9):
                try:
                    Sch.band_shift_units(nq, nk, dl)
                    ok = dl >= 1
                except Sch.ScheduleError:
                    ok = False
                assert (choose_band(nq, nk, (dl, 0), 64, 1, 16)[0] == _lib.SHIFT) == ok, (nq, nk, dl)


# ---- placement (the library's choice; not part of the schedule) ----

def _member_index(lst, sched, N, g, groups, P, gang):
    """(gang, member) of a gang schedule's member list, from its first chain:
    member p of a SHIFT gang starts with key/value tile p, of a SYM_SHIFT gang
    with tile p (and tile N-1-p); gang k serves groups k, k + n_gangs, ..."""
    head, _, kj = lst[0][:3]
    n_gangs = P // gang
    return (head // g) % n_gangs, kj


@pytest.mark.parametrize("sched,N,g,groups,P", [(Sch.SHIFT, 128, 1, 16, 256), (Sch.SHIFT, 32, 1, 48, 256),
                                                (Sch.SYM_SHIFT, 128, 1, 16, 256), (Sch.SYM_SHIFT, 64, 4, 8, 256),
                                                (Sch.SHIFT, 6, 3, 5, 13)])
def test_gang_placement_is_a_bijection_with_chiplet_runs(sched, N, g, groups, P):
    # Workgroup w runs on chiplet w % 8 (round-robin dispatch).  With
    # xcd_local the library places gang members so that (a) no two member
    # lists share a workgroup, (b) for SHIFT gangs on a grid that is a multiple
    # of 128, runs of 16 consecutive members m = gang * size + p sit on one
    # chiplet, and (c) otherwise members of one gang are congruent modulo the
    # gang count.  Without xcd_local gang k occupies k*size .. k*size+size-1.
    mask = Sch.FULL if sched == Sch.SHIFT else Sch.CAUSAL
    gang = N if sched == Sch.SHIFT else N // 2
    for xcd in (True, False):
        lists = Schedule(mask, sched, N, g, groups, P, xcd_local=xcd).lists()
        seen = {}
        for w, lst in enumerate(lists):
            if not lst:
                continue
            k, p = _member_index(lst, sched, N, g, groups, P, gang)
            assert (k, p) not in seen
            seen[(k, p)] = w
        assert len(seen) == min(groups, P // gang) * gang
        for (k, p), w in seen.items():
            m = k * gang + p
            if not xcd:
                assert w == m
            elif sched == Sch.SHIFT and P % 128 == 0:
                assert w % 8 == (m // 16) % 8
            else:
                assert w == p * (P // gang) + k


def test_schedule_generator_is_clean_under_asan_and_ubsan(tmp_path):
    # The host scheduler built with g++ under AddressSanitizer and
    # UndefinedBehaviorSanitizer (host code only), driven over every mask,
    # schedule, grid up to 7 x 9, gang cap and band, plus the workload shapes.
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "sched_san"
    src = [os.path.join(ROOT, "tests", "sanitize", "schedule_driver.cpp"),
           os.path.join(ROOT, "scheduling_persistent_fa_amd", "csrc", "schedule.cpp")]
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", str(exe), *src], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
