"""Pins for the schedule oracle (CPU only).

Against the pages: the four-tile shift example and the two closed-form times
of [news] §2.3 ("DASH如何革新LLM确定性训练"); the lemma of [summary] §2.2.B
("Resumo Técnico: DASH ...") in its checkable lock-step form.  Against
exhaustive enumeration: coverage, chain contiguity and ordinal permutations
for every small tile count.
"""
import os

import pytest

from oracle import schedules as Sch
from oracle.schedules import CAUSAL, DESC_Q, FULL, SERIAL, SHIFT, SYM_SHIFT, Step

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_shift_example():
    rows = []
    for line in open(os.path.join(GOLDEN, "shift_n4_example.txt")):
        line = line.split("#")[0].strip()
        if line:
            vals = [int(x) for x in line.split()]
            rows.append((vals[0], vals[1:]))
    return rows


def test_shift_four_tiles_matches_the_figure():
    lists = Sch.build(FULL, SHIFT, 4, 1, 1, 4)
    for cu, order in _read_shift_example():
        assert [s.kj for s in lists[cu]] == [cu] * 4
        assert [s.qi for s in lists[cu]] == order
        # dQ tile qi receives its t-th contribution at step t: ordinal = position
        assert [s.ord for s in lists[cu]] == [0, 1, 2, 3]


def _closed_form_serial_lists(n, m, mask, walk_desc=False):
    """Chain kj of every head on workgroup kj (the model behind [news] §2.3's formulas)."""
    lists = [[] for _ in range(n)]
    for h in range(m):
        for kj in range(n):
            qs = list(range(kj if mask == CAUSAL else 0, n))
            if walk_desc:
                qs = qs[::-1]
            for i, qi in enumerate(qs):
                lists[kj].append(Step(h, qi, kj, kj, i == 0, i == len(qs) - 1))
    return lists


@pytest.mark.parametrize("n,m", [(2, 1), (4, 3), (8, 5), (16, 2)])
@pytest.mark.parametrize("c,r", [(1.0, 1.0), (3.0, 0.5), (1.0, 2.0)])
def test_serial_causal_matches_T_causal(n, m, c, r):
    # [news] §2.3: T_causal = m*n*(c+r) + (n-1)*r
    mk, _ = Sch.simulate(_closed_form_serial_lists(n, m, CAUSAL), c, r)
    assert abs(mk - (m * n * (c + r) + (n - 1) * r)) < 1e-9


@pytest.mark.parametrize("n,m", [(4, 8), (8, 16), (16, 12)])
def test_desc_q_causal_close_to_T_reversed(n, m):
    # [news] §2.3: T_reversed ~= m*(n+1)*(c+r)/2 + (n-1)*r, with freed workgroups taking the next heads
    c, r = 1.0, 1.0
    lists = Sch.build(CAUSAL, DESC_Q, n, 1, m, n)
    mk, _ = Sch.simulate(lists, c, r)
    t_rev = m * (n + 1) * (c + r) / 2 + (n - 1) * r
    assert abs(mk - t_rev) <= n * (c + r)
    # and the descending walk beats the serialized baseline's closed form
    assert mk < m * n * (c + r) + (n - 1) * r


@pytest.mark.parametrize("n,m", [(4, 1), (4, 3), (8, 4), (32, 2)])
@pytest.mark.parametrize("c,r", [(1.0, 1.0), (2.0, 0.25)])
def test_shift_full_reaches_the_lower_bound(n, m, c, r):
    # [summary] §2.2.B: shift scheduling is optimal; on one gang every workgroup
    # works m*n steps back to back, so the makespan is exactly m*n*(c+r).
    lists = Sch.build(FULL, SHIFT, n, 1, m, n)
    mk, wait = Sch.simulate(lists, c, r)
    assert abs(mk - m * n * (c + r)) < 1e-9 and wait == 0


@pytest.mark.parametrize("n,m", [(4, 2), (8, 4), (16, 2)])
def test_sym_shift_causal_has_no_waits(n, m):
    # Two heads at a time on n workgroups: each member does n+1 steps per head
    lists = Sch.build(CAUSAL, SYM_SHIFT, n, 1, m, n)
    mk, wait = Sch.simulate(lists, 1.0, 1.0)
    assert wait == 0
    assert abs(mk - m * (n + 1) * 2.0 / 2) < 1e-9


def test_sym_shift_four_tiles_worked_example():
    lists = Sch.build(CAUSAL, SYM_SHIFT, 4, 1, 1, 2)
    assert [(s.kj, s.qi) for s in lists[0]] == [(0, 2), (0, 3), (0, 0), (0, 1), (3, 3)]
    assert [(s.kj, s.qi) for s in lists[1]] == [(1, 3), (1, 2), (1, 1), (2, 3), (2, 2)]
    order = {}
    for lst in lists:
        for s in lst:
            order.setdefault(s.qi, {})[s.ord] = s.kj
    assert [order[q][o] for q in range(4) for o in sorted(order[q])] == [0, 1, 0, 0, 1, 2, 1, 0, 2, 3]


@pytest.mark.parametrize("mask,sched", [(FULL, SERIAL), (FULL, DESC_Q), (FULL, SHIFT),
                                        (CAUSAL, SERIAL), (CAUSAL, DESC_Q), (CAUSAL, SYM_SHIFT)])
def test_exhaustive_small_schedules_are_valid(mask, sched):
    for N in range(1, 11):
        if sched == SYM_SHIFT and N % 2:
            continue
        gang = N if sched == SHIFT else max(1, N // 2)
        for g in (1, 2, 4):
            for groups in (1, 3):
                for P in sorted({gang, gang + 1, 2 * gang + 1, 5}):
                    if sched in (SHIFT, SYM_SHIFT) and P < gang:
                        continue
                    lists = Sch.build(mask, sched, N, g, groups, P)
                    Sch.validate(lists, mask, N, g, groups)
                    if sched in (SERIAL, DESC_Q):
                        assert all(s.ord == s.kj for l in lists for s in l)
                    else:
                        assert Sch.monotone_in_lockstep(lists, g)


def test_serial_and_desc_q_share_ordinals_but_not_walks():
    a = Sch.build(CAUSAL, SERIAL, 6, 1, 2, 4)
    b = Sch.build(CAUSAL, DESC_Q, 6, 1, 2, 4)
    key = lambda lists: sorted((s.head, s.qi, s.kj, s.ord) for l in lists for s in l)
    assert key(a) == key(b)
    assert [s.qi for s in a[0]] != [s.qi for s in b[0]]


def test_validator_rejects_duplicate_ordinal():
    lists = Sch.build(FULL, SHIFT, 4, 1, 1, 4)
    s = lists[1][0]
    lists[1][0] = Step(s.head, s.qi, s.kj, (s.ord + 1) % 4, s.first, s.last)
    with pytest.raises(Sch.ScheduleError):
        Sch.validate(lists, FULL, 4, 1, 1)


def test_validator_rejects_cyclic_wait():
    # Two workgroups, each waiting for the other's later step: a deadlock.
    lists = [
        [Step(0, 0, 0, 1, True, False), Step(0, 1, 0, 0, False, True)],
        [Step(0, 1, 1, 1, True, False), Step(0, 0, 1, 0, False, True)],
    ]
    with pytest.raises(Sch.ScheduleError):
        Sch.simulate(lists, 1.0, 1.0)


def test_validator_rejects_missing_and_split_chains():
    lists = Sch.build(CAUSAL, DESC_Q, 4, 1, 1, 2)
    with pytest.raises(Sch.ScheduleError):
        Sch.validate([l[:-1] for l in lists], CAUSAL, 4, 1, 1)
    moved = [list(l) for l in lists]
    moved[1].append(moved[0].pop(3))  # last step of the four-step chain of tile 0
    with pytest.raises(Sch.ScheduleError):
        Sch.validate(moved, CAUSAL, 4, 1, 1)


def test_rejects_bad_combinations():
    with pytest.raises(Sch.ScheduleError):
        Sch.build(CAUSAL, SHIFT, 4, 1, 1, 4)
    with pytest.raises(Sch.ScheduleError):
        Sch.build(FULL, SYM_SHIFT, 4, 1, 1, 4)
    with pytest.raises(Sch.ScheduleError):
        Sch.build(CAUSAL, SYM_SHIFT, 5, 1, 1, 4)
    with pytest.raises(Sch.ScheduleError):
        Sch.build(FULL, SHIFT, 8, 1, 1, 4)


@pytest.mark.parametrize("mask,sched", [(FULL, SHIFT), (CAUSAL, SYM_SHIFT)])
def test_capped_gangs_are_valid_and_monotone(mask, sched):
    for N in (4, 6, 8, 12, 16):
        units = N if sched == SHIFT else N // 2
        for cap in range(1, units + 1):
            for g in (1, 2):
                lists = Sch.build(mask, sched, N, g, 3, 2 * cap + 1, max_gang=cap)
                Sch.validate(lists, mask, N, g, 3)
                assert Sch.monotone_in_lockstep(lists, g)


@pytest.mark.parametrize("N,cap,m", [(8, 2, 3), (16, 4, 2), (32, 8, 4)])
def test_capped_shift_rounds_keep_the_lower_bound(N, cap, m):
    # one gang of `cap` workgroups takes N/cap rounds per head, each member
    # working back to back: makespan m * N/cap * N * (c + r), no waiting
    lists = Sch.build(FULL, SHIFT, N, 1, m, cap, max_gang=cap)
    mk, wait = Sch.simulate(lists, 1.0, 0.5)
    assert wait == 0 and abs(mk - m * (N // cap) * N * 1.5) < 1e-9


@pytest.mark.parametrize("N,cap,m", [(8, 2, 2), (16, 4, 2), (32, 4, 2)])
def test_capped_sym_shift_rounds_have_no_waits(N, cap, m):
    lists = Sch.build(CAUSAL, SYM_SHIFT, N, 1, m, cap, max_gang=cap)
    mk, wait = Sch.simulate(lists, 1.0, 1.0)
    assert wait == 0 and abs(mk - m * (N // 2 // cap) * (N + 1) * 2.0) < 1e-9


@pytest.mark.parametrize("mask,sched", [(FULL, SERIAL), (FULL, DESC_Q), (FULL, SHIFT), (CAUSAL, SERIAL),
                                        (CAUSAL, DESC_Q), (CAUSAL, SYM_SHIFT)])
def test_rectangular_schedules_valid_exhaustively(mask, sched):
    # Every Nq x Nk grid up to 6 x 8 (causal: Nk >= Nq; symmetric shift: Nq
    # even), two groups, several grid sizes and gang caps.
    for nq in range(1, 7):
        if sched == SYM_SHIFT and nq % 2:
            continue
        for nk in range(1, 9):
            if mask == CAUSAL and nk < nq:
                continue
            gang = min(nq, nk) if sched == SHIFT else (nq // 2 if sched == SYM_SHIFT else 1)
            for P in {gang, nk + 3, 2 * nk}:
                for cap in (0, 1, 2):
                    lists = Sch.build(mask, sched, nq, 2, 2, P, Nk=nk, max_gang=cap)
                    Sch.validate(lists, mask, nq, 2, 2, Nk=nk)


@pytest.mark.parametrize("mask,sched,nq,nk", [(FULL, SHIFT, 5, 13), (FULL, SHIFT, 8, 24), (FULL, SHIFT, 7, 3),
                                              (CAUSAL, SYM_SHIFT, 6, 15), (CAUSAL, SYM_SHIFT, 8, 24),
                                              (CAUSAL, SYM_SHIFT, 8, 8)])
def test_rectangular_gangs_never_meet_on_a_query_tile(mask, sched, nq, nk):
    # Latin property of the uncapped gangs: at every lock-step position the
    # members of a gang sit on distinct query tiles, so in the unit-cost DAG
    # model no step waits for another member (zero total wait).
    P = min(nq, nk) if sched == SHIFT else nq // 2
    lists = Sch.build(mask, sched, nq, 1, 1, P, Nk=nk)
    Sch.validate(lists, mask, nq, 1, 1, Nk=nk)
    longest = max(len(l) for l in lists)
    for t in range(longest):
        at_t = [l[t].qi for l in lists if t < len(l)]
        assert len(at_t) == len(set(at_t)), (t, at_t)
    _, wait = Sch.simulate(lists, 1.0, 0.0)
    assert wait == 0.0
    # every visible (qi, kj) pair once
    pairs = {(s.qi, s.kj) for l in lists for s in l}
    assert len(pairs) == sum(len(l) for l in lists)


@pytest.mark.parametrize("mask,sched,N", [(FULL, SHIFT, 4), (FULL, SHIFT, 8), (CAUSAL, SYM_SHIFT, 4),
                                           (CAUSAL, SYM_SHIFT, 8), (CAUSAL, SYM_SHIFT, 16)])
@pytest.mark.parametrize("g", [2, 4])
def test_gqa_chains_keep_a_dq_tile_g_steps_apart(mask, sched, N, g):
    # A chain takes the g heads of a group at each query tile of its walk, so
    # lock-step position t of the walk becomes positions g*t .. g*t + g - 1:
    # consecutive contributors to one dQ tile stand at least g positions
    # apart, and a release latency of up to g - 1 steps costs no waiting.
    P = N if sched == SHIFT else N // 2
    lists = Sch.build(mask, sched, N, g, 1, P)
    Sch.validate(lists, mask, N, g, 1)
    pos = {}
    for l in lists:
        for t, s in enumerate(l):
            pos.setdefault((s.head, s.qi), []).append((s.ord, t))
    for tile, lst in pos.items():
        ts = [t for _, t in sorted(lst)]
        assert all(b - a >= g for a, b in zip(ts, ts[1:])), (tile, ts)
    _, wait = Sch.simulate(lists, 1.0, float(g - 1))
    assert wait == 0.0


def test_rectangular_shift_contributions_are_one_per_step_when_nk_le_nq():
    # Latin rectangle: with Nk <= Nq no two members of a shift gang touch one
    # dQ tile at the same step, and tile qi gets its t-th contribution at step t.
    nq, nk = 7, 5
    lists = Sch.build(FULL, SHIFT, nq, 1, 1, nk, Nk=nk)
    for lst in lists:
        for t, s in enumerate(lst):
            assert s.qi == (s.kj + t) % nq
    assert Sch.monotone_in_lockstep(lists, 1)


# ---- band (sliding-window) masks on the tile grid ----

BANDS = [(0, 0), (1, 0), (2, 1), (0, 2), (3, None), (None, 1), (None, 0), (None, None)]


@pytest.mark.parametrize("sched", [SERIAL, DESC_Q])
@pytest.mark.parametrize("band", BANDS)
def test_band_schedules_valid_exhaustively(sched, band):
    for nq in range(1, 7):
        for nk in range(nq, 9):
            for P in (1, 3, nk + 2):
                lists = Sch.build(Sch.BAND, sched, nq, 2, 2, P, Nk=nk, band=band)
                Sch.validate(lists, Sch.BAND, nq, 2, 2, Nk=nk, band=band)
                # only visible tile pairs, and every one of them
                pairs = {(s.head, s.qi, s.kj) for l in lists for s in l}
                for h in range(4):
                    for qi in range(nq):
                        for kj in range(nk):
                            d = kj - qi - (nk - nq)
                            vis = (band[0] is None or d >= -band[0]) and (band[1] is None or d <= band[1])
                            assert ((h, qi, kj) in pairs) == vis


def test_band_reduces_to_causal_and_full():
    for sched in (SERIAL, DESC_Q):
        for nq, nk in ((5, 5), (4, 9)):
            assert (Sch.build(Sch.BAND, sched, nq, 2, 3, 7, Nk=nk, band=(None, 0))
                    == Sch.build(CAUSAL, sched, nq, 2, 3, 7, Nk=nk))
            assert (Sch.build(Sch.BAND, sched, nq, 2, 3, 7, Nk=nk, band=(None, None))
                    == Sch.build(FULL, sched, nq, 2, 3, 7, Nk=nk))


@pytest.mark.parametrize("n,dl", [(12, 3), (16, 5), (9, 0), (20, 19)])
def test_descending_walk_is_a_shift_inside_a_sliding_window(n, dl):
    # Sliding-window causal band (dl, 0) with a workgroup per chain: walked in
    # descending query order, chain kj reaches each dQ tile exactly one step
    # after chain kj - 1, so in the unit-cost model (reduction free) the whole
    # head finishes in dl + 1 steps, the length of an unclipped chain; the
    # ascending walk makes every chain wait for its predecessor's whole walk.
    desc = Sch.build(Sch.BAND, DESC_Q, n, 1, 1, n, band=(dl, 0))
    mk, wait = Sch.simulate(desc, 1.0, 0.0)
    assert mk == dl + 1
    ser = Sch.build(Sch.BAND, SERIAL, n, 1, 1, n, band=(dl, 0))
    _, wait_s = Sch.simulate(ser, 1.0, 0.0)
    assert dl == 0 or wait_s > wait


def test_band_rejects_gang_schedules_and_bad_extents():
    for sched in (SHIFT, SYM_SHIFT):  # (shift needs an even band on a square grid)
        with pytest.raises(Sch.ScheduleError):
            Sch.build(Sch.BAND, sched, 4, 1, 1, 4, band=(1, 0))
    with pytest.raises(Sch.ScheduleError):
        Sch.build(Sch.BAND, SERIAL, 4, 1, 1, 4, band=(-1, 0))
    with pytest.raises(Sch.ScheduleError):
        Sch.build(Sch.BAND, SERIAL, 5, 1, 1, 4, Nk=4, band=(1, 0))


@pytest.mark.parametrize("N,Nk,dl,g,groups,P", [(12, 12, 4, 1, 1, 10), (16, 16, 6, 2, 3, 7), (8, 20, 4, 1, 2, 5),
                                                 (10, 13, 3, 1, 3, 12), (32, 32, 8, 1, 4, 64), (9, 9, 8, 1, 2, 5)])
def test_band_shift_schedule(N, Nk, dl, g, groups, P):
    # Shift inside a sliding-window band: valid, every unit dl + 1 steps per
    # head, and with one round of units per group (P = units) no step waits in
    # the unit-cost model with free reductions; pooled rounds keep every
    # workgroup within one unit of the others.
    lists = Sch.build(Sch.BAND, SHIFT, N, g, groups, P, Nk=Nk, band=(dl, 0))
    Sch.validate(lists, Sch.BAND, N, g, groups, Nk=Nk, band=(dl, 0))
    U = len(Sch.band_shift_units(N, Nk, dl))
    L = (dl + 1) * g
    lengths = sorted(len(l) for l in lists)
    assert lengths[-1] - lengths[0] <= L
    assert sum(lengths) == sum(len(l) for l in Sch.build(Sch.BAND, DESC_Q, N, g, groups, P, Nk=Nk, band=(dl, 0)))
    one = Sch.build(Sch.BAND, SHIFT, N, g, 1, U, Nk=Nk, band=(dl, 0))
    mk, wait = Sch.simulate(one, 1.0, 0.0)
    assert wait == 0.0 and mk == L


@pytest.mark.parametrize("N,Nk,dl,g,groups,P", [(128, 128, 32, 1, 16, 256), (16, 16, 4, 1, 4, 12), (16, 16, 4, 2, 4, 12),
                                                 (16, 16, 4, 1, 4, 5), (32, 32, 8, 1, 4, 24), (20, 28, 4, 1, 3, 8)])
def test_band_shift_triangle_units_never_meet_their_group(N, Nk, dl, g, groups, P):
    # The corner-triangle units are dealt after every group's aligned units,
    # so (with fewer workgroups than a group's aligned units) no round holds
    # a triangle unit beside its own group's unclipped units: consecutive
    # contributors to a dQ tile stand at least g lock-step positions apart,
    # and a release latency below g steps costs no waiting.  (Dealt group by
    # group instead, the sliding-window workload shape has 5.5 % of its
    # contributions at the same position as their predecessor.)
    lists = Sch.build(Sch.BAND, Sch.SHIFT, N, g, groups, P, Nk=Nk, band=(dl, 0))
    Sch.validate(lists, Sch.BAND, N, g, groups, Nk=Nk, band=(dl, 0))
    pos = {}
    for l in lists:
        for t, s in enumerate(l):
            pos[(s.head, s.qi, s.ord)] = t
    gaps = [t - pos[(h, q, o - 1)] for (h, q, o), t in pos.items() if o > 0]
    assert min(gaps) >= g
    _, wait = Sch.simulate(lists, 1.0, g - 0.25)
    assert wait == 0.0


def test_band_shift_rejects_unsupported_bands():
    for N, Nk, band in [(8, 8, (3, 0)), (8, 10, (4, 0)), (8, 8, (2, 1)), (4, 4, (4, 0))]:
        with pytest.raises(Sch.ScheduleError):
            Sch.build(Sch.BAND, SHIFT, N, 1, 1, 4, Nk=Nk, band=band)


def test_splitmix64_matches_its_published_sequence():
    # SplitMix64 seeded with 0 (Steele, Lea and Flood, OOPSLA 2014; the
    # reference generator's first three outputs): the state advances by the
    # golden-ratio increment before each output.
    G = 0x9E3779B97F4A7C15
    assert [Sch.splitmix64((i * G) % 2**64) for i in range(3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_jitter_factors_span_half_to_three_halves():
    xs = [Sch.jitter(99, w, i) for w in range(8) for i in range(500)]
    assert min(xs) >= 0.5 and max(xs) < 1.5
    assert 0.95 < sum(xs) / len(xs) < 1.05
    assert Sch.jitter(0, 3, 4) == 1.0


def test_jittered_shift_keeps_its_lockstep_order():
    # Under any timing the shift gang still reduces each dQ tile in ordinal
    # order (the simulation would raise on a deadlock), and the makespan is at
    # least the slowest member's own work.
    lists = Sch.build(FULL, SHIFT, 8, 1, 2, 8)
    for seed in range(1, 50):
        mk, _ = Sch.simulate(lists, 1.0, 0.25, seed)
        own = max(sum(Sch.jitter(seed, w, i) + 0.25 for i in range(len(l))) for w, l in enumerate(lists))
        assert mk >= own - 1e-9
