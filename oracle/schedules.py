"""DASH tile schedules, dQ accumulation ordinals, validator and DAG simulator.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain Python, written
from the pages' description of the method; it shares nothing with the C++
schedule generator, and the tests compare the two element by element.

Vocabulary.  N tiles per sequence (query and key/value alike).  A *step* is
one (query head, query tile qi, key/value tile kj) pair.  A *chain* is every
step of one key/value tile of one key/value group (batch b, kv head hk): the
query tiles of the walk, and at each of them the g query heads of the group
in ascending order.
A chain runs contiguously on one workgroup so that its dK/dV stay in
registers ([summary] §2.1, restrictions).  The *ordinal* of a step is its
position in the accumulation sequence of its dQ tile (head, qi); a fixed
ordinal per step is what makes dQ bitwise reproducible ([summary] §1).

Schedules ([summary] §2.2; [news] §2.3):
* SERIAL    -- the serialized fixed-order baseline: each chain walks qi
               ascending; dQ_qi accumulates key/value tiles in ascending kj.
* DESC_Q    -- same ordinals, but each chain walks qi descending
               ([summary] §2.2.A).
* SHIFT     -- full mask: a gang of N workgroups handles one kv group; the
               workgroup holding key/value tile p visits query tiles
               p, p+1, ..., N-1, 0, ..., p-1 ([summary] §2.2.B; [news] §2.3
               and its four-tile figure).  dQ_qi's t-th contributor is the
               tile visited at step t, so no two workgroups touch one dQ tile
               at the same step.
* SYM_SHIFT -- causal mask: a gang of N/2 workgroups; workgroup p owns tiles
               p and N-1-p and covers a dense rectangle then a folded
               triangle ([summary] §2.2.B, symmetric shift).  The index
               formulas are this implementation's reading of that sentence.
Gang schedules rank each dQ tile's contributors by their lock-step time key
(position in the workgroup's list for that group), ties broken by kj.
``build`` states how each schedule extends to Nq != Nk grids.

Parity status: pinned by the four-tile example of [news] §2.3, the closed-form
times of [news] §2.3, coverage/Latin/monotonicity properties ([summary]
§2.2.B lemma) and exhaustive small-N checks (tests/test_schedule_oracle.py).
"""
from __future__ import annotations

from dataclasses import dataclass

FULL, CAUSAL, BAND = 0, 1, 2
SERIAL, DESC_Q, SHIFT, SYM_SHIFT = 0, 1, 2, 3
NAMES = {SERIAL: "serial", DESC_Q: "desc_q", SHIFT: "shift", SYM_SHIFT: "sym_shift"}


@dataclass(frozen=True)
class Step:
    head: int    # global query head index (b * Hq + hq)
    qi: int
    kj: int
    ord: int
    first: bool  # first step of its chain
    last: bool   # last step of its chain


class ScheduleError(ValueError):
    pass


def tile_band(mask: int, band=None):
    """(dl, dr): key/value tile kj is visible from query tile qi when
    -dl <= kj - qi - (Nk - N) <= dr; None = unbounded.

    Full mask: everything; causal (aligned at the bottom right): (None, 0);
    BAND: the given pair (a sliding window of rows, rounded out to tiles).
    """
    if mask == FULL:
        return None, None
    if mask == CAUSAL:
        return None, 0
    if mask == BAND:
        if band is None:
            raise ScheduleError("a band mask needs its (left, right) tile extents")
        return band
    raise ScheduleError(f"unknown mask {mask}")


def q_range(mask: int, N: int, Nk: int, kj: int, band=None) -> range:
    """Query tiles that see key/value tile kj (possibly empty)."""
    dl, dr = tile_band(mask, band)
    off = Nk - N
    lo = 0 if dr is None else max(0, kj - off - dr)
    hi = N - 1 if dl is None else min(N - 1, kj - off + dl)
    return range(lo, hi + 1)


def k_range(mask: int, N: int, Nk: int, qi: int, band=None) -> range:
    """Key/value tiles seen by query tile qi."""
    dl, dr = tile_band(mask, band)
    off = Nk - N
    lo = 0 if dl is None else max(0, qi + off - dl)
    hi = Nk - 1 if dr is None else min(Nk - 1, qi + off + dr)
    return range(lo, hi + 1)


def kv_walk(mask: int, sched: int, N: int, kj: int, Nk: int | None = None, band=None) -> list[int]:
    """Query tiles visited by key/value tile kj for the serial/descending walks.

    N query tiles, Nk key/value tiles (default N).  Under the causal mask,
    aligned at the bottom right, query tile qi sees key/value tiles
    0 .. qi + Nk - N; under a band mask those in ``k_range``.
    """
    tiles = list(q_range(mask, N, N if Nk is None else Nk, kj, band))
    return tiles[::-1] if sched == DESC_Q else tiles


def _chain(group: int, g: int, kj: int, walk: list[int]) -> list[tuple[int, int, int]]:
    """The steps of one chain: for each query tile of the walk, the g query
    heads of the group in ascending order (query-tile-major)."""
    return [(group * g + u, qi, kj) for qi in walk for u in range(g)]


def _flagged(chain: list[tuple[int, int, int, int]]) -> list[Step]:
    n = len(chain)
    return [Step(h, qi, kj, o, i == 0, i == n - 1) for i, (h, qi, kj, o) in enumerate(chain)]


def build(mask: int, sched: int, N: int, g: int, groups: int, P: int,
          max_gang: int = 0, Nk: int | None = None, band=None) -> list[list[Step]]:
    """Per-workgroup step lists for ``groups`` kv groups of g query heads, N query
    tiles, Nk key/value tiles (default N), P workgroups.

    With Nk != N the schedules generalise as follows (this implementation's
    reading; the pages describe square grids only):
    * serial / descending: the chain of key/value tile kj walks the query
      tiles that see it.
    * shift: a gang of min(N, Nk) members -- more would meet on a query tile
      at the same step -- and the member holding key/value tile i visits
      query tiles (i + t) mod N.  With Nk > N member p holds key/value tiles
      p, p + N, p + 2N, ... one after another, which keeps the gang a Latin
      rectangle: at every lock-step position its members sit on distinct
      query tiles.
    * symmetric shift (causal, N even, Nk >= N): the key/value tiles
      0 .. R-1, R = Nk - N, see every query tile (a dense block); tiles
      R .. Nk-1 with the N query tiles form the square causal triangle.  The
      gang has N/2 members; member p first runs the square's tile pair
      (R + p, R + N-1-p) exactly as in the square schedule, then the dense
      key/value tiles p, p + N/2, p + N, ... each visiting query tiles
      (tile + t) mod N.

    ``max_gang`` > 0 caps a gang schedule's gang below its natural size;
    member p then takes the units (key/value tiles, or tile pairs)
    p, p + gang, p + 2*gang, ... one after another.

    Gang k (k = group mod the number of gangs) puts member p on workgroup
    k * gang + p.  Which compute unit runs which member list does not change
    what any list computes or the order of any dQ tile; the tests compare
    schedules up to that placement.

    A band mask (``mask`` = BAND, ``band`` = (dl, dr) in tiles) takes the
    serial and descending walks over the visible tiles only: a key/value
    tile that no query tile sees has no chain, and a dQ tile's ordinals rank
    its visible key/value tiles in ascending order.  (Walked descending, the
    chains of neighbouring key/value tiles then reach each dQ tile one step
    apart, in ordinal order: the shift structure inside the band.)
    """
    Nk = N if Nk is None else Nk
    if N < 1 or Nk < 1 or g < 1 or groups < 1 or P < 1:
        raise ScheduleError("sizes must be positive")
    if mask in (CAUSAL, BAND) and Nk < N:
        raise ScheduleError("a causal or band mask needs at least as many key/value tiles as query tiles")
    if mask == BAND:
        dl, dr = tile_band(mask, band)
        if (dl is not None and dl < 0) or (dr is not None and dr < 0):
            raise ScheduleError("band extents must not be negative")
    out: list[list[Step]] = [[] for _ in range(P)]
    if sched in (SERIAL, DESC_Q):
        # Chains in (group, kj) order go to the least-loaded workgroup (unit
        # cost per step, ties to the lowest index): a static stand-in for the
        # in-order dispatch of the baseline's one-block-per-KV-tile launch.
        load = [0] * P
        for grp in range(groups):
            for kj in range(Nk):
                walk = kv_walk(mask, sched, N, kj, Nk, band)
                if not walk:
                    continue
                w = min(range(P), key=lambda x: (load[x], x))
                # every dQ tile accumulates its key/value tiles in ascending order:
                # ordinal = kj minus the first key/value tile the query tile sees
                out[w].extend(_flagged([(h, qi, k, k - k_range(mask, N, Nk, qi, band).start)
                                        for (h, qi, k) in _chain(grp, g, kj, walk)]))
                load[w] += g * len(walk)
        return out
    if sched == SHIFT and mask == BAND:
        return _band_shift(N, Nk, band, g, groups, P)
    if sched == SHIFT:
        if mask != FULL:
            raise ScheduleError("shift scheduling needs a full mask")
        units = min(N, Nk)  # natural gang size; the gang holds all Nk key/value tiles
    elif sched == SYM_SHIFT:
        if mask != CAUSAL:
            raise ScheduleError("symmetric shift needs a causal mask")
        if N % 2:
            raise ScheduleError("symmetric shift needs an even tile count")
        units = N // 2
    else:
        raise ScheduleError(f"unknown schedule {sched}")
    gang_size = max_gang if 0 < max_gang < units else units
    n_gangs = P // gang_size
    if n_gangs < 1:
        raise ScheduleError("gang larger than the workgroup count")
    M = N // 2   # symmetric shift: tile pairs of the square causal part
    R = Nk - N   # symmetric shift: dense key/value tiles in front of that square
    for grp in range(groups):
        gang = grp % n_gangs
        members = []  # per member: list of chains, each a list of (head, qi, kj)
        for p in range(gang_size):
            chains = []
            if sched == SHIFT:
                for i in range(p, Nk, gang_size):
                    chains.append(_chain(grp, g, i, [(i + t) % N for t in range(N)]))
            else:
                for i in range(p, M, gang_size):
                    # square part, local tile i: query tiles M..N-1 shifted, then i..M-1;
                    # local tile N-1-i: query tiles N-1 down to N-1-i
                    a_walk = [M + (i + t) % M for t in range(M)] + [i + s for s in range(M - i)]
                    b_walk = [N - 1 - s + M - i for s in range(M - i, M + 1)]
                    chains += [_chain(grp, g, R + i, a_walk), _chain(grp, g, R + N - 1 - i, b_walk)]
                for d in range(p, R, gang_size):
                    chains.append(_chain(grp, g, d, [(d + t) % N for t in range(N)]))
            members.append(chains)
        # ordinal = rank of (time key, kj) among each dQ tile's contributors,
        # where the time key is the step's position in its member's list
        keys: dict[tuple[int, int], list[tuple[int, int]]] = {}
        for chains in members:
            pos = 0
            for ch in chains:
                for (h, qi, kj) in ch:
                    keys.setdefault((h, qi), []).append((pos, kj))
                    pos += 1
        rank = {}
        for (h, qi), lst in keys.items():
            for o, (_, kj) in enumerate(sorted(lst)):
                rank[(h, qi, kj)] = o
        for p, chains in enumerate(members):
            w = gang * gang_size + p
            for ch in chains:
                out[w].extend(_flagged([(h, qi, kj, rank[(h, qi, kj)]) for (h, qi, kj) in ch]))
    return out


def band_shift_units(N: int, Nk: int, dl: int) -> list[list[tuple[int, list[int]]]]:
    """Units of the shift schedule on a sliding-window band (dl, 0), one group.

    Every unit is a list of chains (kj, walk of one head) of dl + 1 steps in
    all, walked in descending query order: the chains of neighbouring
    key/value tiles then visit each query tile one step apart.
    * unclipped key/value tiles (their whole band inside the grid): one chain;
    * with Nk - N >= dl, the tiles clipped at the first query tile (band
      start before query tile 0, l steps) pair with those clipped at the last
      one (dl + 1 - l steps); walked in that order each keeps its lock-step
      slots, so the pair fills one unit;
    * with Nk = N, the tiles clipped at the last query tile form a causal
      triangle of side dl, which the symmetric shift covers with dl/2 units
      of dl + 1 steps.
    Other shapes raise ScheduleError (this implementation's reading: the
    pages give no schedule for bands).
    """
    off = Nk - N
    L = dl + 1
    if dl < 1 or N < L:
        raise ScheduleError("band shift needs 1 <= dl < Nq")
    units = [[(kj, [kj - off + dl - t for t in range(L)])] for kj in range(off, off + N - dl)]
    if off >= dl:
        for ell in range(1, dl + 1):
            kb, kt = off - dl - 1 + ell, off + N - dl - 1 + ell
            units.append([(kb, [ell - 1 - t for t in range(ell)]), (kt, [N - 1 - t for t in range(L - ell)])])
    elif off == 0 and dl % 2 == 0:
        M, base = dl // 2, N - dl
        for p in range(M):
            a = [M + (p + t) % M for t in range(M)] + [p + s for s in range(M - p)]
            b = [dl - 1 - s for s in range(p + 1)]
            units.append([(base + p, [base + q for q in a]), (base + dl - 1 - p, [base + q for q in b])])
    else:
        raise ScheduleError("band shift needs Nk = Nq with an even band, or Nk - Nq >= the band")
    return units


def _band_shift(N: int, Nk: int, band, g: int, groups: int, P: int) -> list[list[Step]]:
    """Shift schedule on a sliding-window band: the units of every group are
    dealt round-robin over the P workgroups ("pooled rounds"), the i-th unit
    dealt going to workgroup i mod P in round i // P, so that the rounds stay
    full even when P is not a multiple of the units per group.  The units
    that keep the shift's lock-step slots (unclipped tiles, first/last
    pairs) of all groups are dealt first, then the corner-triangle units of
    all groups: a triangle unit in the same round as its group's unclipped
    units would reach some dQ tiles at the same lock-step position as one of
    them.  A step's lock-step key is its round times the unit length plus
    its position in the unit; each dQ tile ranks its contributors by
    (key, kj)."""
    dl, dr = band
    if dr != 0 or dl is None:
        raise ScheduleError("band shift needs a sliding-window band (dl, 0)")
    units = band_shift_units(N, Nk, dl)
    U, L = len(units), (dl + 1) * g
    n_al = U - (dl // 2 if Nk - N < dl else 0)  # aligned units lead each group's list
    order = [(grp, u) for grp in range(groups) for u in range(n_al)] + \
            [(grp, u) for grp in range(groups) for u in range(n_al, U)]
    placed = []  # (workgroup, key0, group, unit)
    for i, (grp, u) in enumerate(order):
        placed.append((i % P, (i // P) * L, grp, units[u]))
    keys: dict[tuple[int, int], list[tuple[int, int]]] = {}
    for w, key0, grp, chains in placed:
        pos = key0
        for kj, walk in chains:
            for (h, qi, k) in _chain(grp, g, kj, walk):
                keys.setdefault((h, qi), []).append((pos, k))
                pos += 1
    rank = {}
    for (h, qi), lst in keys.items():
        for o, (_, kj) in enumerate(sorted(lst)):
            rank[(h, qi, kj)] = o
    out: list[list[Step]] = [[] for _ in range(P)]
    for w, key0, grp, chains in sorted(placed, key=lambda x: (x[0], x[1])):
        for kj, walk in chains:
            out[w].extend(_flagged([(h, qi, k, rank[(h, qi, k)]) for (h, qi, k) in _chain(grp, g, kj, walk)]))
    return out


def contributors(mask: int, N: int, qi: int, Nk: int | None = None, band=None) -> int:
    """Number of key/value tiles that add into dQ tile qi (N query tiles, Nk
    key/value tiles, causal and band masks aligned at the bottom right)."""
    Nk = N if Nk is None else Nk
    if mask == BAND:
        return len(k_range(mask, N, Nk, qi, band))
    return qi + Nk - N + 1 if mask == CAUSAL else Nk


def validate(lists: list[list[Step]], mask: int, N: int, g: int, groups: int, Nk: int | None = None,
             band=None) -> None:
    """Raise ScheduleError unless the lists are a complete, contiguous, well-ordered, deadlock-free schedule."""
    Nk = N if Nk is None else Nk
    heads = g * groups
    seen = set()
    for lst in lists:
        for s in lst:
            if not (0 <= s.head < heads and 0 <= s.qi < N and 0 <= s.kj < Nk):
                raise ScheduleError(f"index out of range: {s}")
            if s.kj not in k_range(mask, N, Nk, s.qi, band):
                raise ScheduleError(f"masked tile scheduled: {s}")
            key = (s.head, s.qi, s.kj)
            if key in seen:
                raise ScheduleError(f"tile pair scheduled twice: {key}")
            seen.add(key)
    expect = sum(contributors(mask, N, qi, Nk, band) for qi in range(N)) * heads
    if len(seen) != expect:
        raise ScheduleError(f"coverage {len(seen)} != {expect}")
    # chain contiguity: each (group, kj) appears as exactly one run, flagged first..last
    chain_owner = {}
    for w, lst in enumerate(lists):
        run = None
        for i, s in enumerate(lst):
            ck = (s.head // g, s.kj)
            if s.first:
                if run is not None:
                    raise ScheduleError(f"chain {run} not closed before {s}")
                if ck in chain_owner:
                    raise ScheduleError(f"chain {ck} split")
                chain_owner[ck] = w
                run = ck
            if i == 0 and not s.first:
                raise ScheduleError("list does not start a chain")
            if (s.head // g, s.kj) != run:
                raise ScheduleError(f"chain {run} interrupted by {s}")
            if s.last:
                run = None
        if lst and not lst[-1].last:
            raise ScheduleError("list ends inside a chain")
    if len(chain_owner) != groups * sum(1 for kj in range(Nk) if len(q_range(mask, N, Nk, kj, band))):
        raise ScheduleError("chain count mismatch")
    # ordinals: a permutation of 0..count-1 per dQ tile
    ords: dict[tuple[int, int], list[int]] = {}
    for lst in lists:
        for s in lst:
            ords.setdefault((s.head, s.qi), []).append(s.ord)
    for (h, qi), o in ords.items():
        if sorted(o) != list(range(contributors(mask, N, qi, Nk, band))):
            raise ScheduleError(f"ordinals of dQ tile {(h, qi)} are {sorted(o)}")
    simulate(lists, 1.0, 1.0)  # raises on deadlock


_MASK64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """SplitMix64's output function (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014) applied to x advanced by
    one golden-ratio increment."""
    z = (x + 0x9E3779B97F4A7C15) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def jitter(seed: int, w: int, i: int) -> float:
    """Cost factor in [0.5, 1.5) of step i of workgroup w: a counter-based
    draw, seed ^ (w << 32 | i) through SplitMix64 (1.0 when seed is 0)."""
    if seed == 0:
        return 1.0
    x = (seed ^ ((w << 32) | i)) & _MASK64
    return 0.5 + (splitmix64(x) >> 11) * 2.0 ** -53


def simulate(lists: list[list[Step]], c: float, r: float, jitter_seed: int = 0):
    """Unit-cost DAG model of [news] §2.2 / [summary] §2.1.

    Every step costs c of compute and then r of reduction into its dQ tile;
    the reduction may start only after the tile's previous ordinal finished
    its own.  A workgroup runs its list in order and idles while waiting.
    With a non-zero ``jitter_seed`` step i of workgroup w costs
    c * jitter(seed, w, i) of compute instead (timing noise; the order a
    schedule fixes must not deadlock under any of it).
    Returns (makespan, total wait).  Raises ScheduleError on deadlock.
    """
    P = len(lists)
    idx = [0] * P
    t = [0.0] * P
    count: dict[tuple[int, int], int] = {}
    done_at: dict[tuple[int, int], float] = {}
    wait = 0.0
    remaining = sum(len(l) for l in lists)
    while remaining:
        progressed = False
        for w in range(P):
            while idx[w] < len(lists[w]):
                s = lists[w][idx[w]]
                key = (s.head, s.qi)
                if count.get(key, 0) != s.ord:
                    break
                ready = t[w] + c * jitter(jitter_seed, w, idx[w])
                start = max(ready, done_at.get(key, 0.0))
                wait += start - ready
                t[w] = start + r
                done_at[key] = t[w]
                count[key] = s.ord + 1
                idx[w] += 1
                remaining -= 1
                progressed = True
        if not progressed:
            raise ScheduleError("deadlock: no workgroup can make progress")
    return max(t), wait


def monotone_in_lockstep(lists: list[list[Step]], g: int) -> bool:
    """The checkable form of the [summary] §2.2.B lemma for gang schedules:
    along every dQ tile's accumulation sequence the lock-step time key never
    decreases (no zero-weight edge points to a shallower node), and with one
    query head per group it strictly increases (no two workgroups reduce into
    one dQ tile at the same step)."""
    times = {}
    for lst in lists:
        pos, cur = 0, None
        for s in lst:
            grp = s.head // g
            if grp != cur:
                pos, cur = 0, grp
            times[(s.head, s.qi, s.kj)] = pos
            pos += 1
    seq: dict[tuple[int, int], list[tuple[int, int]]] = {}
    for lst in lists:
        for s in lst:
            seq.setdefault((s.head, s.qi), []).append((s.ord, times[(s.head, s.qi, s.kj)]))
    strict = g == 1
    for lst in seq.values():
        lst.sort()
        for (o1, t1), (o2, t2) in zip(lst, lst[1:]):
            if t2 < t1 or (strict and t2 == t1):
                return False
    return True
