"""GPU determinism: deterministic schedules give bit-identical dQ/dK/dV over
50 runs on every workload, and under seeded delays injected around the dQ
semaphore waits; independent of the workgroup count where the order does not
depend on it; serial and descending-Q share their dQ accumulation order and
so their dQ bits; the atomic ceiling agrees with them within tolerance."""
import hashlib

import numpy as np
import pytest

from tests._gpu_helpers import TOL, DeviceProblem, rel_err, say, to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from scheduling_persistent_fa_amd import _lib  # noqa: E402
from scheduling_persistent_fa_amd.attention import (ATOMIC, DESC_Q, SERIAL, SHIFT, SYM_SHIFT, attn_bwd,  # noqa: E402
                                                    attn_fwd, make_opts)

RUNS = 50


def _digest(*ts):
    h = hashlib.sha256()
    for t in ts:
        h.update(t.detach().contiguous().view(torch.int16).cpu().numpy().tobytes())
    return h.hexdigest()


CASES = [  # name, B, Hq, Hkv, S, D, causal, std, tile, workgroups, schedules
    ("full_b1_h1_s256_d64_4wg", 1, 1, 1, 256, 64, False, 1.0, 64, 4, [SERIAL, DESC_Q, SHIFT]),
    ("causal_b4_h16_s2048_d128", 4, 16, 16, 2048, 128, True, 1.0, 0, 0, [SERIAL, DESC_Q, SYM_SHIFT]),
    ("full_b2_h24_s4096_d64", 2, 24, 24, 4096, 64, False, 1.0, 0, 0, [SERIAL, DESC_Q, SHIFT]),
    ("full_b1_h16_s16384_d128", 1, 16, 16, 16384, 128, False, 1.0, 0, 0, [SERIAL, DESC_Q, SHIFT]),
    ("causal_b1_h16_s16384_d128", 1, 16, 16, 16384, 128, True, 1.0, 0, 0, [SERIAL, DESC_Q, SYM_SHIFT]),
    ("gqa_causal_b1_hq32_hkv8_s8192_d128", 1, 32, 8, 8192, 128, True, 0.5, 0, 0, [SERIAL, DESC_Q, SYM_SHIFT]),
]


def _same_bits(a, b) -> bool:
    return all(torch.equal(x.view(torch.int16), y.view(torch.int16)) for x, y in zip(a, b))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fifty_runs_bit_identical(case):
    # Every deterministic schedule of every workload, in the benchmark's launch
    # configuration: 50 runs, each compared on the device with the first.
    from scheduling_persistent_fa_amd.attention import check_async_error
    name, B, Hq, Hkv, S, D, causal, std, tile, wgs, scheds = case
    pb = DeviceProblem(B, Hq, Hkv, S, D, causal, std=std)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, causal)
    outs = {}
    for sched in scheds:
        say(f"[determinism] {name} {_lib.SCHEDULE_NAMES[sched]} x{RUNS}")
        op = make_opts(num_workgroups=wgs, tile=tile)
        first = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched, opts=op)
        first = tuple(t.clone() for t in first)
        dq, dk, dv = (torch.empty_like(t) for t in first)
        for run in range(1, RUNS):
            dq.fill_(float("nan"))
            attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched, dq=dq, dk=dk, dv=dv, opts=op)
            assert _same_bits((dq, dk, dv), first), (name, _lib.SCHEDULE_NAMES[sched], run)
        check_async_error()
        for t in first:
            assert torch.isfinite(t.float()).all()
        outs[sched] = first
    if SERIAL in outs and DESC_Q in outs:
        # same ordinals (ascending key/value order) -> same dQ bits
        assert torch.equal(outs[SERIAL][0].view(torch.int16), outs[DESC_Q][0].view(torch.int16))
    # the non-deterministic ceiling agrees with a deterministic schedule within tolerance
    got = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, ATOMIC, opts=make_opts(num_workgroups=wgs, tile=tile))
    base = outs[scheds[0]]
    for g_, ref in zip(got, base):
        assert rel_err(to_f64(g_), to_f64(ref)) <= TOL


DELAY_CASES = [  # name, B, H, S, D, causal, window, schedules
    ("causal_b4_h16_s2048_d128", 4, 16, 2048, 128, True, None, [SERIAL, DESC_Q, SYM_SHIFT]),
    ("full_b2_h8_s2048_d128", 2, 8, 2048, 128, False, None, [SERIAL, DESC_Q, SHIFT]),
    ("sliding_b2_h4_s2048_w512_d128", 2, 4, 2048, 128, True, (511, 0), [SERIAL, DESC_Q, SHIFT]),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", DELAY_CASES, ids=[c[0] for c in DELAY_CASES])
def test_seeded_delays_do_not_change_the_bits(case):
    # Delay injection: a build of the persistent kernel that sleeps a seeded
    # 0..63 x 64 clocks before every semaphore wait and release.  The order of
    # every dQ accumulation is fixed by the schedule, so any timing must give
    # the undelayed bits ([summary] §1: reproducibility from a fixed order).
    name, B, H, S, D, causal, window, scheds = case
    pb = DeviceProblem(B, H, H, S, D, causal, seed=3)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, causal, window=window)
    for sched in scheds:
        ref = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched, opts=make_opts(sync_check=True),
                       window=window)
        ref = tuple(t.clone() for t in ref)
        for seed in (1, 2, 0xBEEF, 0x9E3779B9):
            say(f"[delay] {name} {_lib.SCHEDULE_NAMES[sched]} seed {seed:#x}")
            got = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched,
                           opts=make_opts(delay_seed=seed, sync_check=True), window=window)
            assert _same_bits(got, ref), (name, _lib.SCHEDULE_NAMES[sched], seed)


def test_delay_injection_needs_a_deterministic_schedule():
    pb = DeviceProblem(1, 1, 1, 512, 64, False)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, False)
    with pytest.raises(_lib.DashError) as ei:
        attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, False, ATOMIC, opts=make_opts(delay_seed=5))
    assert ei.value.status == _lib.ERR_INVALID_ARG


@pytest.mark.parametrize("sched,causal,wgs", [(SERIAL, True, [256, 128, 37]), (DESC_Q, False, [256, 100]),
                                              (SYM_SHIFT, True, [256, 16]), (SHIFT, False, [256, 32])])
def test_result_independent_of_workgroup_count(sched, causal, wgs):
    pb = DeviceProblem(2, 4, 4, 2048 if causal else 4096, 128 if causal else 64, causal)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, causal)
    digests = set()
    for p in wgs:
        say(f"[wg-invariance] {_lib.SCHEDULE_NAMES[sched]} P={p}")
        dq, dk, dv = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched,
                              opts=make_opts(num_workgroups=p, sync_check=True))
        digests.add(_digest(dq, dk, dv))
    assert len(digests) == 1


def test_semaphores_count_every_contribution():
    # After the kernel every semaphore word of each 64-row block (one per wave
    # holding dQ tiles: 8 for D=128 and 128-row tiles) equals its contributor count.
    from scheduling_persistent_fa_amd.attention import workspace_bytes
    B, Hq, S, D, T = 1, 2, 1024, 128, 128
    pb = DeviceProblem(B, Hq, Hq, S, D, True)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, True)
    ws = torch.zeros(workspace_bytes(B, Hq, Hq, S, D, 1) // 4, dtype=torch.int32, device="cuda")
    assert ws.data_ptr() % 256 == 0
    attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, True, SYM_SHIFT, opts=make_opts(workspace=ws, sync_check=True))
    torch.cuda.synchronize()
    align = lambda x: (x + 255) // 256 * 256
    rows = B * Hq * S
    sem_off = align(align(rows * D * 4) + rows * 4) // 4  # after the fp32 dQ accumulator and Delta
    sem = ws[sem_off: sem_off + rows // 64 * 8].cpu().numpy().reshape(B * Hq, S // 64, 8)
    expect = np.array([(blk * 64) // T + 1 for blk in range(S // 64)])
    assert (sem == expect[None, :, None]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_capped_gangs_deterministic_and_correct(causal):
    # A gang cap below the natural gang size makes each gang take its
    # key/value tiles in rounds; the result is still fixed-order and correct.
    from oracle import attention as A
    B, H, S, D = 1, 8, 4096, 128
    pb = DeviceProblem(B, H, H, S, D, causal)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, causal)
    sched = SYM_SHIFT if causal else SHIFT
    digests = set()
    for rep in range(3):
        say(f"[capped] causal={causal} max_gang=16 run {rep}")
        dq, dk, dv = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched,
                              opts=make_opts(max_gang=16, sync_check=True))
        digests.add(_digest(dq, dk, dv))
    assert len(digests) == 1
    ref = A.backward(pb.f64("q"), pb.f64("k"), pb.f64("v"), pb.f64("do"), pb.scale, causal)
    for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert rel_err(to_f64(got), ref[name]) <= TOL


@pytest.mark.parametrize("causal,S,wgs", [(False, 2048, 8), (True, 2048, 0), (True, 1920, 0)])
def test_auto_schedule_runs_the_chosen_schedule(causal, S, wgs):
    # AUTO must give the bits of the schedule (and gang cap) the adaptive rule names.
    from oracle import attention as A
    from scheduling_persistent_fa_amd.attention import AUTO, device_info
    from scheduling_persistent_fa_amd.schedule import choose
    B, H, D, T = 1, 2, 128, 128
    pb = DeviceProblem(B, H, H, S, D, causal)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, causal)
    P = wgs or device_info()["num_cu"]
    kind, cap = choose(1 if causal else 0, S // T, D, 1, P)
    say(f"[auto] causal={causal} S={S} P={P} -> {_lib.SCHEDULE_NAMES[kind]} cap {cap}")
    got = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, AUTO,
                   opts=make_opts(num_workgroups=wgs, sync_check=True))
    d_auto = _digest(*got)
    want = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, kind,
                    opts=make_opts(num_workgroups=wgs, max_gang=cap, sync_check=True))
    assert _digest(*want) == d_auto
    ref = A.backward(pb.f64("q"), pb.f64("k"), pb.f64("v"), pb.f64("do"), pb.scale, causal)
    for t, name in zip(got, ("dq", "dk", "dv")):
        assert rel_err(to_f64(t), ref[name]) <= TOL


def test_windowed_schedules_fifty_runs_bit_identical():
    # Sliding window of 512 keys over 2048 tokens (band of 4 tiles of 128):
    # the band shift and the descending walk, 50 runs each; the descending
    # walk is also independent of the workgroup count.
    B, H, S, D, window = 2, 4, 2048, 128, (511, 0)
    pb = DeviceProblem(B, H, H, S, D, True, seed=7)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, True, window=window)
    for sched in (SHIFT, DESC_Q):
        say(f"[determinism] sliding window {_lib.SCHEDULE_NAMES[sched]} x{RUNS}")
        dq, dk, dv = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, True, sched, opts=make_opts(sync_check=True),
                              window=window)
        ref = _digest(dq, dk, dv)
        for _ in range(RUNS - 1):
            attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, True, sched, dq=dq, dk=dk, dv=dv, window=window)
            assert _digest(dq, dk, dv) == ref
    digests = set()
    for p in (256, 64, 37):
        dq, dk, dv = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, True, DESC_Q,
                              opts=make_opts(num_workgroups=p, sync_check=True), window=window)
        digests.add(_digest(dq, dk, dv))
    assert len(digests) == 1
