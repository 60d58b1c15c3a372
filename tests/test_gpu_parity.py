"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Small shapes span several tiles and are compared element by element; so
are the workload shapes at full size, in the launch configuration the
benchmark times (one workgroup per compute unit).
Tolerance: max|err| / max|ref| <= 2e-2 for dQ, dK, dV and O; LSE and Delta
within 2e-2 * max(1, max|ref|).
"""
import numpy as np
import pytest

from oracle import attention as A
from tests._gpu_helpers import TOL, DeviceProblem, rel_err, say, to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from scheduling_persistent_fa_amd import _lib  # noqa: E402
from scheduling_persistent_fa_amd.attention import (ATOMIC, DESC_Q, SERIAL, SHIFT, SYM_SHIFT, attn_bwd,  # noqa: E402
                                                    attn_fwd, bwd_delta, make_opts)


def _schedules(causal, N):
    det = [SERIAL, DESC_Q] + ([SYM_SHIFT] if causal and N % 2 == 0 else []) + ([] if causal else [SHIFT])
    return det + [ATOMIC]


SMALL = [
    # (name, B, Hq, Hkv, S, D, causal, tile, std, workgroups)
    ("full_b1_h1_s256_d64_shift_4wg", 1, 1, 1, 256, 64, False, 64, 1.0, 4),
    ("full_d128_n4", 1, 2, 2, 512, 128, False, 128, 1.0, 0),
    ("causal_d128_n4", 1, 2, 2, 512, 128, True, 128, 1.0, 0),
    ("gqa4_causal_d128_n4", 2, 8, 2, 512, 128, True, 128, 0.5, 0),
    ("full_d64_n8", 1, 3, 3, 1024, 64, False, 128, 1.0, 0),
    ("causal_d64_t64_n6", 2, 2, 1, 384, 64, True, 64, 1.0, 0),
    ("causal_d128_t64_n5_odd", 1, 2, 2, 320, 128, True, 64, 1.0, 0),
    ("full_d64_t64_n5_few_wg", 1, 2, 1, 320, 64, False, 64, 1.0, 7),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes_match_oracle(case):
    name, B, Hq, Hkv, S, D, causal, tile, std, wgs = case
    say(f"[parity] {name}: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} tile={tile} wgs={wgs}")
    pb = DeviceProblem(B, Hq, Hkv, S, D, causal, std=std)
    ref = A.backward(pb.f64("q"), pb.f64("k"), pb.f64("v"), pb.f64("do"), pb.scale, causal)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, causal)
    torch.cuda.synchronize()
    assert rel_err(to_f64(o), ref["o"]) <= TOL
    assert np.abs(to_f64(lse) - ref["lse"]).max() <= TOL * max(1.0, np.abs(ref["lse"]).max())
    delta = bwd_delta(o, pb.do)
    torch.cuda.synchronize()
    assert np.abs(to_f64(delta) - ref["delta"]).max() <= TOL * max(1.0, np.abs(ref["delta"]).max())
    N = S // tile
    for sched in _schedules(causal, N):
        if sched == SHIFT and wgs and wgs < N:
            continue
        say(f"  schedule {_lib.SCHEDULE_NAMES[sched]}")
        opts = make_opts(num_workgroups=wgs, tile=tile, sync_check=True)
        dq, dk, dv = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched, opts=opts)
        torch.cuda.synchronize()
        for nm, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            e = rel_err(to_f64(got), ref[nm])
            assert e <= TOL, (name, _lib.SCHEDULE_NAMES[sched], nm, e)


FULL_SIZE = [  # name, B, Hq, Hkv, Sq, Sk, D, causal, window, std, schedules
    ("causal_b4_h16_s2048_d128", 4, 16, 16, 2048, 2048, 128, True, None, 1.0, [SERIAL, DESC_Q, SYM_SHIFT, ATOMIC]),
    ("full_b2_h24_s4096_d64", 2, 24, 24, 4096, 4096, 64, False, None, 1.0, [SERIAL, DESC_Q, SHIFT, ATOMIC]),
    ("full_b1_h16_s16384_d128", 1, 16, 16, 16384, 16384, 128, False, None, 1.0, [SERIAL, DESC_Q, SHIFT, ATOMIC]),
    ("causal_b1_h16_s16384_d128", 1, 16, 16, 16384, 16384, 128, True, None, 1.0,
     [SERIAL, DESC_Q, SYM_SHIFT, ATOMIC]),
    ("gqa_causal_b1_hq32_hkv8_s8192_d128", 1, 32, 8, 8192, 8192, 128, True, None, 0.5,
     [SERIAL, DESC_Q, SYM_SHIFT, ATOMIC]),
    # the rectangular and windowed workloads of the benchmark
    ("cross_b1_h16_q4096_k16384_d128", 1, 16, 16, 4096, 16384, 128, False, None, 1.0, [DESC_Q, SHIFT, ATOMIC]),
    ("causal_b1_h16_q4096_k16384_d128", 1, 16, 16, 4096, 16384, 128, True, None, 1.0, [DESC_Q, SYM_SHIFT, ATOMIC]),
    ("sliding_b1_h16_s16384_w4096_d128", 1, 16, 16, 16384, 16384, 128, True, (4095, 0), 1.0,
     [SERIAL, DESC_Q, SHIFT, ATOMIC]),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("case", FULL_SIZE, ids=[c[0] for c in FULL_SIZE])
def test_workload_shapes_every_element(case):
    # Full size, in the benchmark's launch configuration (one workgroup per
    # compute unit), every element of dQ, dK and dV of every schedule against
    # the float64 oracle, and every output finite.
    from tests._oracle_full import full_reference
    name, B, Hq, Hkv, Sq, Sk, D, causal, window, std, scheds = case
    say(f"[parity-full] {name}")
    pb = DeviceProblem(B, Hq, Hkv, Sq, D, causal, std=std, Sk=Sk)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, causal, window=window)
    torch.cuda.synchronize()
    # LSE of the last head against the oracle's row statistics
    q64, k64, v64, do64 = pb.f64("q"), pb.f64("k"), pb.f64("v"), pb.f64("do")
    lse_ref = A.head_stats(q64, k64, v64, do64, B - 1, Hq - 1, pb.scale, causal, window=window)[0]
    assert np.abs(to_f64(lse[B - 1, Hq - 1]) - lse_ref).max() <= TOL * max(1.0, np.abs(lse_ref).max())
    del q64, k64, v64, do64
    outs = {}
    for sched in scheds:  # GPU runs first; the oracle afterwards on the host
        dq, dk, dv = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched, opts=make_opts(sync_check=True),
                              window=window)
        torch.cuda.synchronize()
        for t in (dq, dk, dv):
            assert torch.isfinite(t.float()).all(), (name, _lib.SCHEDULE_NAMES[sched])
        outs[sched] = tuple(t.float().cpu().numpy() for t in (dq, dk, dv))
        del dq, dk, dv
    say("  GPU runs done; oracle over every head")
    ref = full_reference(pb.inp, causal, window=window, label=name)
    for sched, got in outs.items():
        errs = [rel_err(g_, ref[nm]) for g_, nm in zip(got, ("dq", "dk", "dv"))]
        say(f"  {_lib.SCHEDULE_NAMES[sched]}: rel err dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
        assert max(errs) <= TOL, (name, _lib.SCHEDULE_NAMES[sched], errs)


def test_unsupported_shapes_are_rejected_before_launch():
    pb = DeviceProblem(1, 1, 1, 320, 64, True)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, True)
    with pytest.raises(_lib.DashError) as ei:  # tiles are 64 or 128 rows
        attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, True, SERIAL, opts=make_opts(tile=96))
    assert ei.value.status == _lib.ERR_UNSUPPORTED
    with pytest.raises(_lib.DashError) as ei:  # symmetric shift needs an even tile count (ceil(320/128) = 3)
        attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, True, SYM_SHIFT, opts=make_opts(tile=128))
    assert ei.value.status == _lib.ERR_UNSUPPORTED
    with pytest.raises(_lib.DashError) as ei:  # shift needs a full mask
        attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, True, SHIFT, opts=make_opts(tile=64))
    assert ei.value.status == _lib.ERR_UNSUPPORTED
    with pytest.raises(_lib.DashError) as ei:  # symmetric shift needs an even tile count (N = 5)
        attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, True, SYM_SHIFT, opts=make_opts(tile=64))
    assert ei.value.status == _lib.ERR_UNSUPPORTED
    pf = DeviceProblem(1, 1, 1, 256, 64, False)
    of, lf = attn_fwd(pf.q, pf.k, pf.v, False)
    with pytest.raises(_lib.DashError) as ei:  # gang of 4 does not fit 2 workgroups
        attn_bwd(pf.q, pf.k, pf.v, of, pf.do, lf, False, SHIFT, opts=make_opts(tile=64, num_workgroups=2))
    assert ei.value.status == _lib.ERR_UNSUPPORTED


def test_wait_budget_exhaustion_is_loud_and_recovers():
    # A one-cycle wait budget makes the first waiting workgroup give up (forced
    # from the host; every later wait then returns at once, and every
    # workgroup runs to the end of its list).  The failure must show:
    # with sync_check the call returns the timeout; without it the outputs are
    # NaN and the next call (or dash_check_async_error) reports it.  A normal
    # call afterwards is correct again.
    from scheduling_persistent_fa_amd.attention import check_async_error
    pb = DeviceProblem(1, 2, 2, 2048, 128, False)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, False)
    dq, dk, dv = (torch.zeros_like(t) for t in (pb.q, pb.k, pb.v))
    with pytest.raises(_lib.DashError) as ei:
        attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, False, SERIAL, dq=dq, dk=dk, dv=dv,
                 opts=make_opts(spin_timeout_cycles=1, sync_check=True))
    assert ei.value.status == _lib.ERR_TIMEOUT
    for t in (dq, dk, dv):
        assert torch.isnan(t.float()).all()
    check_async_error()  # already reported by the call itself
    # without sync_check: the call returns, the outputs are NaN, the next call fails
    dq, dk, dv = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, False, SERIAL, opts=make_opts(spin_timeout_cycles=1))
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isnan(t.float()).all()
    with pytest.raises(_lib.DashError) as ei:
        attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, False, SERIAL)
    assert ei.value.status == _lib.ERR_TIMEOUT
    # and through dash_check_async_error
    attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, False, DESC_Q, opts=make_opts(spin_timeout_cycles=1))
    with pytest.raises(_lib.DashError) as ei:
        check_async_error()
    assert ei.value.status == _lib.ERR_TIMEOUT
    check_async_error()  # reported once
    ref = A.backward(pb.f64("q"), pb.f64("k"), pb.f64("v"), pb.f64("do"), pb.scale, False)
    dq, dk, dv = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, False, SERIAL, opts=make_opts(sync_check=True))
    torch.cuda.synchronize()
    assert rel_err(to_f64(dq), ref["dq"]) <= TOL and rel_err(to_f64(dk), ref["dk"]) <= TOL
    assert rel_err(to_f64(dv), ref["dv"]) <= TOL


def test_dash_log_reports_each_call():
    # DASH_LOG=1: the library writes one line per step-list build and per
    # backward call to stderr (checked in a child process, so that the
    # setting, read once per process, does not leak into the other tests).
    import os
    import subprocess
    import sys
    code = ("import torch\n"
            "from tests._gpu_helpers import DeviceProblem\n"
            "from scheduling_persistent_fa_amd.attention import attn_fwd, attn_bwd, SYM_SHIFT\n"
            "pb = DeviceProblem(1, 2, 2, 512, 128, True)\n"
            "o, lse = attn_fwd(pb.q, pb.k, pb.v, True)\n"
            "for _ in range(2):\n"
            "    attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, True, SYM_SHIFT)\n"
            "torch.cuda.synchronize()\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, DASH_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[dash]")]
    assert sum(l.startswith("[dash] step lists:") for l in lines) == 1, lines  # built once, then cached
    bwd = [l for l in lines if l.startswith("[dash] bwd ")]
    assert len(bwd) == 2 and "Sq 512 Sk 512 D 128" in bwd[0] and "schedule 3" in bwd[0], lines


def test_concurrent_streams_use_separate_workspaces():
    # Two backward calls in flight at once on two streams, each with the
    # library-managed workspace and 16 workgroups (so both grids are resident
    # together): each must give the bits of the same call run alone.
    B, H, S, D = 1, 4, 2048, 128
    pa = DeviceProblem(B, H, H, S, D, True, seed=1)
    pbb = DeviceProblem(B, H, H, S, D, True, seed=2)
    oa, la = attn_fwd(pa.q, pa.k, pa.v, True)
    ob, lb = attn_fwd(pbb.q, pbb.k, pbb.v, True)
    op = make_opts(num_workgroups=16)
    ref_a = attn_bwd(pa.q, pa.k, pa.v, oa, pa.do, la, True, SERIAL, opts=op)
    ref_b = attn_bwd(pbb.q, pbb.k, pbb.v, ob, pbb.do, lb, True, SERIAL, opts=op)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        say(f"[streams] rep {rep}")
        got_a = attn_bwd(pa.q, pa.k, pa.v, oa, pa.do, la, True, SERIAL, opts=op, stream=s1)
        got_b = attn_bwd(pbb.q, pbb.k, pbb.v, ob, pbb.do, lb, True, SERIAL, opts=op, stream=s2)
        torch.cuda.synchronize()
        for x, y in zip(got_a + got_b, ref_a + ref_b):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_workgroups_record_their_chiplet():
    # Each workgroup reads its chiplet (XCC) id from the hardware register.
    # Dispatch is round-robin over the chiplets, starting where the previous
    # launch's dispatch left off: workgroup w runs on chiplet (c0 + w) mod 8
    # with a launch-dependent c0.  The gang placement relies only on what
    # that implies: workgroups with congruent indices share a chiplet.
    from scheduling_persistent_fa_amd.attention import device_info
    info = device_info()
    P, nx = info["num_cu"], info["num_xcd"]
    say(f"[xcc] {P} compute units, {nx} chiplets")
    assert nx >= 1 and P % nx == 0
    pb = DeviceProblem(1, 4, 4, 2048, 128, False)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, False)
    xcc = torch.full((P,), -1, dtype=torch.int32, device="cuda")
    attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, False, SHIFT, opts=make_opts(xcc=xcc, sync_check=True))
    torch.cuda.synchronize()
    ids = xcc.cpu().numpy()
    assert ((ids >= 0) & (ids < nx)).all()
    assert np.bincount(ids, minlength=nx).tolist() == [P // nx] * nx
    assert (ids == (ids[0] + np.arange(P)) % nx).all(), ids[:32]


@pytest.mark.parametrize("causal", [False, True])
def test_autograd_op_gradients_match_oracle(causal):
    # loss = sum(O * W) makes dO = W; the autograd op's gradients are the
    # library's backward, checked against the float64 oracle.
    from scheduling_persistent_fa_amd.autograd import dash_attention
    B, Hq, Hkv, S, D = 1, 4, 2, 512, 64
    pb = DeviceProblem(B, Hq, Hkv, S, D, causal)
    say(f"[autograd] causal={causal}")
    q, k, v = (t.clone().requires_grad_(True) for t in (pb.q, pb.k, pb.v))
    o = dash_attention(q, k, v, causal=causal)
    (o.float() * pb.do.float()).sum().backward()
    torch.cuda.synchronize()
    ref = A.backward(pb.f64("q"), pb.f64("k"), pb.f64("v"), pb.f64("do"), pb.scale, causal)
    assert rel_err(to_f64(o), ref["o"]) <= TOL
    for t, name in ((q, "dq"), (k, "dk"), (v, "dv")):
        assert rel_err(to_f64(t.grad), ref[name]) <= TOL


RECT = [  # name, B, Hq, Hkv, Sq, Sk, D, causal, tile
    ("full_q256_k768_d64", 1, 2, 1, 256, 768, 64, False, 128),
    ("full_q768_k256_d128", 1, 2, 2, 768, 256, 128, False, 128),
    ("causal_q256_k768_d128", 1, 4, 2, 256, 768, 128, True, 128),
    ("causal_q384_k640_d64_t64", 2, 2, 1, 384, 640, 64, True, 64),
]


@pytest.mark.parametrize("case", RECT, ids=[c[0] for c in RECT])
def test_rectangular_shapes_match_oracle(case):
    from scheduling_persistent_fa_amd.attention import AUTO
    name, B, Hq, Hkv, Sq, Sk, D, causal, tile = case
    say(f"[parity-rect] {name}")
    inp_q = DeviceProblem(B, Hq, Hkv, Sq, D, causal, seed=1)   # Q, dO of Sq rows
    inp_k = DeviceProblem(B, Hq, Hkv, Sk, D, causal, seed=2)   # K, V of Sk rows
    q, do, k, v = inp_q.q, inp_q.do, inp_k.k, inp_k.v
    q64, do64, k64, v64 = inp_q.f64("q"), inp_q.f64("do"), inp_k.f64("k"), inp_k.f64("v")
    scale = 1.0 / np.sqrt(D)
    ref = A.backward(q64, k64, v64, do64, scale, causal)
    o, lse = attn_fwd(q, k, v, causal)
    torch.cuda.synchronize()
    assert rel_err(to_f64(o), ref["o"]) <= TOL
    assert np.abs(to_f64(lse) - ref["lse"]).max() <= TOL * max(1.0, np.abs(ref["lse"]).max())
    scheds = [SERIAL, DESC_Q] + ([SYM_SHIFT] if causal else [SHIFT]) + [ATOMIC, AUTO]
    for sched in scheds:
        say(f"  schedule {_lib.SCHEDULE_NAMES[sched]}")
        opts = make_opts(tile=tile, sync_check=True)
        dq, dk, dv = attn_bwd(q, k, v, o, do, lse, causal, sched, opts=opts)
        torch.cuda.synchronize()
        for nm, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            e = rel_err(to_f64(got), ref[nm])
            assert e <= TOL, (name, _lib.SCHEDULE_NAMES[sched], nm, e)
        if sched != ATOMIC:
            again = attn_bwd(q, k, v, o, do, lse, causal, sched, opts=opts)
            for a_, b_ in zip((dq, dk, dv), again):
                assert torch.equal(a_.view(torch.int16), b_.view(torch.int16))


# ---- ragged lengths (not multiples of the tile) and degenerate sizes ----

RAGGED = [  # name, B, Hq, Hkv, Sq, Sk, D, causal, tile (0 = the library's choice)
    ("full_q200_k333_d64", 1, 2, 1, 200, 333, 64, False, 0),
    ("full_q777_k129_d128_t128", 1, 2, 1, 777, 129, 128, False, 128),
    ("causal_s300_d128_odd_tiles", 1, 2, 2, 300, 300, 128, True, 0),
    ("causal_s333_d64", 2, 2, 1, 333, 333, 64, True, 0),
    ("causal_q250_k700_d64_shift2", 2, 2, 1, 250, 700, 64, True, 0),
    ("causal_q700_k1000_d128_t128_shift44", 1, 4, 2, 700, 1000, 128, True, 128),
    ("full_q1_k1_d128", 1, 1, 1, 1, 1, 128, False, 0),
    ("causal_q1_k1000_d64", 1, 2, 1, 1, 1000, 64, True, 0),
    ("causal_s1_d64", 1, 1, 1, 1, 1, 64, True, 0),
]


def _query_tiles(Sq, Sk, causal, tile):
    """Query tiles of the library's tile grid (causal: aligned with the key tiles)."""
    T = tile or (64 if min(Sq, Sk) < 512 else 128)
    nk = -(-Sk // T)
    return nk - (Sk - Sq) // T if causal else -(-Sq // T)


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_ragged_lengths_match_oracle(case):
    from scheduling_persistent_fa_amd.attention import AUTO
    name, B, Hq, Hkv, Sq, Sk, D, causal, tile = case
    say(f"[parity-ragged] {name}")
    pb = DeviceProblem(B, Hq, Hkv, Sq, D, causal, seed=3, Sk=Sk)
    ref = A.backward(pb.f64("q"), pb.f64("k"), pb.f64("v"), pb.f64("do"), pb.scale, causal)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, causal)
    torch.cuda.synchronize()
    assert rel_err(to_f64(o), ref["o"]) <= TOL
    assert np.abs(to_f64(lse) - ref["lse"]).max() <= TOL * max(1.0, np.abs(ref["lse"]).max())
    nq = _query_tiles(Sq, Sk, causal, tile)
    fast = ([SYM_SHIFT] if nq % 2 == 0 else []) if causal else [SHIFT]
    for sched in [SERIAL, DESC_Q] + fast + [ATOMIC, AUTO]:
        say(f"  schedule {_lib.SCHEDULE_NAMES[sched]}")
        opts = make_opts(tile=tile, sync_check=True)
        # outputs start as NaN so that an element the kernels never write shows
        dq, dk, dv = (torch.full_like(t, float("nan")) for t in (pb.q, pb.k, pb.v))
        attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched, dq=dq, dk=dk, dv=dv, opts=opts)
        torch.cuda.synchronize()
        for nm, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            g64 = to_f64(got)
            if np.abs(ref[nm]).max() == 0.0:
                # One visible key per query (Sk = 1) makes dS exactly zero: dP and
                # Delta are the same dot product, formed twice in fp32 over D terms,
                # so dQ and dK are rounding noise far below 1e-3.
                assert np.isfinite(g64).all() and np.abs(g64).max() <= 1e-3, (name, nm)
                continue
            e = rel_err(g64, ref[nm])
            assert e <= TOL, (name, _lib.SCHEDULE_NAMES[sched], nm, e)
        if sched != ATOMIC:
            again = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched, opts=opts)
            for a_, b_ in zip((dq, dk, dv), again):
                assert torch.equal(a_.view(torch.int16), b_.view(torch.int16))


def test_no_queries_gives_zero_key_gradients():
    # Sq = 0: dQ is empty, and no key or value receives any gradient.
    say("[parity-ragged] no queries")
    k = torch.randn(2, 2, 300, 64, device="cuda").to(torch.bfloat16)
    v = torch.randn(2, 2, 300, 64, device="cuda").to(torch.bfloat16)
    q = torch.empty(2, 4, 0, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = attn_fwd(q, k, v, False)
    assert o.shape == (2, 4, 0, 64) and lse.shape == (2, 4, 0)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    for causal in (False, True):
        dq, dk, dv = attn_bwd(q, k, v, o, torch.empty_like(q), lse, causal, SERIAL, dk=dk, dv=dv)
        torch.cuda.synchronize()
        assert dq.numel() == 0
        assert torch.count_nonzero(dk.float()).item() == 0 and torch.count_nonzero(dv.float()).item() == 0


# ---- banded (sliding-window) masks ----

WINDOWED = [  # name, B, Hq, Hkv, Sq, Sk, D, (left, right), tile (0 = library's choice)
    ("sliding_causal_s300_w50_d64", 1, 2, 1, 300, 300, 64, (50, 0), 0),
    ("sliding_causal_s1000_w300_d128_t128", 1, 4, 2, 1000, 1000, 128, (300, 0), 128),
    ("local_s333_w40_70_d64", 2, 2, 2, 333, 333, 64, (40, 70), 0),
    ("sliding_q250_k700_w100_d64_unseen_keys", 1, 2, 1, 250, 700, 64, (100, 0), 0),
    ("right_only_s200_w5_d128", 1, 2, 1, 200, 200, 128, (None, 5), 0),
    ("zero_width_q64_k200_d64", 1, 1, 1, 64, 200, 64, (0, 0), 0),
    ("sliding_gqa_s1000_w200_d128_t64_band_shift", 1, 4, 2, 1000, 1000, 128, (200, 0), 64),
]


def _band_shift_applies(Sq, Sk, window, tile):
    """Whether the shift schedule covers this window (sliding band, see oracle.schedules)."""
    from oracle import schedules as Sch
    left, right = window
    if left is None or right != 0:
        return False
    T = tile or (64 if min(Sq, Sk) < 512 else 128)
    nk = -(-Sk // T)
    nq = nk - (Sk - Sq) // T
    try:
        Sch.band_shift_units(nq, nk, -(-left // T))
        return True
    except Sch.ScheduleError:
        return False


@pytest.mark.parametrize("case", WINDOWED, ids=[c[0] for c in WINDOWED])
def test_windowed_masks_match_oracle(case):
    from scheduling_persistent_fa_amd.attention import AUTO
    name, B, Hq, Hkv, Sq, Sk, D, window, tile = case
    say(f"[parity-window] {name}")
    pb = DeviceProblem(B, Hq, Hkv, Sq, D, False, seed=5, Sk=Sk)
    ref = A.backward(pb.f64("q"), pb.f64("k"), pb.f64("v"), pb.f64("do"), pb.scale, False, window=window)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, False, window=window)
    torch.cuda.synchronize()
    assert rel_err(to_f64(o), ref["o"]) <= TOL
    assert np.abs(to_f64(lse) - ref["lse"]).max() <= TOL * max(1.0, np.abs(ref["lse"]).max())
    scheds = [SERIAL, DESC_Q] + ([SHIFT] if _band_shift_applies(Sq, Sk, window, tile) else []) + [ATOMIC, AUTO]
    for sched in scheds:
        say(f"  schedule {_lib.SCHEDULE_NAMES[sched]}")
        opts = make_opts(tile=tile, sync_check=True)
        dq, dk, dv = (torch.full_like(t, float("nan")) for t in (pb.q, pb.k, pb.v))
        attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, False, sched, dq=dq, dk=dk, dv=dv, opts=opts, window=window)
        torch.cuda.synchronize()
        for nm, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            g64 = to_f64(got)
            if np.abs(ref[nm]).max() == 0.0:
                # a zero-width window: dS is exactly zero (see the ragged test)
                assert np.isfinite(g64).all() and np.abs(g64).max() <= 1e-3, (name, nm)
                continue
            e = rel_err(g64, ref[nm])
            assert e <= TOL, (name, _lib.SCHEDULE_NAMES[sched], nm, e)
            # keys that no query sees: exactly zero
            unseen = np.abs(ref[nm]).max(axis=-1) == 0.0
            if nm != "dq" and unseen.any():
                assert not g64[unseen].any(), (name, nm)
        if sched != ATOMIC:
            again = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, False, sched, opts=opts, window=window)
            for a_, b_ in zip((dq, dk, dv), again):
                assert torch.equal(a_.view(torch.int16), b_.view(torch.int16))


def test_windows_that_reduce_to_full_or_causal_take_the_gang_schedules():
    # A window wider than the sequence is the full or causal mask, and the
    # shift schedules accept it.
    pb = DeviceProblem(1, 2, 2, 512, 128, True, seed=6)
    ref = A.backward(pb.f64("q"), pb.f64("k"), pb.f64("v"), pb.f64("do"), pb.scale, True)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, False, window=(5000, 0))
    dq, dk, dv = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, False, SYM_SHIFT, window=(5000, 0),
                          opts=make_opts(tile=128, sync_check=True))
    torch.cuda.synchronize()
    for nm, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert rel_err(to_f64(got), ref[nm]) <= TOL
