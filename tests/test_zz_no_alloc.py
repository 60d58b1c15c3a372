"""The allocation-free backward entry point (dash_attn_bwd_qk_noalloc)
against dash_attn_bwd_qk: same bits, on two calls in a row with the second
smaller, from a static scratch array (no device allocation)."""
import pytest

from tests._gpu_helpers import DeviceProblem, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from scheduling_persistent_fa_amd import _lib  # noqa: E402
from scheduling_persistent_fa_amd.attention import (ATOMIC, DESC_Q, SERIAL, SHIFT, SYM_SHIFT, attn_bwd,  # noqa: E402
                                                    attn_bwd_noalloc, attn_fwd, check_async_error, make_opts)


def _bits_equal(a, b):
    return all(torch.equal(x.view(torch.int16), y.view(torch.int16)) for x, y in zip(a, b))


# (B, Hq, Hkv, S, D, causal, schedule): each pair runs big then small
PAIRS = [
    ((1, 16, 16, 16384, 128, False, SHIFT), (2, 4, 4, 2048, 128, False, SHIFT)),
    ((1, 16, 16, 16384, 128, True, SYM_SHIFT), (1, 8, 2, 1000, 64, True, DESC_Q)),
    ((2, 8, 2, 4096, 128, True, SERIAL), (1, 2, 1, 300, 64, False, SERIAL)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=["full_shift", "causal_sym_gqa", "serial_ragged"])
def test_noalloc_matches_the_allocating_entry_point(pair):
    for (B, Hq, Hkv, S, D, causal, sched) in pair:
        say(f"[noalloc] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} {_lib.SCHEDULE_NAMES[sched]}")
        pb = DeviceProblem(B, Hq, Hkv, S, D, causal, std=0.5 if Hq != Hkv else 1.0)
        o, lse = attn_fwd(pb.q, pb.k, pb.v, causal)
        want = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched, opts=make_opts(sync_check=True))
        got = tuple(torch.full_like(t, float("nan")) for t in want)
        attn_bwd_noalloc(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched, *got, opts=make_opts(sync_check=True))
        torch.cuda.synchronize()
        assert _bits_equal(got, want)
        # a second call of the same shape reuses the step lists already in the scratch
        got2 = tuple(torch.full_like(t, float("nan")) for t in want)
        attn_bwd_noalloc(pb.q, pb.k, pb.v, o, pb.do, lse, causal, sched, *got2)
        check_async_error()
        assert _bits_equal(got2, want)


def test_noalloc_atomic_and_errors():
    pb = DeviceProblem(1, 4, 4, 1024, 128, False)
    o, lse = attn_fwd(pb.q, pb.k, pb.v, False)
    dq, dk, dv = (torch.empty_like(t) for t in (pb.q, pb.k, pb.v))
    attn_bwd_noalloc(pb.q, pb.k, pb.v, o, pb.do, lse, False, ATOMIC, dq, dk, dv, opts=make_opts(sync_check=True))
    want = attn_bwd(pb.q, pb.k, pb.v, o, pb.do, lse, False, SERIAL, opts=make_opts(sync_check=True))
    torch.cuda.synchronize()
    for x, y in zip((dq, dk, dv), want):
        assert (x.float() - y.float()).abs().max().item() <= 2e-2 * y.float().abs().max().item()
    # too large for the scratch: rejected before launch
    big = DeviceProblem(1, 32, 32, 16384, 128, False)
    ob = torch.empty_like(big.q)
    lb = torch.zeros((1, 32, 16384), dtype=torch.float32, device="cuda")
    outs = (torch.empty_like(big.q), torch.empty_like(big.k), torch.empty_like(big.v))
    with pytest.raises(_lib.DashError) as ei:
        attn_bwd_noalloc(big.q, big.k, big.v, ob, big.do, lb, False, SHIFT, *outs)
    assert ei.value.status == _lib.ERR_WORKSPACE
    # a caller workspace is refused
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(_lib.DashError) as ei:
        attn_bwd_noalloc(pb.q, pb.k, pb.v, o, pb.do, lse, False, SERIAL, dq, dk, dv, opts=make_opts(workspace=ws))
    assert ei.value.status == _lib.ERR_INVALID_ARG
    # a forced give-up: NaN outputs, reported once by dash_check_async_error
    attn_bwd_noalloc(pb.q, pb.k, pb.v, o, pb.do, lse, False, SERIAL, dq, dk, dv,
                     opts=make_opts(spin_timeout_cycles=1))
    with pytest.raises(_lib.DashError) as ei:
        check_async_error()
    assert ei.value.status == _lib.ERR_TIMEOUT
    for t in (dq, dk, dv):
        assert torch.isnan(t.float()).all()
    check_async_error()
    attn_bwd_noalloc(pb.q, pb.k, pb.v, o, pb.do, lse, False, SERIAL, dq, dk, dv)
    check_async_error()
    assert _bits_equal((dq, dk, dv), want)
