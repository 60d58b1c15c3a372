"""Pins for the float64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: central
finite differences of the forward, row identities that hold exactly in real
arithmetic, closed forms of degenerate inputs, the causal mask against an
explicit -inf bias, and (when importable) torch's autograd in float64.
"""
import math

import numpy as np
import pytest

from oracle import attention as A
from scheduling_persistent_fa_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, make_inputs


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, do, scale, causal):
    o, _ = A.forward(q, k, v, scale, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,D,g", [(1, 2, 1), (3, 4, 1), (5, 3, 2), (8, 8, 2), (6, 4, 3)])
def test_gradients_match_central_differences(S, D, g, causal):
    q = _rand((1, g, S, D), 1)
    k = _rand((1, 1, S, D), 2)
    v = _rand((1, 1, S, D), 3)
    do = _rand((1, g, S, D), 4)
    scale = 1.0 / math.sqrt(D)
    res = A.backward(q, k, v, do, scale, causal)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            key = {"dq": "q", "dk": "k", "dv": "v"}[name]
            args_p = dict(args); args_p[key] = xp
            args_m = dict(args); args_m[key] = xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, scale, causal)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], do, scale, causal)) / (2 * h)
        err = np.abs(num - res[name]).max() / max(1e-12, np.abs(num).max())
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one_and_ds_rows_sum_to_zero(causal):
    S, D = 48, 16
    q, k, v, do = (_rand((S, D), s) for s in range(4))
    p, dp, ds = A.head_matrices(q, k, v, do, 0.25, causal)
    assert np.abs(p.sum(axis=1) - 1).max() < 1e-12
    # sum_j dS_ij = sum_j P_ij dP_ij - Delta_i sum_j P_ij = 0 in exact arithmetic
    # tolerance scaled by the size of the summed terms P_ij * dP_ij
    term_size = (p * np.abs(dp)).sum(axis=1)
    assert (np.abs(ds.sum(axis=1)) <= 1e-12 * term_size).all()
    if causal:
        assert (p[np.triu_indices(S, 1)] == 0).all()


def test_causal_equals_full_with_minus_inf_bias_bitwise():
    B, Hq, Hkv, S, D = 1, 4, 2, 40, 8
    q, do = _rand((B, Hq, S, D), 5), _rand((B, Hq, S, D), 6)
    k, v = _rand((B, Hkv, S, D), 7), _rand((B, Hkv, S, D), 8)
    bias = np.where(np.arange(S)[None, :] > np.arange(S)[:, None], -np.inf, 0.0)
    c = A.backward(q, k, v, do, 0.3, True, row_block=16)
    f = A.backward(q, k, v, do, 0.3, False, row_block=16, bias=bias)
    for name in ("dq", "dk", "dv", "o", "lse", "delta"):
        assert np.array_equal(c[name], f[name]), name


def test_causal_row_equals_full_attention_over_prefix():
    S, D = 24, 8
    q, k, v, do = (_rand((1, 1, S, D), s) for s in range(10, 14))
    c = A.backward(q, k, v, do, 0.5, True)
    for i in (0, 5, 23):
        o, lse = A.forward(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.5, False)
        assert np.allclose(o[0, 0, 0], c["o"][0, 0, i], rtol=1e-12, atol=1e-12)
        assert abs(lse[0, 0, 0] - c["lse"][0, 0, i]) < 1e-12
        pre = A.backward(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], do[:, :, i:i + 1], 0.5, False)
        assert np.allclose(pre["dq"][0, 0, 0], c["dq"][0, 0, i], rtol=1e-12, atol=1e-12)


def test_single_key_closed_form():
    # S = 1: P = 1, O = V, dV = sum over the group's heads of dO, dQ = dK = 0
    g, D = 3, 5
    q, do = _rand((1, g, 1, D), 20), _rand((1, g, 1, D), 21)
    k, v = _rand((1, 1, 1, D), 22), _rand((1, 1, 1, D), 23)
    r = A.backward(q, k, v, do, 0.7, False)
    assert np.allclose(r["o"], np.repeat(v, g, axis=1), atol=1e-15)
    assert np.allclose(r["dv"][0, 0], do[0].sum(axis=0), atol=1e-14)
    assert np.abs(r["dq"]).max() < 1e-15 and np.abs(r["dk"]).max() < 1e-15
    assert np.allclose(r["lse"][0, :, 0], 0.7 * (q[0, :, 0] @ k[0, 0, 0]), atol=1e-14)


def test_equal_keys_give_uniform_softmax_and_zero_dq():
    S, D = 16, 4
    q, v, do = _rand((1, 1, S, D), 30), _rand((1, 1, S, D), 31), _rand((1, 1, S, D), 32)
    k = np.repeat(_rand((1, 1, 1, D), 33), S, axis=2)
    r = A.backward(q, k, v, do, 0.4, False)
    assert np.allclose(r["o"][0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (S, D)), atol=1e-13)
    assert np.abs(r["dq"]).max() < 1e-13


def test_zero_queries_give_mean_values_and_mean_dv():
    S, D = 12, 6
    q = np.zeros((1, 1, S, D))
    k, v, do = _rand((1, 1, S, D), 40), _rand((1, 1, S, D), 41), _rand((1, 1, S, D), 42)
    r = A.backward(q, k, v, do, 0.4, False)
    assert np.allclose(r["o"][0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (S, D)), atol=1e-14)
    assert np.allclose(r["dv"][0, 0], np.broadcast_to(do[0, 0].mean(axis=0), (S, D)), atol=1e-14)
    assert np.allclose(r["lse"], math.log(S), atol=1e-14)


def test_zero_values_give_zero_dq_dk():
    S, D = 10, 4
    q, k, do = _rand((1, 1, S, D), 50), _rand((1, 1, S, D), 51), _rand((1, 1, S, D), 52)
    v = np.zeros((1, 1, S, D))
    for causal in (False, True):
        r = A.backward(q, k, v, do, 0.5, causal)
        assert np.abs(r["dq"]).max() == 0 and np.abs(r["dk"]).max() == 0
        p, _, _ = A.head_matrices(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.5, causal)
        assert np.allclose(r["dv"][0, 0], p.T @ do[0, 0], atol=1e-14)


def test_sampled_rows_match_full_backward():
    B, Hq, Hkv, S, D = 2, 4, 2, 64, 8
    q, do = _rand((B, Hq, S, D), 60), _rand((B, Hq, S, D), 61)
    k, v = _rand((B, Hkv, S, D), 62), _rand((B, Hkv, S, D), 63)
    for causal in (False, True):
        full = A.backward(q, k, v, do, 0.35, causal, row_block=20)
        rows = [0, 17, 63]
        assert np.allclose(A.dq_rows(q, k, v, do, 1, 3, rows, 0.35, causal), full["dq"][1, 3, rows], atol=1e-12)
        dk, dv = A.dkdv_rows(q, k, v, do, 1, 1, rows, 0.35, causal)
        assert np.allclose(dk, full["dk"][1, 1, rows], atol=1e-12)
        assert np.allclose(dv, full["dv"][1, 1, rows], atol=1e-12)
        lse, delta = A.head_stats(q, k, v, do, 0, 2, 0.35, causal, row_block=7)
        assert np.allclose(lse, full["lse"][0, 2], atol=1e-12)
        assert np.allclose(delta, full["delta"][0, 2], atol=1e-12)


def test_matches_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, S, D = 1, 4, 2, 33, 16
    q, do = _rand((B, Hq, S, D), 70), _rand((B, Hq, S, D), 71)
    k, v = _rand((B, Hkv, S, D), 72), _rand((B, Hkv, S, D), 73)
    scale = 1 / math.sqrt(D)
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        g = Hq // Hkv
        s = scale * tq @ tk.repeat_interleave(g, dim=1).transpose(-1, -2)
        if causal:
            s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv.repeat_interleave(g, dim=1)
        o.backward(torch.tensor(do))
        r = A.backward(q, k, v, do, scale, causal)
        assert np.allclose(r["o"], o.detach().numpy(), atol=1e-13)
        assert np.allclose(r["dq"], tq.grad.numpy(), atol=1e-12)
        assert np.allclose(r["dk"], tk.grad.numpy(), atol=1e-12)
        assert np.allclose(r["dv"], tv.grad.numpy(), atol=1e-12)


def test_planted_sign_error_is_caught_by_finite_differences(monkeypatch):
    # A dropped minus sign in dS must fail the finite-difference pin.
    real = A.backward

    def broken(q, k, v, do, scale, causal, row_block=1024, bias=None):
        r = real(q, k, v, do, scale, causal, row_block, bias)
        r["dk"] = -r["dk"]
        return r

    S, D = 4, 3
    q, k, v, do = (_rand((1, 1, S, D), s) for s in range(80, 84))
    r = broken(q, k, v, do, 0.5, False)
    h = 1e-6
    kp = k.copy(); kp[0, 0, 1, 2] += h
    km = k.copy(); km[0, 0, 1, 2] -= h
    num = (_loss(q, kp, v, do, 0.5, False) - _loss(q, km, v, do, 0.5, False)) / (2 * h)
    assert abs(num - r["dk"][0, 0, 1, 2]) > 1e-4 * max(1.0, abs(num))


def test_float32_addition_is_not_associative():
    # [news] §2.1: the same sum in another order gives other bits.
    a = (np.float32(1e8) + np.float32(1e-6)) - np.float32(1e8)
    b = (np.float32(1e8) - np.float32(1e8)) + np.float32(1e-6)
    assert a == 0.0 and b == np.float32(1e-6)


def test_input_recipe_is_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even mantissa (1.0);
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    r = bf16_bits_to_f32(f32_to_bf16_bits(x))
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.015625 and r[3] == -2.5
    inp = make_inputs(1, 2, 1, 8, 4, seed=0)
    assert inp.q.shape == (1, 2, 8, 4) and inp.k.shape == (1, 1, 8, 4) and inp.q.dtype == np.uint16
    again = make_inputs(1, 2, 1, 8, 4, seed=0)
    assert np.array_equal(inp.do, again.do)


# ---- queries and keys of different lengths (bottom-right causal alignment) ----

def _loss_rect(q, k, v, do, scale, causal):
    o, _ = A.forward(q, k, v, scale, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Sk,D,g", [(2, 5, 3, 1), (4, 7, 4, 2), (5, 5, 2, 1)] + [(6, 3, 3, 1)])
def test_rectangular_gradients_match_central_differences(Sq, Sk, D, g, causal):
    if causal and Sk < Sq:
        pytest.skip("a causal mask needs Sk >= Sq (every query row sees a key)")
    q, do = _rand((1, g, Sq, D), 101), _rand((1, g, Sq, D), 102)
    k, v = _rand((1, 1, Sk, D), 103), _rand((1, 1, Sk, D), 104)
    scale = 1.0 / math.sqrt(D)
    res = A.backward(q, k, v, do, scale, causal)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            key = {"dq": "q", "dk": "k", "dv": "v"}[name]
            ap = {"q": q, "k": k, "v": v}; ap[key] = xp
            am = {"q": q, "k": k, "v": v}; am[key] = xm
            num[idx] = (_loss_rect(ap["q"], ap["k"], ap["v"], do, scale, causal)
                        - _loss_rect(am["q"], am["k"], am["v"], do, scale, causal)) / (2 * h)
        err = np.abs(num - res[name]).max() / max(1e-12, np.abs(num).max())
        assert err < 1e-6, (name, err)


def test_bottom_right_causal_row_equals_full_attention_over_its_keys():
    # Query row i of Sq rows against Sk keys sees keys 0 .. i + Sk - Sq.
    Sq, Sk, D = 10, 26, 8
    q, do = _rand((1, 1, Sq, D), 110), _rand((1, 1, Sq, D), 111)
    k, v = _rand((1, 1, Sk, D), 112), _rand((1, 1, Sk, D), 113)
    c = A.backward(q, k, v, do, 0.4, True)
    for i in (0, 3, Sq - 1):
        n = i + Sk - Sq + 1
        pre = A.backward(q[:, :, i:i + 1], k[:, :, :n], v[:, :, :n], do[:, :, i:i + 1], 0.4, False)
        assert np.allclose(pre["o"][0, 0, 0], c["o"][0, 0, i], rtol=1e-12, atol=1e-12)
        assert abs(pre["lse"][0, 0, 0] - c["lse"][0, 0, i]) < 1e-12
        assert np.allclose(pre["dq"][0, 0, 0], c["dq"][0, 0, i], rtol=1e-12, atol=1e-12)
    # the last query row sees every key: it equals the full-mask row
    f = A.backward(q, k, v, do, 0.4, False)
    assert np.allclose(f["o"][0, 0, -1], c["o"][0, 0, -1], atol=1e-12)


def test_rectangular_sampled_rows_match_full_backward():
    B, Hq, Hkv, Sq, Sk, D = 1, 4, 2, 24, 40, 8
    q, do = _rand((B, Hq, Sq, D), 120), _rand((B, Hq, Sq, D), 121)
    k, v = _rand((B, Hkv, Sk, D), 122), _rand((B, Hkv, Sk, D), 123)
    for causal in (False, True):
        full = A.backward(q, k, v, do, 0.35, causal, row_block=7)
        assert np.allclose(A.dq_rows(q, k, v, do, 0, 3, [0, 11, 23], 0.35, causal), full["dq"][0, 3, [0, 11, 23]],
                           atol=1e-12)
        dk, dv = A.dkdv_rows(q, k, v, do, 0, 1, [0, 17, 39], 0.35, causal)
        assert np.allclose(dk, full["dk"][0, 1, [0, 17, 39]], atol=1e-12)
        assert np.allclose(dv, full["dv"][0, 1, [0, 17, 39]], atol=1e-12)


def test_rectangular_matches_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, Sq, Sk, D = 1, 2, 1, 13, 29, 16
    q, do = _rand((B, Hq, Sq, D), 130), _rand((B, Hq, Sq, D), 131)
    k, v = _rand((B, Hkv, Sk, D), 132), _rand((B, Hkv, Sk, D), 133)
    scale = 1 / math.sqrt(D)
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = scale * tq @ tk.repeat_interleave(Hq // Hkv, dim=1).transpose(-1, -2)
        if causal:  # key j hidden from query i when j > i + Sk - Sq
            s = s.masked_fill(torch.ones(Sq, Sk, dtype=torch.bool).triu(Sk - Sq + 1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv.repeat_interleave(Hq // Hkv, dim=1)
        o.backward(torch.tensor(do))
        r = A.backward(q, k, v, do, scale, causal)
        assert np.allclose(r["o"], o.detach().numpy(), atol=1e-13)
        for got, t in ((r["dq"], tq), (r["dk"], tk), (r["dv"], tv)):
            assert np.allclose(got, t.grad.numpy(), atol=1e-12)


# ---- banded (sliding-window) masks: query i sees keys j with
# ---- -left <= j - (i + Sk - Sq) <= right (None = unbounded) ----

WINDOWS = [((1, 0), False), ((2, 1), False), ((0, 2), False), ((3, None), False), ((None, 1), False), ((2, 5), True)]


@pytest.mark.parametrize("window,causal", WINDOWS)
@pytest.mark.parametrize("Sq,Sk,D,g", [(5, 5, 3, 1), (3, 7, 4, 2)])
def test_window_gradients_match_central_differences(window, causal, Sq, Sk, D, g):
    q, do = _rand((1, g, Sq, D), 201), _rand((1, g, Sq, D), 202)
    k, v = _rand((1, 1, Sk, D), 203), _rand((1, 1, Sk, D), 204)
    scale = 1.0 / math.sqrt(D)
    res = A.backward(q, k, v, do, scale, causal, window=window)

    def loss(q_, k_, v_):
        o, _ = A.forward(q_, k_, v_, scale, causal, window=window)
        return float((o * do).sum())

    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            key = {"dq": "q", "dk": "k", "dv": "v"}[name]
            ap = {"q": q, "k": k, "v": v}; ap[key] = xp
            am = {"q": q, "k": k, "v": v}; am[key] = xm
            num[idx] = (loss(ap["q"], ap["k"], ap["v"]) - loss(am["q"], am["k"], am["v"])) / (2 * h)
        err = np.abs(num - res[name]).max() / max(1e-12, np.abs(num).max())
        assert err < 1e-6, (name, err)


def test_window_row_equals_full_attention_over_its_window():
    # Query row i sees the contiguous key range [i + off - left, i + off + right]
    # clipped to the sequence: evaluate that slice with no mask at all.
    Sq, Sk, D, left, right = 9, 21, 8, 4, 2
    off = Sk - Sq
    q, do = _rand((1, 1, Sq, D), 210), _rand((1, 1, Sq, D), 211)
    k, v = _rand((1, 1, Sk, D), 212), _rand((1, 1, Sk, D), 213)
    c = A.backward(q, k, v, do, 0.3, False, window=(left, right))
    for i in range(Sq):
        lo, hi = max(0, i + off - left), min(Sk, i + off + right + 1)
        sl = A.backward(q[:, :, i:i + 1], k[:, :, lo:hi], v[:, :, lo:hi], do[:, :, i:i + 1], 0.3, False)
        assert np.allclose(sl["o"][0, 0, 0], c["o"][0, 0, i], rtol=1e-12, atol=1e-12)
        assert abs(sl["lse"][0, 0, 0] - c["lse"][0, 0, i]) < 1e-12
        assert np.allclose(sl["dq"][0, 0, 0], c["dq"][0, 0, i], rtol=1e-12, atol=1e-12)


def test_zero_width_window_closed_form():
    # window (0, 0): every query sees only its diagonal key i + off, so
    # O_i = V_{i+off}, LSE_i = S_{i,i+off}, dQ = dK = 0 and dV_{i+off} = dO_i.
    Sq, Sk, D = 6, 10, 5
    off = Sk - Sq
    q, do = _rand((1, 1, Sq, D), 220), _rand((1, 1, Sq, D), 221)
    k, v = _rand((1, 1, Sk, D), 222), _rand((1, 1, Sk, D), 223)
    r = A.backward(q, k, v, do, 0.5, False, window=(0, 0))
    assert np.array_equal(r["o"][0, 0], v[0, 0, off:])
    assert np.allclose(r["lse"][0, 0], 0.5 * (q[0, 0] * k[0, 0, off:]).sum(axis=1), atol=1e-14)
    assert np.abs(r["dq"]).max() < 1e-14 and np.abs(r["dk"]).max() < 1e-14
    assert np.array_equal(r["dv"][0, 0, off:], do[0, 0]) and not r["dv"][0, 0, :off].any()


def test_wide_windows_reduce_to_full_and_causal_bitwise():
    Sq, Sk, D = 7, 12, 4
    q, do = _rand((1, 2, Sq, D), 230), _rand((1, 2, Sq, D), 231)
    k, v = _rand((1, 1, Sk, D), 232), _rand((1, 1, Sk, D), 233)
    full = A.backward(q, k, v, do, 0.4, False)
    causal = A.backward(q, k, v, do, 0.4, True)
    for name in ("dq", "dk", "dv", "o", "lse"):
        assert np.array_equal(A.backward(q, k, v, do, 0.4, False, window=(Sk, Sk))[name], full[name])
        assert np.array_equal(A.backward(q, k, v, do, 0.4, False, window=(Sk, 0))[name], causal[name])
        assert np.array_equal(A.backward(q, k, v, do, 0.4, True, window=(None, 3))[name], causal[name])


def test_keys_outside_every_window_get_zero_gradients():
    Sq, Sk, D, left = 4, 20, 6, 2
    q, do = _rand((1, 1, Sq, D), 240), _rand((1, 1, Sq, D), 241)
    k, v = _rand((1, 1, Sk, D), 242), _rand((1, 1, Sk, D), 243)
    r = A.backward(q, k, v, do, 0.5, True, window=(left, None))
    first_seen = Sk - Sq - left  # the first query's window starts here
    assert not r["dk"][0, 0, :first_seen].any() and not r["dv"][0, 0, :first_seen].any()
    assert np.abs(r["dv"][0, 0, first_seen:]).min() > 0


def test_window_matches_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, Sq, Sk, D = 1, 2, 1, 11, 23, 8
    q, do = _rand((B, Hq, Sq, D), 250), _rand((B, Hq, Sq, D), 251)
    k, v = _rand((B, Hkv, Sk, D), 252), _rand((B, Hkv, Sk, D), 253)
    scale = 1 / math.sqrt(D)
    for left, right in ((3, 0), (5, 2), (0, 4)):
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = scale * tq @ tk.repeat_interleave(Hq // Hkv, dim=1).transpose(-1, -2)
        ones = torch.ones(Sq, Sk, dtype=torch.bool)
        # keep keys j with i + off - left <= j <= i + off + right (off = Sk - Sq)
        keep = ones.triu(Sk - Sq - left) & ones.tril(Sk - Sq + right)
        s = s.masked_fill(~keep, float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv.repeat_interleave(Hq // Hkv, dim=1)
        o.backward(torch.tensor(do))
        r = A.backward(q, k, v, do, scale, False, window=(left, right))
        assert np.allclose(r["o"], o.detach().numpy(), atol=1e-13)
        for got, t in ((r["dq"], tq), (r["dk"], tk), (r["dv"], tv)):
            assert np.allclose(got, t.grad.numpy(), atol=1e-12)
        assert np.allclose(A.dq_rows(q, k, v, do, 0, 1, [0, 5, 10], scale, False, window=(left, right)),
                           r["dq"][0, 1, [0, 5, 10]], atol=1e-12)
        dk, dv = A.dkdv_rows(q, k, v, do, 0, 0, [0, 12, 22], scale, False, window=(left, right))
        assert np.allclose(dk, r["dk"][0, 0, [0, 12, 22]], atol=1e-12)
        assert np.allclose(dv, r["dv"][0, 0, [0, 12, 22]], atol=1e-12)
