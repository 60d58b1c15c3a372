"""Torch-facing wrappers of the C ABI (PyTorch supplies device memory and streams).

Every call goes through libdash_attn.so; these functions only allocate
outputs, check shapes and marshal pointers.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import ATOMIC, AUTO, DESC_Q, MASK_CAUSAL, MASK_FULL, SERIAL, SHIFT, SYM_SHIFT  # noqa: F401


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check_bhsd(name, t, shape):
    if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected contiguous bfloat16 CUDA tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()} cuda={t.is_cuda}")


def _window(causal: bool, window):
    """(left, right) for the window entry points, -1 = unbounded; causal forces right = 0."""
    left, right = (None, None) if window is None else window
    if causal:
        right = 0
    return (-1 if left is None else int(left)), (-1 if right is None else int(right))


def attn_fwd(q, k, v, causal: bool, scale: float = 0.0, out=None, lse=None, stream=None, window=None):
    """O [B,Hq,Sq,D] bf16 and LSE [B,Hq,Sq] fp32 from the library's forward kernel.

    K and V are [B,Hkv,Sk,D]; with Sq != Sk the causal mask is aligned at the
    bottom right (query row i sees keys 0 .. i + Sk - Sq).  ``window`` =
    (left, right) restricts row i to keys j with -left <= j - (i + Sk - Sq)
    <= right (None = unbounded side; with causal=True right is 0)."""
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    _check_bhsd("q", q, (B, Hq, Sq, D))
    _check_bhsd("k", k, (B, Hkv, Sk, D))
    _check_bhsd("v", v, (B, Hkv, Sk, D))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if window is None:
        _lib.check(_lib.lib().dash_attn_fwd_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk,
                                               D, float(scale), MASK_CAUSAL if causal else MASK_FULL,
                                               _stream(stream)))
    else:
        wl, wr = _window(causal, window)
        _lib.check(_lib.lib().dash_attn_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq,
                                                   Sk, D, float(scale), wl, wr, _stream(stream)))
    return out, lse


def make_opts(num_workgroups: int = 0, tile: int = 0, atomic_walk: int = -1, xcd_local: bool = True,
              workspace: torch.Tensor | None = None, stall: torch.Tensor | None = None,
              spin_timeout_cycles: int = 0, sync_check: bool = False, events=None,
              max_gang: int = 0, delay_seed: int = 0, xcc: torch.Tensor | None = None) -> _lib.BwdOpts:
    o = _lib.BwdOpts()
    o.struct_size = ctypes.sizeof(_lib.BwdOpts)
    o.num_workgroups = num_workgroups
    o.tile = tile
    o.atomic_walk = atomic_walk
    o.xcd_local = 1 if xcd_local else -1
    if workspace is not None:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel() * workspace.element_size()
    if stall is not None:
        o.stall_cycles_out = stall.data_ptr()
    o.spin_timeout_cycles = spin_timeout_cycles
    o.sync_check = int(sync_check)
    if events is not None:
        o.event_start = events[0].cuda_event
        o.event_stop = events[1].cuda_event
    o.max_gang = max_gang
    o.debug_delay_seed = delay_seed
    if xcc is not None:
        o.xcc_id_out = xcc.data_ptr()
    return o


def attn_bwd(q, k, v, o, do, lse, causal: bool, schedule: int, scale: float = 0.0, dq=None, dk=None, dv=None,
             opts: _lib.BwdOpts | None = None, stream=None, window=None):
    """dQ, dK, dV (bf16) from the library's persistent backward kernel (Sq query
    rows from q, Sk key/value rows from k; ``window`` as in attn_fwd)."""
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    for name, t, shp in (("q", q, (B, Hq, Sq, D)), ("k", k, (B, Hkv, Sk, D)), ("v", v, (B, Hkv, Sk, D)),
                         ("o", o, (B, Hq, Sq, D)), ("do", do, (B, Hq, Sq, D))):
        _check_bhsd(name, t, shp)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq) or not lse.is_contiguous():
        raise ValueError("lse: expected contiguous float32 [B,Hq,Sq]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, shp in (("dq", dq, (B, Hq, Sq, D)), ("dk", dk, (B, Hkv, Sk, D)), ("dv", dv, (B, Hkv, Sk, D))):
        _check_bhsd(name, t, shp)
    op = ctypes.byref(opts) if opts is not None else None
    ptrs = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv))
    if window is None:
        _lib.check(_lib.lib().dash_attn_bwd_qk(*ptrs, B, Hq, Hkv, Sq, Sk, D, float(scale),
                                               MASK_CAUSAL if causal else MASK_FULL, schedule, op, _stream(stream)))
    else:
        wl, wr = _window(causal, window)
        _lib.check(_lib.lib().dash_attn_bwd_window(*ptrs, B, Hq, Hkv, Sq, Sk, D, float(scale), wl, wr, schedule, op,
                                                   _stream(stream)))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, do, lse, causal: bool, schedule: int, dq, dk, dv, scale: float = 0.0,
                     opts: _lib.BwdOpts | None = None, stream=None):
    """dash_attn_bwd_qk_noalloc: the backward pass into caller-allocated dq,
    dk, dv with the library's static scratch (no device allocation)."""
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    for name, t, shp in (("q", q, (B, Hq, Sq, D)), ("k", k, (B, Hkv, Sk, D)), ("v", v, (B, Hkv, Sk, D)),
                         ("o", o, (B, Hq, Sq, D)), ("do", do, (B, Hq, Sq, D)), ("dq", dq, (B, Hq, Sq, D)),
                         ("dk", dk, (B, Hkv, Sk, D)), ("dv", dv, (B, Hkv, Sk, D))):
        _check_bhsd(name, t, shp)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq) or not lse.is_contiguous():
        raise ValueError("lse: expected contiguous float32 [B,Hq,Sq]")
    op = ctypes.byref(opts) if opts is not None else None
    _lib.check(_lib.lib().dash_attn_bwd_qk_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, Sq, Sk, D,
        float(scale), MASK_CAUSAL if causal else MASK_FULL, schedule, op, _stream(stream)))
    return dq, dk, dv


def bwd_delta(o, do, stream=None):
    B, H, S, D = o.shape
    _check_bhsd("o", o, (B, H, S, D))
    _check_bhsd("do", do, (B, H, S, D))
    delta = torch.empty((B, H, S), dtype=torch.float32, device=o.device)
    _lib.check(_lib.lib().dash_attn_bwd_delta(_ptr(o), _ptr(do), _ptr(delta), B, H, S, D, _stream(stream)))
    return delta


def workspace_bytes(B, Hq, Hkv, S, D, mask: int = MASK_FULL, schedule: int = AUTO) -> int:
    n = ctypes.c_size_t()
    _lib.check(_lib.lib().dash_attn_bwd_workspace_bytes(B, Hq, Hkv, S, D, mask, schedule, ctypes.byref(n)))
    return n.value


def check_async_error(stream=None) -> None:
    """Synchronise the stream and raise DashError(ERR_TIMEOUT) if a backward
    call on the device gave up on a dQ semaphore since the last report."""
    _lib.check(_lib.lib().dash_check_async_error(_stream(stream)))


def device_info(device: int = 0):
    cu, xcd, lds, clk = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _lib.check(_lib.lib().dash_device_info(device, ctypes.byref(cu), ctypes.byref(xcd), ctypes.byref(lds),
                                           ctypes.byref(clk)))
    return {"num_cu": cu.value, "num_xcd": xcd.value, "lds_bytes": lds.value, "clock_khz": clk.value}


def bf16_from_bits(bits, device="cuda") -> torch.Tensor:
    """Device bf16 tensor from a numpy uint16 array of bf16 bit patterns."""
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bits_from_bf16(t: torch.Tensor):
    """numpy uint16 bit patterns of a bf16 tensor."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
