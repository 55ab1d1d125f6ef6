"""Kimi Delta Attention (KDA) on AMD Instinct MI355X (gfx950).

Thin Python binding over libkda.so (C ABI in include/kda.h).  The binding
only marshals arguments: it checks dtypes, devices and contiguity, allocates
outputs with torch, and passes raw device pointers and torch's current HIP
stream.  Every step of the computation runs in the library's HIP kernels.

    o, S_T = prefill_chunked(q, k, v, alpha, beta, S0=None, chunk=64)
    o, S   = decode_step(q, k, v, alpha, beta, S)            # in place on S

Layouts (token-major, as the attention projections produce them):
    prefill  q,k [B,T,H,dk]  v [B,T,H,dv]  alpha [B,T,H,dk]  beta [B,T,H]
             S0, S_T [B,H,dk,dv]  o [B,T,H,dv]
    decode   q,k [N,H,dk]    v [N,H,dv]    alpha [N,H,dk]    beta [N,H]
             S [N,H,dk,dv]   o [N,H,dv]
q, k, v, o are bfloat16 or float32 (all the same); alpha, beta and the states
are float32.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import KDAError  # noqa: F401

__all__ = ["prefill_chunked", "decode_step", "prefill_workspace_bytes", "KDAError", "lib"]

_DT = {torch.bfloat16: _lib.KDA_BF16, torch.float32: _lib.KDA_F32}


def lib():
    return _lib.load()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(name, t, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def prefill_workspace_bytes(B, T, H, dk, dv, chunk, dtype=torch.bfloat16) -> int:
    return int(lib().kda_prefill_workspace_bytes(B, T, H, dk, dv, chunk, _DT[dtype]))


def prefill_chunked(q, k, v, alpha, beta, S0=None, chunk=64, out=None, state_out=None,
                    return_state=True):
    """KDA over whole sequences; returns (o, S_T) (S_T None if not requested)."""
    L = lib()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise TypeError(f"q: dtype {q.dtype} not supported")
    dt = q.dtype
    for n, t, d, s in (("q", q, dt, (B, T, H, dk)), ("k", k, dt, (B, T, H, dk)),
                       ("v", v, dt, (B, T, H, dv)), ("alpha", alpha, torch.float32, (B, T, H, dk)),
                       ("beta", beta, torch.float32, (B, T, H))):
        _check(n, t, d, s, dev)
    if S0 is not None:
        _check("S0", S0, torch.float32, (B, H, dk, dv), dev)
    o = torch.empty((B, T, H, dv), dtype=dt, device=dev) if out is None else out
    _check("out", o, dt, (B, T, H, dv), dev)
    S_T = None
    if return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) \
            if state_out is None else state_out
        _check("state_out", S_T, torch.float32, (B, H, dk, dv), dev)
    ws_bytes = int(L.kda_prefill_workspace_bytes(B, T, H, dk, dv, chunk, _DT[dt]))
    if ws_bytes == (1 << 64) - 1:
        raise KDAError(_lib.KDA_ERR_UNSUPPORTED, "kda_prefill_workspace_bytes")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = L.kda_prefill_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0),
                               _ptr(o), _ptr(S_T), B, T, H, dk, dv, chunk, _DT[dt], _ptr(ws),
                               ws_bytes, _stream(dev))
    if st != _lib.KDA_OK:
        raise KDAError(st, "kda_prefill_chunked")
    return o, S_T


def decode_step(q, k, v, alpha, beta, S, out=None, state_out=None):
    """One recurrence step; state_out defaults to S itself (in place)."""
    L = lib()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise TypeError(f"q: dtype {q.dtype} not supported")
    dt = q.dtype
    for n, t, d, s in (("q", q, dt, (N, H, dk)), ("k", k, dt, (N, H, dk)),
                       ("v", v, dt, (N, H, dv)), ("alpha", alpha, torch.float32, (N, H, dk)),
                       ("beta", beta, torch.float32, (N, H)),
                       ("S", S, torch.float32, (N, H, dk, dv))):
        _check(n, t, d, s, dev)
    o = torch.empty((N, H, dv), dtype=dt, device=dev) if out is None else out
    _check("out", o, dt, (N, H, dv), dev)
    S_out = S if state_out is None else state_out
    _check("state_out", S_out, torch.float32, (N, H, dk, dv), dev)
    st = L.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S),
                           _ptr(o), _ptr(S_out), N, H, dk, dv, _DT[dt], _stream(dev))
    if st != _lib.KDA_OK:
        raise KDAError(st, "kda_decode_step")
    return o, S_out
