"""Kimi Delta Attention (KDA) on AMD Instinct MI355X (gfx950).

Thin Python binding over libkda.so (C ABI in include/kda.h).  The binding
only marshals arguments: it checks dtypes, devices and contiguity, allocates
outputs with torch, and passes raw device pointers and torch's current HIP
stream.  Every step of the computation runs in the library's HIP kernels.

    o, S_T = prefill_chunked(q, k, v, alpha, beta, S0=None, chunk=64)
    o, S   = decode_step(q, k, v, alpha, beta, S)            # in place on S

With the input prologue fused into the kernels (raw projections in):

    o, S_T = prefill_chunked_logits(q, k, v, g, b, S0=None, chunk=64, qk_map="l2")
    o, S   = decode_step_logits(q, k, v, g, b, S, qk_map="l2")

where alpha = exp(-softplus(g)) (g has the dtype of q), beta = sigmoid(b)
(b float32), and qk_map is "as_given", "l2" (x / max(|x|, 1e-12)) or
"silu_l2" (the same after SiLU).

Gated DeltaNet (one gate per token and head, a [B,T,H] / [N,H] float32) and
DeltaNet (a=None, gate 1):

    o, S_T = gdn_prefill_chunked(q, k, v, a, beta, S0=None, chunk=64)
    o, S   = gdn_decode_step(q, k, v, a, beta, S)

The adjoint of one decode step (gradients of a loss through it):

    dq, dk, dv, dalpha, dbeta, dS = decode_step_backward(q, k, v, alpha, beta, S, dO, dS_new)

and of a whole prefill (float32 gradients; S0 and dS_T optional):

    dq, dk, dv, dalpha, dbeta, dS0 = prefill_backward(q, k, v, alpha, beta, dO, S0, dS_T)

and from raw projections (the prologue's forward and adjoint as kernels of
their own around the prefill backward):

    dq, dk, dv, dg, db, dS0 = prefill_backward_logits(q, k, v, g, b, dO, S0, dS_T, qk_map)

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

__all__ = ["prefill_chunked", "prefill_chunked_noalloc", "decode_step", "prefill_chunked_logits", "decode_step_logits",
           "gdn_prefill_chunked", "gdn_decode_step", "decode_step_backward",
           "prefill_backward", "prefill_backward_workspace_bytes", "prefill_backward_chunked",
           "prefill_backward_chunked_workspace_bytes", "prologue_forward",
           "prologue_backward", "prefill_backward_logits", "gdn_prefill_backward",
           "gdn_decode_step_backward",
           "prefill_workspace_bytes", "KDAError", "lib"]

_DT = {torch.bfloat16: _lib.KDA_BF16, torch.float32: _lib.KDA_F32}
_QK = {"as_given": _lib.KDA_QK_AS_GIVEN, "l2": _lib.KDA_QK_L2, "silu_l2": _lib.KDA_QK_SILU_L2}


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
                    return_state=True, workspace=None):
    """KDA over whole sequences; returns (o, S_T) (S_T None if not requested).

    workspace: optional uint8 device tensor of at least prefill_workspace_bytes
    bytes, reused instead of a fresh allocation per call."""
    return _prefill(q, k, v, alpha, beta, S0, chunk, out, state_out, return_state, None,
                    workspace)


def prefill_chunked_logits(q, k, v, g, b, S0=None, chunk=64, qk_map="l2", out=None,
                           state_out=None, return_state=True, workspace=None):
    """KDA over whole sequences from raw projections: alpha = exp(-softplus(g)),
    beta = sigmoid(b), q and k mapped by qk_map, all inside the kernels."""
    if qk_map not in _QK:
        raise ValueError(f"qk_map {qk_map!r}: expected one of {sorted(_QK)}")
    return _prefill(q, k, v, g, b, S0, chunk, out, state_out, return_state, _QK[qk_map],
                    workspace)


def gdn_prefill_chunked(q, k, v, a, beta, S0=None, chunk=64, out=None, state_out=None,
                        return_state=True, workspace=None):
    """Gated DeltaNet over whole sequences: one gate per token and head
    (a [B,T,H] float32), or DeltaNet with a=None (gate 1)."""
    return _prefill(q, k, v, a, beta, S0, chunk, out, state_out, return_state, "gdn",
                    workspace)


def prefill_chunked_noalloc(q, k, v, alpha, beta, S0=None, chunk=64, out=None, state_out=None):
    """prefill_chunked through kda_prefill_chunked_noalloc: the library uses its
    own fixed device scratch instead of a workspace, and the C call allocates
    nothing.  Pass `out` and `state_out` to allocate nothing here either.
    Calls overlapping in time on one GPU must not be issued (they share the
    scratch).  Returns (o, S_T)."""
    L = lib()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise TypeError(f"q: dtype {q.dtype} not supported")
    dt = q.dtype
    for n, t, d, sh in (("q", q, dt, (B, T, H, dk)), ("k", k, dt, (B, T, H, dk)),
                        ("v", v, dt, (B, T, H, dv)), ("alpha", alpha, torch.float32, (B, T, H, dk)),
                        ("beta", beta, torch.float32, (B, T, H))):
        _check(n, t, d, sh, dev)
    if S0 is not None:
        _check("S0", S0, torch.float32, (B, H, dk, dv), dev)
    o = torch.empty((B, T, H, dv), dtype=dt, device=dev) if out is None else out
    _check("out", o, dt, (B, T, H, dv), dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) \
        if state_out is None else state_out
    _check("state_out", S_T, torch.float32, (B, H, dk, dv), dev)
    st = L.kda_prefill_chunked_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                       _ptr(S0), _ptr(o), _ptr(S_T), B, T, H, dk, dv, chunk,
                                       _DT[dt], _stream(dev))
    if st != _lib.KDA_OK:
        raise KDAError(st, "kda_prefill_chunked_noalloc")
    return o, S_T


def _workspace(ws, ws_bytes, dev):
    """The caller's workspace tensor (checked), or a fresh one when none is given."""
    if ws is None:
        return torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    if ws.device != dev or not ws.is_contiguous():
        raise ValueError("workspace: must be a contiguous tensor on the inputs' device")
    if ws.numel() * ws.element_size() < ws_bytes:
        raise ValueError(f"workspace: {ws.numel() * ws.element_size()} bytes, "
                         f"{ws_bytes} needed")
    return ws


def _prefill(q, k, v, gate, beta, S0, chunk, out, state_out, return_state, qk, workspace=None):
    """qk: None (per-channel alpha), "gdn" (scalar gate or None), or a QkMap
    code (raw projections with the fused prologue)."""
    L = lib()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise TypeError(f"q: dtype {q.dtype} not supported")
    dt = q.dtype
    checks = [("q", q, dt, (B, T, H, dk)), ("k", k, dt, (B, T, H, dk)),
              ("v", v, dt, (B, T, H, dv)),
              ("b" if isinstance(qk, int) else "beta", beta, torch.float32, (B, T, H))]
    if qk is None:
        checks.append(("alpha", gate, torch.float32, (B, T, H, dk)))
    elif qk == "gdn":
        if gate is not None:
            checks.append(("a", gate, torch.float32, (B, T, H)))
    else:
        checks.append(("g", gate, dt, (B, T, H, dk)))
    for n, t, d, s in checks:
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
    ws = _workspace(workspace, ws_bytes, dev)
    if ws is not None:
        ws_bytes = ws.numel() * ws.element_size()
    if qk is None:
        st = L.kda_prefill_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S0),
                                   _ptr(o), _ptr(S_T), B, T, H, dk, dv, chunk, _DT[dt],
                                   _ptr(ws), ws_bytes, _stream(dev))
        where = "kda_prefill_chunked"
    elif qk == "gdn":
        st = L.kda_gdn_prefill_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                                       _ptr(S0), _ptr(o), _ptr(S_T), B, T, H, dk, dv, chunk,
                                       _DT[dt], _ptr(ws), ws_bytes, _stream(dev))
        where = "kda_gdn_prefill_chunked"
    else:
        st = L.kda_prefill_chunked_logits(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                                          _ptr(S0), _ptr(o), _ptr(S_T), B, T, H, dk, dv, chunk,
                                          _DT[dt], qk, _ptr(ws), ws_bytes, _stream(dev))
        where = "kda_prefill_chunked_logits"
    if st != _lib.KDA_OK:
        raise KDAError(st, where)
    return o, S_T


def decode_step(q, k, v, alpha, beta, S, out=None, state_out=None):
    """One recurrence step; state_out defaults to S itself (in place)."""
    return _decode(q, k, v, alpha, beta, S, out, state_out, None)


def decode_step_logits(q, k, v, g, b, S, qk_map="l2", out=None, state_out=None):
    """One recurrence step from raw projections (see prefill_chunked_logits);
    state_out defaults to S itself (in place)."""
    if qk_map not in _QK:
        raise ValueError(f"qk_map {qk_map!r}: expected one of {sorted(_QK)}")
    return _decode(q, k, v, g, b, S, out, state_out, _QK[qk_map])


def gdn_decode_step(q, k, v, a, beta, S, out=None, state_out=None):
    """One Gated DeltaNet step (a [N,H] float32, or None for DeltaNet);
    state_out defaults to S itself (in place)."""
    return _decode(q, k, v, a, beta, S, out, state_out, "gdn")


def _decode(q, k, v, gate, beta, S, out, state_out, qk):
    L = lib()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise TypeError(f"q: dtype {q.dtype} not supported")
    dt = q.dtype
    checks = [("q", q, dt, (N, H, dk)), ("k", k, dt, (N, H, dk)), ("v", v, dt, (N, H, dv)),
              ("b" if isinstance(qk, int) else "beta", beta, torch.float32, (N, H)),
              ("S", S, torch.float32, (N, H, dk, dv))]
    if qk is None:
        checks.append(("alpha", gate, torch.float32, (N, H, dk)))
    elif qk == "gdn":
        if gate is not None:
            checks.append(("a", gate, torch.float32, (N, H)))
    else:
        checks.append(("g", gate, dt, (N, H, dk)))
    for n, t, d, s in checks:
        _check(n, t, d, s, dev)
    o = torch.empty((N, H, dv), dtype=dt, device=dev) if out is None else out
    _check("out", o, dt, (N, H, dv), dev)
    S_out = S if state_out is None else state_out
    _check("state_out", S_out, torch.float32, (N, H, dk, dv), dev)
    if qk is None:
        st = L.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S),
                               _ptr(o), _ptr(S_out), N, H, dk, dv, _DT[dt], _stream(dev))
        where = "kda_decode_step"
    elif qk == "gdn":
        st = L.kda_gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S),
                                   _ptr(o), _ptr(S_out), N, H, dk, dv, _DT[dt], _stream(dev))
        where = "kda_gdn_decode_step"
    else:
        st = L.kda_decode_step_logits(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                                      _ptr(S), _ptr(o), _ptr(S_out), N, H, dk, dv, _DT[dt], qk,
                                      _stream(dev))
        where = "kda_decode_step_logits"
    if st != _lib.KDA_OK:
        raise KDAError(st, where)
    return o, S_out


def _step_backward(q, k, v, alpha, beta, S, dO, dS_new, in_place, gdn):
    L = lib()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise TypeError(f"q: dtype {q.dtype} not supported")
    dt = q.dtype
    gate_shape = (N, H) if gdn else (N, H, dk)
    for n, t, d, s in (("q", q, dt, (N, H, dk)), ("k", k, dt, (N, H, dk)), ("v", v, dt, (N, H, dv)),
                       ("beta", beta, torch.float32, (N, H)),
                       ("S", S, torch.float32, (N, H, dk, dv)), ("dO", dO, dt, (N, H, dv)),
                       ("dS_new", dS_new, torch.float32, (N, H, dk, dv))):
        _check(n, t, d, s, dev)
    if alpha is not None or not gdn:
        _check("a" if gdn else "alpha", alpha, torch.float32, gate_shape, dev)
    g_q = torch.empty((N, H, dk), dtype=dt, device=dev)
    g_k = torch.empty((N, H, dk), dtype=dt, device=dev)
    g_v = torch.empty((N, H, dv), dtype=dt, device=dev)
    g_a = None if alpha is None else torch.empty(gate_shape, dtype=torch.float32, device=dev)
    g_b = torch.empty((N, H), dtype=torch.float32, device=dev)
    g_S = dS_new if in_place else torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    fn = L.kda_gdn_decode_step_backward if gdn else L.kda_decode_step_backward
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S), _ptr(dO), _ptr(dS_new),
            _ptr(g_q), _ptr(g_k), _ptr(g_v), _ptr(g_a), _ptr(g_b), _ptr(g_S), N, H, dk, dv, _DT[dt],
            _stream(dev))
    if st != _lib.KDA_OK:
        raise KDAError(st, "kda_gdn_decode_step_backward" if gdn else "kda_decode_step_backward")
    return g_q, g_k, g_v, g_a, g_b, g_S


def decode_step_backward(q, k, v, alpha, beta, S, dO, dS_new, in_place=False):
    """Adjoint of decode_step: given dO = dL/do [N,H,dv] (dtype of q) and
    dS_new = dL/dS after the step [N,H,dk,dv] float32, returns (dq, dk, dv,
    dalpha, dbeta, dS) with dS = dL/dS before the step; in_place=True writes
    dS over dS_new."""
    return _step_backward(q, k, v, alpha, beta, S, dO, dS_new, in_place, gdn=False)


def gdn_decode_step_backward(q, k, v, a, beta, S, dO, dS_new, in_place=False):
    """Adjoint of gdn_decode_step (a [N,H] one gate per head, or None for
    DeltaNet): (dq, dk, dv, da, dbeta, dS); da [N,H] is None when a is None."""
    return _step_backward(q, k, v, a, beta, S, dO, dS_new, in_place, gdn=True)


def prefill_backward_workspace_bytes(B, T, H, dk, dv) -> int:
    return int(lib().kda_prefill_backward_workspace_bytes(B, T, H, dk, dv))


def prefill_backward_chunked_workspace_bytes(B, T, H, dk, dv) -> int:
    return int(lib().kda_prefill_backward_chunked_workspace_bytes(B, T, H, dk, dv))


def _prefill_backward(q, k, v, alpha, beta, dO, S0, dS_T, gdn, chunked=False, workspace=None):
    L = lib()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise TypeError(f"q: dtype {q.dtype} not supported")
    dt = q.dtype
    f32 = torch.float32
    gate_shape = (B, T, H) if gdn else (B, T, H, dk)
    for n, t, d, s in (("q", q, dt, (B, T, H, dk)), ("k", k, dt, (B, T, H, dk)),
                       ("v", v, dt, (B, T, H, dv)), ("beta", beta, f32, (B, T, H)),
                       ("dO", dO, dt, (B, T, H, dv))):
        _check(n, t, d, s, dev)
    if alpha is not None or not gdn:
        _check("a" if gdn else "alpha", alpha, f32, gate_shape, dev)
    for n, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None:
            _check(n, t, f32, (B, H, dk, dv), dev)
    g_q = torch.empty((B, T, H, dk), dtype=f32, device=dev)
    g_k = torch.empty((B, T, H, dk), dtype=f32, device=dev)
    g_v = torch.empty((B, T, H, dv), dtype=f32, device=dev)
    g_a = None if alpha is None else torch.empty(gate_shape, dtype=f32, device=dev)
    g_b = torch.empty((B, T, H), dtype=f32, device=dev)
    g_S = torch.empty((B, H, dk, dv), dtype=f32, device=dev)
    wsfn = prefill_backward_chunked_workspace_bytes if chunked else prefill_backward_workspace_bytes
    nws = wsfn(B, T, H, dk, dv)
    if nws == (1 << 64) - 1:                      # (size_t)-1: sizes not supported
        raise KDAError(_lib.KDA_ERR_UNSUPPORTED, wsfn.__name__)
    ws = _workspace(workspace, nws, dev)
    name = ("kda_prefill_backward_chunked" if chunked else
            "kda_gdn_prefill_backward" if gdn else "kda_prefill_backward")
    st = getattr(L, name)(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(dO),
                          _ptr(dS_T), _ptr(g_q), _ptr(g_k), _ptr(g_v), _ptr(g_a), _ptr(g_b),
                          _ptr(g_S), B, T, H, dk, dv, _DT[dt], _ptr(ws), nws, _stream(dev))
    if st != _lib.KDA_OK:
        raise KDAError(st, name)
    return g_q, g_k, g_v, g_a, g_b, g_S


def prefill_backward(q, k, v, alpha, beta, dO, S0=None, dS_T=None):
    """Gradients of a loss L through prefill_chunked: given dO = dL/do
    [B,T,H,dv] (dtype of q) and, optionally, dS_T = dL/dS_T [B,H,dk,dv]
    float32, returns (dq, dk, dv, dalpha, dbeta, dS0), all float32, shaped
    like q, k, v, alpha, beta and the state."""
    return _prefill_backward(q, k, v, alpha, beta, dO, S0, dS_T, gdn=False)


def prefill_backward_chunked(q, k, v, alpha, beta, dO, S0=None, dS_T=None, workspace=None):
    """prefill_backward in chunk form on the matrix cores (bf16, dk = dv =
    128): the same gradients, within the bf16 bar instead of fp32 rounding,
    deterministic, with no float atomics.  `workspace`: an optional uint8
    device tensor of at least prefill_backward_chunked_workspace_bytes."""
    return _prefill_backward(q, k, v, alpha, beta, dO, S0, dS_T, gdn=False, chunked=True,
                             workspace=workspace)


def gdn_prefill_backward(q, k, v, a, beta, dO, S0=None, dS_T=None):
    """Gradients through gdn_prefill_chunked (a [B,T,H] one gate per token
    and head, or None for DeltaNet): (dq, dk, dv, da, dbeta, dS0), all
    float32; da [B,T,H] is None when a is None."""
    return _prefill_backward(q, k, v, a, beta, dO, S0, dS_T, gdn=True)


def _prologue_rows(q, k, g, b):
    if q.dtype not in _DT:
        raise TypeError(f"q: dtype {q.dtype} not supported")
    dk = q.shape[-1]
    lead = tuple(q.shape[:-1])
    for n, t, d, sh in (("q", q, q.dtype, q.shape), ("k", k, q.dtype, q.shape),
                        ("g", g, q.dtype, q.shape), ("b", b, torch.float32, lead)):
        _check(n, t, d, sh, q.device)
    rows = 1
    for x in lead:
        rows *= x
    return rows, dk, lead


def prologue_forward(q, k, g, b, qk_map="l2"):
    """The input prologue alone: raw q, k, g [..., dk] (bf16 or fp32) and b
    [...] fp32 -> (q_hat, k_hat, alpha, beta), the inputs of prefill_chunked
    and prefill_backward."""
    if qk_map not in _QK:
        raise ValueError(f"qk_map must be one of {sorted(_QK)}")
    rows, dk, lead = _prologue_rows(q, k, g, b)
    dev = q.device
    qh, kh = torch.empty_like(q), torch.empty_like(k)
    alpha = torch.empty(q.shape, dtype=torch.float32, device=dev)
    beta = torch.empty(lead, dtype=torch.float32, device=dev)
    st = lib().kda_prologue_forward(_ptr(q), _ptr(k), _ptr(g), _ptr(b), _ptr(qh), _ptr(kh),
                                    _ptr(alpha), _ptr(beta), rows, dk, _DT[q.dtype], _QK[qk_map],
                                    _stream(dev))
    if st != _lib.KDA_OK:
        raise KDAError(st, "kda_prologue_forward")
    return qh, kh, alpha, beta


def prologue_backward(q, k, g, b, dq_hat, dk_hat, dalpha, dbeta, qk_map="l2"):
    """Adjoint of prologue_forward: gradients with respect to (q_hat, k_hat,
    alpha, beta), fp32, -> gradients with respect to the raw (q, k, g, b),
    fp32."""
    if qk_map not in _QK:
        raise ValueError(f"qk_map must be one of {sorted(_QK)}")
    rows, dk, lead = _prologue_rows(q, k, g, b)
    dev = q.device
    f32 = torch.float32
    for n, t, sh in (("dq_hat", dq_hat, q.shape), ("dk_hat", dk_hat, q.shape),
                     ("dalpha", dalpha, q.shape), ("dbeta", dbeta, lead)):
        _check(n, t, f32, sh, dev)
    dq = torch.empty(q.shape, dtype=f32, device=dev)
    dk_ = torch.empty(q.shape, dtype=f32, device=dev)
    dg = torch.empty(q.shape, dtype=f32, device=dev)
    db = torch.empty(lead, dtype=f32, device=dev)
    st = lib().kda_prologue_backward(_ptr(q), _ptr(k), _ptr(g), _ptr(b), _ptr(dq_hat),
                                     _ptr(dk_hat), _ptr(dalpha), _ptr(dbeta), _ptr(dq), _ptr(dk_),
                                     _ptr(dg), _ptr(db), rows, dk, _DT[q.dtype], _QK[qk_map],
                                     _stream(dev))
    if st != _lib.KDA_OK:
        raise KDAError(st, "kda_prologue_backward")
    return dq, dk_, dg, db


def prefill_backward_logits(q, k, v, g, b, dO, S0=None, dS_T=None, qk_map="l2"):
    """Gradients through prefill_chunked_logits: the prologue forward, the
    prefill backward on its outputs, then the prologue's adjoint (three
    library calls).  Returns (dq, dk, dv, dg, db, dS0), all float32, with
    respect to the raw q, k, v, g, b and S0."""
    qh, kh, alpha, beta = prologue_forward(q, k, g, b, qk_map)
    dqh, dkh, dv, da, dbeta, dS0 = prefill_backward(qh, kh, v, alpha, beta, dO, S0=S0, dS_T=dS_T)
    dq, dk_, dg, db = prologue_backward(q, k, g, b, dqh, dkh, da, dbeta, qk_map)
    return dq, dk_, dv, dg, db, dS0
