"""Float64 CPU oracle for the adjoint (backward) of one KDA recurrence step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
CPU-baseline leg of the benchmark may import this module.  The product path
never calls it and shares no code with it.

The forward step (kda_oracle._step; "From GPT-2 to Kimi K3, Explained",
sections "DeltaNet (Fast Weight Programmers)", "Gated Delta Net" and
"KDA/Kimi Linear") is

    S' = Diag(alpha) S,  r = k S',  u = beta (v - r),  S_new = S' + k^T u,  o = q S_new.

Given dO = dL/do and dS_new = dL/dS_new for some scalar L, the chain rule
taken backwards through those five lines gives

    G     = dS_new + q^T dO                 (everything that reaches S_new)
    dq    = S_new dO^T
    du    = k G
    dv    = beta du,   dbeta = du . (v - r),   dr = -beta du
    dk    = G u^T + S' dr^T
    dS'   = G + k^T dr
    dalpha = rowsum(dS' * S),   dS = Diag(alpha) dS'.

The pages describe the forward pass only, so every line here is pinned in
tests/test_backward_pins.py against central finite differences of the
forward oracle (a different computation that a wrong sign, a dropped term or
a transposed product fails), for one step and for a chain of steps that
reproduces the gradient of a whole prefill.

kda_prologue_backward is the chain rule through the input prologue of
kda_prologue.py (alpha = exp(-softplus(g)) = sigmoid(-g), beta = sigmoid(b),
q, k = normalize(phi(x))):

    dg = -dalpha alpha (1 - alpha),   db = dbeta beta (1 - beta)
    normalize, y = x / max(||x||, eps):  dx = (dy - y (y . dy)) / ||x||  if ||x|| > eps,
                                         dx = dy / eps                      otherwise
    silu:  d silu(x) / dx = sigmoid(x) (1 + x (1 - sigmoid(x)))

and kda_prefill_backward_logits chains prologue, prefill backward and
prologue backward.  gdn_prefill_backward is the prefill backward of Gated
DeltaNet (one gate per token and head, broadcast over the key channels) and
DeltaNet (no gate): the gate's gradient is the sum over the channels of the
per-channel one.  Both are pinned against finite differences of the
forward oracle in tests/test_backward_pins.py.

kda_prefill_backward is that chain written out: the forward recurrence
(kda_oracle.kda_recurrence) run once to keep the state before every token,
then the step adjoint applied from the last token to the first, the state
gradient carried from token to token and, after token 0, returned as dS0.
"""
from __future__ import annotations

import numpy as np

from .kda_oracle import _channel_gate, as_f64, kda_decode_step
from .kda_prologue import NORM_EPS, QK_AS_GIVEN, QK_L2, QK_SILU_L2, kda_prologue, sigmoid, silu

__all__ = ["kda_decode_step_backward", "kda_prefill_backward", "kda_prologue_backward",
           "kda_prefill_backward_logits", "gdn_prefill_backward", "gdn_decode_step_backward"]


def kda_decode_step_backward(q, k, v, alpha, beta, S, dO, dS_new):
    """Adjoint of kda_decode_step, float64.

    q, k, alpha: [N, H, dk]; v, dO: [N, H, dv]; beta: [N, H]; S, dS_new:
    [N, H, dk, dv].  Returns (dq, dk, dv, dalpha, dbeta, dS), each shaped
    like the matching forward input."""
    q, k, v, alpha, beta, S, dO, dS_new = (as_f64(x) for x in
                                           (q, k, v, alpha, beta, S, dO, dS_new))
    Sp = alpha[..., :, None] * S                                  # S'
    r = np.einsum("...c,...cj->...j", k, Sp)
    u = beta[..., None] * (v - r)
    S_new = Sp + k[..., :, None] * u[..., None, :]
    G = dS_new + q[..., :, None] * dO[..., None, :]
    dq = np.einsum("...cj,...j->...c", S_new, dO)
    du = np.einsum("...c,...cj->...j", k, G)
    dv = beta[..., None] * du
    dbeta = np.sum(du * (v - r), axis=-1)
    dr = -beta[..., None] * du
    dk = np.einsum("...cj,...j->...c", G, u) + np.einsum("...cj,...j->...c", Sp, dr)
    dSp = G + k[..., :, None] * dr[..., None, :]
    dalpha = np.sum(dSp * S, axis=-1)
    dS = alpha[..., :, None] * dSp
    return dq, dk, dv, dalpha, dbeta, dS


def kda_prefill_backward(q, k, v, alpha, beta, S0, dO, dS_T):
    """Gradients of L through a whole prefill, float64.

    q, k, alpha: [B, T, H, dk]; v, dO: [B, T, H, dv]; beta: [B, T, H];
    S0, dS_T: [B, H, dk, dv] or None (zeros).  dO = dL/do for every token,
    dS_T = dL/dS_T for the final state.  Returns (dq, dk, dv, dalpha, dbeta,
    dS0), shaped like q, k, v, alpha, beta and the state."""
    q, k, v, alpha, beta, dO = (as_f64(x) for x in (q, k, v, alpha, beta, dO))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else as_f64(S0).copy()
    before = []                                   # S_{t-1}: the state token t starts from
    for t in range(T):
        before.append(S)
        _, S = kda_decode_step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], S)
    dS = np.zeros((B, H, dk, dv)) if dS_T is None else as_f64(dS_T).copy()
    dq, dk_, dv_ = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    da, db = np.zeros_like(alpha), np.zeros_like(beta)
    for t in reversed(range(T)):
        dq[:, t], dk_[:, t], dv_[:, t], da[:, t], db[:, t], dS = kda_decode_step_backward(
            q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], before[t], dO[:, t], dS)
    return dq, dk_, dv_, da, db, dS


def _normalize_backward(x, dy):
    """Adjoint of normalize(x) = x / max(||x||, eps) over the last axis."""
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    big = n > NORM_EPS
    y = x / np.where(big, n, NORM_EPS)
    proj = np.sum(y * dy, axis=-1, keepdims=True)
    return np.where(big, (dy - y * proj) / np.where(big, n, 1.0), dy / NORM_EPS)


def kda_prologue_backward(q, k, g, b, dq_hat, dk_hat, dalpha, dbeta, qk_map=QK_L2):
    """Adjoint of kda_prologue, float64: from the gradients with respect to
    its outputs (q_hat, k_hat, alpha, beta) to those with respect to its raw
    inputs.  Returns (dq, dk, dg, db), shaped like q, k, g, b."""
    q, k, g, b = (as_f64(x) for x in (q, k, g, b))
    dq_hat, dk_hat, dalpha, dbeta = (as_f64(x) for x in (dq_hat, dk_hat, dalpha, dbeta))
    alpha = sigmoid(-g)
    beta = sigmoid(b)
    dg = -dalpha * alpha * (1.0 - alpha)
    db = dbeta * beta * (1.0 - beta)

    def feature(x, dy):
        if qk_map == QK_AS_GIVEN:
            return dy
        if qk_map == QK_L2:
            return _normalize_backward(x, dy)
        if qk_map == QK_SILU_L2:
            s = sigmoid(x)
            return _normalize_backward(silu(x), dy) * s * (1.0 + x * (1.0 - s))
        raise ValueError(f"unknown qk_map {qk_map}")

    return feature(q, dq_hat), feature(k, dk_hat), dg, db


def kda_prefill_backward_logits(q, k, v, g, b, S0, dO, dS_T, qk_map=QK_L2):
    """Gradients of L through kda_recurrence_logits (prologue, then the
    recurrence), float64.  Returns (dq, dk, dv, dg, db, dS0) with respect to
    the raw q, k, v, g, b and S0."""
    qn, kn, alpha, beta = kda_prologue(q, k, g, b, qk_map)
    dqh, dkh, dv, da, db_, dS0 = kda_prefill_backward(qn, kn, v, alpha, beta, S0, dO, dS_T)
    dq, dk, dg, db = kda_prologue_backward(q, k, g, b, dqh, dkh, da, db_, qk_map)
    return dq, dk, dv, dg, db, dS0


def gdn_prefill_backward(q, k, v, a, beta, S0, dO, dS_T):
    """Gradients of L through gdn_recurrence, float64.  a: [B, T, H] or None
    (DeltaNet).  Returns (dq, dk, dv, da, dbeta, dS0); da is None when a is."""
    k64 = as_f64(k)
    dq, dk, dv, dalpha, dbeta, dS0 = kda_prefill_backward(q, k64, v, _channel_gate(a, k64), beta,
                                                          S0, dO, dS_T)
    return dq, dk, dv, (None if a is None else dalpha.sum(axis=-1)), dbeta, dS0


def gdn_decode_step_backward(q, k, v, a, beta, S, dO, dS_new):
    """Adjoint of gdn_decode_step (a [N, H], or None for DeltaNet), float64.
    Returns (dq, dk, dv, da, dbeta, dS); da is None when a is."""
    k64 = as_f64(k)
    dq, dk, dv, dalpha, dbeta, dS = kda_decode_step_backward(q, k64, v, _channel_gate(a, k64),
                                                              beta, S, dO, dS_new)
    return dq, dk, dv, (None if a is None else dalpha.sum(axis=-1)), dbeta, dS
