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
"""
from __future__ import annotations

import numpy as np

from .kda_oracle import as_f64

__all__ = ["kda_decode_step_backward"]


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
