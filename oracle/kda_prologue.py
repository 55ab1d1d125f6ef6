"""Float64 CPU oracle for the KDA input prologue: raw gate logits, raw
write-strength logits and raw queries/keys in, the recurrence's inputs out.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
CPU-baseline leg of the benchmark may import this module.  The product path
(the HIP library and its Python binding) never calls it and shares no code
with it.

What is computed, per token and head:

    alpha = exp(-softplus(g)),  softplus(g) = ln(1 + e^g)     one per key channel
    beta  = sigmoid(b) = 1 / (1 + e^-b)                       one per token
    q, k  = normalize(phi(x)),  normalize(x) = x / max(||x||_2, 1e-12)
            over the head dimension, with phi = identity, or phi = silu,
            silu(x) = x * sigmoid(x)

and then the KDA recurrence of kda_oracle.py on (q, k, v, alpha, beta).

Sources (page title, then section):
  * "22580: от GPT-2 до Kimi K3, объяснение", section "DeltaNet, или Fast
    Weight Programmers": the module applies SiLU and then L2 normalisation
    over the head dimension to q and k, and a sigmoid of a projection of x to
    get the per-token write strength beta; the same section explains why a
    unit-length key reads back exactly what was written.
  * "From GPT-2 to Kimi K3, Explained", section "Gated Delta Net": the gate
    must lie in [0, 1] (1 keeps, 0 clears); the pages fix no
    parameterisation.  exp(-softplus(g)) is the one the synthetic prefill
    workloads draw their gates with, and it maps every real g into (0, 1).

Readings taken:
  * normalize follows torch.nn.functional.normalize, which the page's module
    calls: the norm is floored at 1e-12, so a zero vector stays zero;
  * the identity feature map (no SiLU) is also offered, because the
    workloads' q and k are plain L2-normalised Gaussians.

Every function here is pinned in tests/test_prologue_pins.py: special values
that the definitions fix exactly (g = 0 gives alpha = 1/2, g = ln 3 gives
1/4), limits, the odd-part identity of SiLU, unit norm and scale invariance,
and every pin of the recurrence run through exact inverse logits.  The decode
step from logits is pinned on its own: chained over a sequence it must give
the prefill from logits, every recurrence pin must hold through it on exact
inverse logits, a unit key reads back its value in one step, and g = ln 3
with b = -inf only decays the state by 1/4.
"""
from __future__ import annotations

import numpy as np

from .kda_oracle import as_f64, kda_decode_step, kda_recurrence

__all__ = ["QK_AS_GIVEN", "QK_L2", "QK_SILU_L2", "softplus", "sigmoid", "silu", "normalize",
           "kda_prologue", "kda_recurrence_logits", "kda_decode_step_logits"]

QK_AS_GIVEN, QK_L2, QK_SILU_L2 = 0, 1, 2
NORM_EPS = 1e-12


def softplus(x):
    """ln(1 + e^x), written as logaddexp(0, x) so that large x do not
    overflow (the two agree exactly in real arithmetic)."""
    return np.logaddexp(0.0, as_f64(x))


def sigmoid(x):
    """1 / (1 + e^-x) = exp(-softplus(-x)), finite for every x."""
    return np.exp(-softplus(-as_f64(x)))


def silu(x):
    """x * sigmoid(x)."""
    x = as_f64(x)
    return x * sigmoid(x)


def normalize(x):
    """x / max(||x||_2, 1e-12) over the last axis."""
    x = as_f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, NORM_EPS)


def kda_prologue(q, k, g, b, qk_map=QK_L2):
    """Raw projections -> (q, k, alpha, beta) of the recurrence, float64.

    q, k, g: [..., dk]; b: [...].  qk_map is QK_AS_GIVEN (q, k unchanged),
    QK_L2 (normalize) or QK_SILU_L2 (normalize(silu(.)))."""
    q, k = as_f64(q), as_f64(k)
    if qk_map == QK_SILU_L2:
        q, k = normalize(silu(q)), normalize(silu(k))
    elif qk_map == QK_L2:
        q, k = normalize(q), normalize(k)
    elif qk_map != QK_AS_GIVEN:
        raise ValueError(f"unknown qk_map {qk_map}")
    alpha = np.exp(-softplus(g))
    beta = sigmoid(b)
    return q, k, alpha, beta


def kda_recurrence_logits(q, k, v, g, b, S0=None, qk_map=QK_L2):
    """The prologue, then the sequential KDA prefill (kda_recurrence).

    q, k, g: [B, T, H, dk]; v: [B, T, H, dv]; b: [B, T, H];
    S0: [B, H, dk, dv] or None.  Returns (o, S_T) in float64."""
    qn, kn, alpha, beta = kda_prologue(q, k, g, b, qk_map)
    return kda_recurrence(qn, kn, v, alpha, beta, S0)


def kda_decode_step_logits(q, k, v, g, b, S, qk_map=QK_L2):
    """The prologue, then one decode step (kda_decode_step).

    q, k, g: [N, H, dk]; v: [N, H, dv]; b: [N, H]; S: [N, H, dk, dv]."""
    qn, kn, alpha, beta = kda_prologue(q, k, g, b, qk_map)
    return kda_decode_step(qn, kn, v, alpha, beta, S)
