"""Float64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
CPU-baseline leg of the benchmark may import this module.  The product path
(the HIP library and its Python binding) never calls it and shares no code
with it.

What is computed
----------------
One independent chain per (batch b, head h).  Row-vector convention: k_t and
q_t are rows of length dk, v_t a row of length dv, the state S is dk x dv.

    S'_t  = Diag(alpha_t) . S_{t-1}              (decay first)
    r_t   = k_t . S'_t                           (read the state at the key)
    u_t   = beta_t * (v_t - r_t)                 (the delta)
    S_t   = S'_t + k_t^T . u_t                   (write)
    o_t   = q_t . S_t                            (read after the write)

Equivalently S_t = (I - beta_t k_t^T k_t) Diag(alpha_t) S_{t-1} + beta_t k_t^T v_t.

Sources (page title, then section):
  * "From GPT-2 to Kimi K3, Explained", section "DeltaNet (Fast Weight
    Programmers)" and its Russian translation "22580: от GPT-2 до Kimi K3,
    объяснение", section "DeltaNet, или Fast Weight Programmers": read the
    old value at the key, form the difference, write key^T times the
    per-token-scaled difference, then read with q and no denominator.
  * same pages, section "DeltaNet (Parallelizing Linear Transformers with
    Delta Rule)": the sequential prefill writes first and then reads
    o_t = q_t S_t; the Householder form of the transition.
  * "From GPT-2 to Kimi K3, Explained", section "Gated Delta Net", and the
    Chinese digest (wps.hkprog.org), section "Gated DeltaNet": the previous
    state is decayed by alpha and then written precisely; alpha = 1 is pure
    DeltaNet, alpha = 0 clears the memory.
  * same pages, section "KDA/Kimi Linear", and "Kimi Delta Attention (KDA):
    что это за механизм внимания...", section "Как KDA развивает идею Gated
    DeltaNet": alpha becomes one value per channel (a diagonal gate matrix).

Readings taken where the pages are silent (each one is listed in the design
notes of the repository):
  * the per-channel gate scales the key dimension (rows of S) and is applied
    before the read-back (decay first);
  * o_t reads the state after the write (inclusive);
  * no 1/sqrt(dk) scaling, no normaliser, no feature map: q and k are taken
    exactly as given;
  * a missing initial state means zeros;
  * T = 0 returns the initial state unchanged.

Every function here is pinned by tests in tests/test_oracle_pins.py against
closed forms, special cases that reduce to library routines (matmul,
triangular solves), an exact rational evaluation and structural invariants.
"""
from __future__ import annotations

import numpy as np

__all__ = ["kda_recurrence", "kda_decode_step", "gdn_recurrence", "gdn_decode_step", "as_f64"]


def as_f64(x) -> np.ndarray:
    """Upcast a numpy array or a CPU torch tensor (any float dtype) to float64.

    bf16 and fp32 values convert to float64 exactly, so the oracle sees the
    very numbers the GPU received.
    """
    if hasattr(x, "detach"):  # torch tensor, without importing torch here
        x = x.detach().to("cpu")
        x = x.double().numpy()
    return np.asarray(x, dtype=np.float64)


def kda_recurrence(q, k, v, alpha, beta, S0=None):
    """Sequential KDA prefill over T tokens, float64.

    Arguments (token-major, as the projections produce them before the head
    transpose):
      q, k   : [B, T, H, dk]
      v      : [B, T, H, dv]
      alpha  : [B, T, H, dk]   per-channel forget gate, values in [0, 1]
      beta   : [B, T, H]       per-token write strength
      S0     : [B, H, dk, dv]  or None (zeros)

    Returns (o [B, T, H, dv], S_T [B, H, dk, dv]) in float64.
    """
    q, k, v, alpha, beta = (as_f64(x) for x in (q, k, v, alpha, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else as_f64(S0).copy()
    o = np.empty((B, T, H, dv))
    for t in range(T):
        S, o[:, t] = _step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], S)
    return o, S


def kda_decode_step(q, k, v, alpha, beta, S):
    """One KDA decode step for N sequences x H heads, float64.

    q, k: [N, H, dk]; v: [N, H, dv]; alpha: [N, H, dk]; beta: [N, H];
    S: [N, H, dk, dv].  Returns (o [N, H, dv], S_new [N, H, dk, dv]).
    This is exactly one iteration of the prefill recurrence.
    """
    q, k, v, alpha, beta, S = (as_f64(x) for x in (q, k, v, alpha, beta, S))
    S_new, o = _step(q, k, v, alpha, beta, S.copy())
    return o, S_new


def _channel_gate(a, like):
    """A gate that is the same on every key channel: a [...] -> [..., dk];
    None means 1 everywhere."""
    if a is None:
        return np.ones(like.shape)
    return np.broadcast_to(as_f64(a)[..., None], like.shape)


def gdn_recurrence(q, k, v, a, beta, S0=None):
    """Gated DeltaNet (and, with a = None, DeltaNet) prefill, float64.

    a: [B, T, H], one gate per token and head, or None for a = 1.  The other
    arguments and the result are those of kda_recurrence.  GDN is the KDA
    recurrence with the gate equal on every key channel: KDA refines GDN's
    scalar gate into one value per channel ("From GPT-2 to Kimi K3,
    Explained", sections "Gated Delta Net" and "KDA/Kimi Linear"), and a = 1
    is plain DeltaNet (section "Gated Delta Net")."""
    k64 = as_f64(k)
    return kda_recurrence(q, k64, v, _channel_gate(a, k64), beta, S0)


def gdn_decode_step(q, k, v, a, beta, S):
    """One Gated DeltaNet decode step; a: [N, H] or None (DeltaNet)."""
    k64 = as_f64(k)
    return kda_decode_step(q, k64, v, _channel_gate(a, k64), beta, S)


def _step(q, k, v, alpha, beta, S):
    """One token for every chain; leading axes are batch-like.

    q, k: [..., dk]; v: [..., dv]; alpha: [..., dk]; beta: [...];
    S: [..., dk, dv].
    """
    S = alpha[..., :, None] * S                                  # Diag(alpha) S
    r = np.einsum("...c,...cj->...j", k, S)                      # k . S'
    u = beta[..., None] * (v - r)                                # beta (v - k S')
    S = S + k[..., :, None] * u[..., None, :]                    # S' + k^T u
    o = np.einsum("...c,...cj->...j", q, S)                      # q . S_t
    return S, o
