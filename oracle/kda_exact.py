"""Exact rational evaluation of KDA in transition-matrix form.

TEST INFRASTRUCTURE ONLY (see oracle/kda_oracle.py for the rule).

This is a second, independent formulation of the same method, used to pin
the float64 oracle.  Instead of stepping read/delta/write, it builds the
per-token transition matrix of the Householder / diagonal-plus-low-rank form

    A_t = (I - beta_t k_t^T k_t) . Diag(alpha_t)      (dk x dk)
    S_t = A_t . S_{t-1} + beta_t k_t^T v_t
    o_t = q_t . S_t

and multiplies it out with Python Fractions, so the result is exact for
rational inputs.  Sources: "From GPT-2 to Kimi K3, Explained", section
"DeltaNet (Parallelizing Linear Transformers with Delta Rule)" (the
reparameterised update S_t = S_{t-1}(I - beta k k^T) + beta v k^T, written
there in column convention; here transposed to the row convention), and
section "KDA/Kimi Linear" with "Kimi Delta Attention (KDA): что это за
механизм...", section "Как KDA развивает идею Gated DeltaNet" (the scalar
gate becomes a diagonal gate matrix).

All inputs are nested Python lists of Fractions (or ints), one chain only:
q, k: [T][dk]; v: [T][dv]; alpha: [T][dk]; beta: [T]; S0: [dk][dv] or None.
"""
from __future__ import annotations

from fractions import Fraction

__all__ = ["kda_exact", "transition_matrix"]


def _zeros(n, m):
    return [[Fraction(0)] * m for _ in range(n)]


def _matmul(a, b):
    n, kk, m = len(a), len(b), len(b[0])
    return [[sum((a[i][p] * b[p][j] for p in range(kk)), Fraction(0)) for j in range(m)]
            for i in range(n)]


def transition_matrix(k_t, alpha_t, beta_t):
    """A_t = (I - beta k^T k) Diag(alpha), exact, dk x dk."""
    dk = len(k_t)
    house = [[(Fraction(1) if i == j else Fraction(0)) - Fraction(beta_t) * k_t[i] * k_t[j]
              for j in range(dk)] for i in range(dk)]
    diag = [[Fraction(alpha_t[j]) if i == j else Fraction(0) for j in range(dk)]
            for i in range(dk)]
    return _matmul(house, diag)


def kda_exact(q, k, v, alpha, beta, S0=None):
    """Return (o [T][dv], S_T [dk][dv]) as exact Fractions."""
    T = len(k)
    dk = len(k[0]) if T else (len(S0) if S0 is not None else 0)
    dv = len(v[0]) if T else (len(S0[0]) if S0 is not None else 0)
    S = _zeros(dk, dv) if S0 is None else [[Fraction(x) for x in row] for row in S0]
    outs = []
    for t in range(T):
        kt = [Fraction(x) for x in k[t]]
        A = transition_matrix(kt, alpha[t], beta[t])
        S = _matmul(A, S)
        b = Fraction(beta[t])
        for i in range(dk):
            for j in range(dv):
                S[i][j] += b * kt[i] * Fraction(v[t][j])
        qt = [Fraction(x) for x in q[t]]
        outs.append([sum((qt[i] * S[i][j] for i in range(dk)), Fraction(0)) for j in range(dv)])
    return outs, S
