"""Float64 model of the chunked KDA backward that the HIP kernels implement.

A design model, not the oracle: it lets the CPU suite show, independently of
any GPU run, that the chunk form of the adjoint below reproduces the
token-by-token adjoint of the recurrence (oracle.kda_prefill_backward), and
it measures how the gate gradient behaves when the matrix-core operands are
rounded to bf16 (`rnd=True`).

Forward chunk algebra (tests/chunk_model.py; "From GPT-2 to Kimi K3,
Explained", section "DeltaNet (Parallelizing Linear Transformers with Delta
Rule)", with the per-channel decay of section "KDA/Kimi Linear"), for a
chunk of C tokens from state S, with p_r = prod_{j<=r} alpha_j per channel,
Gam[r,i] = p_r / p_i, p'_r = p_{C-1} / p_r:
  A = (K K^T . Gam) strictly lower, P = (Q K^T . Gam) lower
  Y = (I + Diag(beta) A)^-1,  X = V - (K.p) S,  Z = Diag(beta) X,  U = Y Z
  O = (Q.p) S + P U,          S_new = Diag(p_{C-1}) S + (K.p')^T U
Adjoint, given dO and dS_new (= dS):
  dU = P^T dO + (K.p') dS           dZ = Y^T dU          dv = beta dZ
  dP = tril(dO U^T)                 dA = -Diag(beta) strict_tril(dZ U^T)
  dbeta = rowsum(dZ . X) + rowsum(dA/beta . A)   [= rowsum(dL . A), dL = dA/beta]
  dq = p . (dO S^T) + G1,  G1[r] = sum_i dP[r,i] k_i Gam[r,i]
  dk = p . (-Diag(beta) dZ S^T) + G2 + G3 + p' . (U dS^T)
       G2[r] = sum_i dA[r,i] k_i Gam[r,i],  G3[i] = sum_r (dP[r,i] q_r + dA[r,i] k_r) Gam[r,i]
  dS_prev = Diag(p_{C-1}) dS + (Q.p)^T dO - (K.p)^T Diag(beta) dZ
The gate gradient, as the gradient with respect to log alpha_t (every gated
quantity is a product of gates, so each term of it carries alpha_t):
  dlog alpha_t = sum_{r>=t} [q_r p_r (dO S^T)_r - k_r p_r beta_r (dZ S^T)_r]
               + sum_{i<t} k_i p'_i (U dS^T)_i + p_{C-1} rowsum(dS . S)
               + sum_{i<t<=r} (dP[r,i] q_r + dA[r,i] k_r) k_i Gam[r,i]
  dalpha_t = dlog alpha_t / alpha_t
`dlog_by="span"` evaluates this directly (only the pairs that span t);
`dlog_by="cumsum"` takes the usual route of per-row totals and a reverse
cumulative sum, where the pairs that do not span t cancel only up to
rounding.
"""
from __future__ import annotations

import numpy as np

from tests.chunk_model import exact_ratio


def bf16(x):
    """Round float64 values to bf16 (round to nearest even), as float64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _forward_states(q, k, v, alpha, beta, S0, C):
    """State at the start of every chunk (float64, exact chunk algebra)."""
    T, dk = k.shape
    S = S0.copy()
    starts = []
    for c0 in range(0, T, C):
        starts.append(S.copy())
        c1 = min(T, c0 + C)
        ac, Kc, Vc, bc = alpha[c0:c1], k[c0:c1], v[c0:c1], beta[c0:c1]
        R = exact_ratio(ac)
        p = np.cumprod(ac, axis=0)
        A = np.tril(np.einsum("rc,ic,ric->ri", Kc, Kc, R), -1)
        Y = np.linalg.inv(np.eye(c1 - c0) + bc[:, None] * A)
        U = Y @ (bc[:, None] * (Vc - (Kc * p) @ S))
        suf = np.ones_like(p)                       # prod_{j>r} alpha_j, no division
        for r in range(c1 - c0 - 2, -1, -1):
            suf[r] = suf[r + 1] * ac[r + 1]
        S = p[-1][:, None] * S + (Kc * suf).T @ U
    return starts


def chunked_backward(q, k, v, alpha, beta, S0, dO, dST, C=64, rnd=False, dlog_by="span"):
    """One chain: q, k, alpha [T, dk]; v, dO [T, dv]; beta [T]; S0, dST
    [dk, dv].  Returns (dq, dk, dv, dalpha, dbeta, dS0).  With rnd, every
    operand of a matrix product is rounded to bf16 first (products and sums
    stay float64, standing in for fp32 accumulation)."""
    r_ = bf16 if rnd else (lambda x: x)
    T, dk = k.shape
    starts = _forward_states(q, k, v, alpha, beta, S0, C)
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(alpha),
           np.zeros_like(beta)]
    dS = dST.copy()
    for ci in reversed(range(len(starts))):
        c0 = ci * C
        c1 = min(T, c0 + C)
        n = c1 - c0
        S = starts[ci]
        Qc, Kc, Vc, ac, bc, dOc = q[c0:c1], k[c0:c1], v[c0:c1], alpha[c0:c1], beta[c0:c1], dO[c0:c1]
        R = exact_ratio(ac)
        p = np.cumprod(ac, axis=0)
        pC = p[-1]
        pp = np.empty_like(p)                    # prod_{j>r} alpha_j
        acc = np.ones(dk)
        for i in range(n - 1, -1, -1):
            pp[i] = acc
            acc = acc * ac[i]
        A = np.tril(np.einsum("rc,ic,ric->ri", Kc, Kc, R), -1)
        P = np.tril(np.einsum("rc,ic,ric->ri", Qc, Kc, R))
        Y = np.linalg.inv(np.eye(n) + bc[:, None] * A)
        KE, QE, KEp = Kc * p, Qc * p, Kc * pp
        X = Vc - r_(KE) @ r_(S)
        Z = bc[:, None] * X
        U = r_(Y) @ r_(Z)
        dU = r_(P).T @ r_(dOc) + r_(KEp) @ r_(dS)
        dZ = r_(Y).T @ r_(dU)
        dv_ = bc[:, None] * dZ
        dP = np.tril(r_(dOc) @ r_(U).T)
        dL = -np.tril(r_(dZ) @ r_(U).T, -1)
        dA = bc[:, None] * dL
        db = np.sum(dZ * X, axis=1) + np.sum(dL * A, axis=1)
        dOS = r_(dOc) @ r_(S).T
        dZS = r_(dZ) @ r_(S).T
        dUS = r_(U) @ r_(dS).T
        dPr, dAr = r_(dP), r_(dA)
        if rnd:
            # as the kernels form them: the decay split into a row factor and
            # a column factor, each folded into a bf16 operand (ratio form)
            G1 = p * (dPr @ bf16(Kc / p))
            G2 = p * (dAr @ bf16(Kc / p))
            G3 = (dPr.T @ bf16(Qc * p) + dAr.T @ bf16(Kc * p)) / p
        else:
            G1 = np.einsum("ri,ic,ric->rc", dPr, Kc, R)
            G2 = np.einsum("ri,ic,ric->rc", dAr, Kc, R)
            G3 = np.einsum("ri,rc,ric->ic", dPr, Qc, R) + np.einsum("ri,rc,ric->ic", dAr, Kc, R)
        dq = p * dOS + G1
        dk_ = -p * bc[:, None] * dZS + G2 + G3 + pp * dUS
        fin = pC * np.sum(dS * S, axis=1)          # from Diag(p_{C-1}) S
        if dlog_by == "cumsum":
            dlg = Qc * dq + Kc * (-p * bc[:, None] * dZS + G2) - Kc * G3 - Kc * pp * dUS
            dlg[-1] += np.sum(Kc * pp * dUS, axis=0) + fin
            dlog = np.cumsum(dlg[::-1], axis=0)[::-1]
        else:
            row = Qc * p * dOS - Kc * p * bc[:, None] * dZS          # terms carried by p_r
            dlog = np.cumsum(row[::-1], axis=0)[::-1]                 # sum over r >= t
            col = Kc * pp * dUS                                       # terms carried by p'_i
            dlog += np.concatenate([np.zeros((1, dk)), np.cumsum(col, axis=0)[:-1]])
            dlog += fin
            X3 = (np.einsum("ri,rc->ric", dPr, Qc) + np.einsum("ri,rc->ric", dAr, Kc)) \
                * Kc[None, :, :] * R                                  # [r, i, c]
            for t in range(n):                                        # pairs i < t <= r
                dlog[t] += X3[t:, :t].sum(axis=(0, 1))
        da = dlog / ac
        dS = pC[:, None] * dS + r_(QE).T @ r_(dOc) - r_(KE).T @ r_(bc[:, None] * dZ)
        for o, x in zip(out, (dq, dk_, dv_, da, db)):
            o[c0:c1] = x
    return (*out, dS)


def subchunk_backward(q, k, v, alpha, beta, S0, dO, dST, sub=16, rnd=False):
    """The kernels' organisation of the same adjoint: the state gradient
    walks back over sub-chunks of `sub` rows (dS <- Diag(E_last) dS +
    (Q.E)^T dO - W^T (P^T dO + (K.E') dS), W = Y Diag(beta)(K.E)), and each
    sub-chunk's gradients use exact running products of alpha, with the gate
    gradient formed with alpha_t's own factor left out (no division):
      dalpha_t = F_{t-1} sum_{r>=t} rho_r Gam(r,t) + H_t sum_{i<t} sigma_i Gam(t-1,i)
               + F_{t-1} H_t fin + sum_{i<t} k_i Gam(t-1,i) sum_{r>=t} x_ri Gam(r,t)
    Gam(r,i) = prod_{i<j<=r} alpha_j; rho, sigma, fin, x as in the kernels.
    One chain; same arguments and returns as chunked_backward."""
    r_ = bf16 if rnd else (lambda x: x)
    T, dk = k.shape
    starts = _forward_states(q, k, v, alpha, beta, S0, sub)
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(alpha),
           np.zeros_like(beta)]

    def gam(a, r, i):                      # prod_{i<j<=r} a_j, per channel
        g = np.ones(a.shape[1])
        for j in range(i + 1, r + 1):
            g = g * a[j]
        return g

    dS = dST.copy()
    for si in reversed(range(len(starts))):
        c0, c1 = si * sub, min(T, (si + 1) * sub)
        n = c1 - c0
        S = starts[si]
        Qc, Kc, Vc, ac, bc, dOc = q[c0:c1], k[c0:c1], v[c0:c1], alpha[c0:c1], beta[c0:c1], dO[c0:c1]
        F = np.cumprod(ac, axis=0)
        Hs = np.array([gam(ac, n - 1, r) for r in range(n)])
        G = np.array([[gam(ac, r, i) if i <= r else np.zeros(dk) for i in range(n)]
                      for r in range(n)])                             # [r, i, c]
        A = np.tril(np.einsum("rc,ic,ric->ri", Kc, Kc, G), -1)
        P = np.tril(np.einsum("rc,ic,ric->ri", Qc, Kc, G))
        Y = np.linalg.inv(np.eye(n) + bc[:, None] * A)
        KE, KEp, QE = Kc * F, Kc * Hs, Qc * F
        W = Y @ (bc[:, None] * KE)
        U = r_(Y) @ r_(bc[:, None] * Vc) - r_(W) @ r_(S)
        dU = r_(P).T @ r_(dOc) + r_(KEp) @ r_(dS)
        dZ = r_(Y).T @ r_(dU)
        X = Vc - r_(KE) @ r_(S)
        dP = np.tril(r_(dOc) @ r_(U).T)
        dL = -np.tril(r_(dZ) @ r_(U).T, -1)
        dA = bc[:, None] * dL
        OS, ZS, US = r_(dOc) @ r_(S).T, r_(dZ) @ r_(S).T, r_(U) @ r_(dS).T
        fin = np.sum(r_(dS) * r_(S), axis=1)
        dq = F * OS + np.einsum("ri,ic,ric->rc", dP, Kc, G)
        dk_ = (-bc[:, None] * F * ZS + np.einsum("ri,ic,ric->rc", dA, Kc, G)
               + np.einsum("ri,rc,ric->ic", dP, Qc, G) + np.einsum("ri,rc,ric->ic", dA, Kc, G)
               + Hs * US)
        rho = Qc * OS - bc[:, None] * Kc * ZS
        sig = Kc * US
        da = np.zeros((n, dk))
        for t in range(n):
            Fm = gam(ac, t - 1, -1) if t > 0 else np.ones(dk)        # prod_{j<t}
            Ht = Hs[t]
            rowp = sum(rho[r] * gam(ac, r, t) for r in range(t, n))
            colp = sum((sig[i] * gam(ac, t - 1, i) for i in range(t)), np.zeros(dk))
            pair = np.zeros(dk)
            for i in range(t):
                s = sum((dP[r, i] * Qc[r] + dA[r, i] * Kc[r]) * gam(ac, r, t) for r in range(t, n))
                pair += Kc[i] * gam(ac, t - 1, i) * s
            da[t] = Fm * rowp + Ht * colp + Fm * Ht * fin + pair
        db = np.sum(dZ * X, axis=1) + np.sum(dL * A, axis=1)
        for o, x in zip(out, (dq, dk_, bc[:, None] * dZ, da, db)):
            o[c0:c1] = x
        dS = F[-1][:, None] * dS + r_(QE).T @ r_(dOc) - r_(W).T @ r_(dU)
    return (*out, dS)
