"""Float64 model of the chunked KDA algorithm that the HIP kernels implement.

This is a design model, not the oracle: it lets the CPU suite prove, before
and independently of any GPU run, that the chunk algebra and the way the
kernels factor the per-channel decay reproduce the sequential recurrence.

Chunk algebra (one chain, a chunk of C tokens starting from state S):
  gates       p_r = prod_{j<=r} alpha_j            (per channel, cumulative)
              g_C = p_{C-1}                         (the chunk's total decay)
  gated keys  A[r,i] = sum_c k_r[c] k_i[c] p_r[c]/p_i[c]    (i < r)
              P[r,i] = sum_c q_r[c] k_i[c] p_r[c]/p_i[c]    (i <= r)
  UT/WY       L = strict_lower(Diag(beta) A),  T = (I + L)^-1 Diag(beta)
  scan        U = T (V - (K*p) S)
              O = (Q*p) S + P U
              S <- Diag(g_C) S + (K * g_C/p)^T U
With alpha = 1 this is the chunkwise delta-rule listing of "From GPT-2 to Kimi
K3, Explained", section "DeltaNet (Parallelizing Linear Transformers with
Delta Rule)" (T there is built by forward substitution; W = T K_beta and
U = T V_beta).  The per-channel decay ratios p_r/p_i generalise the
cumulative-decay term of section "Gated Delta Net" to the diagonal gate of
section "KDA/Kimi Linear".

`gate_factors` reproduces the kernels' overflow-free factoring of p_r/p_i
into products of numbers <= 1 over 16-row sub-blocks; `blocked_unit_lower_inverse`
reproduces their blocked triangular inverse.
"""
from __future__ import annotations

import numpy as np

SUB = 16


def exact_ratio(alpha_chunk):
    """R[r,i,c] = prod_{j=i+1..r} alpha_j[c] for i <= r (0 above)."""
    C, dk = alpha_chunk.shape
    R = np.zeros((C, C, dk))
    for i in range(C):
        acc = np.ones(dk)
        R[i, i] = acc
        for r in range(i + 1, C):
            acc = acc * alpha_chunk[r]
            R[r, i] = acc
    return R


def gate_factors(alpha_chunk, sub=SUB):
    """The kernels' factoring of the pairwise decay.

    Within each sub-block J of `sub` rows:
      F[r]  = prod of alpha from the block start through r (inclusive)
      Hx[i] = prod of alpha from i+1 through the block end (exclusive of i)
      BT[J] = F at the last row of J (the block's total decay)
    Off-diagonal pair (r in R, i in I < R):
      ratio = F[r] * prod_{I<J<R} BT[J] * Hx[i]         (all factors <= 1)
    Diagonal pair (r, i in the same block, i <= r):
      ratio = F[r] * (1 / F[i])                          (needs F not tiny)
    Returns the reconstructed ratio tensor like exact_ratio, and a flag per
    block telling whether the reciprocal form is safe (block total >= 1e-30).
    """
    C, dk = alpha_chunk.shape
    nb = (C + sub - 1) // sub
    F = np.empty((C, dk))
    Hx = np.empty((C, dk))
    BT = np.empty((nb, dk))
    for J in range(nb):
        lo, hi = J * sub, min(C, (J + 1) * sub)
        acc = np.ones(dk)
        for r in range(lo, hi):
            acc = acc * alpha_chunk[r]
            F[r] = acc
        BT[J] = acc
        acc = np.ones(dk)
        for i in range(hi - 1, lo - 1, -1):
            Hx[i] = acc
            acc = acc * alpha_chunk[i]
    safe = np.array([bool(np.all(BT[J] >= 1e-30)) for J in range(nb)])
    R = np.zeros((C, C, dk))
    for r in range(C):
        Rb = r // sub
        for i in range(r + 1):
            Ib = i // sub
            if Ib == Rb:
                with np.errstate(divide="ignore", invalid="ignore"):
                    R[r, i] = F[r] * (1.0 / F[i])
            else:
                between = np.prod(BT[Ib + 1:Rb], axis=0) if Rb - Ib > 1 else np.ones(dk)
                R[r, i] = F[r] * between * Hx[i]
    return R, safe


def blocked_unit_lower_inverse(L, sub=SUB):
    """(I + L)^-1 for strictly lower L, the way the kernels do it: invert each
    diagonal sub-block by forward substitution, then fill the block rows
    below with Y[R,I] = -Y[R,R] sum_{I<=J<R} L[R,J] Y[J,I]."""
    C = L.shape[0]
    nb = (C + sub - 1) // sub
    Y = np.zeros((C, C))
    blk = [slice(J * sub, min(C, (J + 1) * sub)) for J in range(nb)]
    for J, s in enumerate(blk):
        D = L[s, s]
        n = D.shape[0]
        Yd = np.eye(n)
        for r in range(1, n):
            Yd[r, :r] = -D[r, :r] @ Yd[:r, :r]
        Y[s, s] = Yd
    for d in range(1, nb):
        for I in range(nb - d):
            R = I + d
            acc = np.zeros((Y[blk[R], blk[I]].shape))
            for J in range(I, R):
                acc += L[blk[R], blk[J]] @ Y[blk[J], blk[I]]
            Y[blk[R], blk[I]] = -Y[blk[R], blk[R]] @ acc
    return Y


def chunked_kda(q, k, v, alpha, beta, S0, C, factored=False, blocked=False):
    """One chain: q,k [T,dk], v [T,dv], alpha [T,dk], beta [T], S0 [dk,dv].
    Tokens past the last full chunk are handled as a short chunk (the same
    as padding with alpha = 1, beta = 0 identity steps)."""
    T, dk = k.shape
    S = np.array(S0, dtype=np.float64).copy()
    O = np.empty((T, v.shape[1]))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        Kc, Qc, Vc, ac, bc = k[c0:c1], q[c0:c1], v[c0:c1], alpha[c0:c1], beta[c0:c1]
        n = c1 - c0
        p = np.cumprod(ac, axis=0)
        gC = p[-1]
        if factored:
            R, _ = gate_factors(ac)
        else:
            R = exact_ratio(ac)
        A = np.einsum("rc,ic,ric->ri", Kc, Kc, R)
        P = np.einsum("rc,ic,ric->ri", Qc, Kc, R)
        L = np.tril(bc[:, None] * A, -1)
        if blocked:
            Tm = blocked_unit_lower_inverse(L) * bc[None, :]
        else:
            Tm = np.linalg.solve(np.eye(n) + L, np.diag(bc))
        P = np.tril(P)
        rev = np.empty_like(p)                      # prod_{j>i} alpha_j
        acc = np.ones(dk)
        for i in range(n - 1, -1, -1):
            rev[i] = acc
            acc = acc * ac[i]
        U = Tm @ (Vc - (Kc * p) @ S)
        O[c0:c1] = (Qc * p) @ S + P @ U
        S = gC[:, None] * S + (Kc * rev).T @ U
    return O, S
