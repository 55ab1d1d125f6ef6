"""Pins for the KDA oracle: checks against facts that the pages and the
mathematics fix, independent of the oracle's own code.

Each check takes an implementation `run(q, k, v, alpha, beta, S0) -> (o, S_T)`
working on float64 numpy arrays in the token-major layout (q,k [B,T,H,dk],
v [B,T,H,dv], alpha [B,T,H,dk], beta [B,T,H], S0 [B,H,dk,dv] or None) and
returns the largest relative error it finds.  The tests assert that the real
oracle passes every check, and that copies of the oracle with a planted
mistake fail at least one of them.

Page references (title, section):
  DN-FWP   "From GPT-2 to Kimi K3, Explained", "DeltaNet (Fast Weight Programmers)"
  DN-PAR   "From GPT-2 to Kimi K3, Explained", "DeltaNet (Parallelizing Linear
           Transformers with Delta Rule)"
  GDN      "From GPT-2 to Kimi K3, Explained", "Gated Delta Net"; the Chinese
           digest on wps.hkprog.org, "Gated DeltaNet：现在可以遗忘"
  KDA      "From GPT-2 to Kimi K3, Explained", "KDA/Kimi Linear"; "Kimi Delta
           Attention (KDA): что это за механизм внимания...", "Как KDA
           развивает идею Gated DeltaNet"
  DIGEST   "От GPT-2 до Kimi K3: семь лет эволюции внимания...", "Пять стадий
           памяти" (the DeltaNet rule written as v_old, delta, S_new)
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from oracle.kda_exact import kda_exact

CHECKS = {}


def check(name):
    def deco(fn):
        CHECKS[name] = fn
        return fn
    return deco


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.linalg.norm(b), 1e-300)
    return float(np.linalg.norm(a - b) / den)


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_case(seed, B=2, T=9, H=2, dk=4, dv=3, alo=0.2, ahi=1.0, s0=True, unit_keys=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    if unit_keys:
        k = unit(k)
    v = r.standard_normal((B, T, H, dv))
    alpha = r.uniform(alo, ahi, (B, T, H, dk))
    beta = r.uniform(0.0, 1.0, (B, T, H))
    S0 = r.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, alpha, beta, S0


# ---------------------------------------------------------------- pins ----

@check("deltanet_rule")
def deltanet_rule(run):
    """alpha = 1, beta = 1: the plain delta rule of DIGEST / DN-FWP,
    v_old = k S, delta = v - v_old, S <- S + k^T delta, o = q S (DN-PAR's
    sequential loop reads after the write)."""
    q, k, v, _, _, S0 = rand_case(1, dk=5, dv=3)
    B, T, H, dk = k.shape
    alpha = np.ones_like(k)
    beta = np.ones((B, T, H))
    o, S = run(q, k, v, alpha, beta, S0)
    err = 0.0
    for b in range(B):
        for h in range(H):
            St = S0[b, h].copy()
            for t in range(T):
                kt = k[b, t, h][None, :]               # 1 x dk row
                v_old = kt @ St                        # 1 x dv
                delta = v[b, t, h][None, :] - v_old
                St = St + kt.T @ delta
                err = max(err, rel(o[b, t, h], (q[b, t, h][None, :] @ St)[0]))
            err = max(err, rel(S[b, h], St))
    return err


@check("exact_transition_form")
def exact_transition_form(run):
    """Rational inputs, exact Householder/diagonal transition products
    (oracle.kda_exact) versus the implementation in float64.  Unit keys come
    from Pythagorean triples so that the exact-overwrite property also holds
    exactly."""
    r = np.random.default_rng(11)
    T, dk, dv = 6, 3, 2
    triples = [(Fraction(3, 5), Fraction(4, 5), Fraction(0)),
               (Fraction(0), Fraction(5, 13), Fraction(12, 13)),
               (Fraction(8, 17), Fraction(0), Fraction(15, 17)),
               (Fraction(2, 3), Fraction(1, 3), Fraction(2, 3)),
               (Fraction(-3, 5), Fraction(0), Fraction(4, 5)),
               (Fraction(1, 3), Fraction(-2, 3), Fraction(2, 3))]

    def fr(lo, hi, den):
        return Fraction(int(r.integers(lo, hi)), den)

    k = [list(triples[t]) for t in range(T)]
    q = [[fr(-9, 10, 7) for _ in range(dk)] for _ in range(T)]
    v = [[fr(-9, 10, 5) for _ in range(dv)] for _ in range(T)]
    alpha = [[fr(1, 9, 8) for _ in range(dk)] for _ in range(T)]
    beta = [fr(0, 5, 4) for _ in range(T)]
    S0 = [[fr(-5, 6, 3) for _ in range(dv)] for _ in range(dk)]
    o_ex, S_ex = kda_exact(q, k, v, alpha, beta, S0)

    def arr(x):
        return np.array([[float(y) for y in row] for row in x])

    o, S = run(arr(q)[None, :, None], arr(k)[None, :, None], arr(v)[None, :, None],
               arr(alpha)[None, :, None], np.array([float(b) for b in beta])[None, :, None],
               arr(S0)[None, None])
    return max(rel(o[0, :, 0], arr(o_ex)), rel(S[0, 0], arr(S_ex)))


@check("fixed_point")
def fixed_point(run):
    """alpha = 1 and v_t = k_t S: delta is zero, so the state never changes
    for any beta (DIGEST: if v_new equals v_old nothing changes; the Chinese
    digest, "DeltaNet：现在可以编辑记忆")."""
    q, k, _, _, beta, S0 = rand_case(2, dk=4, dv=6)
    alpha = np.ones_like(k)
    v = np.einsum("bthc,bhcj->bthj", k, S0)
    o, S = run(q, k, v, alpha, beta, S0)
    return max(rel(S, S0), rel(o, np.einsum("bthc,bhcj->bthj", q, S0)))


@check("alpha_zero_clears")
def alpha_zero_clears(run):
    """alpha_t = 0 wipes the memory (GDN): S_t = beta_t k_t^T v_t and
    o_t = beta_t (q_t . k_t) v_t whatever came before."""
    q, k, v, alpha, beta, S0 = rand_case(3, T=8, dk=4, dv=3)
    zero_at = [0, 3, 7]
    alpha[:, zero_at] = 0.0
    o, S = run(q, k, v, alpha, beta, S0)
    err = 0.0
    for t in zero_at:
        want = beta[:, t, :, None] * np.sum(q[:, t] * k[:, t], -1)[..., None] * v[:, t]
        err = max(err, rel(o[:, t], want))
    last = zero_at[-1]
    want_S = beta[:, last, :, None, None] * k[:, last, :, :, None] * v[:, last, :, None, :]
    return max(err, rel(S, want_S))


@check("beta_zero_only_decays")
def beta_zero_only_decays(run):
    """beta = 0: nothing is written; each key-dimension row of S is scaled by
    its own gate (KDA: diagonal gate on the key channels).  dk != dv so a gate
    on the wrong axis cannot pass."""
    q, k, v, alpha, _, S0 = rand_case(4, dk=5, dv=3)
    beta = np.zeros(k.shape[:3])
    o, S = run(q, k, v, alpha, beta, S0)
    cum = np.cumprod(alpha, axis=1)                        # [B,T,H,dk]
    want_o = np.einsum("bthc,bhcj->bthj", q * cum, S0)
    want_S = cum[:, -1, :, :, None] * S0
    return max(rel(o, want_o), rel(S, want_S))


@check("linear_attention_limit")
def linear_attention_limit(run):
    """alpha = 1, beta = 1, orthonormal keys and S0 = 0: the delta rule reduces
    to plain linear attention, S_T = K^T V and O = tril(Q K^T) V with the
    diagonal included (DN-PAR, the chunked linear-attention listing: masked
    q k^T inside a block, tril includes the diagonal)."""
    r = np.random.default_rng(5)
    T, dk, dv = 6, 8, 5
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    K = Qm[:T]                                              # orthonormal rows
    Q = r.standard_normal((T, dk))
    V = r.standard_normal((T, dv))
    o, S = run(Q[None, :, None], K[None, :, None], V[None, :, None],
               np.ones((1, T, 1, dk)), np.ones((1, T, 1)), None)
    want_S = K.T @ V
    want_O = np.tril(Q @ K.T) @ V
    return max(rel(S[0, 0], want_S), rel(o[0, :, 0], want_O))


@check("exact_overwrite")
def exact_overwrite(run):
    """Unit key and beta = 1: reading the new state with the same key returns
    exactly the value just written, whatever the gate and history (DN-FWP:
    with a unit key the read-back gives v exactly).  For general beta,
    k_t S_t = (1 - beta_t) k_t Diag(alpha_t) S_{t-1} + beta_t v_t."""
    q, k, v, alpha, beta, S0 = rand_case(6, B=1, T=6, H=2, dk=4, dv=3)
    err = 0.0
    S_prev = S0
    for t in range(k.shape[1]):
        _, S_t = run(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], alpha[:, :t + 1],
                     beta[:, :t + 1], S0)
        read = np.einsum("bhc,bhcj->bhj", k[:, t], S_t)
        decayed = alpha[:, t][..., None] * S_prev
        want = ((1 - beta[:, t])[..., None] * np.einsum("bhc,bhcj->bhj", k[:, t], decayed)
                + beta[:, t][..., None] * v[:, t])
        err = max(err, rel(read, want))
        S_prev = S_t
    ones = np.ones_like(beta)
    for t in (0, 2, 5):
        _, S_t = run(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], alpha[:, :t + 1],
                     ones[:, :t + 1], S0)
        err = max(err, rel(np.einsum("bhc,bhcj->bhj", k[:, t], S_t), v[:, t]))
    return err


@check("single_association")
def single_association(run):
    """T = 1 from an empty state: S = beta k^T v and o = beta (q . k) v; with
    q = k a unit key and beta = 1 the output is v itself (DN-FWP)."""
    q, k, v, alpha, beta, _ = rand_case(7, T=1, dk=4, dv=6)
    o, S = run(q, k, v, alpha, beta, None)
    want_S = beta[:, 0, :, None, None] * k[:, 0, :, :, None] * v[:, 0, :, None, :]
    want_o = beta[:, 0, :, None] * np.sum(q[:, 0] * k[:, 0], -1)[..., None] * v[:, 0]
    o2, _ = run(k, k, v, alpha, np.ones_like(beta), None)
    return max(rel(S, want_S), rel(o[:, 0], want_o), rel(o2[:, 0], v[:, 0]))


@check("scalar_gate_is_gated_deltanet")
def scalar_gate_is_gated_deltanet(run):
    """A gate equal on every channel is Gated DeltaNet (GDN): S_t = a_t S_{t-1}
    + k_t^T beta_t (v_t - k_t a_t S_{t-1}), written here with explicit
    Householder matrices a_t (I - beta_t k_t^T k_t)."""
    q, k, v, _, beta, S0 = rand_case(8, dk=4, dv=3)
    r = np.random.default_rng(80)
    a = r.uniform(0.0, 1.0, k.shape[:3])
    alpha = np.repeat(a[..., None], k.shape[-1], axis=-1)
    o, S = run(q, k, v, alpha, beta, S0)
    B, T, H, dk = k.shape
    err = 0.0
    for b in range(B):
        for h in range(H):
            St = S0[b, h]
            for t in range(T):
                kt = k[b, t, h][None, :]
                M = a[b, t, h] * (np.eye(dk) - beta[b, t, h] * kt.T @ kt)
                St = M @ St + beta[b, t, h] * kt.T @ v[b, t, h][None, :]
                err = max(err, rel(o[b, t, h], q[b, t, h] @ St))
            err = max(err, rel(S[b, h], St))
    return err


@check("linearity_in_values_and_state")
def linearity_in_values_and_state(run):
    """For fixed q, k, alpha, beta the map (V, S0) -> (O, S_T) is linear."""
    q, k, v1, alpha, beta, S1 = rand_case(9)
    _, _, v2, _, _, S2 = rand_case(10)
    a, b = 0.7, -1.3
    o1, T1 = run(q, k, v1, alpha, beta, S1)
    o2, T2 = run(q, k, v2, alpha, beta, S2)
    o3, T3 = run(q, k, a * v1 + b * v2, alpha, beta, a * S1 + b * S2)
    return max(rel(o3, a * o1 + b * o2), rel(T3, a * T1 + b * T2))


@check("column_separability")
def column_separability(run):
    """Column j of (O, S_T) depends only on column j of (V, S0)."""
    q, k, v, alpha, beta, S0 = rand_case(12, dk=4, dv=5)
    o, S = run(q, k, v, alpha, beta, S0)
    err = 0.0
    for cols in ([0, 1], [4], [2, 3]):
        oc, Sc = run(q, k, v[..., cols], alpha, beta, S0[..., cols])
        err = max(err, rel(oc, o[..., cols]), rel(Sc, S[..., cols]))
    return err


@check("contraction")
def contraction(run):
    """Unit keys, alpha and beta in [0,1]: (I - beta k^T k) Diag(alpha) has
    spectral norm at most 1, so ||S_t|| <= ||S_{t-1}|| + beta_t ||v_t||.
    Returns the worst violation relative to the bound (0 if it holds)."""
    q, k, v, alpha, beta, S0 = rand_case(13, B=1, T=12, H=1, dk=3, dv=2)
    worst = 0.0
    prev = np.linalg.norm(S0[0, 0])
    for t in range(k.shape[1]):
        _, S_t = run(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], alpha[:, :t + 1],
                     beta[:, :t + 1], S0)
        now = np.linalg.norm(S_t[0, 0])
        bound = prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        worst = max(worst, (now - bound) / bound)
        prev = now
    return max(worst, 0.0)


@check("dk1_closed_form")
def dk1_closed_form(run):
    """dk = 1 turns the state into a row s of length dv:
    s_T = s_0 prod_j c_j + sum_i beta_i k_i v_i prod_{j>i} c_j with
    c_j = (1 - beta_j k_j^2) alpha_j, and o_t = q_t s_t."""
    r = np.random.default_rng(14)
    T, dv = 10, 3
    k = r.uniform(-1, 1, T)
    q = r.standard_normal(T)
    v = r.standard_normal((T, dv))
    alpha = r.uniform(0, 1, T)
    beta = r.uniform(0, 1, T)
    s0 = r.standard_normal(dv)
    c = (1 - beta * k * k) * alpha
    err = 0.0
    o, S = run(q[None, :, None, None], k[None, :, None, None], v[None, :, None],
               alpha[None, :, None, None], beta[None, :, None], s0[None, None, None])
    for t in range(T):
        s_t = s0 * np.prod(c[:t + 1])
        for i in range(t + 1):
            s_t = s_t + beta[i] * k[i] * v[i] * np.prod(c[i + 1:t + 1])
        err = max(err, rel(o[0, t, 0], q[t] * s_t))
    return max(err, rel(S[0, 0, 0], s_t))


@check("split_resume_and_causality")
def split_resume_and_causality(run):
    """The state is the whole cache: prefill over [0,T) equals prefill over
    [0,T1) then [T1,T) from S_T1; a prefix run gives the prefix of the
    outputs."""
    q, k, v, alpha, beta, S0 = rand_case(15, T=11)
    o, S = run(q, k, v, alpha, beta, S0)
    T1 = 4
    oa, Sa = run(q[:, :T1], k[:, :T1], v[:, :T1], alpha[:, :T1], beta[:, :T1], S0)
    ob, Sb = run(q[:, T1:], k[:, T1:], v[:, T1:], alpha[:, T1:], beta[:, T1:], Sa)
    return max(rel(np.concatenate([oa, ob], 1), o), rel(Sb, S), rel(oa, o[:, :T1]))


def run_all(run):
    return {name: fn(run) for name, fn in CHECKS.items()}
