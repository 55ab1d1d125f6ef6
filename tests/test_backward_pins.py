"""Pins for the step adjoint (oracle.kda_decode_step_backward) and the pins
against planted mistakes.

The adjoint of a step is fixed by the forward step alone: for the scalar
L = <dO, o> + <dS_new, S_new>, the gradient with respect to each input x
must match the central finite difference (L(x + e h) - L(x - e h)) / (2h)
along random directions e, computed from the forward oracle in float64 (an
O(h^2) truncation, ~1e-10 relative at h = 1e-5).  Chained backwards over T
steps, with the states recomputed by the forward oracle, the adjoint must
give the finite-difference gradient of a whole prefill (kda_recurrence) with
respect to every input, including the initial state.
"""
import numpy as np
import pytest

from oracle import kda_decode_step, kda_recurrence
from oracle.kda_backward import kda_decode_step_backward
from tests import oracle_pins as pins

H_FD = 1e-5
TOL = 1e-7


def _case(seed, N=2, H=3, dk=5, dv=4):
    r = np.random.default_rng(seed)
    k = r.standard_normal((N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(q=r.standard_normal((N, H, dk)), k=k, v=r.standard_normal((N, H, dv)),
                alpha=r.uniform(0.3, 1.0, (N, H, dk)), beta=r.uniform(0.1, 1.0, (N, H)),
                S=r.standard_normal((N, H, dk, dv))), \
        dict(dO=r.standard_normal((N, H, dv)), dS_new=r.standard_normal((N, H, dk, dv)))


def _loss(x, w):
    o, S_new = kda_decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S"])
    return float(np.sum(w["dO"] * o) + np.sum(w["dS_new"] * S_new))


NAMES = ("q", "k", "v", "alpha", "beta", "S")


def step_fd_error(backward, seed=1):
    x, w = _case(seed)
    grads = dict(zip(NAMES, backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S"],
                                     w["dO"], w["dS_new"])))
    r = np.random.default_rng(seed + 100)
    err = 0.0
    for n in NAMES:
        for _ in range(3):
            e = r.standard_normal(x[n].shape)
            xp = dict(x, **{n: x[n] + H_FD * e})
            xm = dict(x, **{n: x[n] - H_FD * e})
            fd = (_loss(xp, w) - _loss(xm, w)) / (2 * H_FD)
            an = float(np.sum(grads[n] * e))
            err = max(err, abs(fd - an) / max(abs(fd), 1e-3))
    return err


def chain_fd_error(backward, seed=2, T=6):
    """Gradient of L = <dO, O> + <dS_T, S_T> for a T-token prefill, by the
    adjoint applied backwards over recomputed states, against finite
    differences of the prefill oracle."""
    r = np.random.default_rng(seed)
    q, k, v, alpha, beta, S0 = pins.rand_case(seed, B=1, T=T, H=2, dk=4, dv=3)
    dO = r.standard_normal((1, T, 2, 3))
    dST = r.standard_normal((1, 2, 4, 3))

    def loss(a):
        o, S = kda_recurrence(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"])
        return float(np.sum(dO * o) + np.sum(dST * S))

    x = dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)
    states = [S0]
    for t in range(T):
        _, S = kda_decode_step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], states[-1])
        states.append(S)
    g = {n: np.zeros_like(x[n]) for n in x}
    dS = dST
    for t in reversed(range(T)):
        dq, dk, dv, da, db, dS = backward(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t],
                                          states[t], dO[:, t], dS)
        g["q"][:, t], g["k"][:, t], g["v"][:, t] = dq, dk, dv
        g["alpha"][:, t], g["beta"][:, t] = da, db
    g["S0"] = dS
    err = 0.0
    for n in x:
        e = r.standard_normal(x[n].shape)
        fd = (loss(dict(x, **{n: x[n] + H_FD * e})) - loss(dict(x, **{n: x[n] - H_FD * e}))) \
            / (2 * H_FD)
        err = max(err, abs(fd - float(np.sum(g[n] * e))) / max(abs(fd), 1e-3))
    return err


def test_step_adjoint_matches_finite_differences():
    for seed in (1, 2, 3):
        assert step_fd_error(kda_decode_step_backward, seed) < TOL


def test_chained_adjoint_is_the_prefill_gradient():
    assert chain_fd_error(kda_decode_step_backward) < TOL


def test_adjoint_is_linear_in_the_incoming_gradients():
    x, w = _case(4)
    _, w2 = _case(5)
    f = lambda ww: kda_decode_step_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"],  # noqa: E731
                                            x["S"], ww["dO"], ww["dS_new"])
    a = f(w)
    b = f(w2)
    c = f({"dO": 2 * w["dO"] - w2["dO"], "dS_new": 2 * w["dS_new"] - w2["dS_new"]})
    for ga, gb, gc in zip(a, b, c):
        assert pins.rel(gc, 2 * ga - gb) < 1e-12


# ------------------------------------------------------- planted mistakes --

def _mutant(kind):
    def bwd(q, k, v, alpha, beta, S, dO, dS_new):
        Sp = alpha[..., :, None] * S
        r = np.einsum("...c,...cj->...j", k, Sp)
        u = beta[..., None] * (v - r)
        S_new = Sp + k[..., :, None] * u[..., None, :]
        G = dS_new + (0 if kind == "no_output_term" else q[..., :, None] * dO[..., None, :])
        dq = np.einsum("...cj,...j->...c", Sp if kind == "dq_from_decayed" else S_new, dO)
        du = np.einsum("...c,...cj->...j", k, G)
        dv = beta[..., None] * du
        dbeta = np.sum(du * (v if kind == "dbeta_without_read" else v - r), axis=-1)
        dr = (1 if kind == "dr_sign" else -1) * beta[..., None] * du
        dk = np.einsum("...cj,...j->...c", G, u)
        if kind != "dk_missing_read":
            dk = dk + np.einsum("...cj,...j->...c", Sp, dr)
        dSp = G + k[..., :, None] * dr[..., None, :]
        dalpha = np.sum(dSp * (Sp if kind == "dalpha_decayed" else S), axis=-1)
        dS = (1 if kind == "dS_undecayed" else alpha[..., :, None]) * dSp
        return dq, dk, dv, dalpha, dbeta, dS
    return bwd


KINDS = ["no_output_term", "dq_from_decayed", "dbeta_without_read", "dr_sign", "dk_missing_read",
         "dalpha_decayed", "dS_undecayed"]


@pytest.mark.parametrize("kind", KINDS)
def test_pins_catch_planted_mistake(kind):
    assert step_fd_error(_mutant(kind)) > 1e-4 or chain_fd_error(_mutant(kind)) > 1e-4
