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


# ------------------------------------------------ whole-prefill backward --
#
# oracle.kda_prefill_backward against central finite differences of the
# prefill oracle, for every input (S0 included), with and without an initial
# state and a final-state gradient; planted mistakes in how the chain is
# walked (wrong state, dropped or frozen state gradient) must fail.

from oracle.kda_backward import kda_prefill_backward  # noqa: E402

PNAMES = ("q", "k", "v", "alpha", "beta", "S0")


def prefill_fd_error(backward, seed=7, T=9, with_S0=True, with_dST=True):
    r = np.random.default_rng(seed)
    q, k, v, alpha, beta, S0 = pins.rand_case(seed, B=2, T=T, H=2, dk=4, dv=3)
    if not with_S0:
        S0 = np.zeros_like(S0)
    dO = r.standard_normal((2, T, 2, 3))
    dST = r.standard_normal((2, 2, 4, 3)) if with_dST else None

    def loss(a):
        o, S = kda_recurrence(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"])
        return float(np.sum(dO * o) + (0.0 if dST is None else np.sum(dST * S)))

    x = dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)
    g = dict(zip(PNAMES, backward(q, k, v, alpha, beta, S0 if with_S0 else None, dO, dST)))
    err = 0.0
    for n in PNAMES:
        for _ in range(2):
            e = r.standard_normal(x[n].shape)
            fd = (loss(dict(x, **{n: x[n] + H_FD * e})) - loss(dict(x, **{n: x[n] - H_FD * e}))) \
                / (2 * H_FD)
            err = max(err, abs(fd - float(np.sum(g[n] * e))) / max(abs(fd), 1e-3))
    return err


@pytest.mark.parametrize("with_S0,with_dST", [(True, True), (False, True), (True, False),
                                              (False, False)])
def test_prefill_backward_matches_finite_differences(with_S0, with_dST):
    assert prefill_fd_error(kda_prefill_backward, with_S0=with_S0, with_dST=with_dST) < TOL


def test_prefill_backward_single_token_is_the_step_adjoint():
    q, k, v, alpha, beta, S0 = pins.rand_case(3, B=1, T=1, H=2, dk=4, dv=3)
    r = np.random.default_rng(3)
    dO, dST = r.standard_normal((1, 1, 2, 3)), r.standard_normal((1, 2, 4, 3))
    a = kda_prefill_backward(q, k, v, alpha, beta, S0, dO, dST)
    b = kda_decode_step_backward(q[:, 0], k[:, 0], v[:, 0], alpha[:, 0], beta[:, 0], S0,
                                 dO[:, 0], dST)
    for x, y in zip(a[:5], b[:5]):
        assert pins.rel(x[:, 0], y) < 1e-15
    assert pins.rel(a[5], b[5]) < 1e-15


def test_prefill_backward_of_zero_gradients_is_zero():
    q, k, v, alpha, beta, S0 = pins.rand_case(4, B=1, T=5, H=1, dk=3, dv=2)
    out = kda_prefill_backward(q, k, v, alpha, beta, S0, np.zeros((1, 5, 1, 2)), None)
    assert all(np.all(x == 0) for x in out)


def _chain_mutant(kind):
    def bwd(q, k, v, alpha, beta, S0, dO, dS_T):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        S = np.zeros((B, H, dk, dv)) if S0 is None else S0
        seq = [S]
        for t in range(T):
            _, S = kda_decode_step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], S)
            seq.append(S)
        dS = np.zeros((B, H, dk, dv)) if (dS_T is None or kind == "drop_dST") else dS_T
        out = [np.zeros_like(x) for x in (q, k, v, alpha, beta)]
        for t in reversed(range(T)):
            st = seq[t + 1] if kind == "state_after" else seq[t]
            res = kda_decode_step_backward(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t],
                                           st, dO[:, t], dS)
            for o_, g_ in zip(out, res[:5]):
                o_[:, t] = g_
            if kind != "frozen_dS":
                dS = res[5]
        return (*out, dS)
    return bwd


@pytest.mark.parametrize("kind", ["state_after", "drop_dST", "frozen_dS"])
def test_prefill_pins_catch_planted_chain_mistake(kind):
    assert prefill_fd_error(_chain_mutant(kind)) > 1e-4


# ------------------------------ Gated DeltaNet / DeltaNet prefill backward --
#
# oracle.gdn_prefill_backward against central finite differences of
# oracle.gdn_recurrence (scalar gate per token and head, and no gate); the
# gate's gradient summing the wrong axis must fail.

from oracle import gdn_recurrence  # noqa: E402
from oracle.kda_backward import gdn_prefill_backward  # noqa: E402


def gdn_fd_error(backward, gated=True, seed=21, T=8):
    r = np.random.default_rng(seed)
    q, k, v, alpha, beta, S0 = pins.rand_case(seed, B=2, T=T, H=2, dk=4, dv=3)
    a = r.uniform(0.3, 1.0, (2, T, 2)) if gated else None
    dO = r.standard_normal((2, T, 2, 3))
    dST = r.standard_normal((2, 2, 4, 3))

    def loss(x):
        o, S = gdn_recurrence(x["q"], x["k"], x["v"], x["a"], x["beta"], x["S0"])
        return float(np.sum(dO * o) + np.sum(dST * S))

    x = dict(q=q, k=k, v=v, a=a, beta=beta, S0=S0)
    g = dict(zip(("q", "k", "v", "a", "beta", "S0"), backward(q, k, v, a, beta, S0, dO, dST)))
    err = 0.0
    for n in x:
        if x[n] is None:
            assert g[n] is None
            continue
        e = r.standard_normal(x[n].shape)
        fd = (loss(dict(x, **{n: x[n] + H_FD * e})) - loss(dict(x, **{n: x[n] - H_FD * e}))) \
            / (2 * H_FD)
        err = max(err, abs(fd - float(np.sum(g[n] * e))) / max(abs(fd), 1e-3))
    return err


@pytest.mark.parametrize("gated", [True, False])
def test_gdn_prefill_backward_matches_finite_differences(gated):
    assert gdn_fd_error(gdn_prefill_backward, gated) < TOL


def test_gdn_pins_catch_gate_gradient_on_the_wrong_axis():
    def bwd(q, k, v, a, beta, S0, dO, dST):
        dq, dk, dv, _, db, dS0 = kda_prefill_backward(q, k, v, np.broadcast_to(
            a[..., None], q.shape), beta, S0, dO, dST)
        _, _, _, dal, _, _ = kda_prefill_backward(q, k, v, np.broadcast_to(a[..., None], q.shape),
                                                  beta, S0, dO, dST)
        return dq, dk, dv, dal.mean(axis=-1), db, dS0     # mean instead of sum
    assert gdn_fd_error(bwd) > 1e-4


@pytest.mark.parametrize("gated", [True, False])
def test_gdn_step_adjoint_matches_finite_differences(gated):
    from oracle import gdn_decode_step
    from oracle.kda_backward import gdn_decode_step_backward
    r = np.random.default_rng(31)
    N, H, dk, dv = 2, 3, 5, 4
    k = r.standard_normal((N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    x = dict(q=r.standard_normal((N, H, dk)), k=k, v=r.standard_normal((N, H, dv)),
             a=r.uniform(0.3, 1.0, (N, H)) if gated else None, beta=r.uniform(0.1, 1.0, (N, H)),
             S=r.standard_normal((N, H, dk, dv)))
    dO, dSn = r.standard_normal((N, H, dv)), r.standard_normal((N, H, dk, dv))

    def loss(y):
        o, S_new = gdn_decode_step(y["q"], y["k"], y["v"], y["a"], y["beta"], y["S"])
        return float(np.sum(dO * o) + np.sum(dSn * S_new))

    g = dict(zip(("q", "k", "v", "a", "beta", "S"),
                 gdn_decode_step_backward(x["q"], x["k"], x["v"], x["a"], x["beta"], x["S"], dO,
                                          dSn)))
    for n in x:
        if x[n] is None:
            assert g[n] is None
            continue
        e = r.standard_normal(x[n].shape)
        fd = (loss(dict(x, **{n: x[n] + H_FD * e})) - loss(dict(x, **{n: x[n] - H_FD * e}))) \
            / (2 * H_FD)
        assert abs(fd - float(np.sum(g[n] * e))) / max(abs(fd), 1e-3) < TOL, n
