"""Pins for the prologue's adjoint (oracle.kda_prologue_backward) and for the
whole backward from raw projections (oracle.kda_prefill_backward_logits).

The adjoint is fixed by the forward prologue alone: for L = <w_q, q_hat> +
<w_k, k_hat> + <w_a, alpha> + <w_b, beta> the gradient with respect to each
raw input must match central finite differences of oracle.kda_prologue, for
every q/k map; chained with the prefill backward it must match finite
differences of oracle.kda_recurrence_logits.  Exact values pin the gate and
strength terms (g = 0 and b = 0 give slope -1/4 and 1/4; g = ln 3 gives
alpha = 1/4 and slope -3/16), and the norm floor is linear (a zero row's
gradient is dy / 1e-12).  Planted mistakes must fail."""
import math

import numpy as np
import pytest

from oracle import kda_prologue, kda_recurrence_logits
from oracle.kda_backward import kda_prefill_backward_logits, kda_prologue_backward
from oracle.kda_prologue import NORM_EPS, QK_AS_GIVEN, QK_L2, QK_SILU_L2, sigmoid

H_FD = 1e-6
TOL = 1e-6
MAPS = (QK_AS_GIVEN, QK_L2, QK_SILU_L2)


def _case(seed, shape=(3, 2, 5)):
    r = np.random.default_rng(seed)
    x = dict(q=r.standard_normal(shape), k=r.standard_normal(shape),
             g=r.standard_normal(shape), b=r.standard_normal(shape[:-1]))
    w = dict(q=r.standard_normal(shape), k=r.standard_normal(shape),
             a=r.standard_normal(shape), b=r.standard_normal(shape[:-1]))
    return x, w


def prologue_fd_error(backward, qk_map, seed=1):
    x, w = _case(seed)

    def loss(a):
        qh, kh, al, be = kda_prologue(a["q"], a["k"], a["g"], a["b"], qk_map)
        return float(np.sum(w["q"] * qh) + np.sum(w["k"] * kh) + np.sum(w["a"] * al)
                     + np.sum(w["b"] * be))

    grads = dict(zip(("q", "k", "g", "b"),
                     backward(x["q"], x["k"], x["g"], x["b"], w["q"], w["k"], w["a"], w["b"],
                              qk_map)))
    r = np.random.default_rng(seed + 50)
    err = 0.0
    for n in ("q", "k", "g", "b"):
        for _ in range(3):
            e = r.standard_normal(x[n].shape)
            fd = (loss(dict(x, **{n: x[n] + H_FD * e})) - loss(dict(x, **{n: x[n] - H_FD * e}))) \
                / (2 * H_FD)
            err = max(err, abs(fd - float(np.sum(grads[n] * e))) / max(abs(fd), 1e-3))
    return err


@pytest.mark.parametrize("qk_map", MAPS)
def test_prologue_adjoint_matches_finite_differences(qk_map):
    for seed in (1, 2):
        assert prologue_fd_error(kda_prologue_backward, qk_map, seed) < TOL


def test_gate_and_strength_slopes_are_exact():
    g = np.array([0.0, math.log(3.0), -math.log(3.0)])
    one = np.ones(3)
    _, _, dg, db = kda_prologue_backward(np.ones((3, 1)), np.ones((3, 1)), g[:, None], g,
                                         np.zeros((3, 1)), np.zeros((3, 1)), one[:, None], one)
    assert np.allclose(dg[:, 0], [-0.25, -3.0 / 16.0, -3.0 / 16.0], rtol=0, atol=1e-15)
    # beta = sigmoid(b): slope 1/4 at 0, 3/16 at +-ln 3
    assert np.allclose(db, [0.25, 3.0 / 16.0, 3.0 / 16.0], rtol=0, atol=1e-15)


def test_zero_row_takes_the_norm_floor():
    dy = np.array([[1.0, -2.0, 0.5]])
    dq, _, _, _ = kda_prologue_backward(np.zeros((1, 3)), np.ones((1, 3)), np.zeros((1, 3)),
                                        np.zeros(1), dy, np.zeros((1, 3)), np.zeros((1, 3)),
                                        np.zeros(1), QK_L2)
    assert np.array_equal(dq, dy / NORM_EPS)


def test_unit_row_gradient_is_the_tangential_part():
    # at a unit row the adjoint of normalize removes the radial part of dy
    x = np.array([[0.6, 0.8]])
    dy = np.array([[1.0, 1.0]])
    dq, _, _, _ = kda_prologue_backward(x, x, np.zeros((1, 2)), np.zeros(1), dy,
                                        np.zeros((1, 2)), np.zeros((1, 2)), np.zeros(1), QK_L2)
    assert np.allclose(dq, dy - x * 1.4, rtol=0, atol=1e-15)
    assert abs(float(np.sum(dq * x))) < 1e-15


@pytest.mark.parametrize("qk_map", MAPS)
def test_backward_from_raw_projections_matches_finite_differences(qk_map):
    r = np.random.default_rng(11)
    B, T, H, dk, dv = 1, 7, 2, 4, 3
    x = dict(q=r.standard_normal((B, T, H, dk)), k=r.standard_normal((B, T, H, dk)),
             v=r.standard_normal((B, T, H, dv)), g=r.standard_normal((B, T, H, dk)),
             b=r.standard_normal((B, T, H)), S0=r.standard_normal((B, H, dk, dv)))
    dO = r.standard_normal((B, T, H, dv))
    dST = r.standard_normal((B, H, dk, dv))

    def loss(a):
        o, S = kda_recurrence_logits(a["q"], a["k"], a["v"], a["g"], a["b"], a["S0"], qk_map)
        return float(np.sum(dO * o) + np.sum(dST * S))

    grads = dict(zip(("q", "k", "v", "g", "b", "S0"),
                     kda_prefill_backward_logits(x["q"], x["k"], x["v"], x["g"], x["b"], x["S0"],
                                                 dO, dST, qk_map)))
    for n in grads:
        e = r.standard_normal(x[n].shape)
        fd = (loss(dict(x, **{n: x[n] + 1e-5 * e})) - loss(dict(x, **{n: x[n] - 1e-5 * e}))) / 2e-5
        assert abs(fd - float(np.sum(grads[n] * e))) / max(abs(fd), 1e-3) < 1e-7, n


# ------------------------------------------------------- planted mistakes --

def _mutant(kind):
    def bwd(q, k, g, b, dqh, dkh, da, dbe, qk_map):
        dq, dk, dg, db = kda_prologue_backward(q, k, g, b, dqh, dkh, da, dbe, qk_map)
        al, be = sigmoid(-g), sigmoid(b)
        if kind == "dg_sign":
            dg = -dg
        elif kind == "dg_alpha_only":
            dg = -da * al
        elif kind == "db_beta_only":
            db = dbe * be
        elif kind == "norm_no_projection" and qk_map == QK_L2:
            n = np.sqrt(np.sum(q * q, axis=-1, keepdims=True))
            dq = dqh / n
        elif kind == "silu_slope_sigmoid_only" and qk_map == QK_SILU_L2:
            s = sigmoid(q)
            dq = dq / (s * (1 + q * (1 - s))) * s
        elif kind == "silu_slope_dropped" and qk_map == QK_SILU_L2:
            s = sigmoid(q)
            dq = dq / (s * (1 + q * (1 - s)))
        return dq, dk, dg, db
    return bwd


@pytest.mark.parametrize("kind,qk_map", [("dg_sign", QK_L2), ("dg_alpha_only", QK_L2),
                                         ("db_beta_only", QK_L2), ("norm_no_projection", QK_L2),
                                         ("silu_slope_sigmoid_only", QK_SILU_L2),
                                         ("silu_slope_dropped", QK_SILU_L2)])
def test_pins_catch_planted_prologue_mistake(kind, qk_map):
    assert prologue_fd_error(_mutant(kind), qk_map) > 1e-3
