"""The float64 oracle against its pins, and the pins against planted mistakes.

Every check in tests/oracle_pins.py must hold for the oracle to ~1e-12.  A
set of copies of the oracle, each with one plausible mistake planted (on the
CPU), must each fail at least one check: that is what makes the pins worth
trusting.
"""
import numpy as np
import pytest

from oracle import kda_recurrence, kda_decode_step
from tests import oracle_pins as pins

TOL = 1e-12


@pytest.mark.parametrize("name", sorted(pins.CHECKS))
def test_oracle_pin(name):
    err = pins.CHECKS[name](kda_recurrence)
    assert err < TOL, f"{name}: {err}"


def test_decode_step_is_one_prefill_step():
    q, k, v, alpha, beta, S0 = pins.rand_case(21, B=3, T=1, H=2, dk=4, dv=5)
    o_p, S_p = kda_recurrence(q, k, v, alpha, beta, S0)
    o_d, S_d = kda_decode_step(q[:, 0], k[:, 0], v[:, 0], alpha[:, 0], beta[:, 0], S0)
    assert pins.rel(o_d, o_p[:, 0]) < TOL and pins.rel(S_d, S_p) < TOL


def test_prefill_then_decode_equals_longer_prefill():
    q, k, v, alpha, beta, S0 = pins.rand_case(22, T=10)
    o, S = kda_recurrence(q, k, v, alpha, beta, S0)
    o7, St = kda_recurrence(q[:, :7], k[:, :7], v[:, :7], alpha[:, :7], beta[:, :7], S0)
    outs = []
    for t in range(7, 10):
        ot, St = kda_decode_step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], St)
        outs.append(ot)
    assert pins.rel(np.stack(outs, 1), o[:, 7:]) < TOL and pins.rel(St, S) < TOL


def test_empty_sequence_returns_initial_state():
    q, k, v, alpha, beta, S0 = pins.rand_case(23, T=0)
    o, S = kda_recurrence(q, k, v, alpha, beta, S0)
    assert o.shape == (2, 0, 2, 3) and np.array_equal(S, S0)
    _, Sz = kda_recurrence(q, k, v, alpha, beta, None)
    assert not Sz.any()


# ------------------------------------------------------- planted mistakes --

def _make_run(step):
    def run(q, k, v, alpha, beta, S0=None):
        q, k, v, alpha, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta))
        B, T, H, dk = k.shape
        dv = v.shape[-1]
        S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
        o = np.empty((B, T, H, dv))
        for t in range(T):
            S, o[:, t] = step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], S)
        return o, S
    return run


def _rd(x, S):
    return np.einsum("...c,...cj->...j", x, S)


def _outer(a, b):
    return a[..., :, None] * b[..., None, :]


def m_read_before_decay(q, k, v, a, b, S):
    r = _rd(k, S)
    S = a[..., :, None] * S + _outer(k, b[..., None] * (v - r))
    return S, _rd(q, S)


def m_decay_after_write(q, k, v, a, b, S):
    S = a[..., :, None] * (S + _outer(k, b[..., None] * (v - _rd(k, S))))
    return S, _rd(q, S)


def m_output_before_write(q, k, v, a, b, S):
    S = a[..., :, None] * S
    o = _rd(q, S)
    S = S + _outer(k, b[..., None] * (v - _rd(k, S)))
    return S, o


def m_gate_on_values(q, k, v, a, b, S):
    S = S * a[..., None, :]              # only shape-valid when dk == dv
    S = S + _outer(k, b[..., None] * (v - _rd(k, S)))
    return S, _rd(q, S)


def m_sign_of_delta(q, k, v, a, b, S):
    S = a[..., :, None] * S
    S = S + _outer(k, b[..., None] * (v + _rd(k, S)))
    return S, _rd(q, S)


def m_beta_only_on_value(q, k, v, a, b, S):
    S = a[..., :, None] * S
    S = S + _outer(k, b[..., None] * v - _rd(k, S))
    return S, _rd(q, S)


def m_no_beta(q, k, v, a, b, S):
    S = a[..., :, None] * S
    S = S + _outer(k, v - _rd(k, S))
    return S, _rd(q, S)


def m_transposed_write(q, k, v, a, b, S):
    S = a[..., :, None] * S
    u = b[..., None] * (v - _rd(k, S))
    S = S + _outer(u, k)                 # only shape-valid when dk == dv
    return S, _rd(q, S)


def m_gate_squared(q, k, v, a, b, S):
    S = (a * a)[..., :, None] * S
    S = S + _outer(k, b[..., None] * (v - _rd(k, S)))
    return S, _rd(q, S)


def m_read_with_query(q, k, v, a, b, S):
    S = a[..., :, None] * S
    S = S + _outer(k, b[..., None] * (v - _rd(q, S)))
    return S, _rd(q, S)


MUTANTS = [m_read_before_decay, m_decay_after_write, m_output_before_write, m_gate_on_values,
           m_sign_of_delta, m_beta_only_on_value, m_no_beta, m_transposed_write,
           m_gate_squared, m_read_with_query]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant):
    run = _make_run(mutant)
    caught = []
    for name, fn in pins.CHECKS.items():
        try:
            err = fn(run)
        except Exception:   # a shape error is a caught mistake too
            err = np.inf
        if not err < 1e-9:
            caught.append(name)
    assert caught, f"no pin catches {mutant.__name__}"
