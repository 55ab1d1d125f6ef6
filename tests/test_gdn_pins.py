"""Pins for the Gated DeltaNet / DeltaNet oracle (oracle.gdn_recurrence),
and the pins against planted mistakes.

What fixes the answers, independent of the oracle's code:
  * with the gate equal on every channel the recurrence is Gated DeltaNet,
    S_t = a_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t, written with
    explicit Householder matrices ("From GPT-2 to Kimi K3, Explained",
    section "Gated Delta Net": decay, then the precise write);
  * with no gate (a = 1) it is the plain delta rule of section "DeltaNet
    (Fast Weight Programmers)", its fixed point, and the linear-attention
    limit with orthonormal keys;
  * the dk = 1 closed form; a = 0 clears the memory; beta = 0 only decays,
    by the product of the scalar gates.
The recurrence pins of tests/oracle_pins.py whose gate is the same on every
channel run here through gdn_recurrence with that scalar gate (or with no
gate when it is 1).
"""
import numpy as np
import pytest

from oracle import gdn_decode_step, gdn_recurrence, kda_recurrence
from tests import oracle_pins as pins

TOL = 1e-12
SCALAR_CHECKS = ["deltanet_rule", "fixed_point", "linear_attention_limit",
                 "scalar_gate_is_gated_deltanet", "dk1_closed_form"]
UNGATED_CHECKS = ["deltanet_rule", "fixed_point", "linear_attention_limit"]


def scalar_run(gdn):
    def run(q, k, v, alpha, beta, S0=None):
        alpha = np.asarray(alpha, float)
        assert np.all(alpha == alpha[..., :1]), "gate differs across channels"
        return gdn(q, k, v, alpha[..., 0], beta, S0)
    return run


def ungated_run(gdn):
    def run(q, k, v, alpha, beta, S0=None):
        assert np.all(np.asarray(alpha) == 1.0)
        return gdn(q, k, v, None, beta, S0)
    return run


def gdn_closed_forms(gdn):
    q, k, v, _, beta, S0 = pins.rand_case(31, T=8, dk=4, dv=3)
    r = np.random.default_rng(32)
    a = r.uniform(0.1, 1.0, k.shape[:3])
    a0 = a.copy()
    a0[:, 5] = 0.0
    o, S = gdn(q, k, v, a0, beta, S0)
    # a = 0 at t = 5: the state restarts from beta k^T v
    want = beta[:, 5, :, None] * np.sum(q[:, 5] * k[:, 5], -1)[..., None] * v[:, 5]
    err = pins.rel(o[:, 5], want)
    # beta = 0: only the decay acts, by the running product of the gates
    o, S = gdn(q, k, v, a, np.zeros_like(beta), S0)
    cum = np.cumprod(a, axis=1)
    err = max(err, pins.rel(o, cum[..., None] * np.einsum("bthc,bhcj->bthj", q, S0)))
    return max(err, pins.rel(S, cum[:, -1, :, None, None] * S0))


@pytest.mark.parametrize("name", SCALAR_CHECKS)
def test_gdn_scalar_gate_pins(name):
    assert pins.CHECKS[name](scalar_run(gdn_recurrence)) < TOL


@pytest.mark.parametrize("name", UNGATED_CHECKS)
def test_deltanet_without_gate_pins(name):
    assert pins.CHECKS[name](ungated_run(gdn_recurrence)) < TOL


def test_gdn_closed_forms():
    assert gdn_closed_forms(gdn_recurrence) < TOL


def test_gdn_decode_step_is_one_prefill_step():
    q, k, v, _, beta, S0 = pins.rand_case(33, B=3, T=1, H=2, dk=4, dv=5)
    a = np.random.default_rng(34).uniform(0, 1, (3, 1, 2))
    for gate in (a, None):
        o_p, S_p = gdn_recurrence(q, k, v, gate, beta, S0)
        o_d, S_d = gdn_decode_step(q[:, 0], k[:, 0], v[:, 0],
                                   None if gate is None else gate[:, 0], beta[:, 0], S0)
        assert pins.rel(o_d, o_p[:, 0]) < TOL and pins.rel(S_d, S_p) < TOL


# ------------------------------------------------------- planted mistakes --

def _gdn_mutant(step):
    def gdn(q, k, v, a, beta, S0=None):
        q, k, v, beta = (np.asarray(x, float) for x in (q, k, v, beta))
        B, T, H, dk = k.shape
        a = np.ones((B, T, H)) if a is None else np.asarray(a, float)
        S = np.zeros((B, H, dk, v.shape[-1])) if S0 is None else np.array(S0, float)
        o = np.empty(v.shape)
        for t in range(T):
            S, o[:, t] = step(q[:, t], k[:, t], v[:, t], a[:, t], beta[:, t], S)
        return o, S
    return gdn


def _rd(x, S):
    return np.einsum("...c,...cj->...j", x, S)


def _wr(k, u):
    return k[..., :, None] * u[..., None, :]


def m_gate_after_write(q, k, v, a, b, S):
    S = a[..., None, None] * (S + _wr(k, b[..., None] * (v - _rd(k, S))))
    return S, _rd(q, S)


def m_read_undecayed(q, k, v, a, b, S):
    u = b[..., None] * (v - _rd(k, S))
    S = a[..., None, None] * S + _wr(k, u)
    return S, _rd(q, S)


def m_gate_on_write_too(q, k, v, a, b, S):
    S = a[..., None, None] * S
    S = S + a[..., None, None] * _wr(k, b[..., None] * (v - _rd(k, S)))
    return S, _rd(q, S)


def m_one_minus_gate(q, k, v, a, b, S):
    S = (1 - a)[..., None, None] * S
    S = S + _wr(k, b[..., None] * (v - _rd(k, S)))
    return S, _rd(q, S)


MUTANTS = [m_gate_after_write, m_read_undecayed, m_gate_on_write_too, m_one_minus_gate]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_gdn_pins_catch_planted_mistake(mutant):
    gdn = _gdn_mutant(mutant)
    errs = [pins.CHECKS[n](scalar_run(gdn)) for n in SCALAR_CHECKS]
    errs.append(gdn_closed_forms(gdn))
    assert max(errs) > 1e-9, mutant.__name__


def test_gdn_equals_kda_with_repeated_gate():
    q, k, v, _, beta, S0 = pins.rand_case(35)
    a = np.random.default_rng(36).uniform(0, 1, k.shape[:3])
    o1, S1 = gdn_recurrence(q, k, v, a, beta, S0)
    o2, S2 = kda_recurrence(q, k, v, np.repeat(a[..., None], k.shape[-1], -1), beta, S0)
    assert pins.rel(o1, o2) == 0 and pins.rel(S1, S2) == 0
