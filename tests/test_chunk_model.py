"""The chunked algorithm the kernels implement equals the sequential oracle.

CPU only.  Checks, in float64:
  * chunk form == recurrence for several chunk sizes, including a ragged
    tail, and with the kernels' overflow-free gate factoring and blocked
    triangular inverse;
  * the UT transform T equals a LAPACK triangular solve (scipy);
  * the gate factoring reproduces exact pairwise decay ratios, stays finite
    where the naive exp(+g) / exp(-g) split overflows, and flags blocks with
    (near-)zero gates as unsafe for the reciprocal form.
"""
import numpy as np
import pytest
import scipy.linalg

from oracle import kda_recurrence
from tests import chunk_model as cm
from tests.oracle_pins import rand_case, rel


@pytest.mark.parametrize("C", [1, 4, 16, 32, 64, 128])
@pytest.mark.parametrize("factored,blocked", [(False, False), (True, True)])
def test_chunk_form_matches_recurrence(C, factored, blocked):
    q, k, v, alpha, beta, S0 = rand_case(31, B=1, T=150, H=1, dk=12, dv=7, alo=0.6)
    o_ref, S_ref = kda_recurrence(q, k, v, alpha, beta, S0)
    o, S = cm.chunked_kda(q[0, :, 0], k[0, :, 0], v[0, :, 0], alpha[0, :, 0], beta[0, :, 0],
                          S0[0, 0], C, factored=factored, blocked=blocked)
    assert rel(o, o_ref[0, :, 0]) < 1e-11
    assert rel(S, S_ref[0, 0]) < 1e-11


def test_ut_transform_is_triangular_solve():
    r = np.random.default_rng(3)
    C, dk = 64, 32
    K = r.standard_normal((C, dk))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    a = r.uniform(0.5, 1.0, (C, dk))
    beta = r.uniform(0, 1, C)
    A = np.einsum("rc,ic,ric->ri", K, K, cm.exact_ratio(a))
    L = np.tril(beta[:, None] * A, -1)
    T_lapack = scipy.linalg.solve_triangular(np.eye(C) + L, np.diag(beta), lower=True)
    T_blocked = cm.blocked_unit_lower_inverse(L) * beta[None, :]
    assert rel(T_blocked, T_lapack) < 1e-12


def test_gate_factoring_exact_and_overflow_free():
    r = np.random.default_rng(4)
    C, dk = 128, 8
    # decays strong enough that exp(-cumulative log gate) overflows float32
    a = np.exp(-r.uniform(0.5, 3.0, (C, dk)))
    R_exact = cm.exact_ratio(a)
    R_fact, safe = cm.gate_factors(a.astype(np.float32).astype(np.float64))
    assert np.all(np.isfinite(R_fact))
    mask = np.tril(np.ones((C, C), bool))
    assert np.max(np.abs(R_fact - R_exact)[mask]) < 1e-6
    with np.errstate(over="ignore"):
        naive = np.exp(-np.cumsum(np.log(a), 0)).astype(np.float32)
    assert not np.all(np.isfinite(naive))
    assert safe.all()


def test_gate_factoring_flags_zero_gates():
    a = np.full((64, 4), 0.9)
    a[20, 2] = 0.0
    _, safe = cm.gate_factors(a)
    assert list(safe) == [True, False, True, True]
