"""Pins for the prologue oracle (oracle/kda_prologue.py), and the pins against
planted mistakes.

Each check takes a prologue `pro(q, k, g, b, qk_map) -> (q', k', alpha, beta)`
on float64 arrays and returns the largest error it finds.  The real prologue
must pass every check; copies with one plausible mistake planted (on the CPU)
must each fail at least one.

What fixes the answers, independent of the oracle's code:
  * exp(-softplus(g)) = 1 / (1 + e^g), so g = 0, ln 3, -ln 3 give alpha =
    1/2, 1/4, 3/4 exactly; sigmoid(0), sigmoid(ln 3), sigmoid(-ln 3) are 1/2,
    3/4, 1/4;
  * silu(ln 3) = (3/4) ln 3 and silu(-ln 3) = -(1/4) ln 3, so
    normalize(silu((ln 3, -ln 3))) = (3, -1) / sqrt(10);
  * L2 normalisation gives unit rows, is invariant to positive rescaling and
    keeps the direction ("22580: от GPT-2 до Kimi K3, объяснение", section
    "DeltaNet, или Fast Weight Programmers": a unit key reads back exactly the
    value written with it);
  * composed with the exact inverse logits g = ln(1 - alpha) - ln(alpha),
    b = ln(beta) - ln(1 - beta), the prologue must hand the recurrence back
    its own alpha and beta: every pin of the recurrence (tests/oracle_pins.py)
    then holds through it.
"""
import numpy as np
import pytest

from oracle import kda_recurrence
from oracle.kda_prologue import (QK_AS_GIVEN, QK_L2, QK_SILU_L2, kda_prologue,
                                 kda_recurrence_logits, normalize, sigmoid, silu, softplus)
from tests import oracle_pins as pins

TOL = 1e-12
LN3 = np.log(3.0)
CHECKS = {}


def check(name):
    def deco(fn):
        CHECKS[name] = fn
        return fn
    return deco


def inverse_logits(alpha, beta):
    """The g and b whose prologue gates are exactly alpha and beta (up to
    rounding); 0 and 1 map to the infinities."""
    with np.errstate(divide="ignore"):
        g = np.log1p(-alpha) - np.log(alpha)
        b = np.log(beta) - np.log1p(-beta)
    return g, b


def _raw(seed, B=2, T=5, H=3, dk=4):
    r = np.random.default_rng(seed)
    return r.standard_normal((B, T, H, dk)) * 3.0, r.standard_normal((B, T, H, dk)) * 0.5


@check("gate_special_values")
def gate_special_values(pro):
    g = np.array([0.0, LN3, -LN3, 40.0, -40.0])
    b = np.array([0.0, LN3, -LN3, 40.0, -40.0])
    z = np.zeros((5, 1))
    _, _, a, be = pro(z, z, g[:, None], b, QK_AS_GIVEN)
    e40 = np.exp(-40.0)
    want_a = np.array([0.5, 0.25, 0.75, e40 / (1 + e40), 1 / (1 + e40)])
    want_b = np.array([0.5, 0.75, 0.25, 1 / (1 + e40), e40 / (1 + e40)])
    return max(float(np.max(np.abs(a[:, 0] / want_a - 1))), float(np.max(np.abs(be / want_b - 1))))


@check("gate_range_and_monotone")
def gate_range_and_monotone(pro):
    g = np.linspace(-30, 30, 601)
    z = np.zeros((g.size, 1))
    _, _, a, be = pro(z, z, g[:, None], g, QK_AS_GIVEN)
    a = a[:, 0]
    bad = (np.any(a <= 0) or np.any(a >= 1) or np.any(np.diff(a) >= 0)
           or np.any(be <= 0) or np.any(be >= 1) or np.any(np.diff(be) <= 0))
    return np.inf if bad else 0.0


@check("silu_then_normalize_exact")
def silu_then_normalize_exact(pro):
    x = np.array([[LN3, -LN3], [-LN3, LN3], [2 * LN3, 0.0]])
    g = np.zeros_like(x)
    q, k, _, _ = pro(x, x[::-1].copy(), g, np.zeros(3), QK_SILU_L2)
    s10 = np.sqrt(10.0)
    want = np.array([[3 / s10, -1 / s10], [-1 / s10, 3 / s10], [1.0, 0.0]])
    return max(float(np.max(np.abs(q - want))), float(np.max(np.abs(k - want[::-1]))))


@check("l2_unit_rows_direction_and_scale")
def l2_unit_rows_direction_and_scale(pro):
    q, k = _raw(1)
    g = np.zeros_like(q)
    b = np.zeros(q.shape[:3])
    qn, kn, _, _ = pro(q, k, g, b, QK_L2)
    err = max(float(np.max(np.abs(np.linalg.norm(qn, axis=-1) - 1))),
              float(np.max(np.abs(np.linalg.norm(kn, axis=-1) - 1))))
    # same direction: x' . x = ||x||
    err = max(err, float(np.max(np.abs(np.sum(qn * q, -1) - np.linalg.norm(q, axis=-1)))))
    err = max(err, float(np.max(np.abs(np.sum(kn * k, -1) - np.linalg.norm(k, axis=-1)))))
    c = np.random.default_rng(2).uniform(0.01, 100.0, q.shape[:3] + (1,))
    qs, ks, _, _ = pro(q * c, k / c, g, b, QK_L2)
    return max(err, pins.rel(qs, qn), pins.rel(ks, kn))


@check("as_given_passes_through")
def as_given_passes_through(pro):
    q, k = _raw(3)
    qn, kn, _, _ = pro(q, k, np.zeros_like(q), np.zeros(q.shape[:3]), QK_AS_GIVEN)
    return max(pins.rel(qn, q), pins.rel(kn, k))


@check("zero_vector_stays_zero")
def zero_vector_stays_zero(pro):
    q = np.zeros((2, 4))
    q[1] = [1e-20, 0.0, 0.0, 0.0]      # below the 1e-12 floor: divided by the floor
    for m in (QK_L2, QK_SILU_L2):
        qn, kn, _, _ = pro(q, q, np.zeros_like(q), np.zeros(2), m)
        if not (np.all(np.isfinite(qn)) and np.all(qn[0] == 0)):
            return np.inf
    qn, _, _, _ = pro(q, q, np.zeros_like(q), np.zeros(2), QK_L2)
    return abs(qn[1, 0] - 1e-8) / 1e-8


@check("recurrence_pins_through_inverse_logits")
def recurrence_pins_through_inverse_logits(pro):
    def run(q, k, v, alpha, beta, S0=None):
        g, b = inverse_logits(np.asarray(alpha, float), np.asarray(beta, float))
        qn, kn, a, be = pro(q, k, g, b, QK_AS_GIVEN)
        return kda_recurrence(qn, kn, v, a, be, S0)
    return max(pins.run_all(run).values())


@check("unit_key_reads_back_value")
def unit_key_reads_back_value(pro):
    """With the L2 map and beta = 1 (b = +inf) the written value reads back
    exactly with the normalised key, whatever the raw key's length."""
    q, k = _raw(4, B=1, T=6, H=2, dk=5)
    r = np.random.default_rng(5)
    v = r.standard_normal((1, 6, 2, 3))
    g = r.standard_normal(k.shape)
    b = np.full(k.shape[:3], np.inf)
    S0 = r.standard_normal((1, 2, 5, 3))
    err = 0.0
    for t in range(6):
        qn, kn, a, be = pro(q[:, :t + 1], k[:, :t + 1], g[:, :t + 1], b[:, :t + 1], QK_L2)
        _, S = kda_recurrence(qn, kn, v[:, :t + 1], a, be, S0)
        kt = k[:, t] / np.linalg.norm(k[:, t], axis=-1, keepdims=True)
        err = max(err, pins.rel(np.einsum("bhc,bhcj->bhj", kt, S), v[:, t]))
    return err


def run_all(pro):
    return {name: fn(pro) for name, fn in CHECKS.items()}


@pytest.mark.parametrize("name", sorted(CHECKS))
def test_prologue_pin(name):
    err = CHECKS[name](kda_prologue)
    assert err < TOL, f"{name}: {err}"


def test_helpers_agree_with_their_definitions_at_exact_points():
    assert softplus(0.0) == np.log(2.0)
    assert abs(sigmoid(LN3) - 0.75) < 1e-16 and abs(silu(LN3) - 0.75 * LN3) < 1e-15
    assert np.allclose(normalize(np.array([3.0, 4.0])), [0.6, 0.8], rtol=0, atol=1e-16)


def test_recurrence_logits_is_prologue_then_recurrence():
    q, k = _raw(6)
    r = np.random.default_rng(7)
    v = r.standard_normal(q.shape[:3] + (3,))
    g = r.standard_normal(q.shape)
    b = r.standard_normal(q.shape[:3])
    S0 = r.standard_normal((2, 3, 4, 3))
    for m in (QK_AS_GIVEN, QK_L2, QK_SILU_L2):
        o, S = kda_recurrence_logits(q, k, v, g, b, S0, qk_map=m)
        o2, S2 = kda_recurrence(*_order(kda_prologue(q, k, g, b, m), v), S0)
        assert pins.rel(o, o2) == 0 and pins.rel(S, S2) == 0


def _order(pro_out, v):
    qn, kn, a, be = pro_out
    return qn, kn, v, a, be


# ------------------------------------------------------- planted mistakes --

def _mut(alpha=None, beta=None, qk=None):
    def pro(q, k, g, b, qk_map):
        qq, kk = np.asarray(q, float), np.asarray(k, float)
        if qk is not None:
            qq, kk = qk(qq, kk, qk_map)
        elif qk_map == QK_SILU_L2:
            qq, kk = normalize(silu(qq)), normalize(silu(kk))
        elif qk_map == QK_L2:
            qq, kk = normalize(qq), normalize(kk)
        a = alpha(np.asarray(g, float)) if alpha else np.exp(-softplus(g))
        be = beta(np.asarray(b, float)) if beta else sigmoid(b)
        return qq, kk, a, be
    return pro


def _no_norm(q, k, m):
    return (silu(q), silu(k)) if m == QK_SILU_L2 else (q, k)


def _norm_token_axis(q, k, m):
    if m == QK_AS_GIVEN:
        return q, k
    f = (lambda x: silu(x)) if m == QK_SILU_L2 else (lambda x: x)
    nt = lambda x: x / np.maximum(np.linalg.norm(x, axis=0, keepdims=True), 1e-12)  # noqa: E731
    return nt(f(q)), nt(f(k))


def _silu_after_norm(q, k, m):
    if m == QK_SILU_L2:
        return silu(normalize(q)), silu(normalize(k))
    return (normalize(q), normalize(k)) if m == QK_L2 else (q, k)


def _no_silu(q, k, m):
    return (normalize(q), normalize(k)) if m != QK_AS_GIVEN else (q, k)


def _norm_squared(q, k, m):
    if m == QK_AS_GIVEN:
        return q, k
    f = (lambda x: silu(x)) if m == QK_SILU_L2 else (lambda x: x)
    n2 = lambda x: x / np.maximum(np.sum(x * x, -1, keepdims=True), 1e-12)  # noqa: E731
    return n2(f(q)), n2(f(k))


def _q_only(q, k, m):
    if m == QK_AS_GIVEN:
        return q, k
    f = (lambda x: silu(x)) if m == QK_SILU_L2 else (lambda x: x)
    return normalize(f(q)), f(k)


MUTANTS = {
    "alpha_is_sigmoid_g": _mut(alpha=lambda g: sigmoid(g)),
    "alpha_missing_softplus": _mut(alpha=lambda g: np.exp(-g)),
    "alpha_exp_plus_softplus_neg": _mut(alpha=lambda g: np.exp(-softplus(-g))),
    "beta_sign": _mut(beta=lambda b: sigmoid(-b)),
    "beta_is_tanh": _mut(beta=lambda b: np.tanh(b)),
    "no_normalisation": _mut(qk=_no_norm),
    "normalise_over_tokens": _mut(qk=_norm_token_axis),
    "silu_after_normalise": _mut(qk=_silu_after_norm),
    "silu_missing": _mut(qk=_no_silu),
    "divide_by_squared_norm": _mut(qk=_norm_squared),
    "key_not_normalised": _mut(qk=_q_only),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_prologue_pins_catch_planted_mistake(name):
    pro = MUTANTS[name]
    caught = []
    for cname, fn in CHECKS.items():
        with np.errstate(all="ignore"):
            try:
                err = fn(pro)
            except Exception:   # a shape error is a caught mistake too
                err = np.inf
        if not err < 1e-9:
            caught.append(cname)
    assert caught, f"no pin catches {name}"


# ------------------------------------------- one decode step from logits --
#
# oracle.kda_decode_step_logits(q, k, v, g, b, S, qk_map) -> (o, S') is one
# token of the recurrence from raw projections.  What fixes its answers:
#   * a run of such steps is the whole prefill from raw projections, so
#     chained over a sequence it must give kda_recurrence_logits' o at every
#     token and its final state, for every q/k map;
#   * through the exact inverse logits it must hand the recurrence back its
#     own alpha and beta, so every recurrence pin (tests/oracle_pins.py)
#     holds for the chained steps;
#   * with the L2 map and b = +inf (beta = 1) the normalised key reads back
#     the written value exactly, whatever the raw key's length ("22580: от
#     GPT-2 до Kimi K3, объяснение", section "DeltaNet, или Fast Weight
#     Programmers");
#   * g = ln 3 gives alpha = 1/4 and b = -inf gives beta = 0: one step then
#     only decays, S' = S / 4, and o = q S / 4.
from oracle.kda_prologue import kda_decode_step_logits  # noqa: E402

STEP_CHECKS = {}


def step_check(name):
    def deco(fn):
        STEP_CHECKS[name] = fn
        return fn
    return deco


def _chain(step, q, k, v, g, b, S0, qk_map):
    """Steps over t = 0..T-1 of [B, T, H, .] arrays -> (o [B, T, H, dv], S_T)."""
    B, T, H, dk = np.shape(k)
    dv = np.shape(v)[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.asarray(S0, float)
    outs = []
    for t in range(T):
        o, S = step(q[:, t], k[:, t], v[:, t], g[:, t], b[:, t], S, qk_map)
        outs.append(o)
    return np.stack(outs, axis=1) if outs else np.zeros((B, 0, H, dv)), S


@step_check("chain_equals_prefill_from_logits")
def chain_equals_prefill_from_logits(step):
    q, k = _raw(11, B=2, T=7, H=3, dk=5)
    r = np.random.default_rng(12)
    v = r.standard_normal(q.shape[:3] + (4,))
    g = r.standard_normal(q.shape) * 2.0
    b = r.standard_normal(q.shape[:3])
    S0 = r.standard_normal((2, 3, 5, 4))
    err = 0.0
    for m in (QK_AS_GIVEN, QK_L2, QK_SILU_L2):
        o, S = _chain(step, q, k, v, g, b, S0, m)
        o_ref, S_ref = kda_recurrence_logits(q, k, v, g, b, S0, qk_map=m)
        err = max(err, pins.rel(o, o_ref), pins.rel(S, S_ref))
    return err


@step_check("recurrence_pins_through_steps")
def recurrence_pins_through_steps(step):
    def run(q, k, v, alpha, beta, S0=None):
        g, b = inverse_logits(np.asarray(alpha, float), np.asarray(beta, float))
        return _chain(step, np.asarray(q, float), np.asarray(k, float), np.asarray(v, float),
                      g, b, S0, QK_AS_GIVEN)
    return max(pins.run_all(run).values())


@step_check("unit_key_reads_back_in_one_step")
def unit_key_reads_back_in_one_step(step):
    r = np.random.default_rng(13)
    q, k = r.standard_normal((3, 2, 6)), r.standard_normal((3, 2, 6)) * 7.0
    v = r.standard_normal((3, 2, 4))
    g = r.standard_normal((3, 2, 6))
    S = r.standard_normal((3, 2, 6, 4))
    _, S1 = step(q, k, v, g, np.full((3, 2), np.inf), S, QK_L2)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    return pins.rel(np.einsum("nhc,nhcj->nhj", kn, S1), v)


@step_check("decay_only_step")
def decay_only_step(step):
    r = np.random.default_rng(14)
    q, k = r.standard_normal((2, 3, 4)), r.standard_normal((2, 3, 4))
    v = r.standard_normal((2, 3, 5))
    S = r.standard_normal((2, 3, 4, 5))
    o, S1 = step(q, k, v, np.full((2, 3, 4), LN3), np.full((2, 3), -np.inf), S, QK_AS_GIVEN)
    return max(pins.rel(S1, S / 4.0), pins.rel(o, np.einsum("nhc,nhcj->nhj", q, S) / 4.0))


@pytest.mark.parametrize("name", sorted(STEP_CHECKS))
def test_decode_step_logits_pin(name):
    err = STEP_CHECKS[name](kda_decode_step_logits)
    assert err < TOL, f"{name}: {err}"


def _step_mut(kind):
    """A copy of the decode step from logits with one mistake planted."""
    def step(q, k, v, g, b, S, qk_map):
        q, k, v, S = (np.asarray(x, float) for x in (q, k, v, S))
        if kind != "no_normalisation" and qk_map != QK_AS_GIVEN:
            f = silu if qk_map == QK_SILU_L2 else (lambda x: x)
            q, k = normalize(f(q)), normalize(f(k))
        alpha = sigmoid(g) if kind == "gate_is_sigmoid" else np.exp(-softplus(g))
        beta = sigmoid(-np.asarray(b, float)) if kind == "beta_sign" else sigmoid(b)
        if kind == "decay_after_write":
            r = np.einsum("nhc,nhcj->nhj", k, S)
            u = beta[..., None] * (v - r)
            S1 = alpha[..., None] * (S + k[..., None] * u[..., None, :])
        else:
            Sd = alpha[..., None] * S
            r = np.einsum("nhc,nhcj->nhj", k, Sd)
            u = beta[..., None] * (v - r)
            S1 = Sd + k[..., None] * u[..., None, :]
        return np.einsum("nhc,nhcj->nhj", q, S1), S1
    return step


STEP_MUTANTS = ["gate_is_sigmoid", "beta_sign", "decay_after_write", "no_normalisation"]


def test_unmutated_step_copy_passes():
    """The mutant harness itself, with no mistake, passes every step pin."""
    for name, fn in STEP_CHECKS.items():
        assert fn(_step_mut("none")) < TOL, name


@pytest.mark.parametrize("kind", STEP_MUTANTS)
def test_decode_step_logits_pins_catch_planted_mistake(kind):
    caught = []
    for cname, fn in STEP_CHECKS.items():
        with np.errstate(all="ignore"):
            try:
                err = fn(_step_mut(kind))
            except Exception:
                err = np.inf
        if not err < 1e-9:
            caught.append(cname)
    assert caught, f"no pin catches {kind}"
