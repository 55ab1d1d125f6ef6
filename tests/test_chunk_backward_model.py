"""CPU checks of the chunked backward's algebra (tests/chunk_backward_model.py)
against the oracle's token-by-token adjoint (oracle.kda_prefill_backward,
itself pinned by finite differences in tests/test_backward_pins.py).

The sub-chunk form is what the HIP kernels compute: the state gradient over
16-row sub-chunks and, inside each, exact running products of alpha with
the gate gradient formed with alpha_t's own factor left out.  It must agree
with the oracle to rounding, closed gates (alpha = 0) and ragged lengths
included; with bf16 matrix-core operands it must stay inside the bf16 bar,
which the usual cumulative-sum route for the gate gradient does not."""
import numpy as np
import pytest

from tests.chunk_backward_model import bf16, chunked_backward, subchunk_backward
from oracle import kda_prefill_backward

NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS0")


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def case(T, dk, dv, seed=0, zero_gates=False):
    rng = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)  # noqa: E731
    q = bf16(unit(rng.standard_normal((T, dk))))
    k = bf16(unit(rng.standard_normal((T, dk))))
    v = bf16(rng.standard_normal((T, dv)))
    alpha = 1.0 / (1.0 + np.exp(rng.standard_normal((T, dk))))
    if zero_gates:
        alpha[min(5, T - 1), : dk // 3] = 0.0
        alpha[T // 2] = 0.0
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = 0.1 * rng.standard_normal((dk, dv))
    dO = bf16(rng.standard_normal((T, dv)))
    dST = rng.standard_normal((dk, dv))
    ref = kda_prefill_backward(q[None, :, None], k[None, :, None], v[None, :, None],
                               alpha[None, :, None], beta[None, :, None], S0[None, None],
                               dO[None, :, None], dST[None, None])
    ref = [r[0, :, 0] for r in ref[:5]] + [ref[5][0, 0]]
    return (q, k, v, alpha, beta, S0, dO, dST), ref


@pytest.mark.parametrize("T,zero", [(64, False), (37, False), (50, True), (16, True), (1, False)])
def test_subchunk_form_equals_the_oracle(T, zero):
    args, ref = case(T, 16, 8, seed=T, zero_gates=zero)
    got = subchunk_backward(*args)
    for n, g, r in zip(NAMES, got, ref):
        assert rel(g, r) < 1e-12, (n, rel(g, r))


def test_chunk_form_equals_the_oracle():
    args, ref = case(96, 16, 8, seed=1)
    for how in ("span", "cumsum"):
        got = chunked_backward(*args, C=32, dlog_by=how)
        for n, g, r in zip(NAMES, got, ref):
            assert rel(g, r) < 1e-12, (how, n, rel(g, r))


def test_bf16_operands_stay_inside_the_bar_without_a_cumsum():
    """bf16 operands: the sub-chunk form keeps every gradient near the bf16
    rounding level; the per-row total + reverse cumulative sum route loses
    the gate gradient to cancellation."""
    args, ref = case(256, 64, 64, seed=0)
    sub = subchunk_backward(*args, rnd=True)
    errs = {n: rel(g, r) for n, g, r in zip(NAMES, sub, ref)}
    assert max(errs.values()) < 6e-3, errs
    cum = chunked_backward(*args, C=64, rnd=True, dlog_by="cumsum")
    assert rel(cum[3], ref[3]) > 3 * errs["dalpha"]
