"""The parity measures of tests/parity.py on the CPU: a mistake confined to
one 64-token chunk of one head passes the whole-slice norm at the bf16 bar
but not the chunk maximum; a wrong state head shows in the head maximum."""
import numpy as np
import pytest

from tests import parity


def _case(seed=0, B=1, T=4096, H=16, dv=32):
    r = np.random.default_rng(seed)
    ref = r.standard_normal((B, T, H, dv))
    return ref, ref * (1.0 + 4e-3 * r.standard_normal(ref.shape))


def test_one_bad_chunk_hides_in_the_norm_but_not_in_the_chunk_max():
    ref, x = _case()
    x[0, 128:192, 5] *= 1.10          # one chunk of one head 10% off
    assert parity.rel(x, ref) < 2e-2
    head, chunk = parity.worst_token_major(x, ref)
    assert chunk > 9e-2 and head < 2e-2     # the head maximum alone would miss it too
    with pytest.raises(AssertionError):
        parity.report("planted", 2e-2, x, ref)


def test_clean_case_passes_every_measure():
    ref, x = _case(1)
    m = parity.report("clean", 2e-2, x, ref)
    assert max(m.values()) < 6e-3


def test_state_head_max_and_steps_major_layout():
    r = np.random.default_rng(2)
    S = r.standard_normal((2, 4, 8, 8))
    S2 = S.copy()
    S2[1, 3] *= 1.05
    assert parity.rel(S2, S) < 2e-2 < parity.worst_state(S2, S)
    o = r.standard_normal((100, 2, 4, 8))       # [steps, N, H, dv]
    o2 = o.copy()
    o2[70:80, 1, 2] *= 1.5                      # steps 70-79 of one head wrong
    with pytest.raises(AssertionError):
        parity.report("decode", 2e-2, o2, o, steps_major=True)


def test_all_zero_reference_heads_and_padding_are_left_out():
    ref, x = _case(3, T=100, H=3)
    ref[:, :, 1] = 0.0
    x[:, :, 1] = 0.0
    ref[:, 90:] = 0.0
    x[:, 90:] = 0.0
    head, chunk = parity.worst_token_major(x, ref)
    assert np.isfinite(head) and np.isfinite(chunk) and chunk < 2e-2
