"""Exact rational fixture (tests/golden/kda_rational_t4.json) against the
float64 oracle, plus the facts about it that follow from the pages by hand.

The pages print no worked numeric example.  The fixture is written by
tests/golden/make_golden.py from the exact transition-matrix evaluation; the
hand checks below tie two of its entries to statements on the pages without
using any code:
  * step 0 ("DeltaNet (Fast Weight Programmers)" of "From GPT-2 to Kimi K3,
    Explained"): alpha = 1, beta = 1, k = (3/5, 4/5, 0) reads back
    k S0 = (3/5, -4/5), the delta is (7/5, -1/5), and q = (1, 0, 2) then reads
    (71/25, 22/25);
  * step 2 ("Gated Delta Net": alpha = 0 clears the memory): the state is
    k^T v with beta = 1, so o = (q . k) v = (2/3) (-1, 1).
"""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import kda_recurrence

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load():
    with open(os.path.join(HERE, "kda_rational_t4.json")) as f:
        d = json.load(f)
    fr = lambda m: [[Fraction(x) for x in row] for row in m]  # noqa: E731
    return {k: (fr(v) if isinstance(v, list) and isinstance(v[0], list) else
                ([Fraction(x) for x in v] if isinstance(v, list) else v)) for k, v in d.items()}


def test_hand_checked_entries():
    d = _load()
    assert d["o"][0] == [Fraction(71, 25), Fraction(22, 25)]
    assert d["o"][2] == [Fraction(-2, 3), Fraction(2, 3)]


def test_oracle_matches_exact_fixture():
    d = _load()
    a = lambda m: np.array([[float(x) for x in row] for row in m])  # noqa: E731
    q, k, v, al = a(d["q"]), a(d["k"]), a(d["v"]), a(d["alpha"])
    beta = np.array([float(x) for x in d["beta"]])
    o, S = kda_recurrence(q[None, :, None], k[None, :, None], v[None, :, None],
                          al[None, :, None], beta[None, :, None], a(d["S0"])[None, None])
    assert np.allclose(o[0, :, 0], a(d["o"]), rtol=1e-14, atol=1e-14)
    assert np.allclose(S[0, 0], a(d["S_T"]), rtol=1e-14, atol=1e-14)
