"""Write the exact rational KDA fixtures in this directory.

Calls only oracle/ (the exact transition-matrix evaluation).  Run from the
repository root:  python tests/golden/make_golden.py

Fixture kda_rational_t4.json: one chain, T=4, dk=3, dv=2.  Keys are unit
vectors built from Pythagorean triples so that the pages' exact read-back
property (a unit key with full write strength reads back exactly the value
just written; "From GPT-2 to Kimi K3, Explained", section "DeltaNet (Fast
Weight Programmers)") holds exactly at the beta = 1 steps; step 2 has a gate
of zero on every channel, which clears the memory ("Gated Delta Net");
step 3 mixes channel gates ("KDA/Kimi Linear").
"""
import json
import os
import sys
from fractions import Fraction as F

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.kda_exact import kda_exact  # noqa: E402


def case():
    k = [[F(3, 5), F(4, 5), F(0)],
         [F(0), F(5, 13), F(12, 13)],
         [F(2, 3), F(1, 3), F(2, 3)],
         [F(8, 17), F(0), F(-15, 17)]]
    q = [[F(1), F(0), F(2)], [F(-1, 2), F(1), F(1, 3)], [F(0), F(0), F(1)], [F(1), F(1), F(1)]]
    v = [[F(2), F(-1)], [F(1, 2), F(3)], [F(-1), F(1)], [F(4), F(1, 4)]]
    alpha = [[F(1), F(1), F(1)], [F(1, 2), F(3, 4), F(1)], [F(0), F(0), F(0)],
             [F(1, 4), F(1), F(7, 8)]]
    beta = [F(1), F(1, 2), F(1), F(3, 4)]
    S0 = [[F(1), F(0)], [F(0), F(-1)], [F(1, 2), F(1, 2)]]
    return q, k, v, alpha, beta, S0


def main():
    q, k, v, alpha, beta, S0 = case()
    o, S = kda_exact(q, k, v, alpha, beta, S0)
    enc = lambda m: [[str(x) for x in row] for row in m]  # noqa: E731
    doc = {
        "source": "exact transition-matrix evaluation (oracle/kda_exact.py); see make_golden.py",
        "q": enc(q), "k": enc(k), "v": enc(v), "alpha": enc(alpha),
        "beta": [str(b) for b in beta], "S0": enc(S0),
        "o": enc(o), "S_T": enc(S),
    }
    with open(os.path.join(HERE, "kda_rational_t4.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
