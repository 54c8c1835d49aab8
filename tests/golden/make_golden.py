"""Write tests/golden/brute_d4_t6.json: an exact-rational worked example of the gated delta rule.

Calls only ``oracle.brute`` (exact ``Fraction`` arithmetic on the sum-of-products closed form).
All inputs are dyadic rationals, so they are exactly representable in fp64 and the fp64 oracle
can be compared against the exact answer.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys
from fractions import Fraction as F

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import brute  # noqa: E402

# dk = dv = 4, T = 6, one sequence, non-zero, non-symmetric initial state.
alpha = [F(3, 4), F(7, 8), F(1, 2), F(15, 16), F(5, 8), F(1, 1)]
beta = [F(1, 2), F(3, 4), F(1, 4), F(1, 1), F(0), F(5, 8)]
k = [[F(1, 2), F(-1, 2), F(1, 2), F(1, 2)],
     [F(1, 1), F(0), F(0), F(0)],
     [F(0), F(3, 4), F(-1, 4), F(1, 2)],
     [F(1, 4), F(1, 4), F(-3, 4), F(1, 8)],
     [F(-1, 2), F(0), F(1, 2), F(1, 4)],
     [F(1, 2), F(1, 2), F(1, 2), F(-1, 2)]]
q = [[F(1, 1), F(1, 2), F(0), F(-1, 4)],
     [F(0), F(1, 1), F(1, 2), F(1, 2)],
     [F(-1, 2), F(1, 4), F(1, 1), F(0)],
     [F(1, 8), F(-1, 1), F(1, 4), F(1, 2)],
     [F(1, 2), F(1, 2), F(-1, 2), F(1, 1)],
     [F(3, 4), F(0), F(1, 4), F(-1, 2)]]
v = [[F(1, 1), F(-2, 1), F(1, 2), F(3, 4)],
     [F(0), F(1, 4), F(-1, 1), F(2, 1)],
     [F(3, 2), F(1, 2), F(0), F(-1, 4)],
     [F(-1, 2), F(1, 1), F(1, 8), F(1, 1)],
     [F(2, 1), F(0), F(-3, 4), F(1, 2)],
     [F(1, 4), F(-1, 2), F(1, 1), F(0)]]
# S0 is dv x dk (value-major); the oracle's h0 is its transpose (key-major).
S0 = [[F(1, 4), F(0), F(-1, 8), F(1, 2)],
      [F(1, 2), F(-1, 4), F(0), F(0)],
      [F(0), F(1, 8), F(1, 4), F(-1, 2)],
      [F(-1, 4), F(1, 2), F(0), F(1, 8)]]

outs, ST = brute.run(alpha, beta, q, k, v, S0)
s = lambda x: f"{x.numerator}/{x.denominator}"
doc = {
    "what": "gated delta rule S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t; "
            "exact rationals from oracle/brute.py (sum-of-products closed form)",
    "alpha": [s(x) for x in alpha], "beta": [s(x) for x in beta],
    "q": [[s(x) for x in r] for r in q], "k": [[s(x) for x in r] for r in k],
    "v": [[s(x) for x in r] for r in v], "S0_value_major": [[s(x) for x in r] for r in S0],
    "o": [[s(x) for x in r] for r in outs], "ST_value_major": [[s(x) for x in r] for r in ST],
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "brute_d4_t6.json"), "w") as f:
    json.dump(doc, f, indent=1)
print("wrote brute_d4_t6.json")
