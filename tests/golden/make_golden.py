"""Writes the exact-arithmetic fixtures in this folder.

Uses only Python's fractions and decimal modules: no numpy, no oracle code,
no GPU code.  The page prints no worked example, so these fixtures are
hand-built cases whose exact values follow from the definitions:

  mlp_exact_example.json
      One MLP block (residual add, RMS row scale, gamma, gate/up GEMMs,
      SwiGLU) with eps = 0 and rows chosen so that mean(h^2) is a perfect
      square (h rows [3, 4, 0, 0] and [2, -2, 2, 2], so r = 2/5 and 1/2).
      h, r, g, u are exact rationals; out = silu(g) * u is given to 40
      significant digits via Decimal.exp.
  closed_forms.json
      ln(128256): the loss of every row when the LM-head weights are zero
      (all logits equal), for the 128256-entry vocabulary.
"""
import json
import os
from decimal import Decimal, getcontext
from fractions import Fraction as F

getcontext().prec = 50
HERE = os.path.dirname(os.path.abspath(__file__))

x = [[1, 2], [3, -1]]
wo = [[1, 0], [0, 1], [1, 1], [1, -1]]
res = [[2, 2, -3, 1], [-1, -1, 0, -2]]
gamma = [F(1), F(2), F(1, 2), F(1)]
wg = [[1, 0, 0, 0], [0, 1, 1, 0]]
wu = [[1, 1, 1, 1], [0, 0, 2, 0]]

y = [[sum(F(x[m][k]) * wo[n][k] for k in range(2)) for n in range(4)] for m in range(2)]
h = [[res[m][n] + y[m][n] for n in range(4)] for m in range(2)]
assert h == [[3, 4, 0, 0], [2, -2, 2, 2]]
ms = [sum(v * v for v in row) / 4 for row in h]
assert ms == [F(25, 4), F(4)]
r = [F(2, 5), F(1, 2)]                 # 1/sqrt(ms), exact because ms is a square
assert all(rr * rr * m == 1 for rr, m in zip(r, ms))
n = [[r[m] * h[m][k] * gamma[k] for k in range(4)] for m in range(2)]
g = [[sum(n[m][k] * wg[j][k] for k in range(4)) for j in range(2)] for m in range(2)]
u = [[sum(n[m][k] * wu[j][k] for k in range(4)) for j in range(2)] for m in range(2)]
assert g == [[F(6, 5), F(16, 5)], [F(1), F(-3, 2)]]
assert u == [[F(22, 5), F(0)], [F(1, 2), F(1)]]


def dec(q):
    return Decimal(q.numerator) / Decimal(q.denominator)


def silu(q):
    z = dec(q)
    return z / (1 + (-z).exp())


out = [[silu(g[m][j]) * dec(u[m][j]) for j in range(2)] for m in range(2)]
s = lambda q: str(q)
ex = {
    "source": "hand-built; exact rationals via fractions, out via decimal at 50 digits",
    "inputs": {"x": [[s(F(v)) for v in row] for row in x],
               "res": [[s(F(v)) for v in row] for row in res],
               "wo": [[s(F(v)) for v in row] for row in wo],
               "wg": [[s(F(v)) for v in row] for row in wg],
               "wu": [[s(F(v)) for v in row] for row in wu],
               "gamma": [s(v) for v in gamma], "eps": "0"},
    "expected": {"h": [[s(v) for v in row] for row in h], "r": [s(v) for v in r],
                 "g": [[s(v) for v in row] for row in g], "u": [[s(v) for v in row] for row in u],
                 "out": [[format(v, ".40g") for v in row] for row in out]},
}
with open(os.path.join(HERE, "mlp_exact_example.json"), "w") as f:
    json.dump(ex, f, indent=1)
with open(os.path.join(HERE, "closed_forms.json"), "w") as f:
    json.dump({"ln_128256": format(Decimal(128256).ln(), ".40g"),
               "source": "loss per row when all 128256 logits are equal = ln V"}, f, indent=1)
print("wrote fixtures")
