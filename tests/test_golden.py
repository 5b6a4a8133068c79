"""Stored oracle fixture (written by tests/golden/make_golden.py, which calls only the oracle)."""
import json
import os
import sys
from fractions import Fraction

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_golden  # noqa: E402


def test_oracle_reproduces_stored_fixture():
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as f:
        gold = {k: np.array(v) for k, v in json.load(f).items()}
    out = make_golden.evaluate(make_golden.case())
    for k, v in out.items():
        assert np.allclose(v, gold[k], rtol=1e-14, atol=1e-15), k


def test_stored_recurrence_matches_exact_rationals():
    """Exact Fraction evaluation of eqs. 1-4 from the stored (q, k, v, alpha, beta, S0)."""
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as f:
        gold = {k: np.array(v) for k, v in json.load(f).items()}
    c = make_golden.case()
    cu, H = c["cu"], c["H"]
    F = Fraction
    for s in range(len(cu) - 1):
        for h in range(H):
            S = [[F(x) for x in row] for row in c["S0"][s, h]]
            for t in range(cu[s], cu[s + 1]):
                a, b = F(gold["alpha"][t, h]), F(gold["beta"][t, h])
                q = [F(x) for x in gold["q"][t, h]]
                k = [F(x) for x in gold["k"][t, h]]
                v = [F(x) for x in gold["v"][t, h]]
                d = len(k)
                St = [[a * S[i][j] for j in range(d)] for i in range(d)]
                e = [v[j] - sum(St[i][j] * k[i] for i in range(d)) for j in range(d)]
                S = [[St[i][j] + b * k[i] * e[j] for j in range(d)] for i in range(d)]
                y = [float(sum(S[i][j] * q[i] for i in range(d))) for j in range(d)]
                assert np.allclose(y, gold["y"][t, h], rtol=1e-13, atol=1e-15)
            assert np.allclose(np.array(S, dtype=float), gold["ST"][s, h], rtol=1e-13, atol=1e-15)
