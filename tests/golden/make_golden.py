"""Writes tests/golden/oracle_tiny.json: a tiny end-to-end token-mixer case evaluated by
the fp64 oracle alone (eqs. 6-11 of section 2.1.1 of the Qwen3.8-Next design reading
notes). The pages print no worked example, so this fixture pins the oracle against its
own later edits; tests/test_golden.py also checks its recurrence part against exact
rational brute force. Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def case():
    rng = np.random.default_rng(20261203)
    ntok, H, d = 9, 2, 4
    cu = [0, 2, 9]
    x = {n: rng.standard_normal((ntok, H, d)).round(3) for n in ("xq", "xk", "xv")}
    w = {n: (0.5 * rng.standard_normal((H * d, 4))).round(3) for n in ("wq", "wk", "wv")}
    a_raw = rng.standard_normal((ntok, H)).round(3)
    b_raw = rng.standard_normal((ntok, H)).round(3)
    A_log = np.log(np.array([1.5, 9.0]))
    dt_bias = np.array([-4.6, -4.6])
    z = rng.standard_normal((ntok, H, d)).round(3)
    nw = (0.1414 * rng.standard_normal(d)).round(4)
    S0 = (0.1 * rng.standard_normal((2, H, d, d))).round(3)
    return dict(cu=cu, H=H, **x, **w, a_raw=a_raw, b_raw=b_raw, A_log=A_log, dt_bias=dt_bias,
                z=z, norm_weight=nw, S0=S0)


def evaluate(c):
    q, k, v = oracle.preprocess(c["xq"], c["xk"], c["xv"], c["wq"], c["wk"], c["wv"], c["cu"], c["H"])
    g, al, be = oracle.gates(c["a_raw"], c["b_raw"], c["A_log"], c["dt_bias"])
    y, ST = oracle.recurrence(q, k, v, al, be, c["S0"], c["cu"])
    o = oracle.output_gate(y, c["z"], c["norm_weight"])
    return dict(q=q, k=k, v=v, g=g, alpha=al, beta=be, y=y, ST=ST, o=o)


if __name__ == "__main__":
    c = case()
    out = evaluate(c)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump({k: np.asarray(v).tolist() for k, v in out.items()}, f, indent=0)
    print("wrote", path)
