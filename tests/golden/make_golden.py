"""Writes tests/golden/exact_tiny.json from oracle/exact_rational.py only.

The fixture is an exact (rational, unrounded) evaluation of update form 2 of
page "Qwen3.8-Flash-Next 技术总结", section 2.1 (Gated DeltaNet), with the
readout o_t = S_t^T q_t, on two tiny hand-picked cases. Run from the repo
root:  python tests/golden/make_golden.py
"""
import json
import os
import sys
from fractions import Fraction as F

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(
    os.path.abspath(__file__)))))

from oracle import exact_rational  # noqa: E402


def case_a():
    # T = 4 tokens, dk = dv = 2, zero initial state
    q = [[F(1), F(0)], [F(3, 5), F(4, 5)], [F(0), F(1)], [F(1, 2), F(-1, 2)]]
    k = [[F(3, 5), F(4, 5)], [F(1), F(0)], [F(-4, 5), F(3, 5)], [F(0), F(1)]]
    v = [[F(1), F(-2)], [F(1, 2), F(3)], [F(-1), F(1, 4)], [F(2), F(0)]]
    alpha = [F(9, 10), F(1, 2), F(4, 5), F(1)]
    beta = [F(1, 2), F(3, 4), F(1), F(1, 3)]
    s0 = [[F(0), F(0)], [F(0), F(0)]]
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, s0=s0)


def case_b():
    # T = 3 tokens, dk = 3, dv = 2, nonzero initial state, beta above 1
    q = [[F(1), F(2), F(-1)], [F(0), F(1, 3), F(2, 3)], [F(-1, 2), F(0), F(1)]]
    k = [[F(2, 3), F(1, 3), F(2, 3)], [F(0), F(3, 5), F(-4, 5)],
         [F(1, 2), F(1, 2), F(0)]]
    v = [[F(1), F(1)], [F(-3), F(1, 7)], [F(2, 9), F(-1)]]
    alpha = [F(7, 8), F(3, 4), F(99, 100)]
    beta = [F(3, 2), F(1, 5), F(9, 10)]
    s0 = [[F(1, 10), F(-1, 5)], [F(0), F(3, 10)], [F(-1, 2), F(1, 4)]]
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, s0=s0)


def _s(x):
    if isinstance(x, list):
        return [_s(y) for y in x]
    return str(x)


def main():
    out = {"source": "exact rational evaluation of update form 2, page "
                     "'Qwen3.8-Flash-Next 技术总结' section 2.1, readout "
                     "o_t = S_t^T q_t; one head, one sequence",
           "cases": {}}
    for name, case in (("a", case_a()), ("b", case_b())):
        o, s = exact_rational.run(case["q"], case["k"], case["v"],
                                  case["alpha"], case["beta"], case["s0"])
        rec = {key: _s(val) for key, val in case.items()}
        rec["o"] = _s(o)
        rec["final"] = _s(s)
        out["cases"][name] = rec
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "exact_tiny.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, ensure_ascii=False)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
