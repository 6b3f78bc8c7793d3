"""Exact rational evaluation of the gated delta rule on tiny inputs.

TEST INFRASTRUCTURE ONLY. Pure-Python loops over fractions.Fraction, so it is
only for a handful of tokens at head dim <= 4. It is used by
``tests/golden/make_golden.py`` to write fixtures with no rounding at all.

It follows update form 2 of page "Qwen3.8-Flash-Next 技术总结", section 2.1
(Gated DeltaNet): S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T, with
a_t given directly as a rational in (0, 1] (not as a logarithm), and the
readout o_t = S_t^T q_t on the post-update state. One head, one sequence.
"""
from fractions import Fraction


def run(q, k, v, alpha, beta, s0):
    """q, k: T lists of dk Fractions; v: T lists of dv Fractions;
    alpha, beta: T Fractions; s0: dk x dv nested list of Fractions.
    Returns (o: T lists of dv Fractions, S_T: dk x dv nested list)."""
    dk = len(s0)
    dv = len(s0[0]) if dk else 0
    S = [[Fraction(x) for x in row] for row in s0]
    outs = []
    for t in range(len(alpha)):
        a, b, kt, vt, qt = alpha[t], beta[t], k[t], v[t], q[t]
        # (I - b k k^T) S, one entry at a time
        kS = [sum(kt[i] * S[i][j] for i in range(dk)) for j in range(dv)]
        S = [[a * (S[i][j] - b * kt[i] * kS[j]) + b * kt[i] * vt[j]
              for j in range(dv)] for i in range(dk)]
        outs.append([sum(S[i][j] * qt[i] for i in range(dk)) for j in range(dv)])
    return outs, S
