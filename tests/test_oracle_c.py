"""Pins of the C oracle (oracle/gdn_ref.c), no GPU.

The C oracle is a second, plain-C writing of update form 1 of page
"Qwen3.8-Flash-Next 技术总结", section 2.1 (the recurrence with readout
o_t = S_t^T q_t), used where the NumPy recurrence would take minutes. It is
tied here to things other than itself: the exact rational fixtures (update
form 2, no rounding at all), the NumPy form-1 and form-2 recurrences (which
test_oracle_pins.py pins to closed forms, LAPACK and those same fixtures),
the pure-decay closed form, and the one-token decode identity. Its inputs
are float32 numbers, so every comparison feeds both sides the same float32
values.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import c_ref as C
from oracle import gdn_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "exact_tiny.json")


def f32(x):
    return np.asarray(x, dtype=np.float32)


def rand_case(seed, lens, h_qk, h_v, dk, dv, init=True, beta_hi=1.0, la_lo=None):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    q = rng.standard_normal((T, h_qk, dk))
    k = rng.standard_normal((T, h_qk, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, h_v, dv))
    la = -np.logaddexp(0.0, rng.normal(-2.0, 1.0, (T, h_v)))
    if la_lo is not None:
        la = rng.uniform(la_lo, 0.0, (T, h_v))
    beta = beta_hi / (1.0 + np.exp(-rng.standard_normal((T, h_v))))
    s0 = rng.normal(0.0, 0.3, (len(lens), h_v, dk, dv)) if init else None
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return [f32(x) for x in (q, k, v, la, beta)] + [s0, cu]


def rel(x, y):
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


def test_c_oracle_matches_exact_rational_fixtures():
    with open(GOLDEN) as f:
        gold = json.load(f)
    for name, case in gold["cases"].items():
        fr = lambda x: np.array([[float(Fraction(y)) for y in row] for row in x])  # noqa: E731
        q, k, v = fr(case["q"]), fr(case["k"]), fr(case["v"])
        alpha = np.array([float(Fraction(x)) for x in case["alpha"]])
        beta = np.array([float(Fraction(x)) for x in case["beta"]])
        s0 = fr(case["s0"])
        o, s = C.recurrent_form1(q[:, None], k[:, None], v[:, None], np.log(alpha)[:, None],
                                 beta[:, None], s0[None, None], threads=1)
        # the inputs pass through float32 (about 6e-8 relative each)
        np.testing.assert_allclose(o[:, 0], fr(case["o"]), rtol=2e-6, atol=2e-6, err_msg=name)
        np.testing.assert_allclose(s[0, 0], fr(case["final"]), rtol=2e-6, atol=2e-6, err_msg=name)


@pytest.mark.parametrize("lens,h_qk,h_v,dk,dv,init", [
    ([37], 1, 1, 16, 16, False),
    ([50, 0, 13, 1], 2, 6, 16, 8, True),      # empty and one-token sequences, dk != dv
    ([70, 41], 1, 3, 32, 32, True),
    ([129], 4, 8, 8, 24, False),
])
def test_c_oracle_equals_numpy_form1_and_form2(lens, h_qk, h_v, dk, dv, init):
    q, k, v, la, b, s0, cu = rand_case(11 + len(lens), lens, h_qk, h_v, dk, dv, init)
    o_c, s_c = C.recurrent_form1(q, k, v, la, b, s0, cu, threads=3)
    for form in (O.recurrent_form1, O.recurrent_form2):
        o_n, s_n = form(q, k, v, la, b, s0, cu)
        assert rel(o_c, o_n) < 1e-12, form.__name__
        assert rel(s_c, s_n) < 1e-12, form.__name__


def test_c_oracle_wide_ranges():
    # beta up to 2 and log alpha down to -30 (alpha underflows toward 0)
    q, k, v, la, b, s0, cu = rand_case(5, [90, 30], 2, 4, 16, 16, True, beta_hi=2.0, la_lo=-30.0)
    o_c, s_c = C.recurrent_form1(q, k, v, la, b, s0, cu, threads=2)
    o_n, s_n = O.recurrent_form1(q, k, v, la, b, s0, cu)
    assert rel(o_c, o_n) < 1e-12 and rel(s_c, s_n) < 1e-12


def test_c_oracle_single_sequence_without_table_and_threads_agree():
    q, k, v, la, b, s0, cu = rand_case(7, [200], 2, 6, 16, 16, True)
    one = C.recurrent_form1(q, k, v, la, b, s0, None, threads=1)
    many = C.recurrent_form1(q, k, v, la, b, s0, cu, threads=4)
    for x, y in zip(one, many):
        assert np.array_equal(x, y)            # each pair runs the same loop, whatever the thread


def test_c_oracle_beta_zero_is_pure_decay():
    q, k, v, la, b, s0, cu = rand_case(9, [40, 25], 1, 2, 8, 8, True)
    b = np.zeros_like(b)
    o, s = C.recurrent_form1(q, k, v, la, b, s0, cu, threads=2)
    for n in range(2):
        t0, t1 = cu[n], cu[n + 1]
        decay = np.exp(np.sum(la[t0:t1].astype(np.float64), axis=0))    # [Hv]
        np.testing.assert_allclose(s[n], decay[:, None, None] * s0[n], rtol=1e-12, atol=1e-300)


def test_c_oracle_decode_steps_equal_single_steps():
    rng = np.random.default_rng(3)
    K, N, hq, hv, d = 5, 3, 1, 3, 8
    q = f32(rng.standard_normal((K, N, hq, d)))
    k = f32(rng.standard_normal((K, N, hq, d)) / np.sqrt(d))
    v = f32(rng.standard_normal((K, N, hv, d)))
    la = f32(-rng.uniform(0, 1, (K, N, hv)))
    b = f32(rng.uniform(0, 1, (K, N, hv)))
    s0 = rng.normal(0, 0.1, (N, hv, d, d))
    o_c, s_c = C.decode_steps(s0, q, k, v, la, b, threads=2)
    s = s0
    for t in range(K):
        o_t, s = O.decode_step(s, q[t], k[t], v[t], la[t], b[t])
        assert rel(o_c[t], o_t) < 1e-12
    assert rel(s_c, s) < 1e-12


def test_c_oracle_rejects_bad_tables():
    q, k, v, la, b, s0, cu = rand_case(1, [10, 10], 1, 1, 4, 4, False)
    for bad in ([0, 12, 10, 20], [1, 10, 20], [0, 10, 21]):
        with pytest.raises(ValueError):
            C.recurrent_form1(q, k, v, la, b, None, np.array(bad))
