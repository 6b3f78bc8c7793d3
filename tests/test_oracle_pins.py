"""Pins of the CPU oracle to facts other than itself (no GPU).

Each test ties the fp64 oracle to something the page or plain mathematics
fixes: the two printed forms of the update (page "Qwen3.8-Flash-Next 技术总结",
section 2.1), closed forms, invariants, a LAPACK routine, brute force in exact
rational arithmetic, and hand-derived values. A plausible slip in the oracle
(dropped term, wrong sign, transposed state, wrong head map, off-by-one in the
chunk prefix sums, pre- instead of post-update readout) fails at least one.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import gdn_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "exact_tiny.json")


def rand_inputs(rng, T, h_qk, h_v, dk, dv, n_init=None, unit=True):
    q = rng.standard_normal((T, h_qk, dk))
    k = rng.standard_normal((T, h_qk, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, h_v, dv))
    la = -np.logaddexp(0.0, rng.normal(-2.0, 1.0, (T, h_v)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, h_v))))
    s0 = None
    if n_init is not None:
        s0 = rng.normal(0.0, 0.3, (n_init, h_v, dk, dv))
    return q, k, v, la, beta, s0


def rel(x, y):
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


# --- the two printed forms ------------------------------------------------

def test_form1_equals_form2():
    rng = np.random.default_rng(1)
    q, k, v, la, b, s0 = rand_inputs(rng, 50, 2, 6, 8, 5, n_init=2)
    cu = [0, 23, 50]
    o1, f1 = O.recurrent_form1(q, k, v, la, b, s0, cu)
    o2, f2 = O.recurrent_form2(q, k, v, la, b, s0, cu)
    assert rel(o1, o2) < 1e-13 and rel(f1, f2) < 1e-13


# --- closed forms and hand values -------------------------------------------

def test_single_token_by_hand():
    # S0 = 0: S_1 = b k v^T, o_1 = S_1^T q = b (k.q) v  (not b (v.q) k)
    rng = np.random.default_rng(2)
    q, k, v, la, b, _ = rand_inputs(rng, 1, 1, 1, 4, 3)
    o, s = O.recurrent_form1(q, k, v, la, b)
    np.testing.assert_allclose(s[0, 0], b[0, 0] * np.outer(k[0, 0], v[0, 0]),
                               rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[0, 0], b[0, 0] * (k[0, 0] @ q[0, 0]) * v[0, 0],
                               rtol=1e-13, atol=1e-15)
    # nonzero S0: S_1 = a S0 + b k (v - a S0^T k)^T
    s0 = rng.standard_normal((1, 1, 4, 3))
    o, s = O.recurrent_form1(q, k, v, la, b, s0)
    a = np.exp(la[0, 0])
    S0 = s0[0, 0]
    want = a * S0 + b[0, 0] * np.outer(k[0, 0], v[0, 0] - a * S0.T @ k[0, 0])
    np.testing.assert_allclose(s[0, 0], want, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o[0, 0], want.T @ q[0, 0], rtol=1e-13, atol=1e-14)


def test_scalar_geometric_closed_form():
    # dk = dv = 1, constant a, b, k, v, q: s_t = rho s_{t-1} + b k v with
    # rho = a (1 - b k^2), so s_t = rho^t s0 + b k v (1 - rho^t) / (1 - rho)
    T, a, b, kk, vv, qq, s0 = 37, 0.93, 0.6, 0.8, -1.7, 0.45, 0.25
    q = np.full((T, 1, 1), qq)
    k = np.full((T, 1, 1), kk)
    v = np.full((T, 1, 1), vv)
    la = np.full((T, 1), np.log(a))
    beta = np.full((T, 1), b)
    o, s = O.recurrent_form1(q, k, v, la, beta, np.full((1, 1, 1, 1), s0))
    rho = a * (1 - b * kk * kk)
    t = np.arange(1, T + 1)
    st = rho ** t * s0 + b * kk * vv * (1 - rho ** t) / (1 - rho)
    np.testing.assert_allclose(o[:, 0, 0], st * qq, rtol=1e-12)
    np.testing.assert_allclose(s[0, 0, 0, 0], st[-1], rtol=1e-12)


def test_constant_key_direction_closed_form():
    # unit k fixed: along k, k^T S_t = rho^t k^T S0 + b v^T (1-rho^t)/(1-rho)
    # with rho = a (1 - b); across k, (I - k k^T) S_t = a^t (I - k k^T) S0.
    rng = np.random.default_rng(3)
    T, dk, dv, a, b = 25, 6, 4, 0.9, 0.35
    kk = rng.standard_normal(dk)
    kk /= np.linalg.norm(kk)
    vv = rng.standard_normal(dv)
    S0 = rng.standard_normal((dk, dv))
    q = np.tile(rng.standard_normal(dk), (T, 1, 1))
    k = np.tile(kk, (T, 1, 1))
    v = np.tile(vv, (T, 1, 1))
    la = np.full((T, 1), np.log(a))
    beta = np.full((T, 1), b)
    _, s = O.recurrent_form1(q, k, v, la, beta, S0[None, None])
    rho = a * (1 - b)
    along = rho ** T * (kk @ S0) + b * vv * (1 - rho ** T) / (1 - rho)
    perp = np.eye(dk) - np.outer(kk, kk)
    np.testing.assert_allclose(kk @ s[0, 0], along, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(perp @ s[0, 0], a ** T * perp @ S0,
                               rtol=1e-11, atol=1e-13)


def test_beta_zero_is_pure_decay():
    # b = 0: S_t = a_t S_{t-1}, so S_t = exp(sum log a) S0 and o_t = S_t^T q_t
    rng = np.random.default_rng(4)
    q, k, v, la, b, s0 = rand_inputs(rng, 40, 2, 4, 8, 8, n_init=1)
    b[:] = 0.0
    for fn in (O.recurrent_form1, O.recurrent_form2):
        o, s = fn(q, k, v, la, b, s0)
        g = np.cumsum(la, axis=0)                                 # [T, Hv]
        grp = O.head_group(2, 4)
        want_o = np.exp(g)[:, :, None] * np.einsum(
            "hkv,thk->thv", s0[0], q[:, grp])
        np.testing.assert_allclose(o, want_o, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(s[0], np.exp(g[-1])[:, None, None] * s0[0],
                                   rtol=1e-12)


def test_exact_recall_unit_key():
    # a = 1, b = 1, |k| = 1: S_t^T k_t = v_t; reading with q_t = k_t returns v_t
    rng = np.random.default_rng(5)
    q, k, v, la, b, s0 = rand_inputs(rng, 30, 1, 3, 16, 16, n_init=1)
    la[:] = 0.0
    b[:] = 1.0
    o, _ = O.recurrent_form1(k, k, v, la, b, s0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_alpha_one_is_plain_delta_rule():
    # a = 1: S_t = S_{t-1} + b k (v - S_{t-1}^T k)^T, i.e. DeltaNet; check on a
    # case where the delta rule's fixed point is known: repeating the same
    # (k, v) with b in (0, 2) drives S^T k to v geometrically: the error
    # e_t = v - S_t^T k obeys e_t = (1 - b) e_{t-1} for |k| = 1.
    rng = np.random.default_rng(6)
    dk, dv, T, b = 8, 5, 12, 0.7
    kk = rng.standard_normal(dk)
    kk /= np.linalg.norm(kk)
    vv = rng.standard_normal(dv)
    S0 = rng.standard_normal((dk, dv))
    k = np.tile(kk, (T, 1, 1))
    v = np.tile(vv, (T, 1, 1))
    o, s = O.recurrent_form1(k, k, v, np.zeros((T, 1)), np.full((T, 1), b),
                             S0[None, None])
    e0 = vv - S0.T @ kk
    t = np.arange(1, T + 1)
    np.testing.assert_allclose(vv - o[:, 0], (1 - b) ** t[:, None] * e0,
                               rtol=1e-10, atol=1e-13)


def test_householder_product_is_qr_q():
    # a = 1, v = 0, S0 = I, k_t = LAPACK Householder vector t, b_t = tau_t:
    # S_n = H_n ... H_1 = (H_1 ... H_n)^T = Q^T of the QR factorisation.
    rng = np.random.default_rng(7)
    n = 6
    M = rng.standard_normal((n, n))
    h, tau = np.linalg.qr(M, mode="raw")
    ref = h.T                           # LAPACK layout: reflectors below diag
    Q, _ = np.linalg.qr(M)
    k = np.zeros((n, 1, n))
    for i in range(n):
        k[i, 0, i] = 1.0
        k[i, 0, i + 1:] = ref[i + 1:, i]
    q = rng.standard_normal((n, 1, n))
    v = np.zeros((n, 1, n))
    la = np.zeros((n, 1))
    beta = tau.reshape(n, 1).astype(np.float64)
    for fn in (O.recurrent_form1, O.recurrent_form2):
        _, s = fn(q, k, v, la, beta, np.eye(n)[None, None])
        np.testing.assert_allclose(s[0, 0], Q.T, rtol=0, atol=1e-13)


def test_exact_rational_golden():
    with open(GOLDEN) as f:
        gold = json.load(f)
    for name, case in gold["cases"].items():
        fr = lambda x: np.array([[float(Fraction(y)) for y in row] for row in x])  # noqa: E731
        q, k, v = fr(case["q"]), fr(case["k"]), fr(case["v"])
        alpha = np.array([float(Fraction(x)) for x in case["alpha"]])
        beta = np.array([float(Fraction(x)) for x in case["beta"]])
        s0 = fr(case["s0"])
        o, s = O.recurrent_form1(q[:, None], k[:, None], v[:, None],
                                 np.log(alpha)[:, None], beta[:, None],
                                 s0[None, None])
        np.testing.assert_allclose(o[:, 0], fr(case["o"]), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(s[0, 0], fr(case["final"]), rtol=1e-13,
                                   atol=1e-15)
    # first token of case a by hand: S1 = b k v^T = [[3/10,-3/5],[2/5,-4/5]]
    a = gold["cases"]["a"]
    assert [Fraction(x) for x in a["o"][0]] == [Fraction(3, 10), Fraction(-3, 5)]


# --- chunkwise evaluation -----------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 2, 16, 64, 200])
def test_chunkwise_equals_recurrence(chunk):
    rng = np.random.default_rng(8)
    q, k, v, la, b, s0 = rand_inputs(rng, 200, 2, 6, 16, 12, n_init=3)
    cu = [0, 77, 77, 200]               # includes an empty sequence
    o1, f1 = O.recurrent_form1(q, k, v, la, b, s0, cu)
    o3, f3, _ = O.chunkwise(q, k, v, la, b, s0, cu, chunk=chunk)
    assert rel(o3, o1) < 1e-12 and rel(f3, f1) < 1e-12
    np.testing.assert_array_equal(f3[1], s0[1])        # empty: final = init


def test_forward_substitution_matches_inverse():
    rng = np.random.default_rng(9)
    A = np.tril(rng.standard_normal((3, 64, 64)) * 0.2, k=-1)
    Tm = O._forward_substitution_inverse(A)
    want = np.linalg.inv(np.eye(64)[None] + A)
    np.testing.assert_allclose(Tm, want, rtol=0, atol=1e-9 * np.abs(want).max())


def test_chunk_stages_match_recurrence_quantities():
    # U rows are the delta vectors u_r = b_r (v_r - a_r S_{r-1}^T k_r) of form 1
    # and Sc is the form-1 state at the chunk start.
    rng = np.random.default_rng(10)
    q, k, v, la, b, s0 = rand_inputs(rng, 40, 1, 3, 8, 8, n_init=1)
    _, _, stages = O.chunkwise(q, k, v, la, b, s0, chunk=16, keep_stages=True)
    grp = O.head_group(1, 3)
    S = s0[0].copy()
    t = 0
    for st in stages:
        np.testing.assert_allclose(st["Sc"], S, rtol=1e-12, atol=1e-14)
        for r in range(st["len"]):
            a = np.exp(la[t])
            kt = k[t, grp]
            u = b[t][:, None] * (v[t] - a[:, None] * np.einsum("hkv,hk->hv", S, kt))
            np.testing.assert_allclose(st["U"][:, r], u, rtol=1e-11, atol=1e-13)
            _, S1 = O.recurrent_form1(q[t:t + 1], k[t:t + 1], v[t:t + 1],
                                      la[t:t + 1], b[t:t + 1], S[None])
            S = S1[0]
            t += 1
        # g is the inclusive in-chunk prefix sum of log a
        np.testing.assert_allclose(
            st["g"], np.cumsum(la[st["start"]:st["start"] + st["len"]].T, axis=1))


# --- structural invariants ------------------------------------------------------

def test_state_carry_split():
    rng = np.random.default_rng(11)
    q, k, v, la, b, s0 = rand_inputs(rng, 96, 2, 6, 8, 8, n_init=1)
    o, f = O.recurrent_form1(q, k, v, la, b, s0)
    oa, fa = O.recurrent_form1(q[:41], k[:41], v[:41], la[:41], b[:41], s0)
    ob, fb = O.recurrent_form1(q[41:], k[41:], v[41:], la[41:], b[41:], fa)
    np.testing.assert_array_equal(np.concatenate([oa, ob]), o)
    np.testing.assert_array_equal(fb, f)
    # chunkwise, split on a chunk boundary
    o3, f3, _ = O.chunkwise(q, k, v, la, b, s0, chunk=16)
    a3, fa3, _ = O.chunkwise(q[:48], k[:48], v[:48], la[:48], b[:48], s0, chunk=16)
    b3, fb3, _ = O.chunkwise(q[48:], k[48:], v[48:], la[48:], b[48:], fa3, chunk=16)
    np.testing.assert_array_equal(np.concatenate([a3, b3]), o3)
    np.testing.assert_array_equal(fb3, f3)


def test_varlen_equals_separate_runs():
    rng = np.random.default_rng(12)
    lens = [5, 33, 1, 20]
    q, k, v, la, b, s0 = rand_inputs(rng, sum(lens), 1, 3, 8, 8, n_init=4)
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, f = O.recurrent_form1(q, k, v, la, b, s0, cu)
    for n in range(4):
        sl = slice(cu[n], cu[n + 1])
        on, fn = O.recurrent_form1(q[sl], k[sl], v[sl], la[sl], b[sl], s0[n:n + 1])
        np.testing.assert_array_equal(o[sl], on)
        np.testing.assert_array_equal(f[n], fn[0])


def test_head_sharing_equals_single_heads():
    # h_qk = 1 shared by h_v = 3 equals three runs with the QK head replicated
    rng = np.random.default_rng(13)
    q, k, v, la, b, s0 = rand_inputs(rng, 30, 1, 3, 8, 8, n_init=1)
    o, f = O.recurrent_form1(q, k, v, la, b, s0)
    for h in range(3):
        oh, fh = O.recurrent_form1(q, k, v[:, h:h + 1], la[:, h:h + 1],
                                   b[:, h:h + 1], s0[:, h:h + 1])
        np.testing.assert_allclose(o[:, h], oh[:, 0], rtol=1e-15, atol=0)
        np.testing.assert_allclose(f[0, h], fh[0, 0], rtol=1e-15, atol=0)
    # and V heads 3..5 of a 2-QK-head layout read QK head 1
    assert list(O.head_group(2, 6)) == [0, 0, 0, 1, 1, 1]


def test_linear_in_state_and_values():
    rng = np.random.default_rng(14)
    q, k, v, la, b, s0 = rand_inputs(rng, 30, 1, 2, 8, 8, n_init=1)
    v2 = rng.standard_normal(v.shape)
    s2 = rng.standard_normal(s0.shape)
    c1, c2 = 0.7, -1.3
    oa, fa = O.recurrent_form1(q, k, v, la, b, s0)
    ob, fb = O.recurrent_form1(q, k, v2, la, b, s2)
    oc, fc = O.recurrent_form1(q, k, c1 * v + c2 * v2, la, b, c1 * s0 + c2 * s2)
    np.testing.assert_allclose(oc, c1 * oa + c2 * ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fc, c1 * fa + c2 * fb, rtol=1e-12, atol=1e-12)


def test_padding_tokens_are_noops():
    # log a = 0 and b = 0 leave the state exactly unchanged
    rng = np.random.default_rng(15)
    q, k, v, la, b, s0 = rand_inputs(rng, 10, 1, 2, 4, 4, n_init=1)
    la[5:] = 0.0
    b[5:] = 0.0
    _, f5 = O.recurrent_form1(q[:5], k[:5], v[:5], la[:5], b[:5], s0)
    _, f10 = O.recurrent_form1(q, k, v, la, b, s0)
    np.testing.assert_array_equal(f5, f10)


def test_decode_steps_equal_prefill():
    rng = np.random.default_rng(16)
    N, steps = 3, 20
    q, k, v, la, b, _ = rand_inputs(rng, N * steps, 2, 6, 8, 8)
    s0 = rng.normal(0, 0.1, (N, 6, 8, 8))
    # token layout for prefill: sequence n holds tokens n*steps .. n*steps+steps-1
    cu = np.arange(N + 1) * steps
    o_pf, f_pf, _ = O.chunkwise(q, k, v, la, b, s0, cu, chunk=8)
    S = s0
    for t in range(steps):
        idx = np.arange(N) * steps + t
        o_t, S = O.decode_step(S, q[idx], k[idx], v[idx], la[idx], b[idx])
        np.testing.assert_allclose(o_t, o_pf[idx], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(S, f_pf, rtol=1e-11, atol=1e-13)


# --- fused input preparation (reading R6) ---------------------------------

def test_prepare_inputs_unit_norm_and_scale_invariance():
    rng = np.random.default_rng(60)
    q = rng.standard_normal((7, 3, 16))
    k = rng.standard_normal((7, 3, 16)) * 5.0
    qn, kn, _, _ = O.prepare_inputs(q, k, np.zeros((7, 2)), np.zeros((7, 2)))
    assert np.allclose(np.linalg.norm(qn, axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(np.linalg.norm(kn, axis=-1), 1.0, rtol=0, atol=1e-14)
    # direction kept: a positive rescaling of the input changes nothing
    qn2, kn2, _, _ = O.prepare_inputs(3.7 * q, 0.01 * k, np.zeros((7, 2)), np.zeros((7, 2)))
    assert np.allclose(qn2, qn, rtol=0, atol=1e-14) and np.allclose(kn2, kn, rtol=0, atol=1e-14)
    assert np.all(np.sum(qn * q, axis=-1) > 0)
    # a zero vector stays zero (the floor on the squared norm)
    z, _, _, _ = O.prepare_inputs(np.zeros((1, 1, 4)), np.ones((1, 1, 4)), np.zeros((1, 1)), np.zeros((1, 1)))
    assert np.all(z == 0)


def test_prepare_inputs_gates_match_library_routines():
    from scipy.special import expit
    a = np.concatenate([np.linspace(-60, 60, 241), np.random.default_rng(61).normal(-2, 1, 50)])
    b = np.concatenate([np.linspace(-60, 60, 241), np.random.default_rng(62).normal(0, 1, 50)])
    _, _, la, beta = O.prepare_inputs(np.ones((1, 1, 2)), np.ones((1, 1, 2)), a, b)
    # log a = -softplus(a) = -log(1 + e^a) (numpy's logaddexp) = log(sigmoid(-a)); b = sigmoid(b)
    assert np.allclose(la, -np.logaddexp(0.0, a), rtol=1e-12, atol=0)
    from scipy.special import log_expit
    assert np.allclose(la, log_expit(-a), rtol=1e-12, atol=0)
    assert np.allclose(beta, expit(b), rtol=1e-12, atol=1e-300)
    assert np.all(la < 0) and np.all(np.isfinite(la))
    assert np.all((beta > 0) & (beta < 1) | (np.abs(b) > 36))
    # the identity sigmoid(b) + sigmoid(-b) = 1 and the asymptote -softplus(a) ~ -a for large a
    _, _, _, beta_neg = O.prepare_inputs(np.ones((1, 1, 2)), np.ones((1, 1, 2)), a, -b)
    assert np.allclose(beta + beta_neg, 1.0, rtol=0, atol=1e-15)
    assert abs(la[-51] + 60.0) < 1e-25 + 1e-12 * 60


def test_prepared_inputs_give_unit_keys_so_recall_is_exact():
    # with prepared (unit) keys, b = 1 (logit +inf approximated by a large
    # value is avoided: use b logits that give b = 1/2) the state stays
    # finite and o matches the recurrence on the prepared arrays
    rng = np.random.default_rng(63)
    T, hq, hv, d = 9, 1, 2, 8
    q, k, la, beta = O.prepare_inputs(rng.standard_normal((T, hq, d)), rng.standard_normal((T, hq, d)),
                                      rng.normal(-2, 1, (T, hv)), rng.normal(0, 1, (T, hv)))
    v = rng.standard_normal((T, hv, d))
    o1, s1 = O.recurrent_form1(q, k, v, la, beta)
    o2, s2 = O.recurrent_form2(q, k, v, la, beta)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-13) and np.allclose(s1, s2, rtol=1e-12, atol=1e-13)
    assert np.all(np.abs(s1) < 1e3)


# --- gate-only variant (reading R7: S <- a S + b k v^T, o = S^T q) ---------

def test_gate_only_equals_masked_attention_closed_form():
    # Unrolling S_t = a_t S_{t-1} + b_t k_t v_t^T gives, with G the running
    # sum of log a over the sequence,
    #   o_t = exp(G_t) S_0^T q_t + sum_{i<=t} exp(G_t - G_i) b_i (q_t . k_i) v_i
    #   S_T = exp(G_T) S_0 + sum_i exp(G_T - G_i) b_i k_i v_i^T,
    # evaluated here as one dense masked product per head.
    rng = np.random.default_rng(41)
    T, h_qk, h_v, d = 23, 2, 4, 5
    q, k, v, la, beta, s0 = rand_inputs(rng, T, h_qk, h_v, d, d, n_init=1)
    o, fin = O.recurrent_gated_no_delta(q, k, v, la, beta, s0)
    for h in range(h_v):
        hq = h // (h_v // h_qk)
        G = np.cumsum(la[:, h])
        mask = np.tril(np.exp(G[:, None] - G[None, :]))
        scores = (q[:, hq] @ k[:, hq].T) * mask
        want_o = scores @ (beta[:, h, None] * v[:, h]) + np.exp(G)[:, None] * (q[:, hq] @ s0[0, h])
        w = np.exp(G[-1] - G) * beta[:, h]
        want_s = np.exp(G[-1]) * s0[0, h] + k[:, hq].T @ (w[:, None] * v[:, h])
        assert rel(o[:, h], want_o) < 1e-12
        assert rel(fin[0, h], want_s) < 1e-12


def test_gate_only_is_causal_linear_attention_when_a_b_are_one():
    # a = b = 1, S_0 = 0: o_t = sum_{i<=t} (q_t . k_i) v_i, written as a loop
    # over pairs
    rng = np.random.default_rng(42)
    T, d = 9, 3
    q, k, v, _, _, _ = rand_inputs(rng, T, 1, 1, d, d, unit=False)
    o, _ = O.recurrent_gated_no_delta(q, k, v, np.zeros((T, 1)), np.ones((T, 1)))
    for t in range(T):
        want = sum(float(q[t, 0] @ k[i, 0]) * v[i, 0] for i in range(t + 1))
        assert np.allclose(o[t, 0], want, rtol=0, atol=1e-13)


def test_gate_only_equals_delta_rule_for_orthogonal_fresh_keys():
    # With S_0 = 0 and mutually orthogonal keys, S_{t-1}^T k_t = 0 at every
    # step, so the delta rule's correction vanishes and both rules agree;
    # with a repeated key they must differ.
    rng = np.random.default_rng(43)
    T, d = 6, 8
    q, _, v, la, beta, _ = rand_inputs(rng, T, 1, 2, d, d)
    k = np.zeros((T, 1, d))
    for t, j in enumerate(rng.permutation(d)[:T]):
        k[t, 0, j] = 1.0
    o1, f1 = O.recurrent_form1(q, k, v, la, beta)
    o2, f2 = O.recurrent_gated_no_delta(q, k, v, la, beta)
    assert rel(o2, o1) < 1e-14 and rel(f2, f1) < 1e-14
    k[3] = k[1]
    o1, _ = O.recurrent_form1(q, k, v, la, beta)
    o2, _ = O.recurrent_gated_no_delta(q, k, v, la, beta)
    assert rel(o2, o1) > 1e-3


def test_gate_only_decode_steps_equal_prefill():
    rng = np.random.default_rng(44)
    T, h_qk, h_v, d = 7, 1, 3, 4
    q, k, v, la, beta, s0 = rand_inputs(rng, T, h_qk, h_v, d, d, n_init=1)
    want_o, want_f = O.recurrent_gated_no_delta(q, k, v, la, beta, s0)
    S = s0
    for t in range(T):
        o, S = O.decode_step_no_delta(S, q[t:t + 1], k[t:t + 1], v[t:t + 1], la[t:t + 1], beta[t:t + 1])
        assert rel(o[0], want_o[t]) < 1e-13
    assert rel(S, want_f) < 1e-13


# --- gradients (reading R8: backpropagation through form 1) ----------------

def _loss(q, k, v, la, beta, s0, cu, ro, rf):
    o, fin = O.recurrent_form1(q, k, v, la, beta, s0, cu)
    return float(np.sum(o * ro) + np.sum(fin * rf))


def test_backward_equals_central_differences_on_every_input():
    # L = <o, R_o> + <S_final, R_f>; each partial derivative is checked by a
    # central difference of the forward oracle (step 1e-5, error O(1e-10))
    rng = np.random.default_rng(51)
    lens = [3, 2]
    T, h_qk, h_v, d = sum(lens), 1, 2, 3
    q, k, v, la, beta, s0 = rand_inputs(rng, T, h_qk, h_v, d, d, n_init=2)
    beta = beta * 1.5                       # b over (0, 1.5): exercises b > 1 too
    cu = np.array([0, 3, 5])
    ro = rng.standard_normal((T, h_v, d))
    rf = rng.standard_normal((2, h_v, d, d))
    g = O.recurrent_form1_backward(q, k, v, la, beta, ro, rf, s0, cu)
    args = dict(q=q, k=k, v=v, la=la, beta=beta, s0=s0)
    names = dict(q="dq", k="dk", v="dv", la="dlog_alpha", beta="dbeta", s0="dinit")
    eps = 1e-5
    for name, x in args.items():
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = _loss(cu=cu, ro=ro, rf=rf, **args)
            x[idx] = keep - eps
            lm = _loss(cu=cu, ro=ro, rf=rf, **args)
            x[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        assert rel(g[names[name]], num) < 1e-8, name


def test_backward_with_head_groups_and_no_final_gradient():
    # two V heads per QK head: dq and dk sum over the group; dfinal = None
    rng = np.random.default_rng(52)
    T, h_qk, h_v, d = 4, 2, 4, 2
    q, k, v, la, beta, s0 = rand_inputs(rng, T, h_qk, h_v, d, d, n_init=1)
    ro = rng.standard_normal((T, h_v, d))
    g = O.recurrent_form1_backward(q, k, v, la, beta, ro, None, s0)
    eps = 1e-5
    for name, x in (("dq", q), ("dk", k)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = _loss(q, k, v, la, beta, s0, None, ro, 0.0)
            x[idx] = keep - eps
            lm = _loss(q, k, v, la, beta, s0, None, ro, 0.0)
            x[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        assert rel(g[name], num) < 1e-8, name


def test_backward_closed_form_for_pure_decay():
    # b = 0 and do = 0: S_T = exp(sum log a) S_0, so dL/dS_0 = exp(sum log a) R
    # and dL/dlog a_t = <S_T, R> for every token; nothing else has gradient
    rng = np.random.default_rng(53)
    T, d = 6, 4
    q, k, v, la, _, s0 = rand_inputs(rng, T, 1, 1, d, d, n_init=1)
    beta = np.zeros((T, 1))
    R = rng.standard_normal((1, 1, d, d))
    g = O.recurrent_form1_backward(q, k, v, la, beta, np.zeros((T, 1, d)), R, s0)
    decay = np.exp(la[:, 0].sum())
    assert rel(g["dinit"], decay * R) < 1e-14
    assert np.allclose(g["dlog_alpha"][:, 0], np.sum(decay * s0 * R), rtol=1e-13, atol=0)
    for name in ("dq", "dk", "dv"):
        assert np.abs(g[name]).max() == 0.0
