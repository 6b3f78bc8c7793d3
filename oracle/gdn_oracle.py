"""fp64 NumPy oracle of the Gated DeltaNet token mixer.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, plain, and
independent of the HIP library.

Method source: page "Qwen3.8-Flash-Next 技术总结：Qwen4 架构的'探路者'",
section 2.1 "Gated DeltaNet", state-update equation:

  form 1 (first line):  S_t = a_t S_{t-1} + b_t k_t (v_t - a_t S_{t-1}^T k_t)^T
  form 2 (second line): S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T

with a_t the forget gate in (0,1) and b_t the write strength. S_t is a
dk x dv matrix (k_t v_t^T is dk x dv and S^T k is a dv-vector). Readings
where the page is silent (each one is listed with the design notes):

  R1 readout   o_t = S_t^T q_t with the post-update state, no 1/sqrt(d)
               scale; q and k arrive already normalised.
  R2 heads     V head h reads QK head h // (H_v / H_qk) (contiguous groups).
  R3 gates     a_t and b_t are per (token, V head); a_t is passed as
               log a_t <= 0 and b_t as any finite real.
  R4 sequences packed sequences (cu_seqlens) are independent; each starts
               from its own initial state (zeros when none is given).
  R5 chunks    the chunkwise evaluation restarts chunks at every sequence
               start; the last chunk of a sequence may be partial.
  R6 prep      fused input preparation (an option of the library): q and
               k arrive raw and are L2-normalised per (token, head) as
               x / sqrt(max(sum x^2, 1e-12)); the gates arrive as logits a,
               b with log a_t = -softplus(a) and b_t = sigmoid(b), the maps
               of the configured input recipe (a_t then lies in (0,1)).
  R7 variants  the section sets the gated delta rule against its two
               parents: the data-dependent forget gate alone (Mamba2) and
               the delta rule alone (DeltaNet). DeltaNet is a_t = 1 in
               form 1 (log a_t = 0, no separate code). The gate alone is
               form 1 without the correction term: the new value is added,
               not corrected, S_t = a_t S_{t-1} + b_t k_t v_t^T, keeping b_t
               as the write strength (b_t = 1 gives plain gated linear
               attention); readout as in R1.
  R8 gradients the pages train the layer but print no backward pass. The
               gradient of a scalar loss L is its definition: given dL/do
               for every token and dL/dS for each sequence's final state,
               backpropagation through the form-1 steps of R1, token by
               token in reverse, gives dL/dq, dL/dk, dL/dv, dL/dlog a, dL/db
               and dL/dS_0. A QK head's dq and dk sum over the V heads that
               read it.

Array conventions (all functions): q, k [T, Hqk, dk]; v [T, Hv, dv];
log_alpha, beta [T, Hv]; init_state / final_state [N, Hv, dk, dv];
o [T, Hv, dv]. Every input is upcast to float64 and every result is
float64.
"""
import numpy as np


def head_group(h_qk, h_v):
    """QK head used by each V head (reading R2): V head h -> h // (h_v/h_qk)."""
    if h_qk <= 0 or h_v <= 0 or h_v % h_qk:
        raise ValueError("h_v must be a positive multiple of h_qk")
    return np.arange(h_v) // (h_v // h_qk)


def seq_bounds(total_tokens, cu_seqlens):
    """(start, end) token ranges of the packed sequences (reading R4)."""
    if cu_seqlens is None:
        return [(0, int(total_tokens))]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


def prepare_inputs(q_raw, k_raw, a_logit, b_logit):
    """Reading R6: (q, k, log_alpha, beta) from raw q, k and gate logits.

    q, k are divided by their Euclidean norm over the last axis (the
    squared norm floored at 1e-12); log_alpha = -softplus(a) =
    -(max(a, 0) + log(1 + exp(-|a|))); beta = sigmoid(b) = 1 / (1 + exp(-b)),
    written in the overflow-free form for either sign of b.
    """
    def unit(x):
        x = np.asarray(x, dtype=np.float64)
        return x / np.sqrt(np.maximum(np.sum(x * x, axis=-1, keepdims=True), 1e-12))
    a = np.asarray(a_logit, dtype=np.float64)
    b = np.asarray(b_logit, dtype=np.float64)
    log_alpha = -(np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a))))
    e = np.exp(-np.abs(b))
    beta = np.where(b >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return unit(q_raw), unit(k_raw), log_alpha, beta


def _prep(q, k, v, log_alpha, beta, init_state, cu_seqlens):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    la = np.asarray(log_alpha, dtype=np.float64)
    b = np.asarray(beta, dtype=np.float64)
    T, h_qk, dk = q.shape
    h_v, dv = v.shape[1], v.shape[2]
    bounds = seq_bounds(T, cu_seqlens)
    n = len(bounds)
    if init_state is None:
        s0 = np.zeros((n, h_v, dk, dv))
    else:
        s0 = np.asarray(init_state, dtype=np.float64).reshape(n, h_v, dk, dv)
    return q, k, v, la, b, s0, bounds, head_group(h_qk, h_v)


def recurrent_form1(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None):
    """Token-serial recurrence, update form 1 of section 2.1, readout R1.

    For each sequence and V head: S <- S_0; per token
      a = exp(log_alpha), p = S^T k, u = b (v - a p), S <- a S + k u^T,
      o = S^T q.
    Returns (o [T,Hv,dv], final_state [N,Hv,dk,dv]).
    """
    q, k, v, la, b, s0, bounds, grp = _prep(q, k, v, log_alpha, beta,
                                            init_state, cu_seqlens)
    o = np.zeros(v.shape)
    final = np.empty_like(s0)
    for n, (t0, t1) in enumerate(bounds):
        S = s0[n].copy()                                  # [Hv, dk, dv]
        for t in range(t0, t1):
            a = np.exp(la[t])                             # [Hv]
            kt = k[t, grp]                                # [Hv, dk]
            qt = q[t, grp]
            pred = np.einsum("hkv,hk->hv", S, kt)         # S_{t-1}^T k_t
            u = b[t][:, None] * (v[t] - a[:, None] * pred)
            S = a[:, None, None] * S + kt[:, :, None] * u[:, None, :]
            o[t] = np.einsum("hkv,hk->hv", S, qt)         # S_t^T q_t
        final[n] = S
    return o, final


def recurrent_gated_no_delta(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None):
    """Token-serial recurrence of the gate-only variant (reading R7).

    For each sequence and V head: S <- S_0; per token
      a = exp(log_alpha), S <- a S + b k v^T, o = S^T q.
    Returns (o [T,Hv,dv], final_state [N,Hv,dk,dv]).
    """
    q, k, v, la, b, s0, bounds, grp = _prep(q, k, v, log_alpha, beta,
                                            init_state, cu_seqlens)
    o = np.zeros(v.shape)
    final = np.empty_like(s0)
    for n, (t0, t1) in enumerate(bounds):
        S = s0[n].copy()                                  # [Hv, dk, dv]
        for t in range(t0, t1):
            a = np.exp(la[t])                             # [Hv]
            kt = k[t, grp]                                # [Hv, dk]
            u = b[t][:, None] * v[t]                      # written as is
            S = a[:, None, None] * S + kt[:, :, None] * u[:, None, :]
            o[t] = np.einsum("hkv,hk->hv", S, q[t, grp])  # S_t^T q_t
        final[n] = S
    return o, final


def recurrent_form1_backward(q, k, v, log_alpha, beta, do, dfinal=None, init_state=None,
                             cu_seqlens=None):
    """Gradients through the form-1 recurrence (reading R8).

    do = dL/do [T,Hv,dv]; dfinal = dL/dS_final [N,Hv,dk,dv] or None (zero).
    Returns a dict: dq, dk [T,Hqk,dk]; dv [T,Hv,dv]; dlog_alpha, dbeta
    [T,Hv]; dinit [N,Hv,dk,dv]. Per token, with G = dL/dS_t carried from the
    end of the sequence backwards:
      o = S_t^T q             ->  G += q do^T,  dq += S_t do
      S_t = a S_{t-1} + k u^T ->  du = G^T k,  dk += G u,
                                  da = <S_{t-1}, G>,  dS_{t-1} = a G
      u = b (v - a p)         ->  db = (v - a p).du,  dv = b du,
                                  da -= b p.du,  dp = -a b du
      p = S_{t-1}^T k         ->  dS_{t-1} += k dp^T,  dk += S_{t-1} dp
      a = exp(log a)          ->  dlog a = a da
    and dL/dS_0 is G after the first token.
    """
    q, k, v, la, b, s0, bounds, grp = _prep(q, k, v, log_alpha, beta,
                                            init_state, cu_seqlens)
    do = np.asarray(do, dtype=np.float64)
    out = dict(dq=np.zeros(q.shape), dk=np.zeros(k.shape), dv=np.zeros(v.shape),
               dlog_alpha=np.zeros(la.shape), dbeta=np.zeros(b.shape), dinit=np.zeros(s0.shape))
    for n, (t0, t1) in enumerate(bounds):
        # forward pass, keeping the state before every token
        S = s0[n].copy()
        before = []
        for t in range(t0, t1):
            before.append(S)
            a = np.exp(la[t])
            kt = k[t, grp]
            pred = np.einsum("hkv,hk->hv", S, kt)
            u = b[t][:, None] * (v[t] - a[:, None] * pred)
            S = a[:, None, None] * S + kt[:, :, None] * u[:, None, :]
        G = np.zeros_like(S) if dfinal is None else np.asarray(dfinal, dtype=np.float64)[n].copy()
        for t in range(t1 - 1, t0 - 1, -1):
            Sp = before[t - t0]
            a = np.exp(la[t])
            kt = k[t, grp]
            qt = q[t, grp]
            pred = np.einsum("hkv,hk->hv", Sp, kt)
            resid = v[t] - a[:, None] * pred
            u = b[t][:, None] * resid
            St = a[:, None, None] * Sp + kt[:, :, None] * u[:, None, :]
            # readout
            G = G + qt[:, :, None] * do[t][:, None, :]
            dq_h = np.einsum("hkv,hv->hk", St, do[t])
            # state update
            du = np.einsum("hkv,hk->hv", G, kt)
            dk_h = np.einsum("hkv,hv->hk", G, u)
            da = np.sum(G * Sp, axis=(1, 2))
            Gp = a[:, None, None] * G
            # corrected value
            out["dbeta"][t] = np.sum(resid * du, axis=1)
            out["dv"][t] = b[t][:, None] * du
            da -= b[t] * np.sum(pred * du, axis=1)
            dp = -(a * b[t])[:, None] * du
            # prediction
            Gp += kt[:, :, None] * dp[:, None, :]
            dk_h += np.einsum("hkv,hv->hk", Sp, dp)
            out["dlog_alpha"][t] = a * da
            np.add.at(out["dq"][t], grp, dq_h)
            np.add.at(out["dk"][t], grp, dk_h)
            G = Gp
        out["dinit"][n] = G
    return out


def recurrent_form2(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None):
    """Token-serial recurrence, update form 2 of section 2.1, readout R1.

      S <- a (I - b k k^T) S + b k v^T,   o = S^T q.
    """
    q, k, v, la, b, s0, bounds, grp = _prep(q, k, v, log_alpha, beta,
                                            init_state, cu_seqlens)
    o = np.zeros(v.shape)
    final = np.empty_like(s0)
    dk = q.shape[2]
    eye = np.eye(dk)
    for n, (t0, t1) in enumerate(bounds):
        S = s0[n].copy()
        for t in range(t0, t1):
            a = np.exp(la[t])
            kt = k[t, grp]
            qt = q[t, grp]
            transition = eye[None] - b[t][:, None, None] * kt[:, :, None] * kt[:, None, :]
            S = a[:, None, None] * np.matmul(transition, S) \
                + b[t][:, None, None] * kt[:, :, None] * v[t][:, None, :]
            o[t] = np.einsum("hkv,hk->hv", S, qt)
        final[n] = S
    return o, final


def _forward_substitution_inverse(A):
    """(I + A)^{-1} for strictly lower-triangular A [..., L, L], row by row:
    row r of the inverse is e_r - sum_{i<r} A[r, i] * (row i of the inverse)."""
    L = A.shape[-1]
    Tm = np.zeros_like(A)
    for r in range(L):
        row = np.zeros(A.shape[:-2] + (L,))
        row[..., r] = 1.0
        if r:
            row -= np.einsum("...i,...ij->...j", A[..., r, :r], Tm[..., :r, :])
        Tm[..., r, :] = row
    return Tm


def chunkwise(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None,
              chunk=64, keep_stages=False):
    """Chunkwise (WY-representation) evaluation in fp64, reading R5.

    Section 2.1 names the chunkwise WY algorithm but prints no formulas; the
    steps below are derived from update form 1. For one V head and one chunk
    of L tokens entering with state S0 (r, i index tokens of the chunk):

      g_r   = sum_{j<=r} log a_j                  (in-chunk prefix sum)
      A[r,i]= b_r (k_r . k_i) exp(g_r - g_i)  for i < r, else 0
      Tinv  = (I + A)^{-1}                        (forward substitution)
      W     = Tinv diag(b * exp(g)) K             [L, dk]
      Ut    = Tinv diag(b) V                      [L, dv]
      U     = Ut - W S0                           (the delta rows u_r)
      O     = diag(exp(g)) Q S0 + (Q K^T * Dincl) U,
              Dincl[r,i] = exp(g_r - g_i) for i <= r, else 0
      S_end = exp(g_L) S0 + (exp(g_L - g) * K)^T U

    Returns (o, final_state, stages); stages is a list with one dict per
    chunk (keys seq, start, len, g, A, T, W, Ut, U, Sc, O) when keep_stages,
    else None. Arrays in a stage dict are [Hv, ...].
    """
    q, k, v, la, b, s0, bounds, grp = _prep(q, k, v, log_alpha, beta,
                                            init_state, cu_seqlens)
    o = np.zeros(v.shape)
    final = np.empty_like(s0)
    stages = [] if keep_stages else None
    for n, (t0, t1) in enumerate(bounds):
        S = s0[n].copy()                                   # [Hv, dk, dv]
        for c0 in range(t0, t1, chunk):
            c1 = min(c0 + chunk, t1)
            L = c1 - c0
            Kc = np.transpose(k[c0:c1, grp], (1, 0, 2))    # [Hv, L, dk]
            Qc = np.transpose(q[c0:c1, grp], (1, 0, 2))
            Vc = np.transpose(v[c0:c1], (1, 0, 2))         # [Hv, L, dv]
            bc = b[c0:c1].T                                # [Hv, L]
            g = np.cumsum(la[c0:c1].T, axis=1)             # [Hv, L]
            diff = g[:, :, None] - g[:, None, :]           # g_r - g_i
            rr, ii = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
            # exponentiate only where i <= r, so the exponent is <= 0
            d_incl = np.where(ii <= rr, np.exp(np.where(ii <= rr, diff, 0.0)), 0.0)
            d_strict = np.where(ii < rr, d_incl, 0.0)
            KK = np.matmul(Kc, np.transpose(Kc, (0, 2, 1)))
            A = bc[:, :, None] * KK * d_strict
            Tm = _forward_substitution_inverse(A)
            gam = np.exp(g)
            W = np.matmul(Tm, (bc * gam)[:, :, None] * Kc)
            Ut = np.matmul(Tm, bc[:, :, None] * Vc)
            U = Ut - np.matmul(W, S)
            QK = np.matmul(Qc, np.transpose(Kc, (0, 2, 1)))
            O = gam[:, :, None] * np.matmul(Qc, S) + np.matmul(QK * d_incl, U)
            o[c0:c1] = np.transpose(O, (1, 0, 2))
            if keep_stages:
                stages.append(dict(seq=n, start=c0, len=L, g=g, A=A, T=Tm, W=W,
                                   Ut=Ut, U=U, Sc=S.copy(), O=O))
            kdec = np.exp(g[:, -1:] - g)[:, :, None] * Kc
            S = np.exp(g[:, -1])[:, None, None] * S \
                + np.matmul(np.transpose(kdec, (0, 2, 1)), U)
        final[n] = S
    return o, final, stages


def decode_step(state, q, k, v, log_alpha, beta):
    """One token per sequence: update form 1 and readout R1.

    state [N, Hv, dk, dv]; q, k [N, Hqk, dk]; v [N, Hv, dv];
    log_alpha, beta [N, Hv]. Returns (o [N, Hv, dv], new_state); the input
    array is not modified.
    """
    n = np.asarray(q).shape[0]
    cu = np.arange(n + 1)
    return recurrent_form1(q, k, v, log_alpha, beta, init_state=state,
                           cu_seqlens=cu)


def decode_step_no_delta(state, q, k, v, log_alpha, beta):
    """One token per sequence of the gate-only variant (reading R7); same
    arguments and results as decode_step."""
    n = np.asarray(q).shape[0]
    cu = np.arange(n + 1)
    return recurrent_gated_no_delta(q, k, v, log_alpha, beta, init_state=state,
                                    cu_seqlens=cu)
