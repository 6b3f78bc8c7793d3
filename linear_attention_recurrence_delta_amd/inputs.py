"""Seeded synthetic inputs for the Gated DeltaNet mixer.

This module holds only the input recipe (random draws and their shaping); it
contains none of the method's arithmetic, and both the HIP-path tests and the
CPU oracle receive the same tensors from it. It imports neither the binding
nor the oracle.

Recipe (head layout from page "Qwen3.8-Flash-Next 技术总结", section 2.1:
48 V heads, 16 QK heads, head dim 128):
  q, k       ~ N(0, 1), then L2-normalised per (token, QK head)
  v          ~ N(0, 1)
  log_alpha  = -softplus(N(-2, 1)) per (token, V head)    (alpha in (0, 1))
  beta       = sigmoid(N(0, 1)) per (token, V head)
  init state ~ N(0, 0.02^2) per entry, when asked for
Draws use numpy's default_rng(seed) in float64 in the fixed order
q, k, v, log_alpha, beta, init; q/k/v are then cast to the requested dtype
by torch (round to nearest even for bfloat16). log_alpha, beta and states
are float32.
"""
import numpy as np
import torch

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _softplus(x):
    return np.logaddexp(0.0, x)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_prefill(seed, seq_lens, h_qk, h_v, d, dtype="bf16", init="zeros"):
    """Packed prefill inputs for sequences of the given lengths.

    init: "zeros" -> init_state None; "randn" -> N(0, 0.02^2) per sequence.
    Returns a dict of CPU tensors: q, k [T,h_qk,d]; v [T,h_v,d];
    log_alpha, beta [T,h_v] f32; init_state [N,h_v,d,d] f32 or None;
    cu_seqlens int32 [N+1].
    """
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in seq_lens]
    T = int(sum(lens))
    tdt = _DTYPES[dtype]
    q = _unit_rows(rng.standard_normal((T, h_qk, d)))
    k = _unit_rows(rng.standard_normal((T, h_qk, d)))
    v = rng.standard_normal((T, h_v, d))
    la = -_softplus(rng.normal(-2.0, 1.0, (T, h_v)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, h_v))))
    init_state = None
    if init == "randn":
        init_state = torch.from_numpy(
            rng.normal(0.0, 0.02, (len(lens), h_v, d, d)).astype(np.float32))
    elif init != "zeros":
        raise ValueError(init)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return dict(
        q=torch.from_numpy(q).to(tdt),
        k=torch.from_numpy(k).to(tdt),
        v=torch.from_numpy(v).to(tdt),
        log_alpha=torch.from_numpy(la.astype(np.float32)),
        beta=torch.from_numpy(beta.astype(np.float32)),
        init_state=init_state,
        cu_seqlens=torch.from_numpy(cu),
    )


def make_varlen_lengths(seed, n, lo, hi):
    """n integer lengths uniform in [lo, hi] (inclusive)."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


def make_decode(seed, batch, steps, h_qk, h_v, d, dtype="bf16"):
    """Inputs for `steps` successive single-token decode steps.

    Returns dict: state0 [batch,h_v,d,d] f32 ~ N(0, 0.02^2); and per-step
    stacks q, k [steps,batch,h_qk,d]; v [steps,batch,h_v,d];
    log_alpha, beta [steps,batch,h_v] f32.
    """
    rng = np.random.default_rng(seed)
    tdt = _DTYPES[dtype]
    state0 = rng.normal(0.0, 0.02, (batch, h_v, d, d)).astype(np.float32)
    q = _unit_rows(rng.standard_normal((steps, batch, h_qk, d)))
    k = _unit_rows(rng.standard_normal((steps, batch, h_qk, d)))
    v = rng.standard_normal((steps, batch, h_v, d))
    la = -_softplus(rng.normal(-2.0, 1.0, (steps, batch, h_v)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((steps, batch, h_v))))
    return dict(
        state0=torch.from_numpy(state0),
        q=torch.from_numpy(q).to(tdt),
        k=torch.from_numpy(k).to(tdt),
        v=torch.from_numpy(v).to(tdt),
        log_alpha=torch.from_numpy(la.astype(np.float32)),
        beta=torch.from_numpy(beta.astype(np.float32)),
    )


def make_backward_seeds(seed, seq_lens, h_v, d, dtype="bf16"):
    """Upstream gradients for the backward pass: d_o = dL/do ~ N(0, 1)
    [T, h_v, d] in the input dtype, and d_final = dL/d(final state) ~ N(0, 1)
    [N, h_v, d, d] fp32 (a loss L = <o, R_o> + <S_final, R_f> with Gaussian
    R). Draw order: d_o, d_final."""
    rng = np.random.default_rng(seed)
    T = int(sum(int(x) for x in seq_lens))
    d_o = torch.from_numpy(rng.standard_normal((T, h_v, d))).to(_DTYPES[dtype])
    d_final = torch.from_numpy(rng.standard_normal((len(seq_lens), h_v, d, d)).astype(np.float32))
    return dict(d_o=d_o, d_final=d_final)


def make_prefill_raw(seed, seq_lens, h_qk, h_v, d, dtype="bf16", init="zeros"):
    """Raw inputs for fused input preparation: q, k ~ N(0, 1) times a
    per-(token, head) scale exp(N(0, 0.5^2)) (not normalised), v ~ N(0, 1),
    gate logits a ~ N(-2, 1) and b ~ N(0, 1) in the log_alpha and beta
    slots, init as in make_prefill. Draw order: q, k, v, a, b, init, the q
    scales, the k scales. Same keys and shapes as make_prefill."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in seq_lens]
    T = int(sum(lens))
    tdt = _DTYPES[dtype]
    q = rng.standard_normal((T, h_qk, d))
    k = rng.standard_normal((T, h_qk, d))
    v = rng.standard_normal((T, h_v, d))
    a = rng.normal(-2.0, 1.0, (T, h_v))
    b = rng.standard_normal((T, h_v))
    init_state = None
    if init == "randn":
        init_state = torch.from_numpy(
            rng.normal(0.0, 0.02, (len(lens), h_v, d, d)).astype(np.float32))
    elif init != "zeros":
        raise ValueError(init)
    q = q * np.exp(rng.normal(0.0, 0.5, (T, h_qk, 1)))
    k = k * np.exp(rng.normal(0.0, 0.5, (T, h_qk, 1)))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return dict(
        q=torch.from_numpy(q).to(tdt),
        k=torch.from_numpy(k).to(tdt),
        v=torch.from_numpy(v).to(tdt),
        log_alpha=torch.from_numpy(a.astype(np.float32)),
        beta=torch.from_numpy(b.astype(np.float32)),
        init_state=init_state,
        cu_seqlens=torch.from_numpy(cu),
    )


def make_decode_raw(seed, batch, steps, h_qk, h_v, d, dtype="bf16"):
    """Raw decode inputs for fused input preparation (see
    make_prefill_raw); same keys and shapes as make_decode. Draw order:
    state0, q, k, v, a, b, the q scales, the k scales."""
    rng = np.random.default_rng(seed)
    tdt = _DTYPES[dtype]
    state0 = rng.normal(0.0, 0.02, (batch, h_v, d, d)).astype(np.float32)
    q = rng.standard_normal((steps, batch, h_qk, d))
    k = rng.standard_normal((steps, batch, h_qk, d))
    v = rng.standard_normal((steps, batch, h_v, d))
    a = rng.normal(-2.0, 1.0, (steps, batch, h_v))
    b = rng.standard_normal((steps, batch, h_v))
    q = q * np.exp(rng.normal(0.0, 0.5, (steps, batch, h_qk, 1)))
    k = k * np.exp(rng.normal(0.0, 0.5, (steps, batch, h_qk, 1)))
    return dict(
        state0=torch.from_numpy(state0),
        q=torch.from_numpy(q).to(tdt),
        k=torch.from_numpy(k).to(tdt),
        v=torch.from_numpy(v).to(tdt),
        log_alpha=torch.from_numpy(a.astype(np.float32)),
        beta=torch.from_numpy(b.astype(np.float32)),
    )


def make_prefill_wide(seed, seq_lens, h_qk, h_v, d, dtype="bf16", kind="beta_to_2"):
    """Prefill inputs outside the main recipe's ranges, for the method's
    edge cases (same keys and shapes as make_prefill, nonzero initial
    states N(0, 0.02^2)). Draw order: q, k, v, log_alpha, beta, init, then
    the kind's extra draws.

    kind "beta_to_2":  beta = 1 + U(0, 1), every seventh (token, head) set
                       to exactly 2 (the write strength above 1; with unit
                       keys the transition still does not expand).
    kind "deep_decay": log_alpha ~ U(-30, 0) (alpha down to about 1e-13),
                       every fifth (token, head) exactly -30.
    kind "raw_qk":     q and k not normalised: unit vectors scaled per
                       (token, head) by U(0.7, 1.3) (k) and exp(N(0, 0.5^2))
                       (q); beta and log_alpha as in the main recipe.
    """
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in seq_lens]
    T = int(sum(lens))
    tdt = _DTYPES[dtype]
    q = _unit_rows(rng.standard_normal((T, h_qk, d)))
    k = _unit_rows(rng.standard_normal((T, h_qk, d)))
    v = rng.standard_normal((T, h_v, d))
    la = -_softplus(rng.normal(-2.0, 1.0, (T, h_v)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, h_v))))
    init_state = rng.normal(0.0, 0.02, (len(lens), h_v, d, d)).astype(np.float32)
    if kind == "beta_to_2":
        beta = 1.0 + rng.uniform(0.0, 1.0, (T, h_v))
        beta.reshape(-1)[::7] = 2.0
    elif kind == "deep_decay":
        la = rng.uniform(-30.0, 0.0, (T, h_v))
        la.reshape(-1)[::5] = -30.0
    elif kind == "raw_qk":
        k = k * rng.uniform(0.7, 1.3, (T, h_qk, 1))
        q = q * np.exp(rng.normal(0.0, 0.5, (T, h_qk, 1)))
    else:
        raise ValueError(kind)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return dict(
        q=torch.from_numpy(q).to(tdt),
        k=torch.from_numpy(k).to(tdt),
        v=torch.from_numpy(v).to(tdt),
        log_alpha=torch.from_numpy(la.astype(np.float32)),
        beta=torch.from_numpy(beta.astype(np.float32)),
        init_state=torch.from_numpy(init_state),
        cu_seqlens=torch.from_numpy(cu),
    )


# The five workloads (sizes as named in the docs). Each entry is the
# keyword arguments of make_prefill / make_decode.
WORKLOADS = {
    "tiny": dict(kind="prefill", seed=1, seq_lens=[64], h_qk=1, h_v=1, d=16,
                 chunk=16, dtype="f32", init="zeros"),
    "layer_4k": dict(kind="prefill", seed=2, seq_lens=[4096], h_qk=16, h_v=48,
                     d=128, chunk=64, dtype="bf16", init="zeros"),
    "long_64k": dict(kind="prefill", seed=3, seq_lens=[65536], h_qk=16,
                     h_v=48, d=128, chunk=64, dtype="bf16", init="randn"),
    "varlen_8": dict(kind="prefill", seed=4, n_seqs=8, len_lo=1024,
                     len_hi=16384, h_qk=16, h_v=48, d=128, chunk=64,
                     dtype="bf16", init="randn"),
    "decode_256": dict(kind="decode", seed=5, batch=256, steps=128, h_qk=16,
                       h_v=48, d=128, dtype="bf16"),
}


def make_prefill_device(seed, seq_lens, h_qk, h_v, d, device, dtype=torch.bfloat16):
    """The recipe above drawn on `device` (for inputs too large to draw on
    the host): torch.Generator(device) seeded with `seed`, float32 draws in
    the order q, k, v, log_alpha, beta, init (N(0, 0.02^2) per sequence), q
    and k normalised in float32, then q/k/v cast to `dtype`. `seq_lens` is
    one length (one sequence, cu_seqlens None) or a list of lengths packed
    via cu_seqlens (int32 on `device`). Same keys and shapes as make_prefill
    with init="randn"; the tensors stay on `device`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    if isinstance(seq_lens, (int, np.integer)):
        lens, cu = [int(seq_lens)], None
    else:
        lens = [int(x) for x in seq_lens]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=device)
    T = int(sum(lens))

    def unit(shape):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x.to(dtype)

    q = unit((T, h_qk, d))
    k = unit((T, h_qk, d))
    v = torch.randn((T, h_v, d), generator=g, device=device, dtype=torch.float32).to(dtype)
    la = -torch.nn.functional.softplus(torch.randn((T, h_v), generator=g, device=device) - 2.0)
    beta = torch.sigmoid(torch.randn((T, h_v), generator=g, device=device))
    init = 0.02 * torch.randn((len(lens), h_v, d, d), generator=g, device=device)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, init_state=init, cu_seqlens=cu)


def make_decode_device(seed, batch, h_qk, h_v, d, device, dtype=torch.bfloat16, steps=None):
    """Decode inputs of the recipe above for `batch` sequences, drawn on
    `device` like make_prefill_device (order: state0, q, k, v, log_alpha,
    beta). With steps=None, one step: state0 [batch,h_v,d,d]; q, k
    [batch,h_qk,d]; v [batch,h_v,d]; log_alpha, beta [batch,h_v]. Otherwise
    the per-step inputs are stacked on a leading axis of `steps`, as in
    make_decode."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    state0 = 0.02 * torch.randn((batch, h_v, d, d), generator=g, device=device)
    lead = () if steps is None else (int(steps),)

    def unit(shape):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x.to(dtype)

    q = unit(lead + (batch, h_qk, d))
    k = unit(lead + (batch, h_qk, d))
    v = torch.randn(lead + (batch, h_v, d), generator=g, device=device, dtype=torch.float32).to(dtype)
    la = -torch.nn.functional.softplus(torch.randn(lead + (batch, h_v), generator=g, device=device) - 2.0)
    beta = torch.sigmoid(torch.randn(lead + (batch, h_v), generator=g, device=device))
    return dict(state0=state0, q=q, k=k, v=v, log_alpha=la, beta=beta)


def make_backward_seeds_device(seed, seq_len, h_v, d, device, dtype=torch.bfloat16):
    """make_backward_seeds for one sequence, drawn on `device` like
    make_prefill_device (float32 draws, order d_o, d_final)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    d_o = torch.randn((int(seq_len), h_v, d), generator=g, device=device, dtype=torch.float32).to(dtype)
    d_final = torch.randn((1, h_v, d, d), generator=g, device=device)
    return dict(d_o=d_o, d_final=d_final)


def workload_inputs(name, **overrides):
    """Inputs of a named workload; overrides replace recipe fields (used to
    shrink a workload for a quick check, e.g. steps=4)."""
    w = dict(WORKLOADS[name])
    w.update(overrides)
    if w["kind"] == "decode":
        return make_decode(w["seed"], w["batch"], w["steps"], w["h_qk"],
                           w["h_v"], w["d"], w["dtype"])
    if "seq_lens" in w:
        lens = w["seq_lens"]
    else:
        lens = make_varlen_lengths(w["seed"] + 1000, w["n_seqs"], w["len_lo"],
                                   w["len_hi"])
    return make_prefill(w["seed"], lens, w["h_qk"], w["h_v"], w["d"],
                        w["dtype"], w["init"])
