"""Where the backward pass's bfloat16 tolerance comes from.

A float64 emulation of the chunkwise evaluation of the gated delta rule
(page "Qwen3.8-Flash-Next 技术总结", section 2.1, update form 1, readout
o_t = S_t^T q_t), differentiated with torch autograd, with the option of
rounding to bfloat16 (round to nearest even) every intermediate that the
library's kernels keep in the input dtype:
  forward:  Tinv, W, U, the state at each chunk start, and every operand of
            a matrix product (the decayed rows exp(g_L - g) U, P = Q K^T *
            Dincl, Tinv diag(b), Tinv diag(b exp(g)));
  backward: dL/dU and dL/dS at each chunk boundary (stored in the input
            dtype between the reverse scan and the gradient kernel).
Accumulation stays in float64, standing in for the kernels' fp32 MFMA
accumulators. Without rounding the emulation's gradients equal the
oracle's backpropagation through the recurrence (test_backward_rounding.py
pins that); with rounding, the relative L2 error of each gradient against
the unrounded one is what a correct bf16 backward can be expected to show.

Test infrastructure only (CPU). Run as a script to print the figures:

    python tests/backward_rounding.py
"""
import numpy as np
import torch


def bf16(x):
    return x.to(torch.bfloat16).to(torch.float64)


class _RoundValue(torch.autograd.Function):
    """Forward: the value rounded to bf16; backward: the gradient unchanged
    (later products use the rounded value, as the kernels do)."""

    @staticmethod
    def forward(ctx, x):
        return bf16(x)

    @staticmethod
    def backward(ctx, g):
        return g


class _RoundGrad(torch.autograd.Function):
    """Forward: identity; backward: the incoming gradient rounded to bf16."""

    @staticmethod
    def forward(ctx, x):
        return x.clone()

    @staticmethod
    def backward(ctx, g):
        return bf16(g)


def chunkwise_forward(q, k, v, log_alpha, beta, s0, chunk, rounded):
    """One head: q, k [T, dk]; v [T, dv]; log_alpha, beta [T]; s0 [dk, dv].
    Returns (o [T, dv], final state [dk, dv]) as autograd tensors."""
    rv = _RoundValue.apply if rounded else (lambda x: x)
    rg = _RoundGrad.apply if rounded else (lambda x: x)
    T = q.shape[0]
    S = s0
    outs = []
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        L = c1 - c0
        Q, K, V = q[c0:c1], k[c0:c1], v[c0:c1]
        b = beta[c0:c1]
        g = torch.cumsum(log_alpha[c0:c1], 0)
        rr, ii = torch.meshgrid(torch.arange(L), torch.arange(L), indexing="ij")
        incl = ii <= rr
        diff = torch.where(incl, g[:, None] - g[None, :], torch.zeros((), dtype=g.dtype))
        gm = torch.where(incl, torch.exp(diff), torch.zeros((), dtype=g.dtype))
        strict = torch.where(ii < rr, gm, torch.zeros((), dtype=g.dtype))
        A = b[:, None] * (K @ K.T) * strict
        Tm = torch.linalg.solve_triangular(torch.eye(L, dtype=q.dtype) + A, torch.eye(L, dtype=q.dtype),
                                           upper=False, unitriangular=True)
        Tm = rv(Tm)
        ea = torch.exp(g)
        W = rv(rv(Tm * (b * ea)[None, :]) @ K)
        Ut = rv(Tm * b[None, :]) @ V
        Sc = rg(rv(S))                                 # state at the chunk start
        U = rg(rv(Ut - W @ Sc))
        P = rv((Q @ K.T) * gm)
        O = ea[:, None] * (Q @ Sc) + P @ U
        outs.append(O)
        ed = torch.exp(g[-1] - g)
        S = torch.exp(g[-1]) * Sc + K.T @ rv(ed[:, None] * U)
    return torch.cat(outs), S


def gradients(inp, d_o, d_final, chunk, rounded):
    """Gradients of <o, d_o> + <S_final, d_final> for one head (dict of
    float64 numpy arrays)."""
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp.items()}
    o, fin = chunkwise_forward(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["s0"], chunk, rounded)
    loss = (o * torch.tensor(d_o)).sum() + (fin * torch.tensor(d_final)).sum()
    loss.backward()
    return {k: v.grad.numpy() for k, v in t.items()}


def random_head(seed, T, d):
    """The input recipe for one head, with q, k, v rounded to bf16 as the
    kernels receive them, and Gaussian upstream gradients (d_o rounded to
    bf16)."""
    rng = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)  # noqa: E731
    as_bf16 = lambda x: bf16(torch.tensor(x)).numpy()  # noqa: E731
    inp = dict(q=as_bf16(unit(rng.standard_normal((T, d)))), k=as_bf16(unit(rng.standard_normal((T, d)))),
               v=as_bf16(rng.standard_normal((T, d))),
               log_alpha=-np.logaddexp(0.0, rng.normal(-2.0, 1.0, T)).astype(np.float32).astype(np.float64),
               beta=(1.0 / (1.0 + np.exp(-rng.standard_normal(T)))).astype(np.float32).astype(np.float64),
               s0=rng.normal(0.0, 0.02, (d, d)).astype(np.float32).astype(np.float64))
    d_o = as_bf16(rng.standard_normal((T, d)))
    d_final = rng.standard_normal((d, d)).astype(np.float32).astype(np.float64)
    return inp, d_o, d_final


def rounding_errors(seed, T, d, chunk):
    """Per gradient: (rel-L2, max |err| / max |ref|) of the rounded
    emulation against the unrounded one."""
    inp, d_o, d_final = random_head(seed, T, d)
    exact = gradients(inp, d_o, d_final, chunk, False)
    rounded = gradients(inp, d_o, d_final, chunk, True)
    out = {}
    for name in exact:
        e = rounded[name] - exact[name]
        out[name] = (float(np.linalg.norm(e) / np.linalg.norm(exact[name])),
                     float(np.abs(e).max() / np.abs(exact[name]).max()))
    return out


if __name__ == "__main__":
    for chunk in (16, 64):
        worst = {}
        for seed in range(3):
            for name, (rel, mx) in rounding_errors(seed, 512, 128, chunk).items():
                w = worst.get(name, (0.0, 0.0))
                worst[name] = (max(w[0], rel), max(w[1], mx))
        print(f"d=128 C={chunk} T=512, worst of 3 seeds:")
        for name, (rel, mx) in worst.items():
            print(f"  d{name:10s} rel-L2 {rel:.2e}  max/max|ref| {mx:.2e}")
