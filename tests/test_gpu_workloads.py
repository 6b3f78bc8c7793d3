"""GPU parity at the five workloads' full sizes, in the launch configuration
bench.py times (one gdn_chunk_fwd over the whole input; gdn_decode_step over
the whole batch), against the fp64 form-1 recurrence (the C oracle,
oracle/gdn_ref.c, pinned in test_oracle_c.py) on every head, every token
and every sequence. Tolerances as in test_gpu_parity.py, applied to each
whole tensor and again to each QK head group (each decode sequence), so
that an error confined to some heads or sequences cannot hide in the
norm of the rest.
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_delta_amd as gdn
from linear_attention_recurrence_delta_amd import inputs as I
from oracle import c_ref as CR
from oracle import gdn_oracle as O

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MAX_ABS, REL_L2 = 2e-2, 5e-3          # bf16 inputs, fp32 state


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def np64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def f32(t):
    return None if t is None else t.detach().to("cpu", torch.float32).numpy()


class Stats:
    """Sums of squares and the largest error, grouped along one axis."""

    def __init__(self, groups):
        self.err = np.zeros(groups)
        self.ref = np.zeros(groups)
        self.mx = np.zeros(groups)

    def add(self, got, want, group_axis_sum):
        e = got - want
        assert np.isfinite(got).all(), "non-finite values"
        self.err += group_axis_sum(e * e)
        self.ref += group_axis_sum(want * want)
        self.mx = np.maximum(self.mx, group_axis_sum(np.abs(e), np.max))

    def verdict(self, what, names):
        rel_all = np.sqrt(self.err.sum() / self.ref.sum())
        mx_all = self.mx.max()
        rel = np.sqrt(self.err / np.maximum(self.ref, 1e-300))
        worst = int(np.argmax(rel))
        print(f"  {what}: rel-L2 {rel_all:.2e} max-abs {mx_all:.2e}; worst {names} {worst}: "
              f"rel-L2 {rel[worst]:.2e}", flush=True)
        assert mx_all <= MAX_ABS and rel_all <= REL_L2, f"{what}: max-abs {mx_all:.3e} rel-L2 {rel_all:.3e}"
        bad = np.nonzero(rel > REL_L2)[0]
        assert bad.size == 0, f"{what}: {names} {bad.tolist()} above rel-L2 {REL_L2}: {rel[bad]}"


def by_group(group):
    """Reducer over everything but the head axis (axis 1), heads binned into
    QK groups of `group` V heads."""
    def red(x, op=np.sum):
        h = op(x.reshape(x.shape[0], x.shape[1], -1), axis=(0, 2))
        return op(h.reshape(-1, group), axis=1)
    return red


def compare_heads(got, want, group, what, rows=2048):
    """got [R, Hv, ...] torch (CPU), want [R, Hv, ...] float64; compared in
    blocks of rows, per QK group of `group` V heads."""
    st = Stats(got.shape[1] // group)
    red = by_group(group)
    for i in range(0, got.shape[0], rows):
        st.add(got[i:i + rows].to(torch.float64).numpy(), want[i:i + rows], red)
    st.verdict(what, "QK group")


def gpu_prefill(inp, chunk):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    cu = d["cu_seqlens"] if inp["cu_seqlens"].numel() > 2 else None
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                               d["init_state"], cu, chunk=chunk)
    torch.cuda.synchronize()
    return o.cpu(), fin.cpu()


def oracle_form1(inp):
    return CR.recurrent_form1(f32(inp["q"]), f32(inp["k"]), f32(inp["v"]), f32(inp["log_alpha"]),
                              f32(inp["beta"]), np64(inp["init_state"]), inp["cu_seqlens"].numpy())


@pytest.mark.parametrize("name", ["layer_4k", "long_64k", "varlen_8"])
def test_workload_prefill_every_head(name):
    inp = I.workload_inputs(name)
    lens = np.diff(inp["cu_seqlens"].numpy()).tolist()
    say(f"{name}: T={sum(lens)} in {len(lens)} sequence(s), 16/48 heads, d=128, C=64, bf16; "
        f"all heads against the form-1 recurrence")
    o, fin = gpu_prefill(inp, 64)
    want_o, want_f = oracle_form1(inp)
    compare_heads(o, want_o, 3, "o")
    compare_heads(fin, want_f, 3, "final state")
    if name == "layer_4k":
        # the chunkwise fp64 evaluation too (tied to the recurrence in the
        # oracle's own pins): same result on every head
        want_o2, want_f2, _ = O.chunkwise(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]),
                                          np64(inp["log_alpha"]), np64(inp["beta"]), None, None, chunk=64)
        compare_heads(o, want_o2, 3, "o vs chunkwise")
        compare_heads(fin, want_f2, 3, "final vs chunkwise")


def per_sequence(x, op=np.sum):
    return op(x.reshape(x.shape[0], -1), axis=1)


def test_workload_decode_256_every_sequence():
    say("decode_256: 256 sequences x 128 steps in place; every step's o and the final state, "
        "every sequence, against the form-1 recurrence")
    dec = I.workload_inputs("decode_256")
    steps = dec["q"].shape[0]
    state = dec["state0"].to(DEV)
    outs = []
    for t in range(steps):
        args = [dec[x][t].to(DEV) for x in ("q", "k", "v", "log_alpha", "beta")]
        outs.append(gdn.gdn_decode_step(*args, state).cpu())
    torch.cuda.synchronize()
    want_o, want_s = CR.decode_steps(np64(dec["state0"]), *(f32(dec[x]) for x in
                                                             ("q", "k", "v", "log_alpha", "beta")))
    worst = 0.0
    for t in range(steps):
        st = Stats(256)
        st.add(outs[t].to(torch.float64).numpy(), want_o[t], per_sequence)
        rel = np.sqrt(st.err.sum() / st.ref.sum())
        assert st.mx.max() <= MAX_ABS and rel <= REL_L2, f"o step {t}: rel {rel:.3e} max {st.mx.max():.3e}"
        bad = np.nonzero(np.sqrt(st.err / st.ref) > REL_L2)[0]
        assert bad.size == 0, f"o step {t}: sequences {bad.tolist()}"
        worst = max(worst, rel)
    print(f"  worst per-step o rel-L2 {worst:.2e}", flush=True)
    st = Stats(256)
    st.add(np64(state), want_s, per_sequence)
    st.verdict("state after 128 steps", "sequence")


def test_workload_decode_256_verify_four_tokens():
    say("decode_256 speculative verify: 4 drafted tokens for all 256 sequences in one pass")
    kt = 4
    dec = I.workload_inputs("decode_256", steps=kt)
    args = [dec[x].to(DEV) for x in ("q", "k", "v", "log_alpha", "beta")]
    single = dec["state0"].to(DEV)
    o_single = [gdn.gdn_decode_step(*[a[t] for a in args], single) for t in range(kt)]
    state = dec["state0"].to(DEV)
    snaps = torch.empty((kt,) + tuple(state.shape), dtype=torch.float32, device=DEV)
    o = gdn.gdn_decode_multi(*args, state, snapshots=snaps)
    torch.cuda.synchronize()
    for t in range(kt):
        assert torch.equal(o[t], o_single[t]), f"o token {t}"
    assert torch.equal(snaps[-1], single)
    assert torch.equal(state, dec["state0"].to(DEV))
    # every sequence against the recurrence, token by token
    for t in range(1, kt + 1):
        want_o, want_s = CR.decode_steps(np64(dec["state0"]), *(f32(dec[x][:t]) for x in
                                                                 ("q", "k", "v", "log_alpha", "beta")))
        st = Stats(256)
        st.add(np64(o[t - 1]), want_o[t - 1], per_sequence)
        st.verdict(f"o token {t - 1}", "sequence")
        st = Stats(256)
        st.add(np64(snaps[t - 1]), want_s, per_sequence)
        st.verdict(f"state after token {t - 1}", "sequence")
