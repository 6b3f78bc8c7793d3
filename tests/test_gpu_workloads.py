"""GPU parity at the five workloads' full sizes, in the launch configuration
bench.py times (one gdn_chunk_fwd over the whole input; decode_step over the
whole batch). The GPU always computes every head and sequence; where the
fp64 oracle would take minutes it checks sampled QK head groups (each with
its V heads, over every token) or sampled sequences, which are independent
of the rest. Tolerances as in test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_delta_amd as gdn
from linear_attention_recurrence_delta_amd import inputs as I
from oracle import gdn_oracle as O

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def np64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def check(got, want, dtype, what):
    got = np64(got) if isinstance(got, torch.Tensor) else got
    err = got - want
    rel = np.linalg.norm(err) / max(np.linalg.norm(want), 1e-30)
    mx = np.abs(err).max()
    assert np.isfinite(got).all(), what
    if dtype == torch.float32:
        assert rel <= 1e-5, f"{what}: rel-L2 {rel:.3e}"
    else:
        assert mx <= 2e-2 and rel <= 5e-3, f"{what}: max-abs {mx:.3e} rel-L2 {rel:.3e}"
    print(f"  {what}: rel-L2 {rel:.2e} max-abs {mx:.2e}", flush=True)


def gpu_prefill(inp, chunk):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    cu = d["cu_seqlens"] if inp["cu_seqlens"].numel() > 2 else None
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                               d["init_state"], cu, chunk=chunk)
    torch.cuda.synchronize()
    return o.cpu(), fin.cpu()


def oracle_group(inp, g, group_size, chunk):
    """Chunkwise fp64 oracle restricted to QK head g and its V heads."""
    hv = slice(g * group_size, (g + 1) * group_size)
    init = None if inp["init_state"] is None else np64(inp["init_state"][:, hv])
    return O.chunkwise(np64(inp["q"][:, g:g + 1]), np64(inp["k"][:, g:g + 1]),
                       np64(inp["v"][:, hv]), np64(inp["log_alpha"][:, hv]),
                       np64(inp["beta"][:, hv]), init, inp["cu_seqlens"].numpy(),
                       chunk=chunk)[:2]


def test_workload_layer_4k_full():
    say("layer_4k: T=4096, 16/48 heads, d=128, C=64, bf16, every head checked")
    inp = I.workload_inputs("layer_4k")
    o, fin = gpu_prefill(inp, 64)
    want_o, want_f, _ = O.chunkwise(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]),
                                    np64(inp["log_alpha"]), np64(inp["beta"]), None, None,
                                    chunk=64)
    check(o, want_o, torch.bfloat16, "o")
    check(fin, want_f, torch.bfloat16, "final")


@pytest.mark.parametrize("name,groups", [("long_64k", (0, 15)), ("varlen_8", (0, 7))])
def test_workload_long_prefill_sampled_heads(name, groups):
    say(f"{name}: full GPU run, oracle on QK groups {groups}")
    inp = I.workload_inputs(name)
    o, fin = gpu_prefill(inp, 64)
    for g in groups:
        want_o, want_f = oracle_group(inp, g, 3, 64)
        check(o[:, 3 * g:3 * g + 3], want_o, torch.bfloat16, f"o group {g}")
        check(fin[:, 3 * g:3 * g + 3], want_f, torch.bfloat16, f"final group {g}")


def test_workload_decode_256_sampled_sequences():
    say("decode_256: 256 x 128 steps in place, oracle on sequences 0, 131, 255")
    dec = I.workload_inputs("decode_256")
    seqs = [0, 131, 255]
    state = dec["state0"].to(DEV)
    ref = np64(dec["state0"][seqs])
    worst = 0.0
    for t in range(dec["q"].shape[0]):
        args = [dec[x][t] for x in ("q", "k", "v", "log_alpha", "beta")]
        o = gdn.gdn_decode_step(*[a.to(DEV) for a in args], state)
        want_o, ref = O.decode_step(ref, *[np64(a[seqs]) for a in args])
        got = np64(o[seqs])
        err = got - want_o
        rel = np.linalg.norm(err) / np.linalg.norm(want_o)
        assert np.abs(err).max() <= 2e-2 and rel <= 5e-3, f"step {t}: rel {rel:.3e}"
        worst = max(worst, rel)
    torch.cuda.synchronize()
    print(f"  worst per-step o rel-L2 {worst:.2e}", flush=True)
    check(state[seqs], ref, torch.bfloat16, "state after 128 steps")


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
    # oracle on sampled sequences
    seqs = [0, 131, 255]
    ref = np64(dec["state0"][seqs])
    for t in range(kt):
        want_o, ref = O.decode_step(ref, *[np64(dec[x][t][seqs]) for x in ("q", "k", "v", "log_alpha", "beta")])
        check(o[t][seqs], want_o, torch.bfloat16, f"o token {t}")
        check(snaps[t][seqs], ref, torch.bfloat16, f"state after token {t}")
