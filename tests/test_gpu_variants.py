"""GPU parity of the two variants that section 2.1 of the Qwen3.8-Flash-Next
summary sets against the gated delta rule, through the C ABI:
  DeltaNet (the delta rule alone): log_alpha = 0, no flag, against the
    oracle's form-1 recurrence;
  the gate alone (GDN_FLAG_NO_DELTA_RULE): S <- a S + b k v^T, against the
    oracle's recurrent_gated_no_delta.
Tolerances as for the gated delta rule (fp32 rel-L2 <= 1e-5; bf16 max-abs <=
2e-2 and rel-L2 <= 5e-3), on o and on the final state separately."""
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
    mx = np.abs(err).max() if err.size else 0.0
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    if dtype == torch.float32:
        assert rel <= 1e-5, f"{what}: rel-L2 {rel:.3e} > 1e-5"
    else:
        assert mx <= 2e-2 and rel <= 5e-3, f"{what}: max-abs {mx:.3e}, rel-L2 {rel:.3e}"


def tdtype(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def prefill(inp, chunk, **kw):
    dv = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o, fin = gdn.gdn_chunk_fwd(dv["q"], dv["k"], dv["v"], dv["log_alpha"], dv["beta"], dv["init_state"],
                               dv["cu_seqlens"], chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o, fin


def oracle(fn, inp):
    return fn(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), np64(inp["log_alpha"]), np64(inp["beta"]),
              np64(inp["init_state"]), inp["cu_seqlens"].numpy())


CONFIGS = [
    (16, 16, "f32", [64]),
    (16, 64, "f32", [77, 123]),
    (128, 16, "f32", [40, 9]),
    (128, 64, "bf16", [300]),
    (128, 16, "bf16", [130]),
    (16, 64, "bf16", [150]),
    (128, 64, "bf16", [0, 1, 63, 64, 65, 200, 0, 7]),
]


# --- DeltaNet: the delta rule alone (a = 1) --------------------------------

@pytest.mark.parametrize("d,chunk,dtype,lens", CONFIGS[:4])
def test_deltanet_prefill(d, chunk, dtype, lens):
    say(f"DeltaNet prefill d={d} C={chunk} {dtype} lens={lens}")
    inp = I.make_prefill(200 + d + chunk, lens, 2, 6, d, dtype, "randn")
    inp["log_alpha"].zero_()
    o, fin = prefill(inp, chunk)
    want_o, want_f = oracle(O.recurrent_form1, inp)
    check(o, want_o, tdtype(dtype), "o")
    check(fin, want_f, tdtype(dtype), "final state")


def test_deltanet_decode():
    say("DeltaNet decode N=5 d=128 bf16 x6 steps")
    inp = I.make_decode(210, 5, 6, 2, 6, 128, "bf16")
    inp["log_alpha"].zero_()
    state = inp["state0"].to(DEV)
    ref = np64(inp["state0"])
    for t in range(6):
        args = [inp[n][t] for n in ("q", "k", "v", "log_alpha", "beta")]
        o = gdn.gdn_decode_step(*[a.to(DEV) for a in args], state)
        torch.cuda.synchronize()
        want_o, ref = O.decode_step(ref, *[np64(a) for a in args])
        check(o, want_o, torch.bfloat16, f"o step {t}")
    check(state, ref, torch.bfloat16, "state after 6 steps")


# --- the gate alone (GDN_FLAG_NO_DELTA_RULE) -------------------------------

@pytest.mark.parametrize("d,chunk,dtype,lens", CONFIGS)
def test_gate_only_prefill(d, chunk, dtype, lens):
    say(f"gate-only prefill d={d} C={chunk} {dtype} lens={lens}")
    inp = I.make_prefill(220 + d + chunk + len(lens), lens, 2, 6, d, dtype, "randn")
    o, fin = prefill(inp, chunk, delta_rule=False)
    want_o, want_f = oracle(O.recurrent_gated_no_delta, inp)
    check(o, want_o, tdtype(dtype), "o")
    check(fin, want_f, tdtype(dtype), "final state")
    for n, ln in enumerate(lens):
        if ln == 0:
            assert torch.equal(fin[n].cpu(), inp["init_state"][n])


def test_gate_only_layer_4k_sampled_heads():
    # 4096 tokens, 16 QK / 48 V heads: every head on the GPU; the oracle runs
    # two sampled QK groups (their six V heads) over every token
    say("gate-only prefill T=4096 16/48 heads d=128 C=64 bf16, sampled groups")
    inp = I.make_prefill(230, [4096], 16, 48, 128, "bf16", "randn")
    o, fin = prefill(inp, 64, delta_rule=False)
    for hq in (0, 11):
        hv = slice(3 * hq, 3 * hq + 3)
        sub = dict(q=inp["q"][:, hq:hq + 1], k=inp["k"][:, hq:hq + 1], v=inp["v"][:, hv],
                   log_alpha=inp["log_alpha"][:, hv], beta=inp["beta"][:, hv],
                   init_state=inp["init_state"][:, hv], cu_seqlens=inp["cu_seqlens"])
        want_o, want_f = oracle(O.recurrent_gated_no_delta, sub)
        check(o[:, hv], want_o, torch.bfloat16, f"o group {hq}")
        check(fin[:, hv], want_f, torch.bfloat16, f"final group {hq}")


@pytest.mark.parametrize("d,chunk,dtype,lens", [(128, 64, "bf16", [77, 0, 130]), (16, 16, "f32", [64])])
def test_gate_only_prefill_with_prepare_inputs(d, chunk, dtype, lens):
    say(f"gate-only + prepare_inputs prefill d={d} C={chunk} {dtype} lens={lens}")
    inp = I.make_prefill_raw(240 + d, lens, 2, 6, d, dtype, "randn")
    o, fin = prefill(inp, chunk, delta_rule=False, prepare_inputs=True)
    q, k, la, beta = O.prepare_inputs(np64(inp["q"]), np64(inp["k"]), np64(inp["log_alpha"]), np64(inp["beta"]))
    want_o, want_f = O.recurrent_gated_no_delta(q, k, np64(inp["v"]), la, beta, np64(inp["init_state"]),
                                                inp["cu_seqlens"].numpy())
    check(o, want_o, tdtype(dtype), "o")
    check(fin, want_f, tdtype(dtype), "final state")


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (128, "f32"), (16, "f32")])
def test_gate_only_decode(d, dtype):
    say(f"gate-only decode N=5 d={d} {dtype} x6 steps")
    inp = I.make_decode(250 + d, 5, 6, 2, 6, d, dtype)
    state = inp["state0"].to(DEV)
    ref = np64(inp["state0"])
    for t in range(6):
        args = [inp[n][t] for n in ("q", "k", "v", "log_alpha", "beta")]
        o = gdn.gdn_decode_step(*[a.to(DEV) for a in args], state, delta_rule=False)
        torch.cuda.synchronize()
        want_o, ref = O.decode_step_no_delta(ref, *[np64(a) for a in args])
        check(o, want_o, tdtype(dtype), f"o step {t}")
    check(state, ref, tdtype(dtype), "state after 6 steps")


@pytest.mark.parametrize("prep", [False, True])
def test_gate_only_decode_multi_equals_single_steps(prep):
    say(f"gate-only decode_multi K=4 d=128 bf16 prepare_inputs={prep} vs single steps")
    kt = 4
    make = I.make_decode_raw if prep else I.make_decode
    inp = make(260, 4, kt, 2, 6, 128, "bf16")
    args = [inp[n].to(DEV) for n in ("q", "k", "v", "log_alpha", "beta")]
    st1 = inp["state0"].to(DEV)
    o1 = [gdn.gdn_decode_step(*[a[t] for a in args], st1, prepare_inputs=prep, delta_rule=False)
          for t in range(kt)]
    st2 = inp["state0"].to(DEV)
    o2 = gdn.gdn_decode_multi(*args, st2, prepare_inputs=prep, delta_rule=False)
    snaps = torch.empty((kt,) + tuple(st2.shape), dtype=torch.float32, device=DEV)
    st3 = inp["state0"].to(DEV)
    o3 = gdn.gdn_decode_multi(*args, st3, snapshots=snaps, prepare_inputs=prep, delta_rule=False)
    torch.cuda.synchronize()
    for t in range(kt):
        assert torch.equal(o2[t], o1[t]), f"o token {t}"
        assert torch.equal(o3[t], o1[t]), f"o token {t} (snapshots)"
    assert torch.equal(st2, st1)
    assert torch.equal(snaps[kt - 1], st1)
    assert torch.equal(st3, inp["state0"].to(DEV))


def test_gate_only_prefill_matches_decode_of_same_tokens():
    say("gate-only: prefill vs decode x40 of the same tokens")
    n, steps = 3, 40
    inp = I.make_decode(270, n, steps, 2, 6, 128, "bf16")
    state = inp["state0"].to(DEV)
    outs = [gdn.gdn_decode_step(*[inp[x][t].to(DEV) for x in ("q", "k", "v", "log_alpha", "beta")], state,
                                delta_rule=False) for t in range(steps)]
    perm = lambda x: x.transpose(0, 1).reshape(n * steps, *x.shape[2:]).contiguous()  # noqa: E731
    cu = torch.arange(n + 1, dtype=torch.int32) * steps
    o_pf, f_pf = gdn.gdn_chunk_fwd(*[perm(inp[x]).to(DEV) for x in ("q", "k", "v", "log_alpha", "beta")],
                                   inp["state0"].to(DEV), cu.to(DEV), chunk=64, delta_rule=False)
    torch.cuda.synchronize()
    o_dec = torch.stack(outs).transpose(0, 1).reshape(n * steps, 6, 128)
    check(o_dec, np64(o_pf), torch.bfloat16, "decode vs prefill o")
    check(state, np64(f_pf), torch.bfloat16, "decode vs prefill state")
