"""GPU parity of the fused input preparation (GDN_FLAG_PREPARE_INPUTS):
raw q, k and gate logits in, against the oracle's preparation
(oracle.gdn_oracle.prepare_inputs) followed by the token-serial recurrence."""
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


def prepared(inp):
    """The oracle's prepared (q, k, log_alpha, beta) from raw inputs."""
    return O.prepare_inputs(np64(inp["q"]), np64(inp["k"]), np64(inp["log_alpha"]), np64(inp["beta"]))


@pytest.mark.parametrize("d,chunk,dtype,lens", [
    (16, 16, "f32", [64]),
    (16, 64, "f32", [77, 123]),
    (128, 16, "f32", [40, 9]),
    (128, 64, "bf16", [200]),
    (128, 64, "bf16", [77, 0, 130]),
    (16, 64, "bf16", [150]),
])
def test_prefill_prepare_inputs(d, chunk, dtype, lens):
    say(f"prefill prepare_inputs d={d} C={chunk} {dtype} lens={lens}")
    inp = I.make_prefill_raw(70 + d + chunk + len(lens), lens, 2, 6, d, dtype, "randn")
    dv = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o, fin = gdn.gdn_chunk_fwd(dv["q"], dv["k"], dv["v"], dv["log_alpha"], dv["beta"], dv["init_state"],
                               dv["cu_seqlens"], chunk=chunk, prepare_inputs=True)
    torch.cuda.synchronize()
    q, k, la, beta = prepared(inp)
    want_o, want_f = O.recurrent_form1(q, k, np64(inp["v"]), la, beta, np64(inp["init_state"]),
                                       inp["cu_seqlens"].numpy())
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    check(o, want_o, tdt, "o")
    check(fin, want_f, tdt, "final state")


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (128, "f32"), (16, "f32")])
def test_decode_prepare_inputs(d, dtype):
    say(f"decode prepare_inputs N=5 d={d} {dtype} x6 steps")
    inp = I.make_decode_raw(80 + d, 5, 6, 2, 6, d, dtype)
    state = inp["state0"].to(DEV)
    ref = np64(inp["state0"])
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, la, beta = prepared(inp)
    for t in range(6):
        args = [inp[n][t].to(DEV) for n in ("q", "k", "v", "log_alpha", "beta")]
        o = gdn.gdn_decode_step(*args, state, prepare_inputs=True)
        torch.cuda.synchronize()
        want_o, ref = O.decode_step(ref, q[t], k[t], np64(inp["v"][t]), la[t], beta[t])
        check(o, want_o, tdt, f"o step {t}")
    check(state, ref, tdt, "state after 6 steps")


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (16, "f32")])
def test_decode_multi_prepare_inputs_equals_single_steps(d, dtype):
    say(f"decode_multi prepare_inputs K=3 d={d} {dtype} vs single steps")
    kt = 3
    inp = I.make_decode_raw(90 + d, 4, kt, 2, 6, d, dtype)
    args = [inp[n].to(DEV) for n in ("q", "k", "v", "log_alpha", "beta")]
    st1 = inp["state0"].to(DEV)
    o1 = [gdn.gdn_decode_step(*[a[t] for a in args], st1, prepare_inputs=True) for t in range(kt)]
    st2 = inp["state0"].to(DEV)
    o2 = gdn.gdn_decode_multi(*args, st2, prepare_inputs=True)
    torch.cuda.synchronize()
    for t in range(kt):
        assert torch.equal(o2[t], o1[t]), f"o token {t}"
    assert torch.equal(st2, st1)


def test_prefill_prepare_inputs_matches_decode_of_same_tokens():
    say("prepare_inputs: prefill vs decode x32 of the same tokens")
    n, steps = 3, 32
    inp = I.make_decode_raw(95, n, steps, 2, 6, 128, "bf16")
    state = inp["state0"].to(DEV)
    outs = [gdn.gdn_decode_step(*[inp[x][t].to(DEV) for x in ("q", "k", "v", "log_alpha", "beta")], state,
                                prepare_inputs=True) for t in range(steps)]
    perm = lambda x: x.transpose(0, 1).reshape(n * steps, *x.shape[2:]).contiguous()  # noqa: E731
    cu = torch.arange(n + 1, dtype=torch.int32) * steps
    o_pf, f_pf = gdn.gdn_chunk_fwd(*[perm(inp[x]).to(DEV) for x in ("q", "k", "v", "log_alpha", "beta")],
                                   inp["state0"].to(DEV), cu.to(DEV), chunk=16, prepare_inputs=True)
    torch.cuda.synchronize()
    o_dec = torch.stack(outs).transpose(0, 1).reshape(n * steps, 6, 128)
    check(o_dec, np64(o_pf), torch.bfloat16, "decode vs prefill o")
    check(state, np64(f_pf), torch.bfloat16, "decode vs prefill state")
