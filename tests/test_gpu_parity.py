"""GPU parity of libgdn against the fp64 CPU oracle, through the C ABI.

Tolerances (per tensor, separately for o and the final state; rel-L2 is
||x - y|| / ||y||, max-abs is max |x - y|):
  fp32 inputs: rel-L2 <= 1e-5
  bf16 inputs (fp32 state and accumulation): max-abs <= 2e-2 and rel-L2 <= 5e-3
The oracle sees exactly the values the GPU sees (bf16 upcast to fp64).
Large workloads are checked on sampled head groups (the oracle runs those
heads over every token) since head groups are independent.
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


def on_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


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
    return rel, mx


def oracle_args(inp):
    return dict(q=np64(inp["q"]), k=np64(inp["k"]), v=np64(inp["v"]),
                log_alpha=np64(inp["log_alpha"]), beta=np64(inp["beta"]),
                init_state=np64(inp.get("init_state")),
                cu_seqlens=None if inp.get("cu_seqlens") is None
                else inp["cu_seqlens"].numpy())


def run_gpu(inp, chunk, use_cu=True):
    d = on_dev(inp)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                               d.get("init_state"), d["cu_seqlens"] if use_cu else None,
                               chunk=chunk)
    torch.cuda.synchronize()
    return o, fin


def random_prefill(seed, lens, h_qk, h_v, d, dtype, init="randn"):
    return I.make_prefill(seed, lens, h_qk, h_v, d, dtype, init)


# --- small shapes: several tiles, ragged tails ---------------------------------

def test_tiny_fp32_workload():
    say("tiny fp32 T=64 d=16 C=16")
    inp = I.workload_inputs("tiny")
    o, fin = run_gpu(inp, 16)
    want_o, want_f = O.recurrent_form1(**oracle_args(inp))
    check(o, want_o, torch.float32, "o")
    check(fin, want_f, torch.float32, "final")


@pytest.mark.parametrize("d,chunk,dtype", [
    (128, 64, "bf16"), (128, 16, "bf16"), (16, 64, "bf16"), (16, 16, "bf16"),
    (16, 16, "f32"), (128, 16, "f32"), (16, 64, "f32"), (128, 64, "f32")])
def test_prefill_ragged_single_sequence(d, chunk, dtype):
    say(f"prefill T=300 d={d} C={chunk} {dtype}")
    inp = random_prefill(100 + d + chunk, [300], 2, 6, d, dtype)
    o, fin = run_gpu(inp, chunk, use_cu=False)
    want_o, want_f = O.recurrent_form1(**{**oracle_args(inp), "cu_seqlens": None})
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    check(o, want_o, tdt, "o")
    check(fin, want_f, tdt, "final")


@pytest.mark.parametrize("dtype,chunk", [("bf16", 64), ("f32", 16)])
def test_prefill_varlen_with_empty_and_short_sequences(dtype, chunk):
    lens = [0, 1, 63, 64, 65, 200, 0, 7, 130]
    say(f"varlen {lens} {dtype} C={chunk}")
    inp = random_prefill(7, lens, 2, 6, 128, dtype)
    o, fin = run_gpu(inp, chunk)
    want_o, want_f = O.recurrent_form1(**oracle_args(inp))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    check(o, want_o, tdt, "o")
    check(fin, want_f, tdt, "final")
    # empty sequences: final state equals the initial state exactly
    for n in (0, 6):
        assert torch.equal(fin[n].cpu(), inp["init_state"][n])


def test_prefill_many_sequences():
    # more sequences than one wave's prefix sum covers (64): the chunk table
    # comes from the block scan, here over two 256-sequence passes
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(0, 41, size=300)]
    say(f"prefill, {len(lens)} sequences, {sum(lens)} tokens, bf16 C=64")
    inp = random_prefill(42, lens, 2, 6, 128, "bf16")
    o, fin = run_gpu(inp, 64)
    want_o, want_f = O.recurrent_form1(**oracle_args(inp))
    check(o, want_o, torch.bfloat16, "o")
    check(fin, want_f, torch.bfloat16, "final")


@pytest.mark.parametrize("chunk", [64, 16])
def test_prefill_reads_only_what_it_writes(chunk):
    # the kernels never read workspace bytes that no kernel wrote (e.g. the
    # fragments that the causal mask makes zero): a workspace full of NaN
    # bytes gives the same outputs, bit for bit, as a zeroed one
    say(f"prefill with a NaN-filled workspace, C={chunk}")
    inp = on_dev(random_prefill(43, [77, 0, 130], 2, 6, 128, "bf16"))
    dims = gdn.make_dims(3, 207, 2, 6, 128, 128, chunk, torch.bfloat16)
    nbytes = gdn.gdn_chunk_fwd_workspace_bytes(dims)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
        outs.append(gdn.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                      inp["init_state"], inp["cu_seqlens"], chunk=chunk, workspace=ws))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("dtype,chunk", [("bf16", 64), ("bf16", 16), ("f32", 16), ("f32", 64)])
@pytest.mark.parametrize("kind", ["beta_to_2", "deep_decay", "raw_qk"])
def test_prefill_wide_input_ranges(kind, dtype, chunk):
    # the method's ranges beyond the main recipe: write strength in (1, 2],
    # forget gates down to exp(-30), keys and queries not of unit length
    lens = [300, 1, 129]
    say(f"prefill {kind} {lens} d=128 C={chunk} {dtype}")
    inp = I.make_prefill_wide(60 + chunk, lens, 2, 6, 128, dtype, kind)
    o, fin = run_gpu(inp, chunk)
    want_o, want_f = O.recurrent_form1(**oracle_args(inp))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    rel_o, mx_o = check(o, want_o, tdt, "o")
    rel_f, mx_f = check(fin, want_f, tdt, "final")
    print(f"  o rel-L2 {rel_o:.2e} max-abs {mx_o:.2e}; final rel-L2 {rel_f:.2e} max-abs {mx_f:.2e}", flush=True)


@pytest.mark.parametrize("kind", ["beta_to_2", "deep_decay", "raw_qk"])
def test_decode_wide_input_ranges(kind):
    # the same ranges through the decode step: 130 sequences, one token each,
    # three successive steps
    say(f"decode {kind} N=130 d=128 bf16 x3 steps")
    steps = [I.make_prefill_wide(70 + t, [130], 2, 6, 128, "bf16", kind) for t in range(3)]
    state0 = I.make_decode(73, 130, 1, 2, 6, 128, "bf16")["state0"]
    state = state0.to(DEV)
    ref = np64(state0)
    for t, inp in enumerate(steps):
        args = [inp[x] for x in ("q", "k", "v", "log_alpha", "beta")]
        o = gdn.gdn_decode_step(*[a.to(DEV) for a in args], state)
        torch.cuda.synchronize()
        want_o, ref = O.decode_step(ref, *[np64(a) for a in args])
        check(o, want_o, torch.bfloat16, f"o step {t}")
    check(state, ref, torch.bfloat16, "state after 3 steps")


def test_debug_check_of_cu_seqlens(monkeypatch):
    # GDN_DEBUG: the prefill entry points read cu_seqlens on the host and
    # reject a table that is not 0 = c_0 <= ... <= c_N = T before enqueueing
    # anything; a valid table gives the same result, bit for bit
    say("GDN_DEBUG cu_seqlens check and GDN_DEBUG_SYNC")
    inp = on_dev(random_prefill(19, [50, 30, 20], 2, 6, 128, "bf16"))
    args = [inp[x] for x in ("q", "k", "v", "log_alpha", "beta", "init_state")]
    o_ref, f_ref = gdn.gdn_chunk_fwd(*args, inp["cu_seqlens"], chunk=64)
    monkeypatch.setenv("GDN_DEBUG", "1")
    monkeypatch.setenv("GDN_DEBUG_SYNC", "1")
    o, f = gdn.gdn_chunk_fwd(*args, inp["cu_seqlens"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(f, f_ref)
    for bad in ([1, 50, 80, 100], [0, 50, 40, 100], [0, 50, 80, 99], [0, 150, 80, 100]):
        cu = torch.tensor(bad, dtype=torch.int32, device=DEV)
        with pytest.raises(gdn.GdnError, match="GDN_DEBUG"):
            gdn.gdn_chunk_fwd(*args, cu, chunk=64)
        seeds = I.make_backward_seeds(20, [50, 30, 20], 6, 128, "bf16")
        with pytest.raises(gdn.GdnError, match="GDN_DEBUG"):
            gdn.gdn_chunk_bwd(*args[:5], seeds["d_o"].to(DEV), args[5], cu, seeds["d_final"].to(DEV), chunk=64)
    torch.cuda.synchronize()


def test_zero_tokens():
    say("T=0, two empty sequences")
    inp = random_prefill(8, [0, 0], 1, 3, 128, "bf16")
    o, fin = run_gpu(inp, 64)
    assert o.numel() == 0
    assert torch.equal(fin.cpu(), inp["init_state"])


def test_head_group_of_four():
    say("h_qk=3 h_v=12 (groups of 4) T=150")
    inp = random_prefill(9, [150], 3, 12, 128, "bf16")
    o, fin = run_gpu(inp, 64, use_cu=False)
    want_o, want_f = O.recurrent_form1(**{**oracle_args(inp), "cu_seqlens": None})
    check(o, want_o, torch.bfloat16, "o")
    check(fin, want_f, torch.bfloat16, "final")


@pytest.mark.parametrize("h_qk,h_v,d,chunk,dtype", [
    (4, 4, 128, 64, "bf16"), (1, 8, 128, 64, "bf16"), (2, 10, 128, 16, "bf16"), (3, 3, 16, 64, "f32"),
    (1, 5, 16, 16, "bf16")])
def test_head_group_sizes(h_qk, h_v, d, chunk, dtype):
    # the forward's kernel 2 takes a QK head's V heads in turn (one per
    # group member, each with its own gates), so group sizes 1, 5 and 8 run
    # that loop a different number of times; two sequences, one ragged
    say(f"h_qk={h_qk} h_v={h_v} (groups of {h_v // h_qk}) d={d} C={chunk} {dtype}, lens [150, 41]")
    inp = random_prefill(500 + h_v + d + chunk, [150, 41], h_qk, h_v, d, dtype)
    o, fin = run_gpu(inp, chunk)
    want_o, want_f = O.recurrent_form1(**oracle_args(inp))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    check(o, want_o, tdt, "o")
    check(fin, want_f, tdt, "final")


@pytest.mark.parametrize("lens", [[70], [300, 0, 1, 129]])
def test_fp32_head_dim_128_chunk_64(lens):
    # fp32 operands at head dim 128 with 64-token chunks: the scan's
    # single-slot instance (16-column slices, compute and copy phases)
    say(f"fp32 d=128 C=64 {lens}")
    inp = random_prefill(18, lens, 2, 6, 128, "f32")
    o, fin = run_gpu(inp, 64)
    want_o, want_f = O.recurrent_form1(**oracle_args(inp))
    check(o, want_o, torch.float32, "o")
    check(fin, want_f, torch.float32, "final")
    # its backward pass is not built
    dims = gdn.make_dims(len(lens), sum(lens), 2, 6, 128, 128, 64, torch.float32)
    with pytest.raises(gdn.GdnError, match="chunk 16"):
        gdn.gdn_chunk_bwd_workspace_bytes(dims)


def test_invariants_beta_zero_and_exact_recall():
    say("beta=0 decay and exact recall, d=128 f32")
    inp = random_prefill(10, [130], 1, 3, 128, "f32")
    inp["beta"].zero_()
    o, fin = run_gpu(inp, 16, use_cu=False)
    g = inp["log_alpha"].double().sum(0)
    want = torch.exp(g)[:, None, None] * inp["init_state"][0].double()
    check(fin[0], want.numpy(), torch.float32, "beta=0 final")
    # a = 1, b = 1, |k| = 1 and q = k: o_t = v_t
    inp = random_prefill(11, [130], 1, 3, 128, "f32")
    inp["log_alpha"].zero_()
    inp["beta"].fill_(1.0)
    inp["q"] = inp["k"].clone()
    o, _ = run_gpu(inp, 16, use_cu=False)
    check(o, np64(inp["v"]), torch.float32, "exact recall")


# --- per-kernel stages (workspace) against the oracle's chunk stages ---------

def frag_k(s, quad, e):
    """Contraction index of fragment element e, 32-step s, lane quad."""
    return 32 * s + (4 * quad + e if e < 4 else 16 + 4 * quad + e - 4)


def unfrag(frags, rows, kdim):
    """[tiles][steps][64][8] fragment array -> dense [rows][kdim] matrix."""
    out = np.zeros((rows, kdim))
    n_t, n_s = frags.shape[0], frags.shape[1]
    for t in range(n_t):
        for s in range(n_s):
            for ln in range(64):
                for e in range(8):
                    k = frag_k(s, ln // 16, e)
                    if k < kdim:
                        out[16 * t + ln % 16, k] = frags[t, s, ln, e]
    return out


@pytest.mark.parametrize("chunk", [64, 16])
def test_stage_outputs_match_oracle_chunks(chunk):
    say(f"stage outputs T=200 d=128 C={chunk} bf16")
    inp = random_prefill(12, [77, 123], 2, 6, 128, "bf16")
    d = on_dev(inp)
    dims = gdn.make_dims(2, 200, 2, 6, 128, 128, chunk, torch.bfloat16)
    lay = gdn.gdn_chunk_fwd_workspace_layout(dims)
    ws = torch.zeros(lay.total, dtype=torch.uint8, device=DEV)
    gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["init_state"],
                      d["cu_seqlens"], chunk=chunk, workspace=ws)
    torch.cuda.synchronize()
    wsc = ws.cpu()
    nc = lay.max_chunks
    ct, cks = chunk // 16, (chunk // 16 + 1) // 2

    def region(off, count, dt):
        return wsc[off:off + count * torch.tensor([], dtype=dt).element_size()].view(dt)

    table = region(lay.chunk_table, nc * 4, torch.int32).view(nc, 4).numpy()
    tf = region(lay.tinv, nc * 6 * ct * cks * 512, torch.bfloat16).view(
        nc, 6, ct, cks, 64, 8).double().numpy()
    wf = region(lay.w, nc * 6 * ct * 4 * 512, torch.bfloat16).view(
        nc, 6, ct, 4, 64, 8).double().numpy()
    kt = region(lay.key_t, nc * 2 * 8 * cks * 512, torch.bfloat16).view(
        nc, 2, 8, cks, 64, 8).double().numpy()
    qf = region(lay.q_frag, nc * 2 * ct * 4 * 512, torch.bfloat16).view(
        nc, 2, ct, 4, 64, 8).double().numpy()
    pm = region(lay.pmask, nc * 6 * ct * cks * 512, torch.bfloat16).view(
        nc, 6, ct, cks, 64, 8).double().numpy()
    dtab = region(lay.dtab, nc * 6 * (2 * chunk + 4), torch.float32).view(
        nc, 6, 2 * chunk + 4).double().numpy()
    _, _, stages = O.chunkwise(**oracle_args(inp), chunk=chunk, keep_stages=True)
    q64, k64, b64 = np64(inp["q"]), np64(inp["k"]), np64(inp["beta"])
    n_seq0 = -(-77 // chunk)
    assert len(stages) == n_seq0 + -(-123 // chunk)
    for c, st in enumerate(stages):
        L, t0 = st["len"], st["start"]
        assert list(table[c]) == [st["seq"], t0, L, c - (0 if st["seq"] == 0 else n_seq0)]
        for h in range(6):
            # Tinv diag(b) against the oracle's Tinv, W against the oracle's W
            bh = b64[t0:t0 + L, h]
            tm = unfrag(tf[c, h], chunk, chunk)
            check(tm[:L, :L], st["T"][h] * bh[None, :], torch.bfloat16, f"Tinv diag(b) chunk {c} head {h}")
            assert np.allclose(tm[L:, :], 0) and np.allclose(tm[:, L:], 0)
            wm = unfrag(wf[c, h], chunk, 128)              # [token r][d]
            check(wm[:L], st["W"][h], torch.bfloat16, f"W chunk {c} head {h}")
            assert (wm[L:] == 0).all()
            # masked, decayed q.k: P[r][j] = q_r . k_j exp(g_r - g_j) for j <= r
            gh = st["g"][h]
            hq_ = h // 3
            qkd = q64[t0:t0 + L, hq_] @ k64[t0:t0 + L, hq_].T
            dec = np.exp(np.minimum(gh[:, None] - gh[None, :], 0.0))
            want_p = np.tril(qkd * dec)
            pmm = unfrag(pm[c, h], chunk, chunk)           # [query r][key j]
            check(pmm[:L, :L], want_p, torch.bfloat16, f"P chunk {c} head {h}")
            assert (pmm[L:] == 0).all() and (pmm[:, L:] == 0).all()
            # row factors exp(g_r), exp(g_L - g_r) (zero past the end), exp(g_L)
            check(dtab[c, h, :L], np.exp(gh), torch.float32, f"exp(g) chunk {c} head {h}")
            check(dtab[c, h, chunk:chunk + L], np.exp(gh[-1] - gh), torch.float32, f"exp(g_L-g) chunk {c} head {h}")
            assert (dtab[c, h, L:chunk] == 0).all() and (dtab[c, h, chunk + L:2 * chunk] == 0).all()
            check(dtab[c, h, 2 * chunk:2 * chunk + 1], np.exp(gh[-1:]), torch.float32, f"exp(g_L) chunk {c} head {h}")
        for hq in range(2):
            ktm = unfrag(kt[c, hq], 128, chunk)            # [d][i]
            assert np.array_equal(ktm[:, :L], k64[t0:t0 + L, hq].T) and (ktm[:, L:] == 0).all()
            qfm = unfrag(qf[c, hq], chunk, 128)            # [r][d]
            assert np.array_equal(qfm[:L], q64[t0:t0 + L, hq]) and (qfm[L:] == 0).all()
    assert (table[len(stages):, 0] == -1).all()


# --- structure: state carry, aliasing, repeatability ---------------------------

def test_split_on_chunk_boundary_is_bitwise_equal():
    say("state carry across calls, split at 192 of 320")
    inp = random_prefill(13, [320], 2, 6, 128, "bf16")
    d = on_dev(inp)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                               d["init_state"])
    s = slice(0, 192)
    t = slice(192, 320)
    oa, fa = gdn.gdn_chunk_fwd(d["q"][s], d["k"][s], d["v"][s], d["log_alpha"][s],
                               d["beta"][s], d["init_state"])
    ob, fb = gdn.gdn_chunk_fwd(d["q"][t].contiguous(), d["k"][t].contiguous(),
                               d["v"][t].contiguous(), d["log_alpha"][t].contiguous(),
                               d["beta"][t].contiguous(), fa)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob]), o)
    assert torch.equal(fb, fin)


def test_final_state_may_alias_init_state():
    say("final_state aliases init_state")
    inp = random_prefill(14, [100, 60], 2, 6, 128, "bf16")
    d = on_dev(inp)
    o_ref, f_ref = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                                     d["init_state"], d["cu_seqlens"])
    st = d["init_state"].clone()
    o, f = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], st,
                             d["cu_seqlens"], final_state=st)
    torch.cuda.synchronize()
    assert f.data_ptr() == st.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(st, f_ref)


def test_repeatable_bitwise():
    say("two identical runs are bitwise equal")
    inp = random_prefill(15, [500, 3, 260], 2, 6, 128, "bf16")
    o1, f1 = run_gpu(inp, 64)
    o2, f2 = run_gpu(inp, 64)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


# --- decode ------------------------------------------------------------------

@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (128, "f32"), (16, "bf16"), (16, "f32")])
def test_decode_steps_small(d, dtype):
    say(f"decode N=5 d={d} {dtype} x6 steps")
    inp = I.make_decode(16 + d, 5, 6, 2, 6, d, dtype)
    state = inp["state0"].to(DEV)
    ref = np64(inp["state0"])
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    for t in range(6):
        args = [inp[n][t] for n in ("q", "k", "v", "log_alpha", "beta")]
        o = gdn.gdn_decode_step(*[a.to(DEV) for a in args], state)
        torch.cuda.synchronize()
        want_o, ref = O.decode_step(ref, *[np64(a) for a in args])
        check(o, want_o, tdt, f"o step {t}")
    check(state, ref, tdt, "state after 6 steps")


def test_decode_matches_prefill_of_same_tokens():
    say("decode x32 vs GPU prefill of the same tokens")
    n, steps = 4, 32
    inp = I.make_decode(17, n, steps, 2, 6, 128, "bf16")
    state = inp["state0"].to(DEV)
    outs = []
    for t in range(steps):
        outs.append(gdn.gdn_decode_step(*[inp[x][t].to(DEV) for x in
                                          ("q", "k", "v", "log_alpha", "beta")], state))
    # same tokens as packed sequences: sequence b holds steps 0..31 of batch b
    perm = lambda x: x.transpose(0, 1).reshape(n * steps, *x.shape[2:]).contiguous()  # noqa: E731
    cu = torch.arange(n + 1, dtype=torch.int32) * steps
    o_pf, f_pf = gdn.gdn_chunk_fwd(*[perm(inp[x]).to(DEV) for x in
                                     ("q", "k", "v", "log_alpha", "beta")],
                                   inp["state0"].to(DEV), cu.to(DEV), chunk=16)
    torch.cuda.synchronize()
    o_dec = torch.stack(outs).transpose(0, 1).reshape(n * steps, 6, 128)
    check(o_dec, np64(o_pf), torch.bfloat16, "decode vs prefill o")
    check(state, np64(f_pf), torch.bfloat16, "decode vs prefill state")


# --- speculative multi-token verify (gdn_decode_multi) --------------------------

@pytest.mark.parametrize("kt", [1, 4])
@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (128, "f32"), (16, "bf16"), (16, "f32")])
def test_decode_multi_equals_single_steps(d, dtype, kt):
    say(f"decode_multi K={kt} N=5 d={d} {dtype} vs single steps")
    inp = I.make_decode(40 + d + kt, 5, kt, 2, 6, d, dtype)
    args = [inp[n].to(DEV) for n in ("q", "k", "v", "log_alpha", "beta")]
    st1 = inp["state0"].to(DEV)
    o1, states = [], []
    for t in range(kt):
        o1.append(gdn.gdn_decode_step(*[a[t] for a in args], st1))
        states.append(st1.clone())
    st2 = inp["state0"].to(DEV)
    snaps = torch.full((kt,) + tuple(st2.shape), float("nan"), dtype=torch.float32, device=DEV)
    o2 = gdn.gdn_decode_multi(*args, st2, snapshots=snaps)
    st3 = inp["state0"].to(DEV)
    o3 = gdn.gdn_decode_multi(*args, st3)
    torch.cuda.synchronize()
    # with snapshots the state is only read; without, it ends after the last token
    assert torch.equal(st2, inp["state0"].to(DEV))
    assert torch.equal(st3, states[-1])
    for t in range(kt):
        assert torch.equal(o2[t], o1[t]) and torch.equal(o3[t], o1[t]), f"o token {t}"
        assert torch.equal(snaps[t], states[t]), f"snapshot {t}"


def test_decode_multi_matches_oracle():
    say("decode_multi K=8 N=3 d=128 bf16 vs oracle")
    kt = 8
    inp = I.make_decode(51, 3, kt, 2, 6, 128, "bf16")
    args = [inp[n].to(DEV) for n in ("q", "k", "v", "log_alpha", "beta")]
    state = inp["state0"].to(DEV)
    snaps = torch.empty((kt,) + tuple(state.shape), dtype=torch.float32, device=DEV)
    o = gdn.gdn_decode_multi(*args, state, snapshots=snaps)
    torch.cuda.synchronize()
    ref = np64(inp["state0"])
    for t in range(kt):
        want_o, ref = O.decode_step(ref, *[np64(inp[n][t]) for n in ("q", "k", "v", "log_alpha", "beta")])
        check(o[t], want_o, torch.bfloat16, f"o token {t}")
        check(snaps[t], ref, torch.bfloat16, f"state after token {t}")
