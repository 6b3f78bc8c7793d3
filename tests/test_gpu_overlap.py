"""Prefill with kernel 2 beside the scan, through the C ABI.

When the scan leaves CUs idle (few heads and sequences) and the input has
enough chunks, gdn_chunk_fwd cuts the chunk slots in two windows: kernel 2
forms the second window on a second stream while the scan runs the first,
and a second scan launch continues from the state the first left in
final_state. The stage-by-stage calls (gdn_chunk_fwd_stages 1..1, then
2..2) never split, so they are the reference here: the arithmetic per chunk
is the same and the carried state is fp32, so every output must be bitwise
equal. Each case first checks that its shape meets the split's conditions
(at least 256 chunk slots, at most four fifths of the CUs held by the
scan's workgroups), so that it exercises the two-window path."""
import pytest
import torch

import linear_attention_recurrence_delta_amd as gdn
from linear_attention_recurrence_delta_amd import binding as B
from linear_attention_recurrence_delta_amd import inputs as I

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def scan_groups(n_seqs, h_v, d, chunk, dtype):
    # one scan workgroup per (sequence, V head, column block): 32 columns,
    # 16 at d = 16 and for fp32 inputs at d = 128 with 64-token chunks
    cols = 16 if d == 16 or (dtype == torch.float32 and chunk == 64) else 32
    return n_seqs * h_v * (d // cols)


def assert_splits(lens, h_v, d, chunk, dtype):
    nc = sum(lens) // chunk + len(lens)
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    g = scan_groups(len(lens), h_v, d, chunk, dtype)
    assert nc >= 256 and 5 * g <= 4 * cus, (nc, g, cus)


def run(d, chunk, stages, final_state, init=None, **kw):
    return gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                             d["init_state"] if init is None else init, d["cu_seqlens"],
                             chunk=chunk, final_state=final_state, stages=stages, **kw)


def serial(d, chunk, init=None, **kw):
    # stage 2 reads what stage 1 left in the workspace: one buffer for both
    flags = (B.GDN_FLAG_PREPARE_INPUTS if kw.get("prepare_inputs") else 0) | \
            (0 if kw.get("delta_rule", True) else B.GDN_FLAG_NO_DELTA_RULE)
    dims = gdn.make_dims(d["cu_seqlens"].numel() - 1, d["q"].shape[0], d["q"].shape[1], d["v"].shape[1],
                         d["q"].shape[2], d["v"].shape[2], chunk, d["q"].dtype, flags)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_bytes(dims), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(d["v"])
    fin = torch.full_like(d["init_state"], float("nan"))
    run(d, chunk, (1, 1), fin, init, workspace=ws, o=o, **kw)
    run(d, chunk, (2, 2), fin, init, workspace=ws, o=o, **kw)
    return o, fin


def whole(d, chunk, init=None, final_state=None, **kw):
    fin = torch.full_like(d["init_state"], float("nan")) if final_state is None else final_state
    o, _ = run(d, chunk, None, fin, init, **kw)
    return o, fin


def assert_bitwise(a, b, what):
    assert torch.equal(a, b), f"{what}: max |diff| {(a.double() - b.double()).abs().max().item():.3e}"


def test_long_sequence_split_equals_serial():
    say("overlap: long_64k (1 x 65536 tokens, 16/48 heads, bf16) whole call vs stage-by-stage")
    inp = I.workload_inputs("long_64k")
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    assert_splits([d["q"].shape[0]], 48, 128, 64, torch.bfloat16)
    o1, f1 = serial(d, 64)
    o2, f2 = whole(d, 64)
    torch.cuda.synchronize()
    assert_bitwise(o2, o1, "o")
    assert_bitwise(f2, f1, "final state")
    # without a final state the launches run one after the other
    o3, f3 = run(d, 64, None, None, output_final_state=False)
    torch.cuda.synchronize()
    assert f3 is None
    assert_bitwise(o3, o1, "o without final state")


# sequences wholly before the window boundary, one across it, and wholly
# after it, with an empty and a one-token sequence among them
LENS = [5000, 0, 1, 7000, 3333, 64, 2500]


@pytest.mark.parametrize("variant", ["plain", "in_place", "gate_only", "prepare"])
def test_packed_sequences_split_equals_serial(variant):
    say(f"overlap: 7 packed sequences (2/6 heads, d=128, C=64, bf16) {variant}")
    assert_splits(LENS, 6, 128, 64, torch.bfloat16)
    make = I.make_prefill_raw if variant == "prepare" else I.make_prefill
    inp = make(71, LENS, 2, 6, 128, "bf16", "randn")
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    kw = {"prepare": {"prepare_inputs": True}, "gate_only": {"delta_rule": False}}.get(variant, {})
    o1, f1 = serial(d, 64, **kw)
    if variant == "in_place":
        st = d["init_state"].clone()
        o2, f2 = whole(d, 64, init=st, final_state=st)
    else:
        o2, f2 = whole(d, 64, **kw)
    torch.cuda.synchronize()
    assert_bitwise(o2, o1, "o")
    assert_bitwise(f2, f1, "final state")
    # the empty sequence's final state is its initial state
    assert_bitwise(f2[1], d["init_state"][1], "empty sequence")


def test_small_head_dim_split_equals_serial():
    say("overlap: 3 sequences (4/8 heads, d=16, C=16, fp32)")
    lens = [2100, 1500, 900]
    assert_splits(lens, 8, 16, 16, torch.float32)
    inp = I.make_prefill(72, lens, 4, 8, 16, "f32", "randn")
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o1, f1 = serial(d, 16)
    o2, f2 = whole(d, 16)
    torch.cuda.synchronize()
    assert_bitwise(o2, o1, "o")
    assert_bitwise(f2, f1, "final state")
