"""gdn_chunk_fwd_noalloc (the prefill entry point that allocates nothing,
its workspace being the library's own device array) against gdn_chunk_fwd
on the same inputs, through the C ABI: two calls in a row, the second with a
smaller input, must give gdn_chunk_fwd's results bit for bit (the same
kernels run on the same workspace layout), and dims beyond the array's size
are rejected before anything is enqueued."""
import pytest
import torch

import linear_attention_recurrence_delta_amd as gdn
from linear_attention_recurrence_delta_amd import binding as B
from linear_attention_recurrence_delta_amd import inputs as I

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def both(inp, chunk):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = [d[x] for x in ("q", "k", "v", "log_alpha", "beta", "init_state")]
    want = gdn.gdn_chunk_fwd(*args, d["cu_seqlens"], chunk=chunk)
    got = gdn.gdn_chunk_fwd_noalloc(*args, d["cu_seqlens"], chunk=chunk)
    torch.cuda.synchronize()
    return got, want


def test_noalloc_equals_chunk_fwd_on_two_calls_then_rejects_oversize():
    # first call: 16 QK / 48 V heads, three sequences (one empty), bf16, C = 64
    lens = [1200, 0, 833]
    say(f"noalloc call 1: {lens} 16/48 heads d=128 C=64 bf16")
    dims = gdn.make_dims(len(lens), sum(lens), 16, 48, 128, 128, 64, torch.bfloat16)
    assert gdn.gdn_chunk_fwd_workspace_bytes(dims) <= B.NOALLOC_SCRATCH_BYTES
    (o1, f1), (o1w, f1w) = both(I.make_prefill(81, lens, 16, 48, 128, "bf16", "randn"), 64)
    assert torch.equal(o1, o1w) and torch.equal(f1, f1w)
    # second call, smaller: it reuses the array the first call filled
    lens = [130, 7]
    say(f"noalloc call 2: {lens} 2/6 heads d=128 C=16 bf16")
    (o2, f2), (o2w, f2w) = both(I.make_prefill(82, lens, 2, 6, 128, "bf16", "randn"), 16)
    assert torch.equal(o2, o2w) and torch.equal(f2, f2w)
    # fp32, head dim 16
    say("noalloc call 3: [64] 1/1 head d=16 C=16 fp32")
    (o3, f3), (o3w, f3w) = both(I.make_prefill(83, [64], 1, 1, 16, "f32", "zeros"), 16)
    assert torch.equal(o3, o3w) and torch.equal(f3, f3w)
    # dims whose workspace exceeds the array: rejected, nothing enqueued
    big = [8192]
    dims = gdn.make_dims(1, sum(big), 16, 48, 128, 128, 64, torch.bfloat16)
    assert gdn.gdn_chunk_fwd_workspace_bytes(dims) > B.NOALLOC_SCRATCH_BYTES
    inp = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
           for k, v in I.make_prefill(84, big, 16, 48, 128, "bf16", "zeros").items()}
    o = torch.full_like(inp["v"], 7.0)
    with pytest.raises(gdn.GdnError, match="GDN_NOALLOC_SCRATCH_BYTES"):
        gdn.gdn_chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], o=o)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
    # and the array still serves a call afterwards
    (o4, f4), (o4w, f4w) = both(I.make_prefill(85, [300], 2, 6, 128, "bf16", "randn"), 64)
    assert torch.equal(o4, o4w) and torch.equal(f4, f4w)
