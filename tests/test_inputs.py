"""The seeded input generators that draw on a device (used where inputs are
too large to draw on the host): the recipe's shapes, dtypes and value
ranges, one sequence or packed lengths, and repeatability for a seed. Run
here on the CPU device. CPU only."""
import numpy as np
import torch

from linear_attention_recurrence_delta_amd import inputs as I


def test_prefill_device_recipe_and_packing():
    one = I.make_prefill_device(5, 300, 2, 6, 16, "cpu")
    assert one["cu_seqlens"] is None and one["init_state"].shape == (1, 6, 16, 16)
    lens = [70, 0, 1, 229]
    d = I.make_prefill_device(5, lens, 2, 6, 16, "cpu")
    assert d["cu_seqlens"].tolist() == [0, 70, 70, 71, 300]
    assert d["q"].shape == (300, 2, 16) and d["k"].shape == (300, 2, 16) and d["v"].shape == (300, 6, 16)
    assert d["q"].dtype == torch.bfloat16 and d["v"].dtype == torch.bfloat16
    assert d["log_alpha"].shape == (300, 6) and d["beta"].shape == (300, 6)
    assert d["log_alpha"].dtype == torch.float32 and d["init_state"].shape == (4, 6, 16, 16)
    # q, k unit rows (to bf16 rounding); log a < 0; b in (0, 1); state ~ N(0, 0.02^2)
    for x in ("q", "k"):
        assert np.allclose(d[x].float().norm(dim=-1).numpy(), 1.0, atol=1e-2)
    assert (d["log_alpha"] < 0).all() and ((d["beta"] > 0) & (d["beta"] < 1)).all()
    assert 0.015 < float(d["init_state"].std()) < 0.025
    # the same seed draws the same tensors; another seed others
    again = I.make_prefill_device(5, lens, 2, 6, 16, "cpu")
    other = I.make_prefill_device(6, lens, 2, 6, 16, "cpu")
    for x in ("q", "k", "v", "log_alpha", "beta", "init_state"):
        assert torch.equal(d[x], again[x])
        assert not torch.equal(d[x], other[x])


def test_decode_and_backward_seed_device_recipes():
    one = I.make_decode_device(7, 5, 2, 6, 16, "cpu")
    assert one["state0"].shape == (5, 6, 16, 16) and one["q"].shape == (5, 2, 16)
    assert one["v"].shape == (5, 6, 16) and one["beta"].shape == (5, 6)
    steps = I.make_decode_device(7, 5, 2, 6, 16, "cpu", steps=3)
    assert steps["q"].shape == (3, 5, 2, 16) and steps["log_alpha"].shape == (3, 5, 6)
    # the state is drawn first, so it does not depend on the step count
    assert torch.equal(one["state0"], steps["state0"])
    assert np.allclose(steps["k"].float().norm(dim=-1).numpy(), 1.0, atol=1e-2)
    assert (steps["log_alpha"] < 0).all() and ((steps["beta"] > 0) & (steps["beta"] < 1)).all()
    s = I.make_backward_seeds_device(8, 40, 6, 16, "cpu")
    assert s["d_o"].shape == (40, 6, 16) and s["d_o"].dtype == torch.bfloat16
    assert s["d_final"].shape == (1, 6, 16, 16) and s["d_final"].dtype == torch.float32
    assert torch.equal(s["d_o"], I.make_backward_seeds_device(8, 40, 6, 16, "cpu")["d_o"])
