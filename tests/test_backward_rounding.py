"""The backward pass's bf16 tolerance, from the rounding emulation in
tests/backward_rounding.py (CPU, no GPU): without rounding the emulation's
chunkwise gradients equal the oracle's backpropagation through the form-1
recurrence (page "Qwen3.8-Flash-Next 技术总结", section 2.1); with the
kernels' bf16 roundings they stay within a few 1e-3 of it, a factor of
about 3-4 under the 1e-2 relative-L2 bound the GPU tests use."""
import numpy as np
import pytest

from oracle import gdn_oracle as O
from tests import backward_rounding as R


def oracle_grads(inp, d_o, d_final):
    g = O.recurrent_form1_backward(inp["q"][:, None], inp["k"][:, None], inp["v"][:, None],
                                   inp["log_alpha"][:, None], inp["beta"][:, None], d_o[:, None],
                                   d_final[None, None], inp["s0"][None, None])
    return dict(q=g["dq"][:, 0], k=g["dk"][:, 0], v=g["dv"][:, 0], log_alpha=g["dlog_alpha"][:, 0],
                beta=g["dbeta"][:, 0], s0=g["dinit"][0, 0])


@pytest.mark.parametrize("T,d,chunk", [(150, 16, 16), (150, 16, 64), (70, 32, 64)])
def test_unrounded_emulation_equals_oracle_backprop(T, d, chunk):
    inp, d_o, d_final = R.random_head(3, T, d)
    got = R.gradients(inp, d_o, d_final, chunk, False)
    want = oracle_grads(inp, d_o, d_final)
    for name in want:
        rel = np.linalg.norm(got[name] - want[name]) / np.linalg.norm(want[name])
        assert rel < 1e-10, (name, rel)


@pytest.mark.parametrize("chunk", [16, 64])
def test_rounded_emulation_is_inside_the_backward_tolerance(chunk):
    errs = R.rounding_errors(5, 256, 128, chunk)
    for name, (rel, mx) in errs.items():
        assert 1e-4 < rel < 5e-3, (name, rel)        # rounding applied, and well under 1e-2
        assert mx < 2e-2, (name, mx)
