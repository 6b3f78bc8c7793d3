"""CPU oracle for the Gated DeltaNet token mixer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with
the HIP library (no kernels, headers, helpers or constants), and it imports
nothing from the ``linear_attention_recurrence_delta_amd`` package.

Source of the method: the web page "Qwen3.8-Flash-Next 技术总结：Qwen4 架构的
'探路者'" (a repost of a CSDN article), section 2.1 "Gated DeltaNet". That
section gives the state update in two algebraically equal forms (the two
lines of its update equation), the meaning of alpha_t (a data-dependent
forget gate in (0,1)) and beta_t (the delta-rule write strength), the head
layout (48 V heads, 16 QK heads, head dim 128), and names -- without
formulas -- the chunkwise WY-representation algorithm used on GPUs.

Modules:
  gdn_oracle      fp64 NumPy: sequential recurrence (form 1 and form 2),
                  a chunkwise fp64 evaluation with per-stage outputs, the
                  one-token decode step.
  exact_rational  exact rational arithmetic (fractions.Fraction) on tiny
                  inputs, used to write golden fixtures.
"""
from .gdn_oracle import (  # noqa: F401
    head_group,
    seq_bounds,
    recurrent_form1,
    recurrent_form2,
    chunkwise,
    decode_step,
)
