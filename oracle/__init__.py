"""fp64 CPU oracle for the complex-valued attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything here: only the tests, the smoke check and the benchmark's
CPU-baseline leg do.  The oracle shares no code with the HIP path; it reads
the same seeded host inputs (already rounded to the device dtype and promoted
to fp64) and computes the plain definitions in complex128:

* :mod:`oracle.born`  -- Born-rule attention ("CNet: A Complex-Valued Deep
  Learning Framework ...", section 11.2, paragraph "Closing it: Born-rule
  attention", and Figure 2).
* :mod:`oracle.pct`   -- phase-coherent (PCT) attention ("Complex-valued
  Phase-Coherent Transformers", section 1 and Appendix D.2), and the family's
  L2-softmax and screening gates (Appendix D.2).
* :mod:`oracle.born_density` -- a second, independent formulation of Born
  attention through causal density-matrix prefix states ("The Quantum
  Shortcut", section 2, the Born rule as a linear functional of the density
  matrix; "Show HN: CNET", BornAttention, its exact finite feature map).  It is
  used only to pin :mod:`oracle.born`.
* :mod:`oracle.born_grad`, :mod:`oracle.pct_grad` -- the backward of both
  operators in closed form (gradients dL/d(conj z) as in "CNet ...", section 3,
  rule (2)), derived from the forward definitions and pinned by finite
  differences.
* :mod:`oracle.rotary` -- the rotary phase embedding ("Show HN: CNET",
  RotaryEmbed).
* :mod:`oracle.born_linear` -- Born attention with a carried density state:
  state build, prefill with an incoming state, and the one-token step
  ("Show HN: CNET", BornAttention's linear and step modes).

Every function here is pinned by the CPU tests against closed forms,
invariants, hand-derived worked examples and the second formulation.
"""
from .born import born_attention, born_attention_rows
from .pct import pct_attention, pct_attention_rows, pct_scores, pct_screen_attention, pct_softmax_attention
from .born_density import born_attention_density
from .born_grad import born_attention_bwd
from .pct_grad import pct_attention_bwd
from .rotary import rotary
from .born_linear import (born_prefill, born_state, born_step, pack_hermitian, pack_state,
                          unpack_hermitian, unpack_state)

__all__ = [
    "born_attention", "born_attention_rows",
    "pct_attention", "pct_attention_rows", "pct_scores", "pct_softmax_attention", "pct_screen_attention",
    "born_attention_density",
    "born_attention_bwd", "pct_attention_bwd",
    "rotary", "born_state", "born_step", "born_prefill",
    "pack_hermitian", "unpack_hermitian", "pack_state", "unpack_state",
]
