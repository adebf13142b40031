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
  Phase-Coherent Transformers", section 1 and Appendix D.2).
* :mod:`oracle.born_density` -- a second, independent formulation of Born
  attention through causal density-matrix prefix states ("The Quantum
  Shortcut", section 2, the Born rule as a linear functional of the density
  matrix; "Show HN: CNET", BornAttention, its exact finite feature map).  It is
  used only to pin :mod:`oracle.born`.

Every function here is pinned by the CPU tests against closed forms,
invariants, hand-derived worked examples and the second formulation.
"""
from .born import born_attention, born_attention_rows
from .pct import pct_attention, pct_attention_rows, pct_scores
from .born_density import born_attention_density

__all__ = [
    "born_attention", "born_attention_rows",
    "pct_attention", "pct_attention_rows", "pct_scores",
    "born_attention_density",
]
