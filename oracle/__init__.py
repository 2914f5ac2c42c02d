"""CPU oracle for the draft-sampling / verification hot path.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
The product path (the HIP library and its Python binding) never imports, calls or links it, and
this package imports nothing from the product path.

Three parts:
  ref    plain float64 numpy restatement of each step, run with the supplied uniforms, so it
         makes the same draws as the GPU path and can be compared draw by draw;
  exact  the same rule over exact rationals (fractions.Fraction) for tiny vocabularies, giving
         the output *distribution*, used to pin `ref` to the mathematics;
  keepset  the offline step before the path: token counting, Top-K / Top-P / minimum-frequency
         selection of the kept vocabulary, and the trimmed head's row gather.

Pages cited (by title and section):
  [VT] "VocabTrim: Vocabulary Pruning for Efficient Speculative Decoding in LLMs" (arXiv 2506.22694v2)
  [GL] "Speculative decoding" (glossary page)
  [RR] "A rejection rule keeps speculative decoding's output exact" (build-from-scratch article)

Every function is pinned by tests under tests/ (test_oracle_*.py); none is "parity unpinned"
except the synthetic input recipe itself, which both sides read as identical arrays.
"""
from . import exact, keepset, ref, stats  # noqa: F401
