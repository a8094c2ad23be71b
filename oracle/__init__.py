"""Plain CPU oracle for the DSA indexer + top-k + absorbed sparse-MLA path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library; both sides receive the same seeded
inputs and compute independently.

Everything here is written for a reader checking it against the pages by eye:
NumPy, float64 arithmetic, no blocking, no fusion, no reordering beyond what a
library primitive (matmul, lexsort) does.  Where the pages fix a precision
(the FP8 cache write rounds in fp32 and e4m3) the oracle reproduces that
rounding explicitly.

Modules
  codecs     bf16 and OCP e4m3fn value codecs
  indexer    key-cache write, indexer score, deterministic top-k
  fp8_indexer  the FP8-query variant: Hadamard rotation, per-row activation
             quantisation, score over e4m3 queries and keys
  prologue   the indexer's inputs: q / k / w projections, RMSNorm k_norm,
             rotate-half RoPE
  mla        absorbed sparse MLA over selected latent rows, and a dense
             causal MLA used only for the sparse == dense invariant
  indexshare GLM-5.2 IndexShare source-layer resolution and layer stack

Pins (what each function is checked against, in tests/test_oracle_*.py):
  codecs      OCP e4m3fn end points and hand-decoded codes (tests/golden),
              bf16 round-to-nearest-even examples
  indexer     brute-force full sort with Python integer/tuple comparison on
              tiny inputs, hand-computed worked example (tests/golden),
              exact-integer scores, threshold certificate, invariants; a
              hand-worked batch of two requests with permuted block tables
              and an FP8 cache with distinct per-slot scales (key values,
              scores and top-k rows)
  mla         sparse == dense when k covers the context, pos == 0 row,
              uniform-logit closed form, permutation invariance, convex hull;
              the same two-request batch with hand-computed outputs
Planted mistakes (a dropped ReLU, the tie rule flipped, the scale divided
or taken from the wrong row, one request's block table used for all, an
off-by-one request lookup, prefill positions for decode queries) each fail
one of these pins.
  indexshare  hand-derived source maps and every rejection case
  fp8_indexer Hadamard orders 2 and 4 by hand, orthogonality and involution,
              dot products kept, the fp32 butterflies within their rounding
              bound, a hand-worked rotation / quantisation / score example
              (tests/golden), brute-force top-k over e4m3 codes
  prologue    a hand-worked two-token example (tests/golden) with every
              intermediate step; RMSNorm unit RMS and scale freedom; RoPE
              norm keeping, identity at angle 0, inverse angle, dependence on
              relative position only; planted interleaved pairs, RoPE on the
              last dims and LayerNorm each fail the example
No oracle function is "parity unpinned".
"""

from . import codecs, indexer, mla, indexshare, fp8_indexer, prologue  # noqa: F401
