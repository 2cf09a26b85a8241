"""Plain, slow CPU oracle of the LoReS quantized recurrent-state decode step.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  The product (the HIP library and
its Python binding) never imports, links or calls it, and it shares no code
with the product: it is written from the pages, in NumPy, and checked against
closed forms, exact rational arithmetic, published test vectors and the
pages' propositions (tests/test_oracle_*.py).

Source pages, cited by title and section:
  [LoReS] "Quantizing Recurrent Language Models Is Easier Than You Think",
          structured summary page: sections "Introduction and Theoretical
          Foundation" (general recurrence form; error propagation),
          "Intra-State Quantization (Section 4)" (scale grouping,
          Proposition 1, decay-based mixed precision, Proposition 2,
          rounding, Proposition 3) and the paper abstract (value-axis
          scale grouping, decay-based mixed precision, stochastic rounding).
  [PACE]  "PACE: Periodic and Channel-Aligned Encoding of Four-Bit Recurrent
          States", abstract (rounding once every few tokens with a buffer;
          column scales); [LeapQuant] abstract (per-window quantization).

Parity status per function (what pins it is listed in each module):
  exact.fma32 / exact.rd_div32 / exact.rn_div32 .... pinned (Fraction brute force)
  rng.mix64 / rng.fmix32 ........................... pinned (published test vectors)
  rng.unit_key / rng.noise16 ....................... PARITY UNPINNED by the pages
       (the pages fix no generator; only distribution tests apply)
  step.reference_step64 ............................ pinned (closed forms, Fraction)
  step.decode_step (fp32 heads) .................... pinned (closed forms, bounds)
  step.decode_step (int8 / int4 / bf16 heads) ...... pinned (exhaustive SR in even and
       odd columns, the antithetic pair probabilities, bounds, Propositions 1-3)
  step.quantize_rows / decode_step, axis="key" ..... pinned (hand-worked codes,
       rank-one structure, transpose identity, unbiasedness, variance)
  assign.decay_stat / assign.assign_precision ...... pinned (hand-worked cases)
  window.window_step / replay ...................... pinned (W = 1 is the per-step
       step; closed forms for delta = 0; the fp64 recurrence inside a window;
       one rounding per window)
"""
from . import exact, rng, step, assign, window  # noqa: F401
