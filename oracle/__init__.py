"""fp64 CPU oracle for the Zebra3D global multi-view attention stage.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library (no
kernels, headers, tables or helpers); both sides only read the same seeded
inputs from `zebra_synth`.

Everything here is plain, slow and written to be checked by eye against the
source pages ("How Hybrid Attention Lets Feed-Forward 3D Models Scale to Many
Views", wispaper.ai, and its translations). All floating-point work is
float64; bf16 inputs are widened exactly before use.

  layout.py  tile map: frames, special tokens, 8x8-patch tiles with partial
             edge tiles ("Linear-centered stages plus tile-sparse stages").
  sparse.py  mean-K/V landmarks, top-k tile selection, tile-sparse softmax
             attention with landmarks, special keys/rows and the self key,
             and dense softmax attention ("Linear-centered stages plus
             tile-sparse stages"; "Global attention dominates runtime").
  coverage.py  attention-mass coverage of the kept tiles and the landmark
             error of the omitted ones, per query tile ("Sensitive stages
             also concentrate their attention").
  block.py   frame-wise attention, and the RMSNorm + 2D-rotary prologue of
             the queries and keys of a sparse stage ("Global attention
             dominates runtime as views grow"; "Linear-centered stages plus
             tile-sparse stages").
  backward.py  gradients of the linear and the tile-sparse stages with
             respect to Q, K and V: the chain rule of linear.py and
             sparse.py taken back step by step ("A closed-form fit avoids
             retraining from scratch": the optional training stage after
             conversion).
  linear.py  RMSNorm, 2D rotary, channel-softmax feature map, linear
             attention and the centred affine output correction
             ("Speedup scales with the number of input views" for the fused
             normalisation/rotation/feature map; "A closed-form fit avoids
             retraining from scratch" for the centred affine correction).

Pins: every function is checked in tests/test_oracle_*.py against something
other than itself (brute force, closed forms, invariants, hand-derived
golden fixtures). The exact outputs at the synthetic 32..1,024-view shapes
are not printed anywhere on the pages; only those invariants pin them.
"""
from . import layout, sparse, linear, coverage, block, backward  # noqa: F401
