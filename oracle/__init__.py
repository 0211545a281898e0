"""Plain, slow, fp64 CPU oracle for sparse block / offset attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers or tables),
and it imports nothing from ``long_context_sparse_block_amd``.

Every function follows a passage of the source pages, cited by page title and
section / equation / algorithm:

* "Parameter-free Adaptive Sparse Attention via Compression-Based Content
  Selection" (arXiv 2607.21752) -- block mask M = M^lit U M^local U I (Sec. 3.2,
  Eq. 3; Appendix B, Algorithm 1), expansion to tokens and causal AND (Sec. 3.4
  "Block-to-token expansion"; Algorithm 1 step 4), literal flags from per-block
  gzip sizes and the mean threshold (Sec. 3.1, Eq. 1-2; Algorithm 1 steps 1-2).
* "BigBird" (llm-arch-kb) -- window / global / random graphs and their edge
  counts (Sec. 2 "Derivation"), and the dense-masked formulation (Sec. 3
  "Reference implementation").
* "Depth-Staggered Fibonacci Spacing for Sparse Attention" (arXiv 2606.28560)
  -- attended set {0..W} U {alpha * f_k} (Sec. 2 "Attended set", "The per-layer
  scalar").

Modules:
  rng         SplitMix64 and the counter-keyed draws built on it
  literal     literal flags from byte content (gzip block sizes, mean threshold)
  block_mask  mask components, union, CSR, longest-first schedule
  attention   block-sparse attention: CSR-gather form and dense-masked form
  offsets     offset table and token-level offset attention (and variants)
  backward    gradients (dq, dk, dv) of both: dense-masked, CSR-gather, offsets
  tiny        pure-Python loop versions for tiny inputs (brute force)
"""

from . import rng, literal, block_mask, attention, offsets, tiny, backward  # noqa: F401
