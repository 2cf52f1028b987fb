"""CPU oracle for the EAGLE-3 / EAGLE-4 speculation step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
numpy implementation of what the speculation step computes.  Only the tests,
the smoke check and the CPU-baseline leg of the benchmark may import it; the
product path (the HIP library and its Python binding) never does, and this
package imports nothing from the product path.

Precision: tensors the workload holds in bfloat16 are float32 arrays rounded
to bfloat16 (nearest even); large contractions are float32 BLAS matmuls on
those values; attention, softmax, RMSNorm, RoPE and every reduction that
decides a discrete choice run in float64 and are rounded once.

Modules
  numerics  rounding, RMSNorm, RoPE, SiLU
  draft     one draft decoder pass (FC fusion, decoder layer, LM head,
            EAGLE-4 candidate head)
  tree      vocab top-k with log-probs, tree expansion and selection
  verify    greedy and stochastic acceptance, Philox4x32-10
  sampling  flat (variable-length chain) batches: metadata bookkeeping,
            per-request temperature / top-k / top-p rejection sampling
  target    the target's verification forward over the tree (logits and
            aux states)
  compact   KV compaction of the accepted path

Parity status of each function is stated in its docstring; every function is
pinned by a CPU test except where a docstring says "parity unpinned".
"""

from . import numerics, draft, tree, verify, compact, sampling, target  # noqa: F401
