"""MI355X-native EAGLE-3 / EAGLE-4 speculation step.

The hot path (draft tree construction, verification, KV compaction) runs in
hand-written HIP kernels for gfx950 behind the C ABI of include/spec.h;
this package is the thin Python binding (``spec``) plus the build script.
"""

from .spec import (KVCache, SpecContext, SpecError, Tree, Weights, spec_build_tree,  # noqa: F401
                   spec_compact_kv, spec_draft_step, spec_topk_logprobs, spec_tree_from_topk,
                   spec_verify_tree)
