"""KV compaction of the accepted path (TEST INFRASTRUCTURE).

After verification the K/V rows of the accepted tree nodes move to the slots
right after the root, so the cache again holds one contiguous sequence.  The
vLLM Neuron design page fixes the slot arithmetic ("KV Cache Sharing":
slot = block_table[pos // block_size] * block_size + pos % block_size); with
one contiguous block per sequence, tree node n of a sequence whose root sits at
slot ``base`` lives at slot base + n.  Compaction reads every accepted row
first, then writes row j to slot base + 1 + j; rows at or below base and all
rows beyond the accepted ones are untouched.

Pinned by tests/test_oracle_compact.py (the invariant holds for every layer,
sequence and head, including a case where one row's source is another's
destination).
"""

from __future__ import annotations

import numpy as np


def compact_kv(k, v, tree_base, accepted_nodes, accepted_len):
    """k, v: [layers, B, n_kv, S, hd] arrays, modified in place."""
    B = k.shape[1]
    for b in range(B):
        a = int(accepted_len[b])
        base = int(tree_base[b])
        src = [base + int(accepted_nodes[b, j]) for j in range(a)]
        rows_k = [k[:, b, :, s, :].copy() for s in src]
        rows_v = [v[:, b, :, s, :].copy() for s in src]
        for j in range(a):
            k[:, b, :, base + 1 + j, :] = rows_k[j]
            v[:, b, :, base + 1 + j, :] = rows_v[j]
    return k, v
