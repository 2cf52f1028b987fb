"""P9: the compaction invariant (CPU only)."""

import numpy as np

from oracle.compact import compact_kv


def test_compaction_moves_accepted_rows_and_nothing_else():
    rng = np.random.default_rng(0)
    L, B, H, S, hd = 3, 4, 2, 40, 8
    k = rng.normal(size=(L, B, H, S, hd)).astype(np.float32)
    v = rng.normal(size=(L, B, H, S, hd)).astype(np.float32)
    base = np.array([5, 10, 0, 20])
    D = 4
    nodes = np.array([[2, 5, 9, -1],   # sources 7,10,14 -> 6,7,8: slot 7 is read and written
                      [1, 2, 3, 4],    # identity moves
                      [-1, -1, -1, -1],
                      [3, 4, -1, -1]])
    alen = np.array([3, 4, 0, 2])
    k0, v0 = k.copy(), v.copy()
    compact_kv(k, v, base, nodes, alen)
    for b in range(B):
        dest = set(range(base[b] + 1, base[b] + 1 + alen[b]))
        for s in range(S):
            if s in dest:
                j = s - base[b] - 1
                src = base[b] + nodes[b, j]
                np.testing.assert_array_equal(k[:, b, :, s], k0[:, b, :, src])
                np.testing.assert_array_equal(v[:, b, :, s], v0[:, b, :, src])
            else:
                np.testing.assert_array_equal(k[:, b, :, s], k0[:, b, :, s])
                np.testing.assert_array_equal(v[:, b, :, s], v0[:, b, :, s])
