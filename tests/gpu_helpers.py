"""Shared helpers of the GPU parity tests (HIP path through the C ABI vs the
oracle on the same seeded inputs)."""

import numpy as np
import torch

from speculative_decoding_aux_amd import spec as S
from speculative_decoding_aux_amd.tensors import from_device, to_device, upload_kv, upload_weights

DEV = "cuda"


def announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


def tree_to_device(t: dict, ctx: S.SpecContext) -> S.Tree:
    B, n1 = t["tokens"].shape
    tr = S.Tree(B, n1, DEV)
    for f in ("tokens", "parent", "num_nodes"):
        getattr(tr, f).copy_(torch.from_numpy(np.ascontiguousarray(t[f], dtype=np.int32)))
    for f in ("depth", "position", "draft_slot"):
        if f in t:
            getattr(tr, f).copy_(torch.from_numpy(np.ascontiguousarray(t[f], dtype=np.int32)))
    return tr


def compare_tree(got: dict, want: dict, fields=("tokens", "parent", "depth", "position", "draft_slot",
                                                 "num_nodes", "score", "anc_mask")):
    for f in fields:
        g, w = np.asarray(got[f]), np.asarray(want[f])
        if f == "score":
            g, w = g.astype(np.float32), w.astype(np.float32)
        if not np.array_equal(g, w):
            idx = np.argwhere(g != w)[:5]
            raise AssertionError(f"tree field {f} differs at {idx.tolist()}: got {g[tuple(idx[0])]}, "
                                 f"want {w[tuple(idx[0])]}")


def ids_match_where_gap_allows(gpu_ids, ora_logits, k, tol, d2t=None):
    """Top-k ids must equal the oracle's wherever the oracle's logits leave a
    gap larger than tol around each rank; elsewhere the GPU choice must be
    within tol of optimal under the oracle's logits."""
    M = gpu_ids.shape[0]
    for r in range(M):
        z = ora_logits[r].astype(np.float64)
        order = np.argsort(-z, kind="stable")
        top = order[: k + 1]
        want = top[:k] if d2t is None else d2t[top[:k]]
        zs = z[top]
        gaps = np.abs(np.diff(zs))
        for j in range(k):
            safe = gaps[j] > tol and (j == 0 or gaps[j - 1] > tol)
            if safe:
                assert gpu_ids[r, j] == want[j], (r, j, gpu_ids[r], want)
        # every GPU id is near-optimal under the oracle's logits
        inv = {int(t): i for i, t in enumerate(d2t)} if d2t is not None else None
        for j in range(k):
            pos = int(gpu_ids[r, j]) if inv is None else inv[int(gpu_ids[r, j])]
            assert z[pos] >= zs[j] - 2 * tol, (r, j)
