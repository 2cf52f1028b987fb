"""End-to-end draft trees at full size against the oracle, by the replay
protocol: spec_build_tree runs a whole step of the Llama-3.1-8B chain, the
Qwen3-4B tree (trimmed vocabulary) and the Qwen3-8B tree (32 sequences); the
oracle then builds the same step from the same inputs, and wherever one of
its own decisions is a near-tie - a top-k boundary or rank, a beam boundary,
the final selection boundary, with a gap below 4e-2 in its own values (bf16
logits agree only to 2e-2) - it takes the library's choice, after checking
that the choice is within 4e-2 of optimal under its own values, per pass
(the input state of pass d has gone through d - 1 recurrent passes on each
side, and a cumulative score sums d log-probs).  Everything
else must agree exactly: tokens, parents, depths, positions, draft slots,
ancestor masks and kept-node counts; cumulative scores within 4e-2 per
depth level.  The
library's choices come from its candidate table (spec_tree_candidates).  The
number of replayed decisions is printed."""

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from gpu_helpers import DEV, announce
from oracle import tree as ot
from speculative_decoding_aux_amd import spec as S
from speculative_decoding_aux_amd.tensors import to_device, upload_kv, upload_weights
from synth import configs, gen

pytestmark = pytest.mark.gpu

TOL = 4e-2


class Replay:
    """Decision hooks of the oracle that adopt the library's choice at
    near-ties (checked against the oracle's own values)."""

    def __init__(self, cfg, cands, tree, d2t):
        self.k, self.D, self.N = cfg["top_k"], cfg["depth"], cfg["total_tokens"]
        self.c = cands
        self.tree = tree
        self.inv = None if d2t is None else {int(t): i for i, t in enumerate(d2t)}
        self.count = {"topk": 0, "beam": 0, "select": 0}

    def depth_of(self, ci):
        k = self.k
        if k == 1:
            return ci + 1
        return 1 if ci < k else 2 + (ci - k) // (k * k)

    def topk(self, d, row, z, ids, lp):
        b = row["b"]
        par = self.c["parent"][b]
        kids = [ci for ci in range(len(par)) if self.depth_of(ci) == d and
                (par[ci] == row["cand"] if d > 1 else par[ci] == -1)]
        gids = self.c["tokens"][b][kids]
        if np.array_equal(gids, np.asarray(ids)):
            return ids, lp
        pos = gids if self.inv is None else np.array([self.inv[int(t)] for t in gids])
        z64 = z.astype(np.float64)
        v = np.sort(z64)[::-1]
        # pass d's input state went through d - 1 recurrent passes on each side
        tol = TOL * d
        for j, p in enumerate(pos):
            assert abs(z64[p] - v[j]) <= tol, f"pass {d} seq {b}: library's rank-{j} child is {v[j] - z64[p]} off"
        self.count["topk"] += 1
        lse = np.float32(logsumexp(z64))
        return gids.astype(np.int64), (z[pos] - lse).astype(np.float32)

    def choose(self, kind, b, depth, ranked, C):
        # a cumulative score sums `depth` log-probs, each within TOL
        tol = TOL * depth
        sc = {ci: float(C[ci]["score"]) for ci in ranked}
        if kind == "beam":
            slot = self.c["slot"][b]
            exp = [ci for ci in range(len(slot)) if self.depth_of(ci) == depth and slot[ci] >= 0]
            lib = sorted(exp, key=lambda ci: slot[ci])
            want = ranked[:self.k]
        else:
            lib = self.selected(b)
            want = ranked[:self.N]
            if sorted(lib) == sorted(want):
                return want
        if lib == want:
            return want
        cut = sc[want[-1]]
        for j, ci in enumerate(lib):
            assert sc[ci] >= cut - tol, f"{kind} of seq {b}: candidate {ci} is {cut - sc[ci]} below the cut"
            if kind == "beam":
                assert abs(sc[ci] - sc[want[j]]) <= tol, f"beam of seq {b}: rank {j} differs by more than {tol}"
        self.count[kind] += 1
        return lib

    def selected(self, b):
        """Candidate indices of the library's tree nodes."""
        toks, par = self.tree["tokens"][b], self.tree["parent"][b]
        ct, cp = self.c["tokens"][b], self.c["parent"][b]
        cand_of = {0: -1}
        out = []
        for n in range(1, int(self.tree["num_nodes"][b]) + 1):
            pc = cand_of[int(par[n])]
            hit = [ci for ci in range(len(ct)) if ct[ci] == toks[n] and cp[ci] == pc and
                   (pc >= 0 or self.depth_of(ci) == 1)]
            assert len(hit) == 1, f"seq {b} node {n}: {len(hit)} candidates match"
            cand_of[n] = hit[0]
            out.append(hit[0])
        return out


@pytest.mark.parametrize("name", ["llama8b_chain", "qwen4b_tree", "qwen8b_tree"])
def test_full_size_tree_by_replay(name):
    announce(f"full-size tree {name}: generating inputs")
    cfg = configs.get(name)
    B = cfg["batch"]
    seed = configs.SEEDS[name] + 31
    W = gen.make_weights(cfg, seed)
    inp = gen.make_step_inputs(cfg, seed)
    announce(f"full-size tree {name}: GPU build")
    ctx = S.SpecContext(cfg, max_batch=B)
    w = upload_weights(cfg, W)
    cache = upload_kv(cfg, inp["k_cache"], inp["v_cache"])
    tr = S.spec_build_tree(ctx, w, cache, to_device(inp["aux"], cfg["dtype"]),
                           torch.from_numpy(inp["in_tokens"]).to(DEV), torch.from_numpy(inp["ctx_len"]).to(DEV))
    cands = {f: v.cpu().numpy() for f, v in S.spec_tree_candidates(ctx, B).items()}
    got = tr.numpy()
    del cache, w
    ctx.close()
    torch.cuda.empty_cache()
    announce(f"full-size tree {name}: oracle build with replay")
    rp = Replay(cfg, cands, got, W.get("d2t"))
    want = ot.build_tree(cfg, W, inp["k_cache"].copy(), inp["v_cache"].copy(), inp["aux"], inp["in_tokens"],
                         inp["ctx_len"], topk_fn=rp.topk, choose=rp.choose)
    announce(f"full-size tree {name}: replayed decisions {rp.count}")
    for f in ("tokens", "parent", "depth", "position", "draft_slot", "num_nodes", "anc_mask"):
        np.testing.assert_array_equal(got[f], want[f], err_msg=f)
    np.testing.assert_allclose(got["score"], want["score"], rtol=0, atol=TOL * cfg["depth"])
    assert got["num_nodes"].min() == cfg["total_tokens"]
