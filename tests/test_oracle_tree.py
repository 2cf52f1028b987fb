"""Pins of the oracle's top-k and tree construction (CPU only)."""

import itertools
import zlib

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import draft as od
from oracle import tree as ot
from synth import configs, gen


# --------------------------------------------------- top-k and log-probs
def test_topk_logprobs_against_sorting_and_logsumexp():
    rng = np.random.default_rng(0)
    z = rng.normal(0, 2, 5000).astype(np.float32)
    z[[10, 20, 30]] = z.max() + 1  # a three-way tie at the top
    top, lp = ot.topk_logprobs(z, 8)
    assert top[:3].tolist() == [10, 20, 30]  # ties broken by id ascending
    ref = np.argsort(-z.astype(np.float64), kind="stable")[:8]
    assert top.tolist() == ref.tolist()
    np.testing.assert_allclose(lp, z[top] - logsumexp(z.astype(np.float64)), atol=2e-6)
    assert lp.dtype == np.float32 and np.all(lp <= 0)


def test_topk_tie_break_uses_given_ids():
    z = np.array([1.0, 3.0, 3.0, 2.0], np.float32)
    top, _ = ot.topk_logprobs(z, 2, ids=np.array([9, 8, 7, 6]))
    assert top.tolist() == [2, 1]


# ---------------------------------------------- P5: brute-force enumeration
def _toy_children(path, V, k):
    rng = np.random.default_rng(zlib.crc32(np.asarray(path, np.int64).tobytes()) + 99)
    z = rng.normal(0, 1, V)
    if len(path) % 2:  # exact ties in some nodes exercise the tie-breaks
        z[1] = z[0]
    order = np.argsort(-z, kind="stable")[:k]
    lse = np.float32(logsumexp(z))
    return order, (z[order].astype(np.float32) - lse).astype(np.float32)


def _toy_pass(V, k, root):
    def fn(d, rows):
        return [_toy_children((root,) + r["path"], V, k) for r in rows]
    return fn


def _brute_tree(root, V, k, D, N):
    """Every token sequence of length 1..D is enumerated and kept iff its last
    token is a top-k child of its prefix and its prefix was in the beam of the
    previous depth; beams and the final choice rank by (score desc, (depth,
    parent beam rank, child rank) asc)."""
    def kids(prefix):
        ids, lp = _toy_children((root,) + prefix, V, k)
        return {int(t): (r, l) for r, (t, l) in enumerate(zip(ids, lp))}

    score, key = {}, {}
    beam_rank = {(): 0}
    for d in range(1, D + 1):
        level = []
        for seq in itertools.product(range(V), repeat=d):
            pre = seq[:-1]
            if pre not in beam_rank:
                continue
            ch = kids(pre)
            if seq[-1] not in ch:
                continue
            r, l = ch[seq[-1]]
            score[seq] = np.float32(l) if d == 1 else np.float32(score[pre] + l)
            key[seq] = (d, beam_rank[pre], r)
            level.append(seq)
        ranked = sorted(level, key=lambda s: (-float(score[s]), key[s]))
        beam_rank = {s: j for j, s in enumerate(ranked[:k])}
    best = sorted(score, key=lambda s: (-float(score[s]), key[s]))[:N]
    return sorted(best, key=lambda s: key[s]), score


def _paths(tree, b=0):
    out = []
    for n in range(1, tree["num_nodes"][b] + 1):
        p, c = [], n
        while c > 0:
            p.append(int(tree["tokens"][b, c]))
            c = int(tree["parent"][b, c])
        out.append(tuple(p[::-1]))
    return out


@pytest.mark.parametrize("k,D,N", [(2, 3, 5), (3, 3, 7), (3, 2, 12), (1, 3, 3), (3, 1, 2), (2, 2, 6)])
def test_tree_matches_brute_force(k, D, N):
    V = 6
    cfg = dict(top_k=k, depth=D, total_tokens=N, kv_capacity=10**6)
    for root in range(V):
        tree = ot.build_tree_core(cfg, 1, 1, np.array([0]), np.array([[root]]), _toy_pass(V, k, root))
        want, score = _brute_tree(root, V, k, D, N)
        got = _paths(tree)
        assert got == want
        for n, p in enumerate(got, start=1):
            assert tree["score"][0, n] == score[p]


# ------------------------------------- invariants on the real draft model
def _tiny_tree_cfg(**kw):
    base = dict(hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32, intermediate=96, vocab=512,
                draft_vocab=512, top_k=3, depth=3, total_tokens=7, dtype="bf16", batch=3, ctx=20)
    base.update(kw)
    return configs.get("tiny_chain", **base)


def _check_invariants(cfg, tree, ctx_len, n_new=1):
    B = tree["tokens"].shape[0]
    k, D, N = cfg["top_k"], cfg["depth"], cfg["total_tokens"]
    for b in range(B):
        nn = int(tree["num_nodes"][b])
        ncand = k + (D - 1) * k * k
        active = ctx_len[b] + n_new + (D - 1) * k <= cfg["kv_capacity"]
        assert nn == (min(N, ncand) if active else 0)
        assert tree["anc_mask"][b, 0] == 1 and tree["parent"][b, 0] == -1
        sib = {}
        for n in range(1, nn + 1):
            p = int(tree["parent"][b, n])
            assert 0 <= p < n  # parents precede children (ancestor-closed)
            assert tree["depth"][b, n] == tree["depth"][b, p] + 1 <= D
            assert tree["position"][b, n] == ctx_len[b] + n_new - 1 + tree["depth"][b, n]
            assert tree["score"][b, n] <= tree["score"][b, p] or p == 0
            assert tree["anc_mask"][b, n] == tree["anc_mask"][b, p] | np.uint64(1 << n)
            sib.setdefault(p, []).append(int(tree["tokens"][b, n]))
        for toks in sib.values():
            assert len(set(toks)) == len(toks)
        for n in range(nn + 1, N + 1):
            assert tree["tokens"][b, n] == -1 and tree["anc_mask"][b, n] == 0


def test_tree_invariants_with_the_draft_model_and_capacity_cutoff():
    cfg = _tiny_tree_cfg()
    W = gen.make_weights(cfg, 7)
    inp = gen.make_step_inputs(cfg, 7, ctx_len=[20, 5, cfg["kv_capacity"] - 3])
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    tree = ot.build_tree(cfg, W, kc, vc, inp["aux"], inp["in_tokens"], inp["ctx_len"])
    _check_invariants(cfg, tree, inp["ctx_len"])
    assert tree["num_nodes"][2] == 0  # near capacity: no drafts, no KV writes
    np.testing.assert_array_equal(kc[2], inp["k_cache"][2])


def test_depth_one_is_plain_top_n():
    cfg = _tiny_tree_cfg(top_k=5, depth=1, total_tokens=3)
    W = gen.make_weights(cfg, 8)
    inp = gen.make_step_inputs(cfg, 8)
    rec = []
    tree = ot.build_tree(cfg, W, inp["k_cache"], inp["v_cache"], inp["aux"], inp["in_tokens"],
                         inp["ctx_len"], record=rec)
    logits = rec[0][1]["logits"]
    for b in range(cfg["batch"]):
        want = np.argsort(-logits[b].astype(np.float64), kind="stable")[:3]
        assert tree["tokens"][b, 1:4].tolist() == want.tolist()


def test_top1_is_the_propose_chain():
    """k = 1: the tree is the page's propose() loop - the initial pass on the
    aux states, then recurrent passes at positions +1 on the pre-norm state,
    each taking the argmax."""
    cfg = _tiny_tree_cfg(top_k=1, depth=4, total_tokens=4, dtype="f32", batch=2)
    W = gen.make_weights(cfg, 9)
    inp = gen.make_step_inputs(cfg, 9)
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    tree = ot.build_tree(cfg, W, kc, vc, inp["aux"], inp["in_tokens"], inp["ctx_len"])
    kc2, vc2 = inp["k_cache"].copy(), inp["v_cache"].copy()
    for b in range(2):
        c0 = int(inp["ctx_len"][b])
        hidden, tok, mode, chain = inp["aux"][b], [int(inp["in_tokens"][b, 0])], 0, []
        for i in range(4):
            pos = c0 + i
            out = od.draft_pass(cfg, W, kc2, vc2, mode, hidden, tok, [b], [pos], [pos],
                                inp["ctx_len"], [list(range(c0, pos + 1))])
            t = int(np.argmax(out["logits"][0]))
            chain.append(t)
            hidden, tok, mode = out["h_out"], [t], 1
        assert tree["tokens"][b, 1:].tolist() == chain
        assert tree["parent"][b].tolist() == [-1, 0, 1, 2, 3]
    # batched (2-row) and single-row float32 BLAS products round differently
    np.testing.assert_allclose(kc, kc2, atol=1e-5, rtol=0)


def test_tree_from_table_equals_model_build():
    """The table-driven draft reproduces the model-driven tree when the
    table holds the model's own per-pass outputs."""
    cfg = _tiny_tree_cfg()
    W = gen.make_weights(cfg, 10)
    inp = gen.make_step_inputs(cfg, 10)
    rec = []
    tree = ot.build_tree(cfg, W, inp["k_cache"].copy(), inp["v_cache"].copy(), inp["aux"],
                         inp["in_tokens"], inp["ctx_len"], record=rec)
    B, k, D = cfg["batch"], cfg["top_k"], cfg["depth"]
    ids = np.zeros((D, B, k, k), np.int64)
    lps = np.zeros((D, B, k, k), np.float32)
    for d, (rows, out) in enumerate(rec, start=1):
        for i, r in enumerate(rows):
            top, lp = ot.topk_logprobs(out["logits"][i], k)
            ids[d - 1, r["b"], r["rank"]] = top
            lps[d - 1, r["b"], r["rank"]] = lp
    t2 = ot.build_tree_from_topk(cfg, inp["ctx_len"], inp["in_tokens"], ids, lps)
    for key in ("tokens", "parent", "depth", "position", "draft_slot", "score", "anc_mask", "num_nodes"):
        np.testing.assert_array_equal(t2[key], tree[key])
