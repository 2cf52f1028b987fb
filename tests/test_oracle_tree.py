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


# ------------------------------------------------ trimmed draft vocabulary
def _masked_full_head_pass(cfg_full, W_full, kc, vc, aux, ctx_len, d2t, k, seen):
    """Reference draft for the trimmed-vocabulary pin: the full head's logits
    restricted to the subset (the normed row against the full head's rows at
    the subset's target ids, gathered so that the float32 product has the
    trimmed head's shape and rounds alike); ranking by a stable sort of
    the subset's logits in draft-id order (so equal logits keep the smaller
    draft id first), log-probs against scipy's logsumexp over the subset, then
    the draft ids mapped to target ids.  ``seen`` receives the subset logits
    of every row."""
    state = {}

    def fn(d, rows):
        hidden = (np.stack([aux[r["b"], r["i"]] for r in rows]) if d == 1
                  else state["h"][[r["src"] for r in rows]])
        A = max(len(r["anc"]) for r in rows)
        anc = np.full((len(rows), A), -1, np.int64)
        for i, r in enumerate(rows):
            anc[i, :len(r["anc"])] = r["anc"]
        out = od.draft_pass(cfg_full, W_full, kc, vc, 0 if d == 1 else 1, hidden,
                            [r["token"] for r in rows], [r["b"] for r in rows],
                            [r["pos"] for r in rows], [r["slot"] for r in rows], ctx_len, anc)
        state["h"] = out["h_out"]
        res = []
        zs = (out["normed"] @ W_full["lm_head"][d2t].T).astype(np.float32)
        for i in range(len(rows)):
            z = zs[i]
            seen.append(z)
            order = np.argsort(-z.astype(np.float64), kind="stable")[:k]
            lp = (z[order] - np.float32(logsumexp(z.astype(np.float64)))).astype(np.float32)
            res.append((d2t[order].astype(np.int64), lp))
        return res

    return fn


@pytest.mark.parametrize("sorted_map", [True, False])
def test_trimmed_vocabulary_equals_the_masked_full_head(sorted_map):
    """A trimmed head whose rows are the full head's rows at the d2t ids must
    give the tree chosen from the full head's logits restricted to that subset
    ("Eaglet", "Approach 1: YAML Recipe": trimmed draft vocabulary with an id
    map).  With an unsorted map the tie-break runs in draft-id order: two
    trimmed rows are made identical so their logits tie exactly."""
    V, Vd = 512, 96
    cfg_t = _tiny_tree_cfg(vocab=V, draft_vocab=Vd, top_k=3, depth=3, total_tokens=9, batch=2)
    cfg_f = _tiny_tree_cfg(vocab=V, draft_vocab=V, top_k=3, depth=3, total_tokens=9, batch=2)
    W = gen.make_weights(cfg_f, 31)
    rng = np.random.default_rng(31)
    d2t = np.sort(rng.choice(V, Vd, replace=False)) if sorted_map else rng.choice(V, Vd, replace=False)
    d2t = d2t.astype(np.int32)
    if not sorted_map:
        # draft ids 5 and 6 tie everywhere (identical rows, scaled up so that
        # both often reach the top 3); their target ids run the other way
        lo, hi = sorted(d2t[5:7])
        d2t[5], d2t[6] = hi, lo
        W["lm_head"][d2t[5]] *= np.float32(32.0)
        W["lm_head"][d2t[6]] = W["lm_head"][d2t[5]]
    Wt = dict(W, lm_head=np.ascontiguousarray(W["lm_head"][d2t]), d2t=d2t)
    inp = gen.make_step_inputs(cfg_f, 31)
    rec = []
    got = ot.build_tree(cfg_t, Wt, inp["k_cache"].copy(), inp["v_cache"].copy(), inp["aux"],
                        inp["in_tokens"], inp["ctx_len"], record=rec)
    seen = []
    fn = _masked_full_head_pass(cfg_f, W, inp["k_cache"].copy(), inp["v_cache"].copy(), inp["aux"],
                                inp["ctx_len"], d2t, cfg_f["top_k"], seen)
    want = ot.build_tree_core(cfg_f, 2, 1, inp["ctx_len"], inp["in_tokens"], fn)
    # precondition: the two heads computed bit-identical logits on the subset
    trimmed = np.concatenate([out["logits"] for _, out in rec])
    np.testing.assert_array_equal(trimmed, np.stack(seen))
    for key in ("tokens", "parent", "depth", "position", "draft_slot", "anc_mask", "num_nodes"):
        np.testing.assert_array_equal(got[key], want[key], err_msg=key)
    np.testing.assert_allclose(got["score"], want["score"], rtol=0, atol=1e-6)
    assert set(got["tokens"][:, 1:].ravel().tolist()) - {-1} <= set(d2t.tolist())
    if not sorted_map:
        # the tie between draft ids 5 and 6: the smaller draft id (the larger
        # target id) is the earlier child wherever both were drafted
        assert all(z[5] == z[6] for z in seen)
        hits = 0
        for b in range(2):
            toks = got["tokens"][b].tolist()
            par = got["parent"][b].tolist()
            nodes = range(1, int(got["num_nodes"][b]) + 1)
            for n in nodes:
                if toks[n] != d2t[6]:
                    continue
                twin = [m for m in nodes if par[m] == par[n] and toks[m] == d2t[5]]
                if twin:
                    assert twin[0] < n
                    hits += 1
        assert hits > 0, "no node drafted both tied ids"


# ------------------------------------------- root pass over several new rows
def test_root_pass_over_new_rows_equals_sequential_single_rows():
    """n_new > 1 ("The propose() Method": the prefill runs the shifted ids of
    the new tokens): the root pass over n rows equals n one-row passes run in
    order, row i at position and slot ctx + i seeing the context and rows
    0..i; the last row seeds depth 1; a beam node of depth 1 at rank j runs at
    position ctx + n - 1 + 1 and slot ctx + n + j and sees every root row.
    Every candidate is selected (N = k + k*k), so the whole tree is checked."""
    n_new, k = 3, 2
    cfg = _tiny_tree_cfg(top_k=k, depth=2, total_tokens=k + k * k, batch=2, n_new=n_new, dtype="bf16")
    W = gen.make_weights(cfg, 33)
    inp = gen.make_step_inputs(cfg, 33, ctx_len=[20, 11])
    tree = ot.build_tree(cfg, W, inp["k_cache"].copy(), inp["v_cache"].copy(), inp["aux"],
                         inp["in_tokens"], inp["ctx_len"])
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    for b in range(2):
        c = int(inp["ctx_len"][b])
        for i in range(n_new):  # one row at a time, in order
            out = od.draft_pass(cfg, W, kc, vc, 0, inp["aux"][b, i:i + 1], [int(inp["in_tokens"][b, i])],
                                [b], [c + i], [c + i], inp["ctx_len"], [list(range(c, c + i + 1))])
        z = out["logits"][0].astype(np.float64)
        top = np.argsort(-z, kind="stable")[:k]
        assert z[top[-1]] - np.sort(z)[::-1][k] > 1e-3  # no near-tie at the cut
        lse = logsumexp(z)
        assert tree["tokens"][b, 0] == inp["in_tokens"][b, n_new - 1]
        assert tree["position"][b, 0] == c + n_new - 1 and tree["draft_slot"][b, 0] == c + n_new - 1
        d1 = [n for n in range(1, k + k * k + 1) if tree["depth"][b, n] == 1]
        assert [int(tree["tokens"][b, n]) for n in d1] == top.tolist()
        np.testing.assert_allclose([tree["score"][b, n] for n in d1], z[top] - lse, atol=2e-5)
        # depth 1 is the beam (k nodes); rank j by score runs at slot c + n + j
        ranked = sorted(d1, key=lambda n: (-float(tree["score"][b, n]), n))
        h_root = out["h_out"]
        for j, n in enumerate(ranked):
            slot = c + n_new + j
            assert tree["draft_slot"][b, n] == slot and tree["position"][b, n] == c + n_new
            o2 = od.draft_pass(cfg, W, kc, vc, 1, h_root, [int(tree["tokens"][b, n])], [b], [c + n_new],
                               [slot], inp["ctx_len"], [list(range(c, c + n_new)) + [slot]])
            z2 = o2["logits"][0].astype(np.float64)
            top2 = np.argsort(-z2, kind="stable")[:k]
            kids = [m for m in range(1, k + k * k + 1) if tree["parent"][b, m] == n]
            assert [int(tree["tokens"][b, m]) for m in kids] == top2.tolist()
            np.testing.assert_allclose([tree["score"][b, m] for m in kids],
                                       tree["score"][b, n] + (z2[top2] - logsumexp(z2)), atol=3e-5)
            for m in kids:
                assert tree["position"][b, m] == c + n_new + 1 and tree["draft_slot"][b, m] == -1


# ----------------------------------------- draft logits of every tree node
def test_node_draft_logits_of_a_chain_equal_the_next_pass():
    """The last node of a depth-D chain was never expanded; its logits (one
    extra recurrent pass at its position, on its parent's state) equal the
    logits of pass D + 1 of the depth-(D+1) chain built from the same inputs,
    where the node is run by the tree construction itself.  Expanded nodes
    carry the logits their children were ranked by."""
    D = 3
    cfg = _tiny_tree_cfg(top_k=1, depth=D, total_tokens=D, dtype="f32", batch=2)
    cfg2 = _tiny_tree_cfg(top_k=1, depth=D + 1, total_tokens=D + 1, dtype="f32", batch=2)
    W = gen.make_weights(cfg, 34)
    inp = gen.make_step_inputs(cfg2, 34)
    rec, rec2 = [], []
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    tree = ot.build_tree(cfg, W, kc, vc, inp["aux"], inp["in_tokens"], inp["ctx_len"], record=rec)
    z = ot.node_draft_logits(cfg, W, kc, vc, inp["ctx_len"], tree, rec)
    ot.build_tree(cfg2, W, inp["k_cache"].copy(), inp["v_cache"].copy(), inp["aux"], inp["in_tokens"],
                  inp["ctx_len"], record=rec2)
    for b in range(2):
        for n in range(D):  # expanded nodes: the argmax of row n is node n + 1
            assert int(np.argmax(z[b, n])) == tree["tokens"][b, n + 1]
            np.testing.assert_array_equal(z[b, n], rec[n][1]["logits"][b])
        np.testing.assert_allclose(z[b, D], rec2[D][1]["logits"][b], rtol=0, atol=1e-5)


def test_node_draft_logits_of_a_tree():
    """In a tree, every node with children ranks them as the top-k of its
    row; rows of unused nodes are zero; never-expanded nodes get finite rows
    whose values differ from their parent's."""
    cfg = _tiny_tree_cfg(top_k=3, depth=3, total_tokens=9, batch=2)
    W = gen.make_weights(cfg, 35)
    inp = gen.make_step_inputs(cfg, 35)
    rec = []
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    tree = ot.build_tree(cfg, W, kc, vc, inp["aux"], inp["in_tokens"], inp["ctx_len"], record=rec)
    z = ot.node_draft_logits(cfg, W, kc, vc, inp["ctx_len"], tree, rec)
    for b in range(2):
        nn = int(tree["num_nodes"][b])
        for n in range(nn + 1):
            kids = [m for m in range(1, nn + 1) if tree["parent"][b, m] == n]
            top = np.argsort(-z[b, n].astype(np.float64), kind="stable")[:3].tolist()
            for m in kids:
                assert tree["tokens"][b, m] in top
            assert np.isfinite(z[b, n]).all() and np.abs(z[b, n]).max() > 0
            if n:
                assert not np.array_equal(z[b, n], z[b, tree["parent"][b, n]])
        assert not z[b, nn + 1:].any()
