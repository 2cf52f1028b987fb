"""Draft-tree construction (TEST INFRASTRUCTURE).

What the pages fix: the draft proposes tokens greedily (vLLM Neuron design
page, "Design Choices": the draft always takes the argmax; "The propose()
Method": a prefill pass on the shifted ids gives the first draft token, then
K-1 recurrent passes at positions +1 each give the rest, returning
[batch, num_speculative_tokens]); a tree is described by draft_top_k,
draft_depth and total_draft_tokens ("Eaglet" page, "Approach 1: YAML Recipe"),
verified by the target as 1 + total_draft_tokens tokens ("Block Efficiency
(BE) Evaluation": eval_tm_arn [128, 32]).

Expansion rule (a reading; the pages give only the three parameters):
  * the root pass runs the n_new new rows of each sequence at positions
    ctx .. ctx+n_new-1 (slots equal to positions); the top-k of its last row
    are the depth-1 candidates, scored by their log-probabilities;
  * for depth d = 2..D the beam is the top-k depth-(d-1) candidates by
    (score desc, candidate index asc); beam node j of depth d-1 sits at
    position ctx+n_new-1+(d-1) and slot ctx+n_new+(d-2)*k+j, runs in recurrent
    mode on its parent's pre-norm state and its own token, sees the context,
    the root rows, its ancestors' slots and its own slot, and appends its top-k
    children with score = parent score + log-prob (float32 add);
  * candidate index is append order (depth-major, beam order, child rank);
  * the tree is the top-N candidates by (score desc, index asc), emitted in
    index order as nodes 1..N; node 0 is the root (the last input token).
    Parents precede children and the set is ancestor-closed because
    log-probabilities are <= 0 and a parent's index is smaller.
  * a sequence with ctx + n_new + (D-1)*k > kv_capacity gets no drafts (the
    position-aware cutoff of the vLLM Neuron design page, "Design Choices").
  * top_k = 1 is the chain of "The propose() Method".

Top-k order is (value desc, id asc) over draft ids; log-probs are
z - logsumexp(z), with logsumexp accumulated in float64 and rounded to
float32 once, then the subtraction in float32.

Pinned by tests/test_oracle_tree.py: brute-force enumeration of every token
sequence on tiny vocabularies, the structural invariants (ancestor closure,
scores non-increasing along paths, depth and position of every node), the
D = 1 and k = 1 reductions, numpy sorting of the log-probs; the trimmed
vocabulary (d2t) against the full head's logits restricted to the subset,
ranked by a stable sort in draft-id order (sorted and unsorted maps, exact
ties); a root pass over several new rows against one-row passes run in order,
with the beam's positions and slots.
"""

from __future__ import annotations

import numpy as np

from .draft import draft_pass, topk_desc


def topk_logprobs(z, k: int, ids=None):
    """Top-k of one row of logits and their log-probabilities.

    Returns (positions in z of the k best by (z desc, tie id asc), their
    float32 log-probs).  ``ids`` are the tie-break ids (default: positions)."""
    z = np.asarray(z, dtype=np.float32)
    top = topk_desc(z, k, ids)
    z64 = z.astype(np.float64)
    m = float(np.max(z64))
    lse = np.float32(m + np.log(np.sum(np.exp(z64 - m))))
    return top, (z[top] - lse).astype(np.float32)


def _ancestor_slots(cands, ci):
    out = []
    p = cands[ci]["parent"]
    while p >= 0:
        out.append(cands[p]["slot"])
        p = cands[p]["parent"]
    return out[::-1]


def build_tree_core(cfg, B, n_new, ctx_len, in_tokens, pass_fn, choose=None):
    """Tree construction with a pluggable draft.

    ``pass_fn(d, rows)`` runs draft pass d (1 = root) over ``rows`` (dicts with
    b, token, pos, slot, anc, src, cand, rank, i, path) and returns one
    (ids[k], logp[k]) pair per row, ids in the target vocabulary.

    ``choose(kind, b, depth, ranked, C)``, if given, may replace a ranking
    decision: kind "beam" (the beam of depth ``depth``, the first k of
    ``ranked``) or "select" (the tree, the first N of ``ranked``); ``ranked``
    lists candidate indices by (score desc, index asc) and ``C`` is the
    sequence's candidate list.  It returns the chosen indices (a test that
    replays another implementation's choices at near-ties uses it); without
    it the rule above applies."""
    k, D, N = cfg["top_k"], cfg["depth"], cfg["total_tokens"]
    cap = cfg["kv_capacity"]
    ctx_len = np.asarray(ctx_len)
    active = [b for b in range(B) if ctx_len[b] + n_new + (D - 1) * k <= cap]
    cands = {b: [] for b in active}

    rows = []
    for b in active:
        c0 = int(ctx_len[b])
        for i in range(n_new):
            rows.append(dict(b=b, i=i, token=int(in_tokens[b, i]), pos=c0 + i, slot=c0 + i,
                             anc=[c0 + j for j in range(i + 1)], src=None, cand=-1, rank=0,
                             path=()))
    res = pass_fn(1, rows) if rows else []
    for idx, r in enumerate(rows):
        if r["i"] != n_new - 1:
            continue
        ids, lp = res[idx]
        for t, l in zip(ids, lp):
            cands[r["b"]].append(dict(token=int(t), parent=-1, depth=1, score=np.float32(l),
                                      slot=-1, src=idx, path=(int(t),)))

    for d in range(2, D + 1):
        rows = []
        for b in active:
            c0 = int(ctx_len[b])
            C = cands[b]
            pool = [ci for ci, c in enumerate(C) if c["depth"] == d - 1]
            ranked = sorted(pool, key=lambda ci: (-float(C[ci]["score"]), ci))
            beam = ranked[:k] if choose is None else choose("beam", b, d - 1, ranked, C)
            for j, ci in enumerate(beam):
                C[ci]["slot"] = c0 + n_new + (d - 2) * k + j
                anc = [c0 + i for i in range(n_new)] + _ancestor_slots(C, ci) + [C[ci]["slot"]]
                rows.append(dict(b=b, i=0, token=C[ci]["token"], pos=c0 + n_new - 1 + (d - 1),
                                 slot=C[ci]["slot"], anc=anc, src=C[ci]["src"], cand=ci, rank=j,
                                 path=C[ci]["path"]))
        res = pass_fn(d, rows) if rows else []
        for idx, r in enumerate(rows):
            ids, lp = res[idx]
            C = cands[r["b"]]
            ps = C[r["cand"]]["score"]
            for t, l in zip(ids, lp):
                C.append(dict(token=int(t), parent=r["cand"], depth=d,
                              score=np.float32(np.float32(ps) + np.float32(l)), slot=-1, src=idx,
                              path=r["path"] + (int(t),)))

    n1 = N + 1
    tree = {
        "tokens": np.full((B, n1), -1, np.int32),
        "parent": np.full((B, n1), -1, np.int32),
        "depth": np.full((B, n1), -1, np.int32),
        "position": np.full((B, n1), -1, np.int32),
        "draft_slot": np.full((B, n1), -1, np.int32),
        "score": np.zeros((B, n1), np.float32),
        "anc_mask": np.zeros((B, n1), np.uint64),
        "num_nodes": np.zeros(B, np.int32),
        "node_cand": np.full((B, n1), -1, np.int64),  # candidate index of each draft node
        "cands": cands,
    }
    for b in range(B):
        c0 = int(ctx_len[b])
        tree["tokens"][b, 0] = in_tokens[b, n_new - 1]
        tree["depth"][b, 0] = 0
        tree["position"][b, 0] = c0 + n_new - 1
        tree["anc_mask"][b, 0] = 1
        if b not in cands:
            continue
        tree["draft_slot"][b, 0] = c0 + n_new - 1
        C = cands[b]
        ranked = sorted(range(len(C)), key=lambda ci: (-float(C[ci]["score"]), ci))
        best = ranked[:N] if choose is None else choose("select", b, D, ranked, C)
        sel = sorted(best)
        node_of = {ci: n + 1 for n, ci in enumerate(sel)}
        tree["num_nodes"][b] = len(sel)
        for ci in sel:
            n = node_of[ci]
            c = C[ci]
            par = 0 if c["parent"] < 0 else node_of[c["parent"]]
            tree["tokens"][b, n] = c["token"]
            tree["parent"][b, n] = par
            tree["depth"][b, n] = c["depth"]
            tree["position"][b, n] = c0 + n_new - 1 + c["depth"]
            tree["draft_slot"][b, n] = c["slot"]
            tree["score"][b, n] = c["score"]
            tree["anc_mask"][b, n] = tree["anc_mask"][b, par] | np.uint64(1 << n)
            tree["node_cand"][b, n] = ci
    return tree


def model_pass_fn(cfg, W, kcache, vcache, aux, ctx_len, record=None, topk_fn=None):
    """The draft model as a pass function for build_tree_core.

    ``record``, if given, is a list that receives each pass's rows and output
    dict (for tests that compare stage by stage).  ``topk_fn(d, row, z, ids,
    lp)``, if given, may replace a row's top-k (ids in the target vocabulary,
    log-probs) given its logits z over the head's rows (EAGLE-3 heads)."""
    k = cfg["top_k"]
    d2t = W.get("d2t")
    state = {}

    def fn(d, rows):
        M = len(rows)
        if d == 1:
            hidden = np.stack([aux[r["b"], r["i"]] for r in rows])
        else:
            hidden = state["h"][[r["src"] for r in rows]]
        A = max(len(r["anc"]) for r in rows)
        anc = np.full((M, A), -1, np.int64)
        for i, r in enumerate(rows):
            anc[i, : len(r["anc"])] = r["anc"]
        out = draft_pass(cfg, W, kcache, vcache, 0 if d == 1 else 1, hidden,
                         [r["token"] for r in rows], [r["b"] for r in rows],
                         [r["pos"] for r in rows], [r["slot"] for r in rows], ctx_len, anc)
        state["h"] = out["h_out"]
        if record is not None:
            record.append((rows, out))
        res = []
        for i in range(M):
            if cfg["cand_rank"]:
                pos, lp = topk_logprobs(out["cand_logits"][i], k, ids=out["cand_ids"][i])
                ids = out["cand_ids"][i][pos]
            else:
                pos, lp = topk_logprobs(out["logits"][i], k)
                ids = d2t[pos] if d2t is not None else pos
                if topk_fn is not None:
                    ids, lp = topk_fn(d, rows[i], out["logits"][i], ids, lp)
            res.append((np.asarray(ids, np.int64), lp))
        return res

    return fn


def build_tree(cfg, W, kcache, vcache, aux, in_tokens, ctx_len, record=None, topk_fn=None,
               choose=None):
    """Full draft side of one speculation step: root pass, D-1 expansions and
    the final selection.  kcache/vcache are updated in place.  ``topk_fn``
    and ``choose`` are the decision hooks of model_pass_fn and
    build_tree_core (identity when None)."""
    in_tokens = np.asarray(in_tokens)
    B, n_new = in_tokens.shape
    fn = model_pass_fn(cfg, W, kcache, vcache, aux, ctx_len, record, topk_fn)
    return build_tree_core(cfg, B, n_new, ctx_len, in_tokens, fn, choose)


def table_pass_fn(ids_tab, lp_tab):
    """A draft given as a table: pass d, sequence b and beam rank j produce
    ids_tab[d-1, b, j] and lp_tab[d-1, b, j] (the root pass uses rank 0)."""
    def fn(d, rows):
        return [(np.asarray(ids_tab[d - 1, r["b"], r["rank"]], np.int64),
                 np.asarray(lp_tab[d - 1, r["b"], r["rank"]], np.float32)) for r in rows]
    return fn


def build_tree_from_topk(cfg, ctx_len, in_tokens, ids_tab, lp_tab):
    in_tokens = np.asarray(in_tokens)
    B, n_new = in_tokens.shape
    return build_tree_core(cfg, B, n_new, ctx_len, in_tokens, table_pass_fn(ids_tab, lp_tab))


def node_draft_logits(cfg, W, kcache, vcache, ctx_len, tree, record):
    """The draft's logits at every node of the trees: row n of sequence b is
    the distribution node n's children are ranked by (used to make target
    logits that resemble the draft's).  ``record`` is the pass record of the
    build_tree call that made ``tree``; kcache/vcache are the caches it left.

    The root takes the logits of its sequence's last new row; an expanded
    node those of the pass that expanded it.  Selected nodes that were never
    expanded run one more recurrent pass here, each on its parent's pre-norm
    state and its own token at its tree position, seeing the context, the
    root rows, its ancestors' slots and itself; their own K/V go to scratch
    slots past the cache (the caches are not changed).  EAGLE-3 heads only.
    Unused nodes get zero rows.  Returns [B, N+1, Vd] float32."""
    assert not cfg["cand_rank"]
    B, n1 = tree["tokens"].shape
    Vd = cfg["draft_vocab"]
    S = kcache.shape[2]
    out = np.zeros((B, n1, Vd), np.float32)
    # where each candidate's row sits in the recorded passes
    h_of, z_of = {}, {}
    rows0, out0 = record[0]
    n_new = max(r["i"] for r in rows0) + 1
    for idx, r in enumerate(rows0):
        if r["i"] == n_new - 1:
            h_of[(r["b"], -1)] = out0["h_out"][idx]
            z_of[(r["b"], -1)] = out0["logits"][idx]
    for rows, o in record[1:]:
        for idx, r in enumerate(rows):
            h_of[(r["b"], r["cand"])] = o["h_out"][idx]
            z_of[(r["b"], r["cand"])] = o["logits"][idx]
    extra = []  # (b, n) of selected nodes never expanded
    for b in range(B):
        if (b, -1) not in z_of:
            continue
        out[b, 0] = z_of[(b, -1)]
        for n in range(1, int(tree["num_nodes"][b]) + 1):
            ci = int(tree["node_cand"][b, n])
            if (b, ci) in z_of:
                out[b, n] = z_of[(b, ci)]
            else:
                extra.append((b, n))
    if not extra:
        return out
    pad = ((0, 0), (0, 0), (0, n1), (0, 0))
    kx, vx = np.pad(kcache, pad), np.pad(vcache, pad)
    hidden, toks, seq, pos, slot, anc = [], [], [], [], [], []
    for b, n in extra:
        c = int(ctx_len[b])
        p = int(tree["parent"][b, n])
        hidden.append(h_of[(b, -1 if p == 0 else int(tree["node_cand"][b, p]))])
        toks.append(int(tree["tokens"][b, n]))
        seq.append(b)
        pos.append(int(tree["position"][b, n]))
        slot.append(S + n)
        chain, a = [], p
        while a > 0:
            chain.append(int(tree["draft_slot"][b, a]))
            a = int(tree["parent"][b, a])
        anc.append([c + i for i in range(n_new)] + chain[::-1] + [S + n])
    A = max(len(a) for a in anc)
    anc_arr = np.full((len(extra), A), -1, np.int64)
    for i, a in enumerate(anc):
        anc_arr[i, :len(a)] = a
    res = draft_pass(cfg, W, kx, vx, 1, np.stack(hidden), toks, seq, pos, slot, ctx_len, anc_arr)
    for i, (b, n) in enumerate(extra):
        out[b, n] = res["logits"][i]
    return out
