"""The whole speculative loop on the GPU against the oracle's loop: the draft
model proposes, the target verifies, and the target's aux states feed the
draft's next step (vLLM Neuron page: "What is Speculative Decoding?", one
target pass over the drafts; "Auxiliary Hidden State Extraction", the aux
states the draft consumes; "KV Cache Sharing").

Pairing of the draft's rows: the row of verified position p carries the
target's aux state at p and the token emitted after p, and sits at draft
position p + 1 (the token's own position).  After the prompt's prefill the
first draft step takes one row per prompt position; after a step that
accepted a drafts it takes the a + 1 rows of the root and the accepted
nodes (n_new = a + 1).  Each step then: spec_build_tree (draft) ->
spec_target_forward over the tree (target KV at ctx + node) -> greedy
spec_verify_tree -> spec_compact_kv of the target cache.  The oracle runs the
same loop on its own outputs (oracle.tree, oracle.target, oracle.verify,
oracle.compact).  Every step's tree, accepted length and emitted tokens must
be identical; logits and aux states close.  Both LM heads have the rows of a
few tokens scaled up, so that each model mostly prefers a few tokens, and the
draft's LM-head rows are permuted so that it tends to propose the target's
token: the accepted lengths of the loop run 3, 2, 2, 2, 1, ..., 0, so the
re-prefill takes 6, 4, 3, 2 and 1 rows.  The seed is one on which every
discrete decision of the oracle's loop has a margin of at least 2e-4 (the
float32 draft and target logits agree with the oracle to about 1e-5),
checked here."""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, announce, compare_tree
from oracle import compact as oc
from oracle import target as otg
from oracle import tree as ot
from oracle import verify as ov
from speculative_decoding_aux_amd import spec as S
from speculative_decoding_aux_amd.tensors import upload_kv, upload_target_weights, upload_weights
from synth import configs, gen

pytestmark = pytest.mark.gpu

L, P, STEPS, SEED = 8, 6, 16, 3
NS, SCALE = 4, 5.0
CFG = configs.get("tiny_chain", hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512,
                  vocab=512, draft_vocab=512, top_k=4, depth=3, total_tokens=16, dtype="f32", batch=1,
                  ctx=64, n_new=P)


def make_models(cfg, seed, prompt, draft_k, draft_v):
    """Draft and target weights with the LM-head rows of tokens 0..NS-1
    scaled by SCALE in both, so that each model mostly prefers a few tokens;
    then the draft's LM-head rows of its first proposal and of the target's
    first token are swapped, so that the draft tends to propose what the
    target emits."""
    W = gen.make_weights(cfg, seed)
    WT = gen.make_target_weights(cfg, seed + 1, L)
    for w in (W, WT):
        w["lm_head"] = w["lm_head"].copy()
        w["lm_head"][:NS] *= SCALE
    n1 = cfg["total_tokens"] + 1
    tk = np.zeros((L, 1, cfg["n_kv_heads"], cfg["kv_capacity"], cfg["head_dim"]), np.float32)
    z, aux = otg.target_forward(cfg, WT, tk, tk.copy(), _chain_tree(prompt, n1), np.array([0]))
    x = int(np.argmax(z[0, P - 1]))
    tree = ot.build_tree(cfg, W, draft_k.copy(), draft_v.copy(), aux[:, :P],
                         np.array([prompt[1:] + [x]], np.int32), np.array([1]))
    y = int(tree["tokens"][0, 1])
    W["lm_head"][[x, y]] = W["lm_head"][[y, x]]
    return W, WT


def _chain_tree(tokens, n1):
    """The prompt as a chain tree at positions 0.. (prefill with ctx 0)."""
    n = len(tokens)
    t = {"tokens": np.full((1, n1), -1, np.int32), "parent": np.full((1, n1), -1, np.int32),
         "depth": np.full((1, n1), -1, np.int32), "position": np.full((1, n1), -1, np.int32),
         "num_nodes": np.array([n - 1], np.int32), "anc_mask": np.zeros((1, n1), np.uint64)}
    for j, tok in enumerate(tokens):
        t["tokens"][0, j] = tok
        t["parent"][0, j] = j - 1
        t["depth"][0, j] = j
        t["position"][0, j] = j
        t["anc_mask"][0, j] = np.uint64((1 << (j + 1)) - 1)
    return t


def _to_tree(t, n1):
    tr = S.Tree(1, n1, DEV)
    for f in ("tokens", "parent", "depth", "position", "num_nodes"):
        getattr(tr, f).copy_(torch.from_numpy(np.ascontiguousarray(t[f])))
    tr.anc_mask.copy_(torch.from_numpy(np.ascontiguousarray(t["anc_mask"]).view(np.int64)))
    return tr


def _margins(record, tree, logits, nodes_path, k, N):
    """Smallest gap of the oracle's discrete choices in one step: each draft
    row's top-k order and boundary, each depth's beam order and boundary, the
    final top-N boundary, and the target's top-2 at every node on the
    verified path."""
    gaps = []
    for _, out in record:
        for r in range(out["logits"].shape[0]):
            s = np.sort(out["logits"][r].astype(np.float64))[::-1][: k + 1]
            gaps.extend(np.abs(np.diff(s)).tolist())
    for _, C in tree["cands"].items():
        sc = np.array([c["score"] for c in C], np.float64)
        depth = np.array([c["depth"] for c in C])
        for d in np.unique(depth):
            s = np.sort(sc[depth == d])[::-1][: k + 1]
            gaps.extend(np.abs(np.diff(s)).tolist())
        s = np.sort(sc)[::-1]
        if len(s) > N:
            gaps.append(s[N - 1] - s[N])
    for n in nodes_path:
        s = np.sort(logits[0, n].astype(np.float64))[::-1]
        gaps.append(s[0] - s[1])
    return min(gaps)


def oracle_loop(cfg, W, WT, draft_k, draft_v, prompt):
    """The loop on the oracle; per step (tree, logits, aux, out tokens,
    accepted length, accepted nodes, margin)."""
    n1, D, k, N = cfg["total_tokens"] + 1, cfg["depth"], cfg["top_k"], cfg["total_tokens"]
    S_t = cfg["kv_capacity"]
    tk = np.zeros((L, 1, cfg["n_kv_heads"], S_t, cfg["head_dim"]), np.float32)
    tv = tk.copy()
    kc, vc = draft_k.copy(), draft_v.copy()
    pre = _chain_tree(prompt, n1)
    z, aux = otg.target_forward(cfg, WT, tk, tv, pre, np.array([0]))
    first = int(np.argmax(z[0, P - 1]))
    top2 = np.sort(z[0, P - 1].astype(np.float64))[::-1][:2]
    margin0 = top2[0] - top2[1]
    rows_aux = aux[:, :P]
    rows_tok = np.array([prompt[1:] + [first]], np.int32)
    ctx_t = P
    steps = []
    for i in range(STEPS):
        n_new = rows_tok.shape[1]
        rec = []
        tree = ot.build_tree(cfg, W, kc, vc, rows_aux, rows_tok, np.array([ctx_t - n_new + 1]), record=rec)
        z, aux = otg.target_forward(cfg, WT, tk, tv, tree, np.array([ctx_t]))
        out, alen, nodes = ov.verify_greedy(tree, z, D)
        oc.compact_kv(tk, tv, np.array([ctx_t]), nodes, alen)
        a = int(alen[0])
        path = [0] + [int(x) for x in nodes[0, :a]]
        steps.append(dict(tree=tree, logits=z, aux=aux, out=out, alen=alen, nodes=nodes,
                          margin=min(_margins(rec, tree, z, path, k, N), margin0 if i == 0 else np.inf)))
        rows_aux = aux[:, path]
        rows_tok = out[:, : a + 1].astype(np.int32)
        ctx_t += a + 1
    return first, steps


def test_closed_loop_matches_oracle():
    announce("closed speculative loop: draft + target forward + verify + compaction")
    cfg = CFG
    inp = gen.make_step_inputs(cfg, SEED, ctx_len=[cfg["ctx"]])
    prompt = np.random.default_rng(SEED).integers(0, cfg["vocab"], size=P).tolist()
    W, WT = make_models(cfg, SEED, prompt, inp["k_cache"], inp["v_cache"])
    first, want = oracle_loop(cfg, W, WT, inp["k_cache"], inp["v_cache"], prompt)
    alens = [int(s["alen"][0]) for s in want]
    assert min(s["margin"] for s in want) > 2e-4, "seed has a near-tie decision"
    assert sum(a >= 1 for a in alens) >= 3, f"accepted lengths {alens}"

    n1 = cfg["total_tokens"] + 1
    ctx_d = S.SpecContext(cfg, max_batch=1, max_new=P)
    ctx_t = S.SpecContext(cfg, max_batch=1, max_new=n1)
    w = upload_weights(cfg, W)
    tw = upload_target_weights(cfg, WT)
    draft = upload_kv(cfg, inp["k_cache"], inp["v_cache"])
    shape = (L, 1, cfg["n_kv_heads"], cfg["kv_capacity"], cfg["head_dim"])
    tkv = S.KVCache(torch.zeros(shape, device=DEV), torch.zeros(shape, device=DEV))
    z, aux = S.spec_target_forward(ctx_t, tw, tkv, _to_tree(_chain_tree(prompt, n1), n1), np.array([0], np.int32))
    got_first = int(torch.argmax(z[0, P - 1]).item())
    assert got_first == first
    rows_aux = aux[:, :P].contiguous()
    rows_tok = torch.tensor([prompt[1:] + [got_first]], dtype=torch.int32, device=DEV)
    pos = P
    for i, st in enumerate(want):
        n_new = rows_tok.shape[1]
        tree = S.spec_build_tree(ctx_d, w, draft, rows_aux, rows_tok,
                                 torch.tensor([pos - n_new + 1], dtype=torch.int32, device=DEV))
        z, aux = S.spec_target_forward(ctx_t, tw, tkv, tree, np.array([pos], np.int32))
        toks, alen, nodes = S.spec_verify_tree(ctx_t, tree, z, 0)
        S.spec_compact_kv(ctx_t, tkv, torch.tensor([pos], dtype=torch.int32, device=DEV), nodes, alen)
        torch.cuda.synchronize()
        compare_tree(tree.numpy(), st["tree"], fields=("tokens", "parent", "depth", "position", "num_nodes",
                                                       "anc_mask"))
        np.testing.assert_allclose(z.cpu().numpy(), st["logits"], atol=1e-3, rtol=0, err_msg=f"step {i} logits")
        np.testing.assert_allclose(aux.cpu().numpy(), st["aux"], atol=1e-3, rtol=1e-3, err_msg=f"step {i} aux")
        np.testing.assert_array_equal(alen.cpu().numpy(), st["alen"], err_msg=f"step {i} accepted length")
        np.testing.assert_array_equal(toks.cpu().numpy(), st["out"], err_msg=f"step {i} tokens")
        np.testing.assert_array_equal(nodes.cpu().numpy(), st["nodes"], err_msg=f"step {i} nodes")
        a = int(alen.cpu()[0])
        path = torch.tensor([0] + nodes.cpu().numpy()[0, :a].tolist(), dtype=torch.long, device=DEV)
        rows_aux = aux[:, path].contiguous()
        rows_tok = toks[:, : a + 1].contiguous()
        pos += a + 1
