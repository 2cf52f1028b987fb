"""P7: the EAGLE-4 candidate head (CPU only).

Pins: keeping every vocabulary entry as a candidate reproduces the full-head
EAGLE-3 tree; an lm_head of exact rank r whose factors come from its truncated
SVD gives low-rank scores equal to the full logits, so the full head's top-1
is always among the retrieved candidates (candidate recall 1)."""

import numpy as np

from oracle import draft as od
from oracle import tree as ot
from synth import configs, gen


def _cfg(**kw):
    base = dict(hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32, intermediate=96, vocab=256,
                draft_vocab=256, top_k=3, depth=3, total_tokens=7, dtype="f32", batch=2, ctx=16)
    base.update(kw)
    return configs.get("tiny_chain", **base)


def test_all_candidates_reproduce_full_head_tree():
    c3 = _cfg()
    c4 = _cfg(cand_rank=16, num_candidates=256)
    W = gen.make_weights(c4, 31)
    inp = gen.make_step_inputs(c3, 31)
    t3 = ot.build_tree(c3, W, inp["k_cache"].copy(), inp["v_cache"].copy(), inp["aux"], inp["in_tokens"], inp["ctx_len"])
    t4 = ot.build_tree(c4, W, inp["k_cache"].copy(), inp["v_cache"].copy(), inp["aux"], inp["in_tokens"], inp["ctx_len"])
    for key in ("tokens", "parent", "depth", "num_nodes", "anc_mask"):
        np.testing.assert_array_equal(t3[key], t4[key])
    np.testing.assert_allclose(t3["score"], t4["score"], atol=1e-5)


def test_exact_low_rank_head_has_full_recall():
    r, K = 16, 8
    cfg = _cfg(cand_rank=r, num_candidates=K, batch=2)
    W = gen.make_weights(cfg, 32)
    rng = np.random.default_rng(5)
    G = rng.normal(0, 0.02, size=(cfg["vocab"], r)) @ rng.normal(0, 1, size=(r, cfg["hidden"]))
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    W["cand_down"] = (S[:r, None] * Vt[:r]).astype(np.float32)   # [r, H]
    W["cand_up"] = U[:, :r].astype(np.float32)                  # [V, r]
    W["lm_head"] = (W["cand_up"].astype(np.float64) @ W["cand_down"]).astype(np.float32)
    inp = gen.make_step_inputs(cfg, 32)
    M = 6
    hid = rng.normal(size=(M, cfg["hidden"])).astype(np.float32)
    out = od.draft_pass(cfg, W, inp["k_cache"], inp["v_cache"], 1, hid, np.arange(M), [0] * 3 + [1] * 3,
                        [16] * M, [16, 17, 18, 16, 17, 18], inp["ctx_len"], [[16], [17], [18]] * 2)
    full = out["normed"] @ W["lm_head"].T
    np.testing.assert_allclose(out["scores"], full, atol=1e-4)
    for i in range(M):
        assert int(np.argmax(full[i])) in out["cand_ids"][i].tolist()
        np.testing.assert_allclose(out["cand_logits"][i], full[i, out["cand_ids"][i]], atol=1e-5)
