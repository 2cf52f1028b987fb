"""GPU parity of one draft pass (S1-S9, S8') and of the whole draft side
(spec_build_tree) against the oracle on the same seeded inputs.

Tolerances: float32 workloads 1e-4 on logits; bf16 workloads 2e-2 absolute on
logits (bf16 operands, float32 accumulation), and relative 1e-2 on bf16
activations and cache rows (a one-ulp rounding flip).  Token ids must match
the oracle wherever the oracle's logits leave a gap wider than the tolerance;
end-to-end trees are compared bit-exactly on seeds whose every decision has
such a gap (checked from the oracle's own values)."""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, announce, compare_tree, ids_match_where_gap_allows
from oracle import draft as od
from oracle import tree as ot
from speculative_decoding_aux_amd import spec as S
from speculative_decoding_aux_amd.tensors import from_device, to_device, upload_kv, upload_weights
from synth import configs, gen

pytestmark = pytest.mark.gpu

SMALL = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512, vocab=2048,
             draft_vocab=2048, top_k=3, depth=3, total_tokens=8, dtype="bf16", batch=2, ctx=40)

CASES = {
    "tiny_chain_f32": (configs.get("tiny_chain"), 1e-4),
    "small_bf16": (configs.get("tiny_chain", **SMALL), 2e-2),
    "small_bf16_window": (configs.get("tiny_chain", **dict(SMALL, sliding_window=8)), 2e-2),
    "small_bf16_trimmed": (configs.get("tiny_chain", **dict(SMALL, vocab=4096, draft_vocab=1024)), 2e-2),
    "small_f32_hd128": (configs.get("tiny_chain", **dict(SMALL, head_dim=128, dtype="f32", n_q_heads=8,
                                                         n_kv_heads=2)), 1e-4),
    "small_eagle4": (configs.get("tiny_chain", **dict(SMALL, cand_rank=32, num_candidates=64)), 2e-2),
    # 4 q-heads per kv-head x 8 beam rows = 32 query vectors per kv-head (two MFMA query tiles)
    "small_bf16_gqa4_k8": (configs.get("tiny_chain", **dict(SMALL, n_q_heads=8, n_kv_heads=2, top_k=8,
                                                            total_tokens=20)), 2e-2),
    # several context chunks and key blocks per wave, window start inside the context
    "small_bf16_longctx_window": (configs.get("tiny_chain", **dict(SMALL, ctx=700, sliding_window=300)), 2e-2),
    "small_f32_longctx": (configs.get("tiny_chain", **dict(SMALL, ctx=530, dtype="f32")), 1e-4),
    # 64 beam rows in float32: split-K sum, residual and RMSNorm in one launch per row
    "small_f32_rows64": (configs.get("tiny_chain", **dict(SMALL, dtype="f32", batch=8, top_k=8,
                                                          total_tokens=20)), 1e-4),
    # large draft vocabularies run the LM head unsplit with the top-k fused in its epilogue
    "bigvocab_k1": (configs.get("tiny_chain", **dict(SMALL, vocab=70000, draft_vocab=70000, top_k=1,
                                                     total_tokens=3)), 2e-2),
    "bigvocab_trimmed_k8": (configs.get("tiny_chain", **dict(SMALL, vocab=90000, draft_vocab=70000,
                                                             top_k=8, total_tokens=20)), 2e-2),
    # mid-size draft vocabularies at <= 16 rows: the split-K head, its
    # reduction and the two-stage top-k (a ragged last chunk at 32040)
    "midvocab_trimmed_k8": (configs.get("tiny_chain", **dict(SMALL, vocab=40000, draft_vocab=32000,
                                                             top_k=8, total_tokens=20)), 2e-2),
    "midvocab_k1_ragged": (configs.get("tiny_chain", **dict(SMALL, vocab=32040, draft_vocab=32040, top_k=1,
                                                            total_tokens=3)), 2e-2),
    # 72 beam rows: the LDS-tiled GEMM with ragged row and column tiles; K = 480 of the
    # down projection is not a multiple of 64 and takes the streaming kernel
    "tile_rows72_ragged": (configs.get("tiny_chain", **dict(SMALL, batch=9, top_k=8, total_tokens=20,
                                                            intermediate=480)), 2e-2),
    # 72 beam rows with 128-wide heads (the many-row QKV epilogue, 4 heads in flight)
    "tile_rows72_hd128": (configs.get("tiny_chain", **dict(SMALL, batch=9, top_k=8, total_tokens=20,
                                                           head_dim=128)), 2e-2),
    # EAGLE-4 head at width 2048 and a 70000 vocab: 128 candidates retrieved by
    # the group-maximum select and rescored with 16-byte weight loads
    "eagle4_h2048_v70000": (configs.get("tiny_chain", **dict(SMALL, hidden=2048, n_q_heads=16, n_kv_heads=4,
                                                             head_dim=128, vocab=70000, draft_vocab=70000,
                                                             cand_rank=128, num_candidates=128)), 2e-2),
    "bigvocab_k8_rows512": (configs.get("tiny_chain", **dict(SMALL, vocab=70000, draft_vocab=70000,
                                                             top_k=8, total_tokens=20, batch=64, ctx=24)), 2e-2),
    # hidden 512 (K % 512 == 0): LM heads over 17..64 rows share their
    # activations through LDS (32 beam rows here; a 64-row root pass below)
    "bigvocab_h512_rows32": (configs.get("tiny_chain", **dict(SMALL, hidden=512, vocab=70000,
                                                              draft_vocab=70000, top_k=8,
                                                              total_tokens=20, batch=4)), 2e-2),
    "bigvocab_h512_root64": (configs.get("tiny_chain", **dict(SMALL, hidden=512, vocab=70000,
                                                              draft_vocab=70000, top_k=2, depth=2,
                                                              total_tokens=4, batch=64, ctx=24)), 2e-2),
    # 96 beam rows of an EAGLE-4 head: the low-rank score GEMM has more column
    # tiles than the chip has CUs and runs with persistent workgroups
    "eagle4_rows96_v70000": (configs.get("tiny_chain", **dict(SMALL, vocab=70000, draft_vocab=70000,
                                                              cand_rank=64, num_candidates=64, top_k=8,
                                                              total_tokens=20, batch=12, ctx=24)), 2e-2),
    # EAGLE-3.1 flags: normalised FC output, normed recurrent output
    "small_bf16_eagle31": (configs.get("tiny_chain", **dict(SMALL, fc_norm=1, norm_output=1)), 2e-2),
    "small_f32_eagle31_rows64": (configs.get("tiny_chain", **dict(SMALL, dtype="f32", batch=8, top_k=8,
                                                                  total_tokens=20, fc_norm=1,
                                                                  norm_output=1)), 1e-4),
}


def _act_tol(cfg):
    return dict(rtol=1e-2, atol=1e-2) if cfg["dtype"] == "bf16" else dict(rtol=1e-5, atol=1e-5)


def _rows_root(cfg, inp):
    B, ctx = cfg["batch"], inp["ctx_len"]
    seq = np.arange(B)
    pos = ctx.astype(np.int32)
    anc = pos[:, None].astype(np.int32)
    return seq, pos, pos.copy(), anc


def _run_both(name):
    cfg, tol = CASES[name]
    B, k, H = cfg["batch"], cfg["top_k"], cfg["hidden"]
    seed = 500 + len(name)
    W = gen.make_weights(cfg, seed)
    inp = gen.make_step_inputs(cfg, seed, ctx_len=[cfg["ctx"] - i * 3 for i in range(B)])
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    ctx = S.SpecContext(cfg, max_batch=B, max_new=1)
    w = upload_weights(cfg, W)
    cache = upload_kv(cfg, inp["k_cache"], inp["v_cache"])
    ctx_len = inp["ctx_len"]
    # pass 1: root rows, initial mode
    seq, pos, slot, anc = _rows_root(cfg, inp)
    toks = inp["in_tokens"][:, 0]
    o1 = od.draft_pass(cfg, W, kc, vc, 0, inp["aux"][:, 0], toks, seq, pos, slot, ctx_len, anc)
    aux = to_device(np.ascontiguousarray(inp["aux"][:, 0]), cfg["dtype"])
    g1 = S.spec_draft_step(ctx, w, cache, B, 1, 0, aux, toks, pos, slot, ctx_len, anc, k,
                           want_logits=True, want_candidates=bool(cfg["cand_rank"]))
    # pass 2: k recurrent rows per sequence on the root state, slots after the root
    rng = np.random.default_rng(seed)
    seq2 = np.repeat(np.arange(B), k)
    pos2 = np.repeat(pos + 1, k).astype(np.int32)
    slot2 = (np.repeat(pos + 1, k) + np.tile(np.arange(k), B)).astype(np.int32)
    anc2 = np.stack([np.repeat(pos, k), slot2], axis=1).astype(np.int32)
    toks2 = rng.integers(0, cfg["vocab"], size=B * k).astype(np.int32)
    hid2 = o1["h_out"][seq2]
    o2 = od.draft_pass(cfg, W, kc, vc, 1, hid2, toks2, seq2, pos2, slot2, ctx_len, anc2)
    # both sides take the same pass-2 input: the oracle's pass-1 state
    hid2_dev = to_device(np.ascontiguousarray(hid2), cfg["dtype"])
    g2 = S.spec_draft_step(ctx, w, cache, B, k, 1, hid2_dev, toks2, pos2, slot2, ctx_len, anc2, k,
                           want_logits=True, want_candidates=bool(cfg["cand_rank"]))
    torch.cuda.synchronize()
    return cfg, tol, W, (o1, g1), (o2, g2), (kc, vc), cache


@pytest.mark.parametrize("name", list(CASES))
def test_draft_step_matches_oracle(name):
    announce(f"draft step {name}")
    cfg, tol, W, p1, p2, (kc, vc), cache = _run_both(name)
    at = _act_tol(cfg)
    k = cfg["top_k"]
    d2t = W.get("d2t")
    for o, g in (p1, p2):
        np.testing.assert_allclose(from_device(g["h_out"]), o["h_out"], **at)
        if cfg["cand_rank"]:
            np.testing.assert_allclose(g["logits"].cpu().numpy(), o["scores"], atol=tol, rtol=0)
            ids_match_where_gap_allows(g["cand_ids"].cpu().numpy(), o["scores"], cfg["num_candidates"], tol)
            gi, gz = g["cand_ids"].cpu().numpy(), g["cand_logits"].cpu().numpy()
            for r in range(gi.shape[0]):
                common = {int(c): j for j, c in enumerate(o["cand_ids"][r])}
                for j, c in enumerate(gi[r]):
                    if int(c) in common:
                        assert abs(gz[r, j] - o["cand_logits"][r, common[int(c)]]) <= tol
        else:
            np.testing.assert_allclose(g["logits"].cpu().numpy(), o["logits"], atol=tol, rtol=0)
            ids_match_where_gap_allows(g["ids"].cpu().numpy(), o["logits"], k, tol, d2t)
        assert np.all(g["logp"].cpu().numpy() <= 0)
    np.testing.assert_allclose(from_device(cache.k)[0], kc, **at)
    np.testing.assert_allclose(from_device(cache.v)[0], vc, **at)


# ------------------------------------------------------------ whole draft side
def _decision_gaps(cfg, record, tree):
    """Smallest margin of every discrete choice the oracle made: the order of
    each row's top-k (and its boundary), each beam's order and boundary, the
    boundary of the final selection, and - with a candidate head - the
    retrieval boundary of the low-rank scores, relative to their spread
    (returned separately)."""
    k, N = cfg["top_k"], cfg["total_tokens"]
    gaps, rel = [], [np.inf]
    for rows, out in record:
        z = out["cand_logits"] if cfg["cand_rank"] else out["logits"]
        for r in range(z.shape[0]):
            s = np.sort(z[r].astype(np.float64))[::-1][: k + 1]
            gaps.extend(np.abs(np.diff(s)).tolist())
        if cfg["cand_rank"]:
            K = cfg["num_candidates"]
            for r in range(out["scores"].shape[0]):
                sr = out["scores"][r].astype(np.float64)
                s = np.sort(sr)[::-1]
                rel.append((s[K - 1] - s[K]) / sr.std())
    for b, C in tree["cands"].items():
        sc = np.array([c["score"] for c in C], np.float64)
        depth = np.array([c["depth"] for c in C])
        for d in np.unique(depth):
            s = np.sort(sc[depth == d])[::-1][: k + 1]
            gaps.extend(np.abs(np.diff(s)).tolist())
        s = np.sort(sc)[::-1]
        if len(s) > N:
            gaps.append(s[N - 1] - s[N])
    return (min(gaps) if gaps else np.inf), min(rel)


# End-to-end trees: a small vocabulary and tree keep the number of discrete
# decisions low enough that seeds with no near-tie exist.
SMALLB = dict(SMALL, vocab=512, draft_vocab=512, top_k=2, depth=3, total_tokens=5)
BUILD = {
    "tiny_chain_f32": (configs.get("tiny_chain"), 1e-4),
    "small_bf16_tree": (configs.get("tiny_chain", **SMALLB), 2e-2),
    "small_bf16_window_tree": (configs.get("tiny_chain", **dict(SMALLB, sliding_window=16, depth=4,
                                                               total_tokens=6)), 2e-2),
    "small_trimmed_tree": (configs.get("tiny_chain", **dict(SMALLB, vocab=4096, draft_vocab=512)), 2e-2),
    "small_eagle4_tree": (configs.get("tiny_chain", **dict(SMALLB, cand_rank=32, num_candidates=64)), 2e-2),
    "small_two_new_rows": (configs.get("tiny_chain", **dict(SMALLB, n_new=2)), 2e-2),
    # deep trees: up to 10 extra keys per row (root rows, ancestors, itself),
    # more than one batch of the attention combine
    "deep_tree_two_new": (configs.get("tiny_chain", **dict(SMALLB, depth=8, total_tokens=10, n_new=2)), 2e-2),
    "deep_chain": (configs.get("tiny_chain", **dict(SMALLB, top_k=1, depth=9, total_tokens=9)), 2e-2),
    "eagle31_tree": (configs.get("tiny_chain", **dict(SMALLB, fc_norm=1, norm_output=1)), 2e-2),
    # chains over a vocab-wide LM head: its records are merged, the tree step
    # taken and the next pass's inputs built in one launch per pass
    "bigvocab_chain": (configs.get("tiny_chain", **dict(SMALL, vocab=70000, draft_vocab=70000, top_k=1,
                                                        depth=3, total_tokens=3)), 2e-2),
    "bigvocab_chain_two_new": (configs.get("tiny_chain", **dict(SMALL, vocab=70000, draft_vocab=70000,
                                                                top_k=1, depth=3, total_tokens=3,
                                                                n_new=2)), 2e-2),
    # the first sequence has an empty context (its rows see only the root
    # rows and their ancestors)
    "small_tree_empty_ctx": (configs.get("tiny_chain", **SMALLB), 2e-2),
    "bigvocab_chain_empty_ctx": (configs.get("tiny_chain", **dict(SMALL, vocab=70000, draft_vocab=70000,
                                                                  top_k=1, depth=3, total_tokens=3)), 2e-2),
    # a chain over a mid-size vocabulary (split head, separate top-k and tree step)
    "midvocab_chain": (configs.get("tiny_chain", **dict(SMALL, vocab=32000, draft_vocab=32000, top_k=1,
                                                        depth=3, total_tokens=3)), 2e-2),
    # a chain whose second sequence is past the capacity cutoff (root only, no
    # KV writes) while the others draft
    "bigvocab_chain_cutoff": (configs.get("tiny_chain", **dict(SMALL, vocab=70000, draft_vocab=70000,
                                                               top_k=1, depth=3, total_tokens=3,
                                                               n_new=2)), 2e-2),
    # the chain's one-launch tail builds the next pass from the normed output
    "bigvocab_chain_eagle31": (configs.get("tiny_chain", **dict(SMALL, vocab=70000, draft_vocab=70000,
                                                                top_k=1, depth=3, total_tokens=3,
                                                                fc_norm=1, norm_output=1)), 2e-2),
}


@pytest.mark.parametrize("name", list(BUILD))
def test_build_tree_matches_oracle(name):
    announce(f"build tree {name}")
    cfg, tol = BUILD[name]
    B, n_new = cfg["batch"], cfg["n_new"]
    margin = 2e-3 if cfg["dtype"] == "bf16" else 1e-5
    # first seed (of a fixed list) on which every oracle decision has a safe margin
    for seed in range(700, 800):
        W = gen.make_weights(cfg, seed)
        ctx_len = [cfg["ctx"] - 3 * i for i in range(B)]
        if name.endswith("_cutoff"):
            ctx_len[1] = cfg["kv_capacity"] - 2
        if name.endswith("_empty_ctx"):
            ctx_len[0] = 0
        inp = gen.make_step_inputs(cfg, seed, ctx_len=ctx_len)
        kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
        rec = []
        want = ot.build_tree(cfg, W, kc, vc, inp["aux"], inp["in_tokens"], inp["ctx_len"], record=rec)
        gap, rel = _decision_gaps(cfg, rec, want)
        if gap > margin and rel > 2e-3:
            break
    else:
        pytest.fail("no seed with safe decision margins")
    ctx = S.SpecContext(cfg, max_batch=B, max_new=n_new)
    w = upload_weights(cfg, W)
    cache = upload_kv(cfg, inp["k_cache"], inp["v_cache"])
    aux = to_device(inp["aux"], cfg["dtype"])
    tr = S.spec_build_tree(ctx, w, cache, aux, torch.from_numpy(inp["in_tokens"]).to(DEV),
                           torch.from_numpy(inp["ctx_len"]).to(DEV))
    torch.cuda.synchronize()
    got = tr.numpy()
    compare_tree(got, want, fields=("tokens", "parent", "depth", "position", "draft_slot", "num_nodes",
                                    "anc_mask"))
    np.testing.assert_allclose(got["score"], want["score"], atol=5e-3 if cfg["dtype"] == "bf16" else 1e-5)
    at = _act_tol(cfg)
    np.testing.assert_allclose(from_device(cache.k)[0], kc, **at)
    np.testing.assert_allclose(from_device(cache.v)[0], vc, **at)
