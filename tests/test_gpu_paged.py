"""Paged KV caches on the GPU (the vLLM Neuron page, "KV Cache Sharing":
physical slot = block_table[pos // block_size] * block_size + pos %
block_size).

The oracle works on the logical, contiguous cache.  The GPU gets the same
cache scattered into a pool of blocks in a shuffled order (with spare blocks
in between), and must (1) match the oracle on two draft passes, as the
contiguous draft tests do, (2) give bit-identical trees, verification and
written cache rows as the contiguous GPU path on whole steps, and (3) compact
a paged multi-layer target cache exactly as the oracle compacts the
contiguous one.  Block sizes 16, 24 (16-key attention blocks straddle pages)
and 64; windows starting inside the context; float32 (scalar attention) and
bf16 (MFMA attention); 72 beam rows (the many-row QKV epilogue)."""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, announce, compare_tree, ids_match_where_gap_allows
from oracle import compact as oc
from oracle import draft as od
from oracle import verify as ov
from speculative_decoding_aux_amd import spec as S
from speculative_decoding_aux_amd.tensors import from_device, to_device, upload_kv, upload_weights
from synth import configs, gen

pytestmark = pytest.mark.gpu

SMALL = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512, vocab=2048,
             draft_vocab=2048, top_k=3, depth=3, total_tokens=8, dtype="bf16", batch=2, ctx=40)


def _paged(cfg, k, v, bs, seed):
    """[L, B, nkv, S, hd] -> pools [L, NB, nkv, bs, hd] with shuffled blocks
    and a [B, max_blocks] table (S rounded up to whole blocks)."""
    Lr, B, nkv, Sl, hd = k.shape
    mb = -(-Sl // bs)
    nb = B * mb + 5  # spare blocks nothing points to
    rng = np.random.default_rng(seed)
    table = rng.permutation(nb)[: B * mb].reshape(B, mb).astype(np.int32)
    pools = []
    for a in (k, v):
        pad = np.zeros((Lr, B, nkv, mb * bs, hd), np.float32)
        pad[:, :, :, :Sl] = a
        pool = np.full((Lr, nb, nkv, bs, hd), 7.0, np.float32)
        for b in range(B):
            for j in range(mb):
                pool[:, table[b, j]] = pad[:, b, :, j * bs:(j + 1) * bs]
        pools.append(pool)
    kc = S.PagedKVCache(to_device(pools[0], cfg["dtype"]), to_device(pools[1], cfg["dtype"]),
                        torch.from_numpy(table).to(DEV))
    return kc, mb * bs


def _gather(cache: S.PagedKVCache, Sl):
    """Paged pools back to [L, B, nkv, Sl, hd] (logical slots)."""
    table = cache.block_table.cpu().numpy()
    out = []
    for pool in (from_device(cache.k), from_device(cache.v)):
        Lr, nb, nkv, bs, hd = pool.shape
        B, mb = table.shape
        a = np.empty((Lr, B, nkv, mb * bs, hd), np.float32)
        for b in range(B):
            for j in range(mb):
                a[:, b, :, j * bs:(j + 1) * bs] = pool[:, table[b, j]]
        out.append(a[:, :, :, :Sl])
    return out


def _act_tol(cfg):
    return dict(rtol=1e-2, atol=1e-2) if cfg["dtype"] == "bf16" else dict(rtol=1e-5, atol=1e-5)


DRAFT = {
    "bf16_bs16": (dict(SMALL), 16, 2e-2),
    "bf16_window_bs24": (dict(SMALL, ctx=700, sliding_window=300), 24, 2e-2),
    "f32_bs16": (dict(SMALL, dtype="f32", ctx=530), 16, 1e-4),
    "bf16_rows72_bs64": (dict(SMALL, batch=9, top_k=8, total_tokens=20, head_dim=128), 64, 2e-2),
}


@pytest.mark.parametrize("name", list(DRAFT))
def test_paged_draft_passes_match_oracle(name):
    over, bs, tol = DRAFT[name]
    announce(f"paged draft passes {name}")
    cfg = configs.get("tiny_chain", **over)
    B, k = cfg["batch"], cfg["top_k"]
    seed = 700 + len(name)
    W = gen.make_weights(cfg, seed)
    inp = gen.make_step_inputs(cfg, seed, ctx_len=[cfg["ctx"] - 3 * i for i in range(B)])
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    ctx = S.SpecContext(cfg, max_batch=B, max_new=1)
    w = upload_weights(cfg, W)
    Sl = cfg["kv_capacity"]
    cache, _ = _paged(cfg, inp["k_cache"][None], inp["v_cache"][None], bs, seed)
    ctx_len = inp["ctx_len"]
    pos = ctx_len.astype(np.int32)
    anc = pos[:, None].astype(np.int32)
    toks = inp["in_tokens"][:, 0]
    o1 = od.draft_pass(cfg, W, kc, vc, 0, inp["aux"][:, 0], toks, np.arange(B), pos, pos, ctx_len, anc)
    aux = to_device(np.ascontiguousarray(inp["aux"][:, 0]), cfg["dtype"])
    g1 = S.spec_draft_step(ctx, w, cache, B, 1, 0, aux, toks, pos, pos, ctx_len, anc, k, want_logits=True)
    rng = np.random.default_rng(seed)
    seq2 = np.repeat(np.arange(B), k)
    pos2 = np.repeat(pos + 1, k).astype(np.int32)
    slot2 = (np.repeat(pos + 1, k) + np.tile(np.arange(k), B)).astype(np.int32)
    anc2 = np.stack([np.repeat(pos, k), slot2], axis=1).astype(np.int32)
    toks2 = rng.integers(0, cfg["vocab"], size=B * k).astype(np.int32)
    hid2 = o1["h_out"][seq2]
    o2 = od.draft_pass(cfg, W, kc, vc, 1, hid2, toks2, seq2, pos2, slot2, ctx_len, anc2)
    g2 = S.spec_draft_step(ctx, w, cache, B, k, 1, to_device(np.ascontiguousarray(hid2), cfg["dtype"]),
                           toks2, pos2, slot2, ctx_len, anc2, k, want_logits=True)
    torch.cuda.synchronize()
    at = _act_tol(cfg)
    for o, g in ((o1, g1), (o2, g2)):
        np.testing.assert_allclose(from_device(g["h_out"]), o["h_out"], **at)
        np.testing.assert_allclose(g["logits"].cpu().numpy(), o["logits"], atol=tol, rtol=0)
        ids_match_where_gap_allows(g["ids"].cpu().numpy(), o["logits"], k, tol)
    gk, gv = _gather(cache, Sl)
    np.testing.assert_allclose(gk[0], kc, **at)
    np.testing.assert_allclose(gv[0], vc, **at)


STEP = {
    "bf16_tree_bs16": (dict(SMALL, vocab=512, draft_vocab=512, top_k=2, depth=3, total_tokens=5), 16),
    "bf16_window_tree_bs24": (dict(SMALL, vocab=512, draft_vocab=512, top_k=2, depth=4, total_tokens=6,
                                   ctx=300, sliding_window=100), 24),
    "f32_chain_bs32": (dict(SMALL, dtype="f32", vocab=512, draft_vocab=512, top_k=1, depth=4,
                            total_tokens=4), 32),
}


@pytest.mark.parametrize("name", list(STEP))
def test_paged_step_equals_contiguous_step(name):
    over, bs = STEP[name]
    announce(f"paged whole step {name}")
    cfg = configs.get("tiny_chain", **over)
    B = cfg["batch"]
    seed = 800 + len(name)
    W = gen.make_weights(cfg, seed)
    inp = gen.make_step_inputs(cfg, seed, ctx_len=[cfg["ctx"] - 5 * i for i in range(B)])
    w = upload_weights(cfg, W)
    aux = to_device(inp["aux"], cfg["dtype"])
    tok = torch.from_numpy(inp["in_tokens"]).to(DEV)
    cl = torch.from_numpy(inp["ctx_len"]).to(DEV)
    Sl = cfg["kv_capacity"]
    outs = []
    for paged in (False, True):
        ctx = S.SpecContext(cfg, max_batch=B, max_new=1)
        if paged:
            cache, _ = _paged(cfg, inp["k_cache"][None], inp["v_cache"][None], bs, seed)
        else:
            cache = upload_kv(cfg, inp["k_cache"], inp["v_cache"])
        tree = S.spec_build_tree(ctx, w, cache, aux, tok, cl)
        tnp = tree.numpy()
        logits = gen.plant_target_logits(cfg, tnp, seed)
        vt = S.spec_verify_tree(ctx, tree, torch.from_numpy(logits).to(DEV), 0)
        torch.cuda.synchronize()
        kv = _gather(cache, Sl) if paged else (from_device(cache.k), from_device(cache.v))
        outs.append((tnp, [t.cpu().numpy() for t in vt], kv))
    (t0, v0, kv0), (t1, v1, kv1) = outs
    compare_tree(t1, t0)
    for a, b in zip(v1, v0):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(kv1[0], kv0[0])
    np.testing.assert_array_equal(kv1[1], kv0[1])


@pytest.mark.parametrize("bs", [16, 24])
def test_paged_target_compaction_matches_oracle(bs):
    announce(f"paged compaction bs={bs}")
    cfg = configs.get("qwen8b_tree", batch=3)
    B, D = 3, cfg["depth"]
    slots = cfg["ctx"] + cfg["total_tokens"] + 8
    tkv = gen.make_target_kv(cfg, 91, slots, layers=4)
    base = np.full(B, cfg["ctx"], np.int32)
    tree = gen.random_tree(cfg, 91, batch=B)
    logits = gen.plant_target_logits(cfg, tree, 91)
    _, alen, nodes = ov.verify_greedy(tree, logits, D)
    want_k, want_v = tkv["k"].copy(), tkv["v"].copy()
    oc.compact_kv(want_k, want_v, base, nodes, alen)
    ctx = S.SpecContext(cfg, max_batch=B)
    cache, _ = _paged(cfg, tkv["k"], tkv["v"], bs, 92)
    S.spec_compact_kv(ctx, cache, torch.from_numpy(base).to(DEV), torch.from_numpy(nodes).to(DEV),
                      torch.from_numpy(alen).to(DEV))
    torch.cuda.synchronize()
    gk, gv = _gather(cache, slots)
    np.testing.assert_array_equal(gk, want_k)
    np.testing.assert_array_equal(gv, want_v)
    assert alen.max() > 0
