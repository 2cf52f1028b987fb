"""Pins of the target-side verification forward (oracle/target.py): a chain
tree equals the causal forward of its token sequence, written independently
in torch (F.rms_norm, F.scaled_dot_product_attention with a causal mask,
complex-number RoPE) including the aux states entering layers (2, L//2, L-3);
siblings do not see each other; the tree writes each node's K/V at its slot."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import target as ot
from synth import configs, gen

L = 8


def _cfg(dtype, **kw):
    base = dict(hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32, intermediate=96, vocab=300,
                draft_vocab=300, top_k=2, depth=3, total_tokens=5, dtype=dtype, batch=2, ctx=10)
    base.update(kw)
    return configs.get("tiny_chain", **base)


def _rope_c(x, pos, base):
    """Rotate-half RoPE written with complex numbers: pair (i, i + hd/2)."""
    hd = x.shape[-1]
    half = hd // 2
    inv = base ** (-torch.arange(half, dtype=torch.float64) * 2 / hd)
    ang = pos[:, None, None].double() * inv[None, None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def _torch_causal(cfg, W, kc, vc, toks, ctx, ctx_only=False):
    """One sequence: context keys [0, ctx) already in the cache (positions =
    slots), then the token run at positions ctx.. with causal attention (with
    ``ctx_only`` every token sees the context alone, not even itself)."""
    dt = cfg["dtype"]
    rnd = (lambda a: torch.from_numpy(gen.round_bf16_inplace(a.float().numpy().copy())).double()) \
        if dt == "bf16" else (lambda a: a.float().double())
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    H, nq, nkv, hd, I = (cfg[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "intermediate"))
    eps = cfg["rms_eps"]
    T = len(toks)
    pos = torch.arange(ctx, ctx + T)
    h = rnd(t(W["embed"][toks]))
    auxes = {}
    for l, Wl in enumerate(W["layers"]):
        if l in ot.aux_layer_ids(L):
            auxes[l] = h.clone()
        x = rnd(F.rms_norm(h, (H,), t(Wl["attn_norm"]), eps))
        qkv = rnd(x @ t(Wl["wqkv"]).T)
        q = qkv[:, : nq * hd].reshape(T, nq, hd)
        k = qkv[:, nq * hd:(nq + nkv) * hd].reshape(T, nkv, hd)
        v = qkv[:, (nq + nkv) * hd:].reshape(T, nkv, hd)
        q, k = rnd(_rope_c(q, pos, cfg["rope_base"])), rnd(_rope_c(k, pos, cfg["rope_base"]))
        K = torch.cat([t(kc[l, :, :ctx]).permute(1, 0, 2), k], 0)  # [ctx+T, nkv, hd]
        Vv = torch.cat([t(vc[l, :, :ctx]).permute(1, 0, 2), v], 0)
        mask = torch.ones(T, ctx + T, dtype=torch.bool)
        mask[:, ctx:] = False if ctx_only else torch.tril(torch.ones(T, T, dtype=torch.bool))
        g = nq // nkv
        Kh = K.permute(1, 0, 2).repeat_interleave(g, 0)[None]
        Vh = Vv.permute(1, 0, 2).repeat_interleave(g, 0)[None]
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], Kh, Vh, attn_mask=mask[None, None])
        o = rnd(o[0].permute(1, 0, 2).reshape(T, nq * hd))
        h1 = rnd(h + o @ t(Wl["wo"]).T)
        m = rnd(F.rms_norm(h1, (H,), t(Wl["mlp_norm"]), eps))
        gu = m @ t(Wl["w_gate_up"]).T
        s = rnd(F.silu(gu[:, :I]) * gu[:, I:])
        h = rnd(h1 + s @ t(Wl["w_down"]).T)
    n = rnd(F.rms_norm(h, (H,), t(W["final_norm"]), eps))
    aux = torch.cat([auxes[i] for i in ot.aux_layer_ids(L)], dim=1)
    return (n @ t(W["lm_head"]).T).numpy(), aux.numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_tree_is_the_causal_forward(dtype):
    cfg = _cfg(dtype)
    B, K = 2, 4
    W = gen.make_target_weights(cfg, 41, L)
    ctx = np.array([10, 7])
    S = 24
    kc = np.stack([gen.random_states(41, f"tk{l}", (B, cfg["n_kv_heads"], S, cfg["head_dim"]), dtype)
                   for l in range(L)])
    vc = np.stack([gen.random_states(41, f"tv{l}", (B, cfg["n_kv_heads"], S, cfg["head_dim"]), dtype)
                   for l in range(L)])
    tree = gen.chain_tree(B, K, cfg["vocab"], ctx, 41)
    k1, v1 = kc.copy(), vc.copy()
    logits, aux = ot.target_forward(cfg, W, k1, v1, tree, ctx)
    tol = dict(atol=1e-5, rtol=1e-5) if dtype == "f32" else dict(atol=2e-2, rtol=0)
    for b in range(B):
        z, a = _torch_causal(cfg, W, kc[:, b], vc[:, b], tree["tokens"][b], int(ctx[b]))
        np.testing.assert_allclose(logits[b], z, **tol)
        np.testing.assert_allclose(aux[b], a, **(tol if dtype == "f32" else dict(atol=2e-2, rtol=2e-2)))
        # each node's K/V went to slot ctx + n; the other slots are untouched
        for l in range(L):
            assert not np.array_equal(k1[l, b, :, ctx[b]:ctx[b] + K + 1], kc[l, b, :, ctx[b]:ctx[b] + K + 1])
            np.testing.assert_array_equal(k1[l, b, :, :ctx[b]], kc[l, b, :, :ctx[b]])
            np.testing.assert_array_equal(k1[l, b, :, ctx[b] + K + 1:], kc[l, b, :, ctx[b] + K + 1:])


def test_siblings_do_not_see_each_other():
    cfg = _cfg("f32")
    W = gen.make_target_weights(cfg, 42, L)
    ctx = np.array([6])
    S = 16
    kc = np.stack([gen.random_states(42, f"tk{l}", (1, 2, S, 32), "f32") for l in range(L)])
    vc = np.stack([gen.random_states(42, f"tv{l}", (1, 2, S, 32), "f32") for l in range(L)])
    # root 0 with children 1, 2; node 3 a child of 1
    tree = {"tokens": np.array([[5, 11, 17, 23]], np.int32), "parent": np.array([[-1, 0, 0, 1]], np.int32),
            "depth": np.array([[0, 1, 1, 2]], np.int32), "position": np.array([[6, 7, 7, 8]], np.int32),
            "num_nodes": np.array([3], np.int32),
            "anc_mask": np.array([[0b1, 0b11, 0b101, 0b1011]], np.uint64)}
    a, _ = ot.target_forward(cfg, W, kc.copy(), vc.copy(), tree, ctx)
    tree2 = dict(tree, tokens=np.array([[5, 11, 99, 23]], np.int32))  # change sibling 2
    b, _ = ot.target_forward(cfg, W, kc.copy(), vc.copy(), tree2, ctx)
    np.testing.assert_array_equal(a[0, [0, 1, 3]], b[0, [0, 1, 3]])
    assert not np.array_equal(a[0, 2], b[0, 2])


def test_nodes_past_num_nodes_see_the_context_only():
    """Rows of a tree past num_nodes (unused nodes) are computed as a token 0
    at position ctx that attends to the context alone and writes no K/V; the
    live nodes are the causal forward of their own chain."""
    cfg = _cfg("f32")
    W = gen.make_target_weights(cfg, 43, L)
    ctx = np.array([9])
    S = 20
    kc = np.stack([gen.random_states(43, f"tk{l}", (1, 2, S, 32), "f32") for l in range(L)])
    vc = np.stack([gen.random_states(43, f"tv{l}", (1, 2, S, 32), "f32") for l in range(L)])
    tree = gen.chain_tree(1, 5, cfg["vocab"], ctx, 43)
    live = 2  # nodes 0..2 live, 3..5 unused
    for key in ("tokens", "parent", "depth", "position"):
        tree[key][0, live + 1:] = -1
    tree["anc_mask"][0, live + 1:] = 0
    tree["num_nodes"][:] = live
    k1, v1 = kc.copy(), vc.copy()
    logits, aux = ot.target_forward(cfg, W, k1, v1, tree, ctx)
    z_live, a_live = _torch_causal(cfg, W, kc[:, 0], vc[:, 0], tree["tokens"][0, :live + 1], 9)
    np.testing.assert_allclose(logits[0, :live + 1], z_live, atol=1e-5, rtol=1e-5)
    z_dead, a_dead = _torch_causal(cfg, W, kc[:, 0], vc[:, 0], [0], 9, ctx_only=True)
    for n in range(live + 1, 6):
        np.testing.assert_allclose(logits[0, n], z_dead[0], atol=1e-5, rtol=1e-5)
        np.testing.assert_allclose(aux[0, n], a_dead[0], atol=1e-5, rtol=1e-5)
    # no K/V written at the unused nodes' slots (or anywhere past the live ones)
    np.testing.assert_array_equal(k1[:, :, :, 9 + live + 1:], kc[:, :, :, 9 + live + 1:])
    np.testing.assert_array_equal(v1[:, :, :, 9 + live + 1:], vc[:, :, :, 9 + live + 1:])
