"""GPU parity of the target's verification forward over draft trees
(spec_target_forward) against the oracle (oracle/target.py) on the same
seeded weights, caches and trees: logits within 1e-4 (float32) / 2e-2
(bf16) absolute, aux states and the K/V rows written at the nodes' slots
within the activation tolerance of the draft tests, greedy verification
with the GPU's logits equal to verification with the oracle's wherever the
oracle's argmax gaps exceed the tolerance.  Chains (also deeper than the
config's draft depth) and random trees, float32 and bf16, 8 layers (aux
layers 2, 4, 5); trees and chains of 32 and 64 nodes with 4 q-heads per
kv-head (more query vectors than one attention launch takes)."""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, announce
from oracle import target as otg
from oracle import verify as ov
from speculative_decoding_aux_amd import spec as S
from speculative_decoding_aux_amd.tensors import from_device, to_device, upload_target_weights
from synth import configs, gen

pytestmark = pytest.mark.gpu

L = 8
BASE = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512, vocab=2048,
            draft_vocab=2048, batch=3, ctx=40)
CASES = {
    "chain_f32": (dict(BASE, dtype="f32", top_k=1, depth=5, total_tokens=5), "chain", 1e-4),
    "chain_bf16": (dict(BASE, dtype="bf16", top_k=1, depth=5, total_tokens=5), "chain", 2e-2),
    "tree_bf16": (dict(BASE, dtype="bf16", top_k=3, depth=3, total_tokens=9), "tree", 2e-2),
    # a chain of 17 tokens (a prompt's prefill) under a config whose draft
    # trees are 3 deep: every node sees all the chain before it
    "deep_chain_f32": (dict(BASE, dtype="f32", top_k=4, depth=3, total_tokens=16), "chain", 1e-4),
    "tree_bf16_hd128": (dict(BASE, dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, top_k=2,
                             depth=4, total_tokens=7), "tree", 2e-2),
    # the verified trees of the Qwen3-4B (1 + 31 nodes) and Qwen3-8B (1 + 63
    # nodes) workloads with 4 q-heads per kv-head: 128 and 256 query vectors
    # per kv-head, taken by the attention in groups of rows
    "tree31_gqa4_bf16": (dict(BASE, dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, top_k=8,
                              depth=5, total_tokens=31), "tree", 2e-2),
    "tree63_gqa4_bf16": (dict(BASE, dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, top_k=8,
                              depth=7, total_tokens=63, batch=2), "tree", 2e-2),
    "tree31_gqa4_f32": (dict(BASE, dtype="f32", n_q_heads=8, n_kv_heads=2, top_k=8, depth=5,
                             total_tokens=31, batch=2), "tree", 1e-4),
    "chain63_gqa4_bf16": (dict(BASE, dtype="bf16", n_q_heads=8, n_kv_heads=2, top_k=8, depth=7,
                               total_tokens=63, batch=2), "chain", 2e-2),
}


def _tree_to_device(t, B, n1):
    tr = S.Tree(B, n1, DEV)
    for f in ("tokens", "parent", "depth", "position", "num_nodes"):
        getattr(tr, f).copy_(torch.from_numpy(np.ascontiguousarray(t[f], dtype=np.int32)))
    tr.anc_mask.copy_(torch.from_numpy(np.ascontiguousarray(t["anc_mask"]).view(np.int64)))
    return tr


@pytest.mark.parametrize("name", list(CASES))
def test_target_forward_matches_oracle(name):
    over, shape, tol = CASES[name]
    announce(f"target forward {name}")
    cfg = configs.get("tiny_chain", **over)
    B, N, dt = cfg["batch"], cfg["total_tokens"], cfg["dtype"]
    n1 = N + 1
    seed = 1300 + len(name)
    W = gen.make_target_weights(cfg, seed, L)
    ctx_len = np.array([cfg["ctx"] - 4 * b for b in range(B)])
    S_ = cfg["ctx"] + n1 + 3
    shape5 = (L, B, cfg["n_kv_heads"], S_, cfg["head_dim"])
    kc = gen.random_states(seed, "target_k", shape5, dt)
    vc = gen.random_states(seed, "target_v", shape5, dt)
    if shape == "chain":
        tree = gen.chain_tree(B, N, cfg["vocab"], ctx_len, seed)
    else:
        tree = gen.with_positions(gen.random_tree(cfg, seed, batch=B), ctx_len)
    k1, v1 = kc.copy(), vc.copy()
    want_z, want_aux = otg.target_forward(cfg, W, k1, v1, tree, ctx_len)
    ctx = S.SpecContext(cfg, max_batch=B, max_new=n1)
    tw = upload_target_weights(cfg, W)
    cache = S.KVCache(to_device(kc, dt), to_device(vc, dt))
    tr = _tree_to_device(tree, B, n1)
    z, aux = S.spec_target_forward(ctx, tw, cache, tr, ctx_len)
    torch.cuda.synchronize()
    z = z.cpu().numpy()
    act = dict(rtol=1e-2, atol=1e-2) if dt == "bf16" else dict(rtol=1e-5, atol=1e-5)
    for b in range(B):
        live = np.arange(int(tree["num_nodes"][b]) + 1)
        np.testing.assert_allclose(z[b, live], want_z[b, live], atol=tol, rtol=0, err_msg=f"seq {b}")
        np.testing.assert_allclose(from_device(aux[b, live]), want_aux[b, live], **act, err_msg=f"seq {b}")
        sl = ctx_len[b] + live
        np.testing.assert_allclose(from_device(cache.k[:, b][:, :, sl]), k1[:, b][:, :, sl], **act)
        np.testing.assert_allclose(from_device(cache.v[:, b][:, :, sl]), v1[:, b][:, :, sl], **act)
    # greedy verification on either side's logits, where the oracle's argmax is clear
    D = cfg["depth"]
    o_gpu = ov.verify_greedy(tree, z, D)
    o_ora = ov.verify_greedy(tree, want_z, D)
    for b in range(B):
        srt = np.sort(want_z[b], axis=1)
        if np.all(srt[:, -1] - srt[:, -2] > 2 * tol):
            np.testing.assert_array_equal(o_gpu[0][b], o_ora[0][b])
