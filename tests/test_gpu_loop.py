"""Losslessness of the target side on the GPU (vLLM Neuron page, "What is
Speculative Decoding?": greedy speculation is bit-exact with the target
alone).

Two loops over the same target (8 float32 layers) and prompt:
  * plain greedy decoding: one target forward per token over a one-node tree;
  * speculation: each step the target verifies a chain of K drafts in one
    forward (spec_target_forward), greedy verification accepts a prefix and
    adds the correction or bonus token (spec_verify_tree), and the accepted
    rows' K/V are compacted next to the root (spec_compact_kv).
The drafts are the plain loop's next K tokens, with one of them replaced by a
wrong token on some steps, so accepted lengths 0..K all occur.  The emitted
sequence must equal the plain one token for token, up to the first position
whose plain-path argmax is a near-tie (gap below 1e-4; none is expected)."""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, announce
from speculative_decoding_aux_amd import spec as S
from speculative_decoding_aux_amd.tensors import upload_target_weights
from synth import configs, gen

pytestmark = pytest.mark.gpu

L, K, P, T = 8, 5, 6, 40


def _chain(tokens, ctx, n1):
    """A chain tree over `tokens` (root first) at positions ctx.., as device
    arrays of width n1."""
    n = len(tokens)
    t = {"tokens": np.full((1, n1), -1, np.int32), "parent": np.full((1, n1), -1, np.int32),
         "depth": np.full((1, n1), -1, np.int32), "position": np.full((1, n1), -1, np.int32),
         "num_nodes": np.array([n - 1], np.int32), "anc_mask": np.zeros((1, n1), np.uint64)}
    for j, tok in enumerate(tokens):
        t["tokens"][0, j] = tok
        t["parent"][0, j] = j - 1
        t["depth"][0, j] = j
        t["position"][0, j] = ctx + j
        t["anc_mask"][0, j] = np.uint64((1 << (j + 1)) - 1)
    tr = S.Tree(1, n1, DEV)
    for f in ("tokens", "parent", "depth", "position", "num_nodes"):
        getattr(tr, f).copy_(torch.from_numpy(t[f]))
    tr.anc_mask.copy_(torch.from_numpy(t["anc_mask"].view(np.int64)))
    return tr


def test_speculative_loop_equals_plain_greedy():
    announce("speculative loop vs plain greedy")
    cfg = configs.get("tiny_chain", hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512,
                      vocab=512, draft_vocab=512, top_k=1, depth=K, total_tokens=K, dtype="f32", batch=1,
                      ctx=80)
    n1 = K + 1
    W = gen.make_target_weights(cfg, 77, L)
    tw = upload_target_weights(cfg, W)
    ctx = S.SpecContext(cfg, max_batch=1, max_new=n1)
    slots = cfg["kv_capacity"]
    shape = (L, 1, cfg["n_kv_heads"], slots, cfg["head_dim"])
    rng = np.random.default_rng(78)
    prompt = rng.integers(0, cfg["vocab"], size=P).tolist()
    assert P <= n1

    def fresh_kv():
        return S.KVCache(torch.zeros(shape, device=DEV), torch.zeros(shape, device=DEV))

    def forward(kv, tokens, c):
        z, _ = S.spec_target_forward(ctx, tw, kv, _chain(tokens, c, n1), np.array([c], np.int32))
        return z[0].cpu().numpy()

    # plain greedy: prefill the prompt, then one token per forward
    kv = fresh_kv()
    z = forward(kv, prompt, 0)
    plain, gaps = [int(np.argmax(z[P - 1]))], [float(np.diff(np.sort(z[P - 1])[-2:])[0])]
    seq = prompt + plain
    while len(plain) < T:
        z = forward(kv, [seq[-1]], len(seq) - 1)
        plain.append(int(np.argmax(z[0])))
        gaps.append(float(np.diff(np.sort(z[0])[-2:])[0]))
        seq.append(plain[-1])
    clear = next((i for i, g in enumerate(gaps) if g < 1e-4), T)
    assert clear > 10, f"the plain path hits a near-tie at token {clear}"

    # speculation: chains of K drafts verified in one forward each
    kv = fresh_kv()
    z = forward(kv, prompt, 0)
    out = [int(np.argmax(z[P - 1]))]
    seq = prompt + out
    seen = set()
    step = 0
    while len(out) < T:
        c = len(seq) - 1
        g = len(out)
        drafts = [plain[g + j] if g + j < T else 0 for j in range(K)]
        if step % 3 != 2:  # corrupt one draft on two steps of three
            j = step % (K + 1)
            if j < K:
                drafts[j] = (drafts[j] + 1 + int(rng.integers(0, cfg["vocab"] - 1))) % cfg["vocab"]
        tree = _chain([seq[-1]] + drafts, c, n1)
        zt, _ = S.spec_target_forward(ctx, tw, kv, tree, np.array([c], np.int32))
        toks, alen, nodes = S.spec_verify_tree(ctx, tree, zt, 0)
        S.spec_compact_kv(ctx, kv, torch.tensor([c], dtype=torch.int32, device=DEV), nodes, alen)
        torch.cuda.synchronize()
        a = int(alen.cpu()[0])
        emitted = toks.cpu().numpy()[0, :a + 1].tolist()
        seen.add(a)
        out += emitted
        seq += emitted
        step += 1
    assert out[:clear] == plain[:clear]
    assert len(seen) >= 3, f"accepted lengths seen: {sorted(seen)}"
    assert K in seen
