"""Target-side verification forward over the draft tree (TEST INFRASTRUCTURE).

Follows the vLLM Neuron design page: "What is Speculative Decoding?" (the
target processes the original token and all draft tokens in one forward pass,
producing logits for each position), "Auxiliary Hidden State Extraction"
(during the forward the hidden states entering the layers at indices
(2, L // 2, L - 3) are captured and concatenated as the draft's aux input;
the hidden state entering layer idx is recorded before that layer runs) and
"KV Cache Sharing" (each tree token's K/V goes to its own slot).

Each tree node n of sequence b is one row: its token, position
tree["position"][b, n] and KV slot ctx_len[b] + n; it attends to the
sequence's context slots [0, ctx_len) and to the slots of its ancestors and
itself (bits of tree["anc_mask"][b, n]), which is the tree mask.  Nodes past
num_nodes are computed over the context alone and write no K/V.

Readings: the target decoder layer is the Llama layer of the draft without the
2H concatenation (input norm, QKV of the H-wide normed state, RoPE
rotate-half, GQA attention, O projection plus residual, post-attention norm,
SwiGLU MLP plus residual); final norm and LM head give float32 logits; the
rounding points are those of the draft (storage precision after every
projection, norm and residual).  Pinned by tests/test_oracle_target.py: a
chain tree is the causal forward of the token sequence (each position sees
the context and the previous chain tokens), checked against an independent
torch formulation with F.scaled_dot_product_attention and a causal mask;
sibling nodes do not see each other (a node's output is unchanged when a
sibling's token changes); the aux states at layer 0 are the embeddings; rows
past num_nodes equal an independent one-token forward (token 0 at position
ctx) that sees the context alone, and leave the cache untouched.
"""

from __future__ import annotations

import numpy as np

from .draft import attention_row
from .numerics import rmsnorm, rope, silu, to_storage


def aux_layer_ids(L: int):
    """The page's default aux layers of an L-layer target."""
    return (2, L // 2, L - 3)


def target_layer(cfg, Wl, h, kcache, vcache, seq, pos, slot, visible):
    """One Llama decoder layer over rows h [M, H]; K/V written to
    kcache/vcache[seq, :, slot] (slot < 0: not written) before any row
    attends; visible[r] lists the slots row r attends to."""
    dt = cfg["dtype"]
    H, nq, nkv, hd, I = (cfg[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "intermediate"))
    eps = cfg["rms_eps"]
    M = h.shape[0]
    x = to_storage(rmsnorm(h, Wl["attn_norm"], eps), dt)
    qkv = to_storage(x @ Wl["wqkv"].T, dt)
    q = qkv[:, : nq * hd].reshape(M, nq, hd)
    k = qkv[:, nq * hd:(nq + nkv) * hd].reshape(M, nkv, hd)
    v = qkv[:, (nq + nkv) * hd:].reshape(M, nkv, hd)
    q = to_storage(rope(q, pos[:, None], cfg["rope_base"]), dt)
    k = to_storage(rope(k, pos[:, None], cfg["rope_base"]), dt)
    for r in range(M):
        if slot[r] >= 0:
            kcache[seq[r], :, slot[r], :] = k[r]
            vcache[seq[r], :, slot[r], :] = v[r]
    o = np.empty((M, nq * hd), dtype=np.float32)
    for r in range(M):
        o[r] = to_storage(attention_row(q[r], kcache[seq[r]], vcache[seq[r]], visible[r], nkv).reshape(-1), dt)
    h1 = to_storage(h.astype(np.float64) + (o @ Wl["wo"].T).astype(np.float64), dt)
    m = to_storage(rmsnorm(h1, Wl["mlp_norm"], eps), dt)
    gu = (m @ Wl["w_gate_up"].T).astype(np.float64)
    s = to_storage(silu(gu[:, :I]) * gu[:, I:], dt)
    return to_storage(h1.astype(np.float64) + (s @ Wl["w_down"].T).astype(np.float64), dt)


def tree_rows(tree, ctx_len):
    """Per row (b, n): token, position, slot and visible slots."""
    B, n1 = tree["tokens"].shape
    seq, tok, pos, slot, vis = [], [], [], [], []
    for b in range(B):
        nn = int(tree["num_nodes"][b])
        c = int(ctx_len[b])
        for n in range(n1):
            seq.append(b)
            live = n <= nn
            tok.append(int(tree["tokens"][b, n]) if live else 0)
            pos.append(int(tree["position"][b, n]) if live else c)
            slot.append(c + n if live else -1)
            mask = int(tree["anc_mask"][b, n]) if live else 0
            extra = [c + j for j in range(n1) if (mask >> j) & 1]
            vis.append(np.array(list(range(c)) + extra, dtype=np.int64))
    return (np.array(seq), np.array(tok), np.array(pos, dtype=np.int64), np.array(slot), vis)


def target_forward(cfg, W, kcache, vcache, tree, ctx_len):
    """The target forward over every tree node.  W: embed [V, H], final_norm,
    lm_head [V, H], layers = list of per-layer dicts (attn_norm, wqkv
    [(nq+2nkv)hd, H], wo, mlp_norm, w_gate_up, w_down).  kcache/vcache:
    [L, B, nkv, S, hd] (updated in place).  Returns logits [B, N+1, V]
    float32 and aux [B, N+1, 3H] (hidden states entering the aux layers)."""
    dt = cfg["dtype"]
    B, n1 = tree["tokens"].shape
    L = len(W["layers"])
    seq, tok, pos, slot, vis = tree_rows(tree, ctx_len)
    h = to_storage(W["embed"][tok], dt)
    aux = {}
    ids = aux_layer_ids(L)
    for l, Wl in enumerate(W["layers"]):
        if l in ids:
            aux[l] = h.copy()
        h = target_layer(cfg, Wl, h, kcache[l], vcache[l], seq, pos, slot, vis)
    n = to_storage(rmsnorm(h, W["final_norm"], cfg["rms_eps"]), dt)
    logits = (n @ W["lm_head"].T).astype(np.float32).reshape(B, n1, -1)
    H = cfg["hidden"]
    a = np.concatenate([aux[i] for i in ids], axis=1).reshape(B, n1, 3 * H)
    return logits, a
