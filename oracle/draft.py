"""One pass of the EAGLE-3 draft over a set of rows (TEST INFRASTRUCTURE).

Follows the vLLM Neuron design page, "Speculative Decoding (EAGLE3) in the
vLLM Neuron Framework":
  * "What is EAGLE3?" - three auxiliary target hidden states are concatenated
    and fused by one linear projection;
  * "Eagle3 Draft Model Architecture" - the decoder layer normalises the token
    embedding and the target hidden state separately, concatenates them to a
    2H-wide input, runs attention (QKV sized for 2H, output H), adds the
    residual, then the MLP on the post-attention norm with a second residual;
    the model returns the pre-norm state as the recurrent input and applies the
    final norm and the LM head; the FC is Linear(3H, H) with no bias shown;
  * two forward modes: initial (FC of the [T, 3H] aux states) and recurrent
    ([T, H] pre-norm state of the previous pass).
EAGLE-4 additions follow the NeMo AutoModel "eagle4" page: a sliding-window
draft attention (Eagle4Config.sliding_window: the keys a draft query sees,
itself and its chain included) and a low-rank candidate head
(Eagle4CandidateHeadConfig: rank r, num_candidates K; the serving engine keeps
K candidates from the low-rank scores and rescores them exactly with the full
lm_head).

Readings (the pages are silent): the residual of the attention block is the
layer's hidden input (FC output or recurrent state); no biases; no QK-norm;
RMSNorm gains as given; RoPE rotate-half on q and k before the K/V store; the
MLP is SwiGLU with the gate rows first in w_gate_up; the low-rank product
n @ cand_down^T is rounded to storage precision and there is no nonlinearity
between the two factors.

EAGLE-3.1 flags (the AMD Quark "EAGLE-3" page, "Background: EAGLE-3 and
EAGLE-3.1": extra normalisation inside the draft head, named fc_norm and
norm_output; where it sits is not stated).  Readings: fc_norm is an RMSNorm
with its own gain (W["fc_norm"]) on the FC output, so the initial pass's layer
input g (and residual) is the normalised fusion; norm_output makes the
recurrent output the final-normed row n (the LM head's input) instead of the
pre-norm state.  Both are off unless the configuration sets them.

Rounding points (storage precision = bf16 or f32 by workload):
  g, c, qkv, rotated q/k, attention output, h1, post-attention norm, the SwiGLU
  product, h_out and the final-normed n are rounded; logits stay float32.

Pinned by tests/test_oracle_draft.py: an independent torch formulation with
F.scaled_dot_product_attention and an explicit boolean mask; special cases
(one visible key returns that value row; q = 0 averages the visible values;
window >= context equals full attention; window 1 sees only itself).
"""

from __future__ import annotations

import numpy as np

from .numerics import rmsnorm, rope, silu, to_storage


def visible_slots(cfg: dict, pq: int, ctx: int, anc_row) -> np.ndarray:
    """Slots a query at position pq may attend to.

    Context slots [0, ctx) hold keys at positions equal to their slot index.
    ``anc_row`` lists extra slots (root rows, tree ancestors, itself; -1
    padded) whose positions form a consecutive run ending at pq, in order.
    With a window W > 0 a key at position pk is visible iff pq - W < pk <= pq
    (the window counts the query itself)."""
    W = int(cfg["sliding_window"])
    lo = 0 if W == 0 else max(0, pq - W + 1)
    extra = [int(s) for s in anc_row if s >= 0]
    n = len(extra)
    keep = [s for j, s in enumerate(extra) if W == 0 or (pq - (n - 1 - j)) > pq - W]
    return np.array(list(range(lo, ctx)) + keep, dtype=np.int64)


def attention_row(q, kc, vc, slots, n_kv: int) -> np.ndarray:
    """softmax(q k^T / sqrt(hd)) v over the given slots, float64, per q-head;
    q-head h reads kv-head h // (n_q / n_kv).  No visible key gives zeros."""
    nq, hd = q.shape
    out = np.zeros((nq, hd), dtype=np.float64)
    if len(slots) == 0:
        return out
    group = nq // n_kv
    K = kc[:, slots, :].astype(np.float64)
    V = vc[:, slots, :].astype(np.float64)
    for h in range(nq):
        kv = h // group
        s = K[kv] @ q[h].astype(np.float64) / np.sqrt(hd)
        s -= s.max()
        p = np.exp(s)
        p /= p.sum()
        out[h] = p @ V[kv]
    return out


def topk_desc(values, k: int, ids=None) -> np.ndarray:
    """Positions of the k best entries ordered by (value desc, id asc)."""
    values = np.asarray(values)
    ids = np.arange(values.shape[0]) if ids is None else np.asarray(ids)
    order = np.lexsort((ids, -values.astype(np.float64)))
    return order[:k]


def draft_pass(cfg, W, kcache, vcache, mode, hidden_in, tokens, seq, pos, slot, ctx_len, anc):
    """Run the draft decoder over M rows; returns a dict.

    mode 0 (initial): hidden_in is [M, 3H], the concatenated low|mid|high aux
    states; mode 1 (recurrent): hidden_in is [M, H].  Each row's k/v are
    written to kcache/vcache[seq, :, slot] (slot < 0: not written) before any
    row attends.  Returns h_out [M, H] (pre-norm recurrent state) and either
    logits [M, Vd] float32 (EAGLE-3 head) or, with a candidate head,
    scores [M, V], cand_ids [M, K] and cand_logits [M, K]."""
    dt = cfg["dtype"]
    H, nq, nkv, hd, I = (cfg[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "intermediate"))
    eps = cfg["rms_eps"]
    x = np.asarray(hidden_in, dtype=np.float32)
    M = x.shape[0]
    tokens = np.asarray(tokens)
    seq = np.asarray(seq)
    pos = np.asarray(pos)
    slot = np.asarray(slot)
    anc = np.asarray(anc).reshape(M, -1)

    # S1: FC fusion of the aux states, or the recurrent state as given
    g = to_storage(x @ W["fc"].T, dt) if mode == 0 else to_storage(x, dt)
    if mode == 0 and cfg.get("fc_norm"):
        g = to_storage(rmsnorm(g, W["fc_norm"], eps), dt)
    # S2: normalised token embedding | normalised hidden -> [M, 2H]
    e = W["embed"][tokens]
    a = to_storage(rmsnorm(e, W["input_norm"], eps), dt)
    b = to_storage(rmsnorm(g, W["hidden_norm"], eps), dt)
    c = np.concatenate([a, b], axis=1)
    # S3: QKV of the 2H-wide input
    qkv = to_storage(c @ W["wqkv"].T, dt)
    q = qkv[:, : nq * hd].reshape(M, nq, hd)
    k = qkv[:, nq * hd:(nq + nkv) * hd].reshape(M, nkv, hd)
    v = qkv[:, (nq + nkv) * hd:].reshape(M, nkv, hd)
    # S4: RoPE at each row's position, then store k, v at the row's slot
    q = to_storage(rope(q, pos[:, None], cfg["rope_base"]), dt)
    k = to_storage(rope(k, pos[:, None], cfg["rope_base"]), dt)
    for r in range(M):
        if slot[r] >= 0:
            kcache[seq[r], :, slot[r], :] = k[r]
            vcache[seq[r], :, slot[r], :] = v[r]
    # S5: tree-masked (and optionally windowed) GQA attention
    o = np.empty((M, nq * hd), dtype=np.float32)
    for r in range(M):
        vis = visible_slots(cfg, int(pos[r]), int(ctx_len[seq[r]]), anc[r])
        o[r] = to_storage(attention_row(q[r], kcache[seq[r]], vcache[seq[r]], vis, nkv).reshape(-1), dt)
    # S6: output projection plus the residual (the layer's hidden input)
    h1 = to_storage(g.astype(np.float64) + (o @ W["wo"].T).astype(np.float64), dt)
    # S7: SwiGLU MLP on the post-attention norm, second residual
    m = to_storage(rmsnorm(h1, W["post_attn_norm"], eps), dt)
    gu = (m @ W["w_gate_up"].T).astype(np.float64)
    s = to_storage(silu(gu[:, :I]) * gu[:, I:], dt)
    h_out = to_storage(h1.astype(np.float64) + (s @ W["w_down"].T).astype(np.float64), dt)
    # S8: final norm and LM head
    n = to_storage(rmsnorm(h_out, W["final_norm"], eps), dt)
    out = {"h_out": n if cfg.get("norm_output") else h_out, "normed": n}
    if not cfg["cand_rank"]:
        out["logits"] = (n @ W["lm_head"].T).astype(np.float32)
        return out
    # S8': low-rank scores, top-K retrieval, exact rescoring of the candidates
    t = to_storage(n @ W["cand_down"].T, dt)
    scores = (t @ W["cand_up"].T).astype(np.float32)
    K = cfg["num_candidates"]
    cand = np.stack([topk_desc(scores[r], K) for r in range(M)]).astype(np.int64)
    cand_logits = np.stack([(W["lm_head"][cand[r]] @ n[r]).astype(np.float32) for r in range(M)])
    out.update(scores=scores, cand_ids=cand, cand_logits=cand_logits)
    return out
