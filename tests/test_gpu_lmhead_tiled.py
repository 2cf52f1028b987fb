"""GPU test of the beam-pass LM head above 64 rows (the tiled GEMM, which
leaves a (max, sum exp) record per row and 128-column strip, and the top-k
that rescans only the k best strips of each row): on the same pass inputs,
its ids equal the top-k that the library computes over the full
materialised logits (the same float32 values), and its log-probs agree
within 2e-6; the logits match the oracle's for every sequence, and the ids
match the oracle's top-k where the gaps allow.  Cases: ragged rows (72), one
and two 256-row blocks, a vocabulary with a ragged last 128-column strip, 23
strips (a short last group when two row blocks share strips), trimmed
vocabularies, and exact ties inside and across strips (duplicated lm_head
rows)."""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, announce, ids_match_where_gap_allows
from oracle import draft as od
from speculative_decoding_aux_amd import spec as S
from speculative_decoding_aux_amd.tensors import to_device, upload_kv, upload_weights
from synth import configs, gen

pytestmark = pytest.mark.gpu

BASE = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512, top_k=8, depth=3,
            total_tokens=20, dtype="bf16", ctx=40)

CASES = [
    # (batch -> rows = batch * top_k, vocab, draft vocab, ties)
    (9, 1000, 1000, False),      # 72 rows; 7 full strips + 104 columns
    (32, 5000, 5000, True),      # 256 rows, ties inside and across strips
    (64, 3000, 2900, False),     # 512 rows (two row blocks), trimmed vocabulary, ragged strip
    (64, 2944, 2944, False),     # 512 rows, 23 strips: a short last group of the strip-to-block map
    (32, 151936, 151936, True),  # the Qwen3-8B vocabulary at 256 rows
]


@pytest.mark.parametrize("B,V,Vd,ties", CASES)
def test_tiled_head_topk_equals_topk_of_logits(B, V, Vd, ties):
    announce(f"tiled LM-head top-k B={B} V={V} Vd={Vd} ties={ties}")
    cfg = configs.get("tiny_chain", **dict(BASE, batch=B, vocab=V, draft_vocab=Vd))
    k, H = cfg["top_k"], cfg["hidden"]
    seed = 4100 + B
    W = gen.make_weights(cfg, seed)
    if ties:
        lm = W["lm_head"]
        lm[5:13] = lm[4]          # a 9-way tie inside strip 0
        lm[[130, 300, Vd - 1]] = lm[4]  # and in three other strips (the last one ragged or not)
    inp = gen.make_step_inputs(cfg, seed)
    ctx_len = inp["ctx_len"]
    ctx = S.SpecContext(cfg, max_batch=B)
    w = upload_weights(cfg, W)
    M = B * k
    rng = np.random.default_rng(seed)
    pos = np.repeat(ctx_len + 1, k).astype(np.int32)
    slot = (np.repeat(ctx_len + 1, k) + np.tile(np.arange(k), B)).astype(np.int32)
    anc = np.stack([np.repeat(ctx_len, k), slot], axis=1).astype(np.int32)
    toks = rng.integers(0, V, size=M).astype(np.int32)
    hid = gen.random_states(seed, "beam_states", (M, H), "bf16")
    outs = []
    for want_logits in (False, True):
        cache = upload_kv(cfg, inp["k_cache"], inp["v_cache"])
        outs.append(S.spec_draft_step(ctx, w, cache, B, k, 1, to_device(hid, "bf16"), toks, pos, slot, ctx_len,
                                      anc, k, want_logits=want_logits))
    torch.cuda.synchronize()
    fused, plain = outs
    np.testing.assert_array_equal(fused["ids"].cpu().numpy(), plain["ids"].cpu().numpy())
    np.testing.assert_allclose(fused["logp"].cpu().numpy(), plain["logp"].cpu().numpy(), rtol=0, atol=2e-6)
    np.testing.assert_array_equal(fused["h_out"].float().cpu().numpy(), plain["h_out"].float().cpu().numpy())
    # the tie-break: within the tie the smaller id ranks first, wherever it shows
    z = plain["logits"].cpu().numpy()
    gi = fused["ids"].cpu().numpy()
    d2t = W.get("d2t")
    for r in range(M):
        top = np.argsort(-z[r].astype(np.float64), kind="stable")[:k]
        want = top if d2t is None else d2t[top]
        assert gi[r].tolist() == want.tolist(), f"row {r}"
    # against the oracle: every sequence's logits (every (strip, row block)
    # tile was computed), ids where the gaps allow
    for b in range(B):
        kc = inp["k_cache"][b:b + 1].copy()
        vc = inp["v_cache"][b:b + 1].copy()
        r2 = np.arange(b * k, (b + 1) * k)
        o = od.draft_pass(cfg, W, kc, vc, 1, hid[r2], toks[r2], np.zeros(k, np.int64), pos[r2], slot[r2],
                          ctx_len[b:b + 1], anc[r2])
        np.testing.assert_allclose(z[r2], o["logits"], rtol=0, atol=2e-2, err_msg=f"logits of sequence {b}")
        ids_match_where_gap_allows(gi[r2], o["logits"], k, 2e-2, d2t)
    ctx.close()
