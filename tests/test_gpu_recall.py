"""EAGLE-4 candidate recall on the GPU (both heads through the C ABI).

With an lm_head of exact rank r built from the candidate head's own factors
(lm_head = cand_up . cand_down, rounded to bf16), the low-rank scores equal
the full logits up to bf16 rounding of the rank-r intermediate, so the full
EAGLE-3 head's top-k over the same rows (same weights, same inputs) lies
inside the retrieved candidates: recall 1 at 1 and at top_k.  With an
unrelated lm_head the recall falls to about K / V, which shows that the
measurement can tell the two apart."""

import numpy as np
import pytest
import torch

from gpu_helpers import announce
from speculative_decoding_aux_amd import spec as S
from speculative_decoding_aux_amd.tensors import to_device, upload_kv, upload_weights
from synth import configs, gen

pytestmark = pytest.mark.gpu


def _recall(cfg, W, inp):
    B, k = cfg["batch"], cfg["top_k"]
    ctx4 = S.SpecContext(cfg, max_batch=B)
    ctx3 = S.SpecContext(dict(cfg, cand_rank=0, num_candidates=0), max_batch=B)
    w = upload_weights(cfg, W)
    kv = upload_kv(cfg, inp["k_cache"], inp["v_cache"])
    pos = inp["ctx_len"].astype(np.int32)
    aux = to_device(np.ascontiguousarray(inp["aux"][:, 0]), cfg["dtype"])
    toks = inp["in_tokens"][:, 0]
    g4 = S.spec_draft_step(ctx4, w, kv, B, 1, 0, aux, toks, pos, pos, inp["ctx_len"], pos[:, None], k,
                           want_candidates=True)
    g3 = S.spec_draft_step(ctx3, w, kv, B, 1, 0, aux, toks, pos, pos, inp["ctx_len"], pos[:, None], k)
    torch.cuda.synchronize()
    full, cands = g3["ids"].cpu().numpy(), g4["cand_ids"].cpu().numpy()
    at1 = np.mean([full[r, 0] in set(cands[r].tolist()) for r in range(B)])
    atk = np.mean([len(set(full[r].tolist()) & set(cands[r].tolist())) / k for r in range(B)])
    return at1, atk


@pytest.mark.parametrize("V", [4096, 70000])
def test_exact_low_rank_head_has_full_recall(V):
    announce(f"candidate recall V={V}")
    cfg = configs.get("tiny_chain", hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512,
                      vocab=V, draft_vocab=V, top_k=8, depth=3, total_tokens=20, dtype="bf16", batch=6,
                      ctx=40, cand_rank=32, num_candidates=128)
    W = gen.make_weights(cfg, 61)
    inp = gen.make_step_inputs(cfg, 61)
    exact = dict(W, lm_head=gen.round_bf16_inplace(
        (W["cand_up"].astype(np.float64) @ W["cand_down"].astype(np.float64)).astype(np.float32)))
    at1, atk = _recall(cfg, exact, inp)
    assert at1 == 1.0 and atk == 1.0, (at1, atk)
    at1r, atkr = _recall(cfg, W, inp)
    assert atkr < 0.5, atkr
