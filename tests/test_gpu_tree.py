"""GPU parity of vocab top-k with log-probs (S9) and of tree expansion and
selection (S10) on identical inputs: ids and topology bit-exact."""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, announce, compare_tree
from oracle import draft as od
from oracle import tree as ot
from speculative_decoding_aux_amd import spec as S
from synth import configs, gen

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,n,k,mapped", [(4, 128256, 1, False), (1, 32000, 8, True), (8, 32000, 8, True),
                                          (256, 151936, 8, False), (3, 1000, 16, False), (2, 37, 5, False),
                                          (64, 4096, 3, False), (5, 128, 8, True), (7, 500, 16, False),
                                          (2, 512, 4, False)])
def test_topk_logprobs_match_oracle(M, n, k, mapped):
    announce(f"topk M={M} n={n} k={k}")
    z = gen.random_logits(M * 7 + n, "topk", (M, n))
    z[0, 3] = z[0, 9] = z[0].max() + 0.5      # exact tie at the top: lower id first
    if n > 100:
        z[-1, 50:60] = z[-1].max()            # a ten-way tie
    d2t = np.sort(np.random.default_rng(n).choice(151936, size=n, replace=False)).astype(np.int32) if mapped else None
    cfg = configs.get("tiny_chain", top_k=min(k, 16), total_tokens=max(3, k), depth=3, vocab=max(n, 4096),
                      draft_vocab=max(n, 4096))
    ctx = S.SpecContext(cfg, max_batch=M)
    ids, lp = S.spec_topk_logprobs(ctx, torch.from_numpy(z).to(DEV), k,
                                   None if d2t is None else torch.from_numpy(d2t).to(DEV))
    torch.cuda.synchronize()
    ids, lp = ids.cpu().numpy(), lp.cpu().numpy()
    for r in range(M):
        top, want_lp = ot.topk_logprobs(z[r], k)
        want_ids = top if d2t is None else d2t[top]
        np.testing.assert_array_equal(ids[r], want_ids)
        np.testing.assert_allclose(lp[r], want_lp, atol=2e-6, rtol=0)


@pytest.mark.parametrize("n,k", [(151936, 8), (151936, 16), (5000, 8), (4999, 2)])
def test_topk_adversarial_layouts(n, k):
    """Value layouts aimed at the batched scan (a thread reads 16-value batches
    at x0 + 1024 i + e): ramps, all-equal rows, the k best packed into one
    batch, ties across chunks, -inf runs; rows of 4999 are not 16-byte aligned."""
    announce(f"topk adversarial n={n} k={k}")
    rng = np.random.default_rng(n + k)
    M = 6
    z = rng.normal(0, 2, (M, n)).astype(np.float32)
    z[0] = np.linspace(-3, 3, n, dtype=np.float32)              # best values at the end
    z[1] = np.linspace(3, -3, n, dtype=np.float32)              # best values at the start
    z[2] = 0.25                                                 # all equal: lowest ids win
    x0 = 4096 + 4 * 37                                          # one thread's batch
    batch = [x0 + 1024 * i + e for i in range(4) for e in range(4)]
    batch = [x for x in batch if x < n]
    z[3, batch] = 10.0 + np.arange(len(batch), dtype=np.float32)[::-1] * 0.5
    z[4, ::997] = z[4].max() + 1.0                              # ties spread over chunks
    z[5, : n // 2] = -np.inf
    cfg = configs.get("tiny_chain", top_k=min(k, 16), total_tokens=max(3, k), depth=3, vocab=n, draft_vocab=n)
    ctx = S.SpecContext(cfg, max_batch=M)
    ids, lp = S.spec_topk_logprobs(ctx, torch.from_numpy(z).to(DEV), k)
    torch.cuda.synchronize()
    ids, lp = ids.cpu().numpy(), lp.cpu().numpy()
    for r in range(M):
        top, want_lp = ot.topk_logprobs(z[r], k)
        np.testing.assert_array_equal(ids[r], top, err_msg=f"row {r}")
        np.testing.assert_allclose(lp[r], want_lp, atol=2e-6, rtol=0, err_msg=f"row {r}")


@pytest.mark.parametrize("n,K", [(128256, 128), (70000, 128), (2048, 64), (128256, 256), (5001, 100)])
def test_candidate_retrieval_matches_oracle(n, K):
    """Retrieval of the K best scores per row (EAGLE-4 head): random rows, a
    ramp, the K best packed into few 16-value batches, ties at the threshold,
    and an all-equal row (far more tied batches than the fast path keeps, so
    the full-row select runs); 5001 is not a multiple of 4 (unaligned rows)."""
    announce(f"candidate retrieval n={n} K={K}")
    rng = np.random.default_rng(n * 3 + K)
    M = 7
    z = rng.normal(0, 1, (M, n)).astype(np.float32)
    z[1] = np.linspace(-1, 1, n, dtype=np.float32)
    z[2, : min(n, 3 * K)] += 8.0                                    # best values contiguous
    z[3] = np.round(z[3] * 2) / 2                                   # heavy ties everywhere
    z[4] = 0.5                                                      # all equal
    z[5, rng.choice(n, size=min(n, 4 * K), replace=False)] = 3.0    # ties at the threshold
    cfg = configs.get("tiny_chain", vocab=max(n, 4096), draft_vocab=max(n, 4096))
    ctx = S.SpecContext(cfg, max_batch=M)
    ids = S.spec_retrieve_candidates(ctx, torch.from_numpy(z).to(DEV), K)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    for r in range(M):
        np.testing.assert_array_equal(ids[r], od.topk_desc(z[r], K), err_msg=f"row {r}")


def _table(cfg, B, seed, quantise):
    """Per-pass top-k tables: distinct ids per row, log-probs sorted
    descending; quantised log-probs create exact score ties."""
    rng = np.random.default_rng(seed)
    k, D, V = cfg["top_k"], cfg["depth"], cfg["vocab"]
    ids = np.zeros((D, B, k, k), np.int32)
    lp = np.zeros((D, B, k, k), np.float32)
    for d in range(D):
        for b in range(B):
            for j in range(k):
                ids[d, b, j] = rng.choice(V, size=k, replace=False)
                v = -rng.exponential(1.5, size=k)
                if quantise:
                    v = np.round(v * 4) / 4
                lp[d, b, j] = np.sort(v)[::-1]
    return ids, lp


@pytest.mark.parametrize("name,B,n_new,quantise", [
    ("llama8b_chain", 4, 1, False), ("qwen4b_tree", 1, 1, False), ("qwen4b_tree", 3, 2, True),
    ("qwen8b_tree", 32, 1, True), ("eagle4_llama8b", 64, 1, False),
])
def test_tree_from_topk_matches_oracle(name, B, n_new, quantise):
    announce(f"tree from table {name} B={B} n_new={n_new}")
    cfg = configs.get(name, batch=B, n_new=n_new)
    seed = configs.SEEDS[name] + 13
    ids, lp = _table(cfg, B, seed, quantise)
    ctx_len = np.full(B, cfg["ctx"], np.int32)
    if B > 1:
        ctx_len[1] = cfg["kv_capacity"] - 2          # past the capacity cutoff: root only
        ctx_len[-1] = 17
    in_tokens = np.random.default_rng(seed).integers(0, cfg["vocab"], size=(B, n_new)).astype(np.int32)
    want = ot.build_tree_from_topk(cfg, ctx_len, in_tokens, ids, lp)
    ctx = S.SpecContext(cfg, max_batch=B, max_new=n_new)
    tr = S.spec_tree_from_topk(ctx, B, n_new, torch.from_numpy(in_tokens).to(DEV),
                               torch.from_numpy(ctx_len).to(DEV), torch.from_numpy(ids).to(DEV),
                               torch.from_numpy(lp).to(DEV))
    torch.cuda.synchronize()
    compare_tree(tr.numpy(), want)
    if B > 1:
        assert want["num_nodes"][1] == 0
