"""GPU parity of the flat-batch index bookkeeping and of rejection sampling
with per-request temperature, top-k and top-p, against the oracle.

The bookkeeping is integer work and bit-exact.  Sampling must give the same
tokens and accepted counts on identical inputs; the seeds used keep every
random decision away from its threshold (checked on the oracle alone):
|u - p_f(x)| > 1e-5, the top-p mass more than 1e-5 (relative) from its
target, and Gumbel winners ahead by more than 1e-4.  The GPU computes
l/T and exp in float32 with float64 sums, the oracle in float64."""

import os

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, announce
from oracle import sampling as osm
from speculative_decoding_aux_amd import spec as S
from synth import configs, gen

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _ctx(V, B, L):
    cfg = configs.get("tiny_chain", vocab=V, draft_vocab=V, total_tokens=L, depth=L, batch=B)
    return S.SpecContext(cfg, max_batch=B)


def test_metadata_matches_the_pages_example_on_gpu():
    announce("decode metadata: page example")
    vals = {}
    with open(os.path.join(GOLDEN, "spec_decode_metadata_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, *nums = line.split()
                vals[name] = [int(x) for x in nums]
    ctx = _ctx(4096, 8, 4)
    nd = vals["num_draft_tokens"]
    got = S.spec_decode_metadata(ctx, vals["cu_num_scheduled_tokens"], nd, sum(nd))
    torch.cuda.synchronize()
    for name, g in zip(("cu_num_draft_tokens", "logits_indices", "target_logits_indices",
                        "bonus_logits_indices"), got):
        assert g.cpu().tolist() == vals[name], name


@pytest.mark.parametrize("B,L", [(1, 0), (300, 7), (1000, 3)])
def test_metadata_matches_oracle(B, L):
    announce(f"decode metadata B={B} L={L}")
    rng = np.random.default_rng(B)
    nd = rng.integers(0, L + 1, B).astype(np.int32)
    cu_s = np.cumsum(nd + 1 + rng.integers(0, 9, B)).astype(np.int32)
    want = osm.spec_decode_metadata(cu_s, nd)
    ctx = _ctx(4096, 8, 4)
    got = S.spec_decode_metadata(ctx, cu_s, nd, int(nd.sum()))
    torch.cuda.synchronize()
    for g, w in zip(got, want):
        np.testing.assert_array_equal(g.cpu().numpy(), w)


def _margins_ok(d, meta):
    cu, _, tgt, bonus = meta
    m_u, m_p, m_g = osm.decision_margins(cu, d["draft_token_ids"], d["logits"], tgt, bonus,
                                         d["temperature"], d["top_k"], d["top_p"], d["uniform"],
                                         d["seed"])
    return m_u > 1e-5 and m_p > 1e-5 and m_g > 1e-4


CASES = [
    # V, B, L, ties, greedy fraction, crowded
    (151936, 8, 5, False, 0.25, False),
    (128256, 6, 7, False, 0.0, False),
    (4099, 16, 4, True, 0.3, False),     # ragged vocabulary (scalar loads), tied logits
    (1000, 32, 6, False, 0.5, False),
    (100000, 8, 4, False, 0.0, True),    # one first-level bin holds almost every token
]


@pytest.mark.parametrize("V,B,L,ties,gf,crowded", CASES)
def test_rejection_sample_matches_oracle(V, B, L, ties, gf, crowded):
    chosen = None
    for s in range(40):
        d = gen.flat_batch(9000 + 31 * s + V % 97, B, L, V, ties=ties, greedy_frac=gf, crowded=crowded)
        meta = osm.spec_decode_metadata(d["cu_num_scheduled_tokens"], d["num_draft_tokens"])
        if _margins_ok(d, meta):
            chosen = (s, d, meta)
            break
    assert chosen is not None, "no seed with clear decision margins"
    s, d, meta = chosen
    announce(f"rejection sample V={V} B={B} L={L} ties={ties} crowded={crowded} seed-index={s}")
    cu, _, tgt, bonus = meta
    want_out, want_acc = osm.rejection_sample(cu, d["draft_token_ids"], d["logits"], tgt, bonus,
                                              d["temperature"], d["top_k"], d["top_p"], d["uniform"],
                                              d["seed"], L)
    ctx = _ctx(V, B, L)
    lg = torch.from_numpy(d["logits"]).to(DEV)
    out, acc = S.spec_rejection_sample(ctx, cu, d["draft_token_ids"], lg, tgt, bonus, d["temperature"],
                                       d["top_k"], d["top_p"], d["uniform"], d["seed"], L)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), want_acc)
    np.testing.assert_array_equal(out.cpu().numpy(), want_out)
    # the batch exercises acceptances and rejections of random requests
    rnd = d["temperature"] > 0
    assert want_acc[rnd].max() > 0


def test_all_greedy_when_uniforms_are_absent():
    announce("rejection sample without uniforms (greedy)")
    V, B, L = 32000, 12, 5
    d = gen.flat_batch(4242, B, L, V)
    cu, _, tgt, bonus = osm.spec_decode_metadata(d["cu_num_scheduled_tokens"], d["num_draft_tokens"])
    # an exact tie at the argmax of the first row exercises the first-index rule
    lg_np = d["logits"].copy()
    a = int(np.argmax(lg_np[0]))
    lg_np[0, max(0, a - 3)] = lg_np[0, a]
    zeros = np.zeros(B, np.float32)
    want_out, want_acc = osm.rejection_sample(cu, d["draft_token_ids"], lg_np, tgt, bonus, zeros,
                                              d["top_k"], d["top_p"], None, 0, L)
    ctx = _ctx(V, B, L)
    out, acc = S.spec_rejection_sample(ctx, cu, d["draft_token_ids"], torch.from_numpy(lg_np).to(DEV),
                                       tgt, bonus, d["temperature"], d["top_k"], d["top_p"], None, 0, L)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), want_out)
    np.testing.assert_array_equal(acc.cpu().numpy(), want_acc)
    assert want_acc.max() > 0


@pytest.mark.parametrize("k,p,T", [(1, 1.0, 1.0), (0, 0.0, 0.8), (3, 0.999, 0.05), (0, 1.0, 4.0)])
def test_degenerate_filters(k, p, T):
    """top-k 1 and top-p 0 keep only the best token; a tiny temperature
    concentrates the mass; a large one flattens it."""
    announce(f"rejection sample degenerate k={k} p={p} T={T}")
    V, B, L = 50000, 8, 4
    for s in range(40):
        d = gen.flat_batch(777 + s, B, L, V, greedy_frac=0.0)
        d["temperature"][:] = T
        d["top_k"][:] = k
        d["top_p"][:] = p
        meta = osm.spec_decode_metadata(d["cu_num_scheduled_tokens"], d["num_draft_tokens"])
        if _margins_ok(d, meta):
            break
    else:
        pytest.fail("no seed with clear decision margins")
    cu, _, tgt, bonus = meta
    want_out, want_acc = osm.rejection_sample(cu, d["draft_token_ids"], d["logits"], tgt, bonus,
                                              d["temperature"], d["top_k"], d["top_p"], d["uniform"],
                                              d["seed"], L)
    ctx = _ctx(V, B, L)
    out, acc = S.spec_rejection_sample(ctx, cu, d["draft_token_ids"], torch.from_numpy(d["logits"]).to(DEV),
                                       tgt, bonus, d["temperature"], d["top_k"], d["top_p"], d["uniform"],
                                       d["seed"], L)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), want_out)
    np.testing.assert_array_equal(acc.cpu().numpy(), want_acc)


@pytest.mark.parametrize("k,p", [(5000, 1.0), (5000, 0.9), (9000, 1.0), (40000, 0.5)])
def test_large_top_k_sets(k, p):
    """Logits uniform on [0, 16) put 4096 of the 65536 tokens in each of the
    eight first-level bins of [8, 16) (sign, exponent and three mantissa
    bits): with top-k 5000 the keys of the cut's bin and the bins above it
    fill the 8192 that LDS holds, with 9000 and 40000 the tokens above the
    cut are more than LDS holds and only the cut's bin is collected.  The
    draft tokens are raised above the rest, so that some are accepted."""
    announce(f"rejection sample large top-k k={k} p={p}")
    V, B, L = 65536, 8, 4
    rng = np.random.default_rng(4100 + k)
    for s in range(40):
        d = gen.flat_batch(5300 + s, B, L, V, greedy_frac=0.0)
        meta = osm.spec_decode_metadata(d["cu_num_scheduled_tokens"], d["num_draft_tokens"])
        cu, _, tgt, bonus = meta
        lg = rng.uniform(0.0, 16.0, d["logits"].shape).astype(np.float32)
        lg[tgt, d["draft_token_ids"]] = rng.uniform(17.0, 26.0, len(tgt)).astype(np.float32)
        d["logits"] = lg
        d["temperature"][:] = 1.0
        d["top_k"][:] = k
        d["top_p"][:] = p
        if _margins_ok(d, meta):
            break
    else:
        pytest.fail("no seed with clear decision margins")
    want_out, want_acc = osm.rejection_sample(cu, d["draft_token_ids"], d["logits"], tgt, bonus,
                                              d["temperature"], d["top_k"], d["top_p"], d["uniform"],
                                              d["seed"], L)
    ctx = _ctx(V, B, L)
    out, acc = S.spec_rejection_sample(ctx, cu, d["draft_token_ids"], torch.from_numpy(d["logits"]).to(DEV),
                                       tgt, bonus, d["temperature"], d["top_k"], d["top_p"], d["uniform"],
                                       d["seed"], L)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), want_out)
    np.testing.assert_array_equal(acc.cpu().numpy(), want_acc)
