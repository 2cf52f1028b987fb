"""Pins of the flat-batch rejection sampler with per-request sampling
parameters (oracle/sampling.py) against the page's printed metadata example,
brute force, a library softmax, plain greedy decoding and the lossless-sampling
law."""

import itertools
import os

import numpy as np
import pytest
from scipy import special, stats

from oracle import sampling as osm
from oracle import verify as ov

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_metadata():
    vals = {}
    with open(os.path.join(GOLDEN, "spec_decode_metadata_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, *nums = line.split()
                vals[name] = [int(x) for x in nums]
    return vals


def test_metadata_matches_the_pages_example():
    g = _golden_metadata()
    cu, li, tgt, bonus = osm.spec_decode_metadata(g["cu_num_scheduled_tokens"], g["num_draft_tokens"])
    assert cu.tolist() == g["cu_num_draft_tokens"]
    assert li.tolist() == g["logits_indices"]
    assert tgt.tolist() == g["target_logits_indices"]
    assert bonus.tolist() == g["bonus_logits_indices"]


def test_metadata_empty_and_all_zero_drafts():
    cu, li, tgt, bonus = osm.spec_decode_metadata([1, 2, 3], [0, 0, 0])
    assert cu.tolist() == [0, 0, 0] and tgt.tolist() == [] and bonus.tolist() == [0, 1, 2]
    assert li.tolist() == [0, 1, 2]
    cu, li, tgt, bonus = osm.spec_decode_metadata([], [])
    assert len(cu) == len(li) == len(tgt) == len(bonus) == 0


def _beats(l, a, b):
    return l[a] > l[b] or (l[a] == l[b] and a < b)


@pytest.mark.parametrize("seed", range(12))
def test_top_k_then_top_p_brute_force(seed):
    """The kept set is, within the top-k set, a smallest subset whose mass
    reaches p; among the smallest such subsets it has the largest mass, and
    every kept token beats every dropped one in (logit desc, id asc)."""
    rng = np.random.default_rng(seed)
    V = 7
    # few distinct values so that ties occur
    l = rng.integers(-3, 3, V).astype(np.float32) * np.float32(0.75)
    T = [0.5, 1.0, 1.7][seed % 3]
    for k in (0, 1, 3, 5, V):
        # top-k by pairwise dominance: exactly the tokens beaten by fewer than k others
        ids = list(range(V))
        if 0 < k < V:
            topk = [a for a in ids if sum(_beats(l, b, a) for b in ids if b != a) < k]
        else:
            topk = ids
        assert len(topk) == (k if 0 < k < V else V)
        z = l.astype(np.float64) / T
        e = {a: np.exp(z[a] - z.max()) for a in ids}
        sk = sum(e[a] for a in topk)
        for p in (0.05, 0.3, 0.5, 0.77, 0.95, 1.0):
            kept = set(osm.kept_prefix(l, T, k, p).tolist())
            if p >= 1.0:
                assert kept == set(topk)
                continue
            target = p * sk
            best = None
            for m in range(1, len(topk) + 1):
                cands = [set(s) for s in itertools.combinations(topk, m)
                         if sum(e[a] for a in s) >= target * (1 - 1e-12)]
                if cands:
                    best = (m, max(sum(e[a] for a in s) for s in cands))
                    break
            assert len(kept) == best[0]
            assert abs(sum(e[a] for a in kept) - best[1]) <= 1e-12 * sk
            assert kept <= set(topk)
            for a in kept:
                for b in set(topk) - kept:
                    assert _beats(l, a, b)


@pytest.mark.parametrize("T", [0.3, 1.0, 2.5])
def test_unfiltered_distribution_is_softmax(T):
    rng = np.random.default_rng(7)
    l = rng.normal(0, 2, 50).astype(np.float32)
    p = osm.filtered_probs(l, T, 0, 1.0)
    assert np.allclose(p, special.softmax(l.astype(np.float64) / T), rtol=1e-12, atol=0)
    # top-k = 1 keeps only the argmax
    p1 = osm.filtered_probs(l, T, 1, 1.0)
    assert p1[np.argmax(l)] == 1.0 and p1.sum() == 1.0


def _synthetic_target(prefix, V=11):
    """A deterministic stand-in for a target model: logits from a hash of the
    prefix (integer-valued so argmax ties happen and resolve to the first id)."""
    h = 1469598103934665603
    for t in prefix:
        h = ((h ^ (int(t) + 1)) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    rng = np.random.default_rng(h)
    return rng.integers(0, 6, V).astype(np.float32)


def test_greedy_rows_equal_plain_greedy_decoding():
    """Mixed variable-length greedy chains over many speculation steps give
    exactly the tokens of plain greedy decoding of the same target."""
    rng = np.random.default_rng(3)
    B, L, K = 4, 40, 5
    seqs = [[int(rng.integers(0, 11))] for _ in range(B)]
    want = []
    for b in range(B):
        s = list(seqs[b])
        while len(s) < L:
            s.append(int(np.argmax(_synthetic_target(s))))
        want.append(s)
    while min(len(s) for s in seqs) < L:
        nd = rng.integers(0, K + 1, B)
        drafts, rows, tgt, bonus = [], [], [], []
        for b in range(B):
            s = list(seqs[b])
            d = []
            for j in range(nd[b]):
                # right with probability 0.6, else a random token
                t = int(np.argmax(_synthetic_target(s))) if rng.random() < 0.6 else int(rng.integers(0, 11))
                d.append(t)
                s.append(t)
            for j in range(nd[b] + 1):
                (tgt if j < nd[b] else bonus).append(len(rows))
                rows.append(_synthetic_target(seqs[b] + d[:j]))
            drafts += d
        out, acc = osm.rejection_sample(np.cumsum(nd), np.array(drafts, np.int32), np.stack(rows),
                                        np.array(tgt), np.array(bonus), np.zeros(B), np.zeros(B, np.int32),
                                        np.ones(B), None, 0, K)
        for b in range(B):
            emitted = [t for t in out[b].tolist() if t >= 0]
            assert len(emitted) == acc[b] + 1
            seqs[b] += emitted
    for b in range(B):
        assert seqs[b][:L] == want[b][:L]


def _one_request(l_rows, drafts, T, k, p, u, seed):
    n = len(drafts)
    return osm.rejection_sample(np.array([n]), np.array(drafts, np.int32), np.stack(l_rows),
                                np.arange(n), np.array([n]), np.array([T]), np.array([k]),
                                np.array([p]), np.array(u, np.float64), seed, max(n, 1))


@pytest.mark.parametrize("T,k,p,xk", [(1.0, 0, 1.0, 0), (0.7, 4, 1.0, 1), (1.3, 0, 0.8, 0),
                                      (0.9, 5, 0.7, 2), (1.0, 3, 0.9, -1)])
def test_emitted_token_follows_filtered_target(T, k, p, xk):
    """One draft token x (a kept token, or a dropped one when xk = -1): the
    first emitted token is distributed as p_f whatever x is (lossless)."""
    rng = np.random.default_rng(11)
    V = 8
    l = rng.normal(0, 1.5, V).astype(np.float32)
    pf = osm.filtered_probs(l, T, k, p)
    kept = osm.kept_prefix(l, T, k, p)
    if xk >= 0:
        x = int(kept[min(xk, len(kept) - 1)])
    else:
        dropped = [v for v in range(V) if pf[v] == 0]
        assert dropped
        x = dropped[0]
    trials = 6000
    us = rng.random(trials)
    counts = np.zeros(V)
    for s in range(trials):
        out, _ = _one_request([l, l], [x], T, k, p, [us[s]], seed=1000 + s)
        counts[out[0, 0]] += 1
    assert np.all(counts[pf == 0] == 0)
    sup = pf > 0
    assert stats.chisquare(counts[sup], pf[sup] * trials).pvalue > 1e-4


def test_bonus_token_follows_filtered_target():
    rng = np.random.default_rng(12)
    V = 9
    l = rng.normal(0, 1.0, V).astype(np.float32)
    T, k, p = 0.8, 6, 0.85
    pf = osm.filtered_probs(l, T, k, p)
    trials = 5000
    counts = np.zeros(V)
    for s in range(trials):
        out, acc = _one_request([l], [], T, k, p, [], seed=77 + 13 * s)
        assert acc[0] == 0
        counts[out[0, 0]] += 1
    sup = pf > 0
    assert np.all(counts[~sup] == 0)
    assert stats.chisquare(counts[sup], pf[sup] * trials).pvalue > 1e-4


def test_acceptance_boundary_is_inclusive():
    l = np.array([0.0, np.log(3.0)], np.float32)
    pf = osm.filtered_probs(l, 1.0, 0, 1.0)
    out, acc = _one_request([l, l], [0], 1.0, 0, 1.0, [pf[0]], seed=5)
    assert acc[0] == 1 and out[0, 0] == 0
    out, acc = _one_request([l, l], [0], 1.0, 0, 1.0, [np.nextafter(pf[0], 1.0)], seed=5)
    assert acc[0] == 0 and out[0, 0] == 1


def test_chain_agrees_with_the_tree_sampler():
    """Without filters, a chain verified by the flat sampler and by the tree
    sampler (same uniforms and Philox stream) emits the same tokens."""
    rng = np.random.default_rng(21)
    V, n, T = 30, 4, 0.9
    for trial in range(30):
        logits = rng.normal(0, 1.0, (n + 1, V)).astype(np.float32)
        drafts = [int(np.argmax(logits[j])) if rng.random() < 0.7 else int(rng.integers(0, V))
                  for j in range(n)]
        u = rng.random(n)
        out, acc = _one_request(list(logits), drafts, T, 0, 1.0, u, seed=trial)
        tree = {"tokens": np.array([[0] + drafts], np.int32),
                "parent": np.array([[-1] + list(range(n))], np.int32),
                "num_nodes": np.array([n], np.int32)}
        au = np.zeros((1, n + 1, 1))
        au[0, :n, 0] = u
        o2, a2, _ = ov.verify_stochastic(tree, logits[None], n, T, au, trial)
        assert acc[0] == a2[0]
        assert out[0].tolist() == o2[0].tolist()
