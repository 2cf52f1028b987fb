"""Pins of the oracle's verification step (CPU only).

Each test fixes the oracle against something other than itself: published
known-answer vectors, an independent formulation of the vLLM Neuron page's
six-step on-device sampler, plain greedy decoding of a synthetic target, and
closed-form distributions (chi-square / binomial)."""

import os
import zlib

import numpy as np
import pytest
from scipy import stats

from conftest import GOLDEN
from oracle import verify as ov
from oracle.tree import build_tree_core
from synth import gen


# ---------------------------------------------------------------- Philox KAT
def test_philox_known_answers():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x, 16) for x in line.split()])
    assert len(rows) == 3
    for r in rows:
        out = ov.philox4x32_10(*r[:6])
        assert [int(x) for x in out] == r[6:]


def test_uniforms_in_open_interval_and_word_selection():
    v = np.arange(64)
    u = ov.uniforms(12345, 3, 7, v)
    assert np.all(u > 0) and np.all(u < 1)
    # v and v+1 inside one block use different words of the same block
    blk = ov.philox4x32_10(np.uint64(5), 7, 3, 0, 12345, 0)
    for w in range(4):
        x = int(blk[w])
        assert ov.uniforms(12345, 3, 7, [20 + w])[0] == ((x >> 8) + 0.5) * 2.0 ** -24


# ------------------------------------------------- P2: chain six-step sampler
def six_step_chain(draft_tokens, target_argmax):
    """Independent formulation of the page's on-device greedy sampler:
    bonus tokens, reshape to [B, K], match mask, first mismatch via argmax on
    the inverted mask with a sentinel column, accept up to and including the
    mismatch, bonus when all matched; -1 elsewhere."""
    B, K = draft_tokens.shape
    targets = target_argmax[:, :K]
    bonus = target_argmax[:, K]
    match = draft_tokens == targets
    inv = np.concatenate([~match, np.ones((B, 1), bool)], axis=1)
    first = np.argmax(inv, axis=1)  # sentinel at K when all matched
    out = np.full((B, K + 1), -1, np.int64)
    for b in range(B):
        out[b, : first[b]] = draft_tokens[b, : first[b]]
        out[b, first[b]] = targets[b, first[b]] if first[b] < K else bonus[b]
    return out, first


@pytest.mark.parametrize("seed", range(6))
def test_chain_greedy_matches_six_step_sampler(seed):
    rng = np.random.default_rng(seed)
    B, K, V = 16, 5, 11
    drafts = rng.integers(0, V, size=(B, K))
    logits = rng.normal(0, 2, size=(B, K + 1, V)).astype(np.float32)
    # plant agreements so that all accepted lengths occur
    for b in range(B):
        a = b % (K + 1)
        for i in range(a):
            row = logits[b, i]
            j = int(np.argmax(row))
            row[j], row[drafts[b, i]] = row[drafts[b, i]], row[j]
    tree = {
        "tokens": np.concatenate([np.zeros((B, 1), np.int64), drafts], axis=1),
        "parent": np.tile(np.arange(-1, K), (B, 1)),
        "num_nodes": np.full(B, K),
    }
    out, alen, anodes = ov.verify_greedy(tree, logits, K)
    ref, first = six_step_chain(drafts, logits.argmax(-1))
    np.testing.assert_array_equal(out, ref)
    np.testing.assert_array_equal(alen, first)
    for b in range(B):
        np.testing.assert_array_equal(anodes[b, : alen[b]], np.arange(1, alen[b] + 1))


# ------------------------------- P1: speculation == plain greedy decoding
V1 = 12


def _target(prefix):
    """Deterministic synthetic target: logits seeded by the prefix; with
    probability 0.7 the argmax is the successor rule (3*last + 1) mod V."""
    rng = np.random.default_rng(zlib.crc32(np.asarray(prefix, np.int64).tobytes()))
    z = rng.normal(0, 2, V1).astype(np.float32)
    if rng.random() < 0.7:
        t = (3 * prefix[-1] + 1) % V1
        j = int(np.argmax(z))
        z[j], z[t] = z[t], z[j]
    return z


def _toy_draft_pass(root_token):
    def fn(d, rows):
        res = []
        for r in rows:
            last = r["token"] if d == 1 else r["path"][-1]
            rng = np.random.default_rng(zlib.crc32(np.asarray((root_token,) + r["path"], np.int64).tobytes()) + 7)
            z = rng.normal(0, 1, V1)
            z[(3 * last + 1) % V1] += 2.5  # the draft mostly knows the rule
            order = np.argsort(-z, kind="stable")[: r_k[0]]
            lse = np.log(np.sum(np.exp(z - z.max()))) + z.max()
            res.append((order.astype(np.int64), (z[order] - lse).astype(np.float32)))
        return res
    return fn


r_k = [3]


@pytest.mark.parametrize("k,D,N", [(1, 4, 4), (3, 3, 8), (2, 4, 9)])
def test_greedy_speculation_bit_identical_to_greedy_decoding(k, D, N):
    r_k[0] = k
    cfg = dict(top_k=k, depth=D, total_tokens=N, kv_capacity=10**6)
    L = 80
    plain = [5]
    while len(plain) < L:
        plain.append(int(np.argmax(_target(plain))))
    spec = [5]
    accepted = []
    while len(spec) < L:
        tree = build_tree_core(cfg, 1, 1, np.array([0]), np.array([[spec[-1]]]), _toy_draft_pass(spec[-1]))
        n1 = N + 1
        logits = np.zeros((1, n1, V1), np.float32)
        for n in range(n1):
            if n > tree["num_nodes"][0]:
                continue
            path, c = [], n
            while c > 0:
                path.append(int(tree["tokens"][0, c]))
                c = int(tree["parent"][0, c])
            logits[0, n] = _target(spec + path[::-1])
        out, alen, _ = ov.verify_greedy(tree, logits, D)
        emitted = [int(t) for t in out[0] if t >= 0]
        assert len(emitted) == alen[0] + 1
        accepted.append(alen[0])
        spec += emitted
    assert spec[:L] == plain
    assert np.mean(accepted) > 0.5  # the check is not vacuous


# --------------------------------- P3: stochastic verify keeps p_target exact
def _chain_or_tree(V, k, D, seed):
    rng = np.random.default_rng(seed)
    tokens, parent = [int(rng.integers(V))], [-1]
    frontier = [0]
    depth = {0: 0}
    while frontier:
        nxt = []
        for p in frontier:
            if depth[p] >= D:
                continue
            for t in rng.choice(V, size=k, replace=False):
                tokens.append(int(t))
                parent.append(p)
                depth[len(tokens) - 1] = depth[p] + 1
                nxt.append(len(tokens) - 1)
            if len(tokens) > 12:
                break
        frontier = nxt if len(tokens) <= 12 else []
    n = len(tokens) - 1
    return n, np.array(tokens), np.array(parent)


@pytest.mark.parametrize("V,k,D,T", [(5, 1, 3, 1.0), (8, 2, 2, 0.7), (16, 3, 2, 1.3), (8, 0, 0, 1.0)])
def test_stochastic_first_token_follows_target(V, k, D, T):
    n, toks, par = _chain_or_tree(V, k, D, 11 + V + k)
    draws = 12000
    rng = np.random.default_rng(V * 100 + k)
    logits_one = rng.normal(0, 1.5, size=(n + 1, V)).astype(np.float32)
    # make the drafted children likely so acceptance paths are exercised
    for c in range(1, n + 1):
        logits_one[par[c], toks[c]] += 1.0
    tree = {"tokens": np.tile(toks, (draws, 1)), "parent": np.tile(par, (draws, 1)),
            "num_nodes": np.full(draws, n)}
    logits = np.broadcast_to(logits_one, (draws, n + 1, V))
    u = rng.random(size=(draws, n + 1, max(k, 1))).astype(np.float32)
    out, alen, anodes = ov.verify_stochastic(tree, logits, max(D, 1), T, u, seed=4242)
    p0 = ov.node_probs(logits_one[0], T)
    counts = np.bincount(out[:, 0], minlength=V)
    chi = stats.chisquare(counts, p0 * draws)
    assert chi.pvalue > 1e-4, (counts, p0 * draws)
    if k:
        # given the first child accepted, the second token follows p_child
        c1 = [c for c in range(1, n + 1) if par[c] == 0][0]
        sel = anodes[:, 0] == c1
        pc = ov.node_probs(logits_one[c1], T)
        cnt = np.bincount(out[sel, 1], minlength=V)
        keep = pc * sel.sum() > 5
        exp = pc[keep] * sel.sum()
        obs = cnt[keep]
        exp = exp * obs.sum() / exp.sum()
        assert stats.chisquare(obs, exp).pvalue > 1e-4
        # closed form: P(accepted >= 1) = sum of the root children's probs
        kids = [toks[c] for c in range(1, n + 1) if par[c] == 0]
        pa = p0[kids].sum()
        z = (np.mean(alen >= 1) - pa) / np.sqrt(pa * (1 - pa) / draws)
        assert abs(z) < 4.5


def test_accept_on_equality_boundary():
    # V = 2 with equal logits: p = 0.5 exactly; u == p/Z accepts, the next float rejects
    tree = {"tokens": np.array([[0, 1]]), "parent": np.array([[-1, 0]]), "num_nodes": np.array([1])}
    logits = np.zeros((1, 2, 2), np.float32)
    u = np.array([[[0.5], [0.0]]], np.float32)
    _, alen, _ = ov.verify_stochastic(tree, logits, 1, 1.0, u, seed=1)
    assert alen[0] == 1
    u[0, 0, 0] = np.nextafter(np.float32(0.5), np.float32(1))
    out, alen, _ = ov.verify_stochastic(tree, logits, 1, 1.0, u, seed=1)
    assert alen[0] == 0 and out[0, 0] == 0  # the only non-child token


def test_leaf_bonus_is_argmax_or_full_sample():
    tree = {"tokens": np.array([[3]]), "parent": np.array([[-1]]), "num_nodes": np.array([0])}
    logits = np.array([[[0.1, 2.0, -1.0, 0.5]]], np.float32)
    out, alen, nodes = ov.verify_greedy(tree, logits, 2)
    assert out.tolist() == [[1, -1, -1]] and alen[0] == 0 and nodes.tolist() == [[-1, -1]]


# --------------------------- P4: planted acceptance law on the chain workload
def test_planted_acceptance_law_chain():
    K, V, trials = 3, 4096, 600
    cfg = dict(total_tokens=K, vocab=V, plant_p=0.7)
    rng = np.random.default_rng(3)
    toks = np.concatenate([[7], rng.choice(V, size=K, replace=False)])
    tree = {"tokens": toks[None, :], "parent": np.arange(-1, K)[None, :], "num_nodes": np.array([K])}
    lens = []
    for s in range(trials):
        logits = gen.plant_target_logits(cfg, tree, seed=50_000 + s)
        _, alen, _ = ov.verify_greedy(tree, logits, K)
        lens.append(int(alen[0]))
    lens = np.array(lens)
    p = np.array([0.7 ** i * 0.3 for i in range(K)] + [0.7 ** K])
    obs = np.bincount(lens, minlength=K + 1)
    assert stats.chisquare(obs, p * trials).pvalue > 1e-4
    emitted = lens + 1
    mean = sum(0.7 ** i for i in range(K + 1))  # 2.533 for K = 3
    assert abs(emitted.mean() - mean) < 4 * emitted.std() / np.sqrt(trials)


# ---------------------------- P8: worked example of the metadata bookkeeping
def test_spec_decode_metadata_example_is_consistent():
    vals = {}
    with open(os.path.join(GOLDEN, "spec_decode_metadata_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, *nums = line.split()
                vals[name] = [int(x) for x in nums]
    cu = np.array(vals["cu_num_scheduled_tokens"])
    nd = np.array(vals["num_draft_tokens"])
    assert np.cumsum(nd).tolist() == vals["cu_num_draft_tokens"]
    # logits at the last (drafts + 1) positions of every request
    li, tgt, bonus = [], [], []
    for r in range(len(cu)):
        for j in range(nd[r] + 1):
            pos = cu[r] - (nd[r] + 1) + j
            (tgt if j < nd[r] else bonus).append(len(li))
            li.append(int(pos))
    assert li == vals["logits_indices"]
    assert tgt == vals["target_logits_indices"]
    assert bonus == vals["bonus_logits_indices"]
