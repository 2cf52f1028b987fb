"""Verification of a draft tree against target logits (TEST INFRASTRUCTURE).

Greedy acceptance follows the on-device rejection sampler of the vLLM Neuron
design page ("Rejection Sampling", "On-Device Rejection Sampler"): a draft is
accepted while it equals the target's argmax; at the first mismatch the
target's token is emitted, and if every draft is accepted a bonus token from
the last position is appended; rejected positions are -1.  On a tree the walk
moves from the root to the child whose token equals the current node's argmax
(siblings carry distinct tokens).  The correction and the bonus are both the
argmax at the last accepted node.

Stochastic acceptance follows the page's CPU rejection sampler ("CPU Rejection
Sampler", after arXiv:2211.17192): a random request accepts a draft token x
iff u <= p_target(x) / draft_prob with draft_prob = 1, and a rejected position
emits a token drawn by the Gumbel-max trick from the target distribution with
the tested draft token zeroed; the bonus token comes from the target
distribution at the last position.  On a tree the children of the current node
are tested in node order as successive point-mass proposals: with Z = 1, child
c_i is accepted iff u[b, cur, i] <= p(c_i) / Z, else Z -= p(c_i).  If every
child is rejected (or there is none) the emitted token is
argmax over v not a child of cur of l_v / T - log(-log U(seed, b, cur, v)).
The emitted token is therefore distributed exactly as p = softmax(l_cur / T).

Noise: U comes from Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC'11) with key (seed low 32 bits, seed
high 32 bits) and counter (v >> 2, node, b, 0); word v & 3 of the output block
x gives U = ((x >> 8) + 0.5) * 2**-24.

Pinned by tests/test_oracle_verify.py: the published Philox4x32-10 known-answer
vectors (tests/golden/philox4x32_10_kat.txt); a six-step chain formulation of
the on-device sampler; bit-exact equality with plain greedy decoding over many
speculation steps of a synthetic target; chi-square tests of the emitted
distribution on tiny vocabularies; the closed-form acceptance law of planted
logits; the boundary u == p/Z.
"""

from __future__ import annotations

import numpy as np

_MASK = np.uint64(0xFFFFFFFF)
_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x32 rounds on uint32 values held in uint64 arrays.  Each
    round multiplies words 0 and 2 by the two round constants, swaps and
    mixes the high halves with words 1 and 3 and the key; the key is bumped by
    the two Weyl constants between rounds."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3)]
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK
    for _ in range(10):
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
        k0 = (k0 + _W0) & _MASK
        k1 = (k1 + _W1) & _MASK
    return c


def uniforms(seed: int, b: int, node: int, v) -> np.ndarray:
    """U(seed, b, node, v) in (0, 1), float64, for an array of vocab ids v."""
    v = np.asarray(v, dtype=np.uint64)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    out = philox4x32_10(v >> np.uint64(2), node, b, 0, seed & 0xFFFFFFFF, seed >> 32)
    word = (v & np.uint64(3)).astype(np.int64)
    x = np.choose(word, out)
    return ((x >> np.uint64(8)).astype(np.float64) + 0.5) * 2.0 ** -24


def children(tree, b: int, n: int):
    """Children of node n, in node order."""
    nn = int(tree["num_nodes"][b])
    return [c for c in range(1, nn + 1) if tree["parent"][b, c] == n]


def _emit(tree, b, path, last_token, D):
    out = np.full(D + 1, -1, np.int32)
    nodes = np.full(D, -1, np.int32)
    for j, c in enumerate(path):
        out[j] = tree["tokens"][b, c]
        nodes[j] = c
    out[len(path)] = last_token
    return out, nodes


def verify_greedy(tree, target_logits, depth: int):
    """Greedy longest-accepted-path.  Returns (out_tokens [B, D+1] -1 padded,
    accepted_len [B], accepted_nodes [B, D] -1 padded)."""
    B = target_logits.shape[0]
    outs, lens, nodes = [], [], []
    for b in range(B):
        cur, path = 0, []
        while True:
            t = int(np.argmax(target_logits[b, cur]))
            nxt = [c for c in children(tree, b, cur) if tree["tokens"][b, c] == t]
            if not nxt:
                break
            cur = nxt[0]
            path.append(cur)
        o, n = _emit(tree, b, path, t, depth)
        outs.append(o)
        lens.append(len(path))
        nodes.append(n)
    return np.stack(outs), np.array(lens, np.int32), np.stack(nodes)


def node_probs(logits_row, temperature: float) -> np.ndarray:
    z = np.asarray(logits_row, dtype=np.float64) / float(temperature)
    z -= z.max()
    e = np.exp(z)
    return e / e.sum()


def gumbel_pick(logits_row, temperature, seed, b, node, exclude) -> int:
    """argmax over v not in ``exclude`` of l_v / T - log(-log U), first
    index on ties."""
    V = logits_row.shape[0]
    v = np.arange(V)
    u = uniforms(seed, b, node, v)
    score = np.asarray(logits_row, dtype=np.float64) / float(temperature) - np.log(-np.log(u))
    if len(exclude):
        score[np.asarray(exclude, dtype=np.int64)] = -np.inf
    return int(np.argmax(score))


def verify_stochastic(tree, target_logits, depth: int, temperature: float, accept_u, seed: int):
    """Recursive point-mass rejection sampling on the tree (see module doc)."""
    B = target_logits.shape[0]
    outs, lens, nodes = [], [], []
    for b in range(B):
        cur, path = 0, []
        while True:
            ch = children(tree, b, cur)
            p = node_probs(target_logits[b, cur], temperature)
            z = 1.0
            acc = None
            for i, c in enumerate(ch):
                pc = p[tree["tokens"][b, c]]
                if float(accept_u[b, cur, i]) <= pc / z:
                    acc = c
                    break
                z -= pc
            if acc is None:
                t = gumbel_pick(target_logits[b, cur], temperature, seed, b, cur,
                                [tree["tokens"][b, c] for c in ch])
                break
            cur = acc
            path.append(cur)
        o, n = _emit(tree, b, path, t, depth)
        outs.append(o)
        lens.append(len(path))
        nodes.append(n)
    return np.stack(outs), np.array(lens, np.int32), np.stack(nodes)
