"""Rejection sampling of variable-length chain batches with per-request
sampling parameters (TEST INFRASTRUCTURE).

Follows the vLLM Neuron design page, "Rejection Sampling" (the CPU rejection
sampler: mixed greedy / random batches, draft_prob = 1, recovered tokens by
the Gumbel-max trick with the draft token zeroed, bonus token from the target
distribution, per-request temperature, top-k and top-p) and
"SpecDecodeMetadata: Index Bookkeeping" (the flat layout of draft positions
and logits rows).

Flat layout: request r has n_r = num_draft_tokens[r] drafts; its drafts occupy
entries [cu_r - n_r, cu_r) of draft_token_ids (cu = cu_num_draft_tokens), its
draft j is verified against logits row target_logits_indices[cu_r - n_r + j]
and its bonus position is row bonus_logits_indices[r].

Readings taken where the page is silent:
* a request is greedy iff its temperature is 0; greedy ignores top-k/top-p
  (neither can remove the argmax) and takes the first index on ties;
* a random request samples from its filtered distribution p_f: with
  z = l / T in float64 and the tokens ordered by (l desc, id asc), top-k keeps
  the first k tokens (k <= 0 or k >= V: all), then top-p keeps the shortest
  prefix of those whose mass, renormalised over the top-k set, reaches p (the
  token that crosses p is kept; p >= 1: all), and p_f renormalises
  exp(z) over the kept prefix;
* draft j is accepted iff u_j <= p_f(x_j); at the first rejection the
  recovered token is argmax over kept v != x_j of z_v - log(-log U), which
  samples max(p_f - delta_x, 0) renormalised; after n_r acceptances the bonus
  is argmax over kept v of z_v - log(-log U) at the bonus row;
* U = U(seed, r, j, v) is the Philox4x32-10 stream of the tree verifier with
  (node, sequence) = (draft position j, request r), j = n_r at the bonus row;
  on a chain this is the tree verifier's stream exactly.

Pinned by tests/test_oracle_sampling.py: the page's printed metadata example
(tests/golden/spec_decode_metadata_example.txt); top-p against a brute-force
search over every subset of a tiny vocabulary for the smallest set whose mass
reaches p; top-k against a sort; temperature against scipy's softmax; greedy
rows against plain greedy decoding; the emitted token's distribution against
p_f by chi-square (lossless sampling), also through the filters.
"""

from __future__ import annotations

import numpy as np

from .verify import uniforms


def spec_decode_metadata(cu_num_scheduled_tokens, num_draft_tokens):
    """Index bookkeeping of a flat batch: every request has logits at its
    last n_r + 1 scheduled positions (its drafts, then the bonus position).
    Returns (cu_num_draft_tokens, logits_indices, target_logits_indices,
    bonus_logits_indices) as int32 arrays."""
    cu_s = np.asarray(cu_num_scheduled_tokens, dtype=np.int64)
    nd = np.asarray(num_draft_tokens, dtype=np.int64)
    li, tgt, bonus = [], [], []
    for r in range(len(nd)):
        first = cu_s[r] - (nd[r] + 1)
        for j in range(nd[r] + 1):
            if j < nd[r]:
                tgt.append(len(li))
            else:
                bonus.append(len(li))
            li.append(first + j)
    cu_d = np.cumsum(nd)
    return (cu_d.astype(np.int32), np.array(li, np.int32), np.array(tgt, np.int32),
            np.array(bonus, np.int32))


def sampling_order(logits_row) -> np.ndarray:
    """Token ids in the order (logit desc, id asc)."""
    l = np.asarray(logits_row, dtype=np.float64)
    ids = np.arange(l.shape[0])
    return np.lexsort((ids, -l))


def kept_prefix(logits_row, temperature: float, top_k: int, top_p: float) -> np.ndarray:
    """Ids kept by top-k then top-p, in sampling order (see module doc)."""
    order = sampling_order(logits_row)
    V = order.shape[0]
    if 0 < top_k < V:
        order = order[:top_k]
    if top_p < 1.0:
        z = np.asarray(logits_row, dtype=np.float64)[order] / float(temperature)
        e = np.exp(z - z.max())
        target = float(top_p) * e.sum()
        cum = 0.0
        m = len(order)
        for i in range(len(order)):
            cum += e[i]
            if cum >= target:
                m = i + 1
                break
        order = order[:m]
    return order


def filtered_probs(logits_row, temperature: float, top_k: int, top_p: float) -> np.ndarray:
    """p_f over the whole vocabulary (zero outside the kept set), float64."""
    V = len(logits_row)
    kept = kept_prefix(logits_row, temperature, top_k, top_p)
    z = np.asarray(logits_row, dtype=np.float64)[kept] / float(temperature)
    e = np.exp(z - z.max())
    p = np.zeros(V)
    p[kept] = e / e.sum()
    return p


def _gumbel_pick(logits_row, temperature, seed, r, j, kept, exclude):
    z = np.asarray(logits_row, dtype=np.float64) / float(temperature)
    score = np.full(z.shape[0], -np.inf)
    score[kept] = z[kept] - np.log(-np.log(uniforms(seed, r, j, kept)))
    if exclude is not None:
        score[exclude] = -np.inf
    return int(np.argmax(score))


def rejection_sample(cu_num_draft_tokens, draft_token_ids, logits, target_logits_indices,
                     bonus_logits_indices, temperature, top_k, top_p, uniform, seed: int,
                     max_spec_len: int):
    """The CPU rejection sampler on a flat batch.  Returns
    (out_tokens [B, max_spec_len + 1] -1 padded, num_accepted [B])."""
    cu = np.asarray(cu_num_draft_tokens, dtype=np.int64)
    B = cu.shape[0]
    out = np.full((B, max_spec_len + 1), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for r in range(B):
        start = 0 if r == 0 else int(cu[r - 1])
        n = int(cu[r]) - start
        T = float(temperature[r])
        greedy = T == 0.0
        emitted = None
        for j in range(n):
            x = int(draft_token_ids[start + j])
            row = logits[int(target_logits_indices[start + j])]
            if greedy:
                t = int(np.argmax(row))
                if x == t:
                    out[r, j] = x
                    continue
                emitted = (j, t)
                break
            p = filtered_probs(row, T, int(top_k[r]), float(top_p[r]))
            if float(uniform[start + j]) <= p[x]:
                out[r, j] = x
                continue
            kept = kept_prefix(row, T, int(top_k[r]), float(top_p[r]))
            emitted = (j, _gumbel_pick(row, T, seed, r, j, kept, x))
            break
        if emitted is None:
            row = logits[int(bonus_logits_indices[r])]
            if greedy:
                emitted = (n, int(np.argmax(row)))
            else:
                kept = kept_prefix(row, T, int(top_k[r]), float(top_p[r]))
                emitted = (n, _gumbel_pick(row, T, seed, r, n, kept, None))
        j, t = emitted
        out[r, j] = t
        acc[r] = j
    return out, acc


def decision_margins(cu_num_draft_tokens, draft_token_ids, logits, target_logits_indices,
                     bonus_logits_indices, temperature, top_k, top_p, uniform, seed: int):
    """Smallest distances to a decision boundary over the rows the sampler
    visits (for choosing test inputs whose decisions are not knife-edge):
    |u - p_f(x)| of each random acceptance test, the relative gap of the
    top-p mass to its target on both sides of the cut, and the gap between
    the best and second-best Gumbel scores of each random final pick."""
    cu = np.asarray(cu_num_draft_tokens, dtype=np.int64)
    m_u, m_p, m_g = np.inf, np.inf, np.inf
    for r in range(cu.shape[0]):
        start = 0 if r == 0 else int(cu[r - 1])
        n = int(cu[r]) - start
        T = float(temperature[r])
        if T == 0.0:
            continue
        k, pp = int(top_k[r]), float(top_p[r])
        for j in range(n + 1):
            rid = int(target_logits_indices[start + j]) if j < n else int(bonus_logits_indices[r])
            row = logits[rid]
            if pp < 1.0:
                order = sampling_order(row)
                if 0 < k < len(order):
                    order = order[:k]
                z = np.asarray(row, np.float64)[order] / T
                e = np.exp(z - z.max())
                cum = np.cumsum(e) / e.sum()
                m_p = min(m_p, float(np.min(np.abs(cum - pp))))
            x = int(draft_token_ids[start + j]) if j < n else None
            if x is not None:
                d = float(uniform[start + j]) - filtered_probs(row, T, k, pp)[x]
                m_u = min(m_u, abs(d))
                if d <= 0:
                    continue
            kept = kept_prefix(row, T, k, pp)
            z = np.asarray(row, np.float64) / T
            sc = z[kept] - np.log(-np.log(uniforms(seed, r, j, kept)))
            if x is not None:
                sc = np.where(kept == x, -np.inf, sc)
            s = np.sort(sc[np.isfinite(sc)])
            if len(s) >= 2:
                m_g = min(m_g, float(s[-1] - s[-2]))
            break
    return m_u, m_p, m_g
