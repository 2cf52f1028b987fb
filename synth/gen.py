"""Seeded synthetic inputs for the speculation step.

This module is shared by the oracle-side tests and the HIP-side tests and
bench.  It draws random numbers and shapes them into inputs; it holds none of
the method's arithmetic.  Every tensor comes from its own generator seeded by
``(seed, tag)``, so any one input can be regenerated on its own.

Recipe (the readings taken where the workload text is silent):
  * matrices and embeddings ~ N(0, 0.02) (0.02 is the standard deviation);
    RMSNorm gains are 1;
  * aux hidden states and the context K/V ~ N(0, 1), written into slots
    [0, ctx) of each sequence; context keys count as already rotated;
  * root tokens uniform over the target vocabulary;
  * the trimmed-vocabulary map is a seeded random subset of the target ids,
    sorted ascending;
  * target logits ~ N(0, 2) per tree node; at each node that has a drafted
    child, with probability ``plant_p`` the value at the current argmax and
    the value of the node's first child token are swapped, so that token
    becomes the argmax and the multiset of values is unchanged;
  * acceptance uniforms ~ U(0, 1) of shape [B, N+1, top_k].

bf16 workloads store every floating input as float32 arrays whose values are
exactly representable in bfloat16 (round to nearest even of the draw).
"""

from __future__ import annotations

import zlib

import numpy as np

WEIGHT_STD = 0.02


def _rng(seed: int, tag: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), zlib.crc32(tag.encode())])


def round_bf16_inplace(a: np.ndarray) -> np.ndarray:
    """Round a float32 array to bfloat16 values (nearest even), in place."""
    assert a.dtype == np.float32 and a.flags.c_contiguous
    u = a.reshape(-1).view(np.uint32)
    step = 1 << 24
    for i in range(0, u.size, step):
        c = u[i:i + step]
        c += np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1))
        c &= np.uint32(0xFFFF0000)
    return a


# Tensors of at least this many values may be drawn in independently seeded
# chunks on several threads (their values then differ from one sequential
# draw, but are as deterministic).
_PAR_MIN = 1 << 26
_PAR_CHUNK = 1 << 24


def _normal(seed, tag, shape, std, dtype, parallel=False):
    n = int(np.prod(shape))
    if parallel and n >= _PAR_MIN:
        import concurrent.futures as cf
        import os

        a = np.empty(n, dtype=np.float32)

        def fill(i):
            c = a[i * _PAR_CHUNK:(i + 1) * _PAR_CHUNK]
            np.random.default_rng([int(seed), zlib.crc32(tag.encode()), 0x5EED, i]).standard_normal(
                size=c.shape[0], dtype=np.float32, out=c)
            if std != 1.0:
                c *= np.float32(std)
            if dtype == "bf16":
                round_bf16_inplace(c)

        with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range((n + _PAR_CHUNK - 1) // _PAR_CHUNK)))
        return a.reshape(shape)
    a = _rng(seed, tag).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == "bf16":
        round_bf16_inplace(a)
    return a


def qkv_rows(cfg: dict) -> int:
    return (cfg["n_q_heads"] + 2 * cfg["n_kv_heads"]) * cfg["head_dim"]


def weight_shapes(cfg: dict) -> dict:
    H, I = cfg["hidden"], cfg["intermediate"]
    V, Vd = cfg["vocab"], cfg["draft_vocab"]
    nqd = cfg["n_q_heads"] * cfg["head_dim"]
    shapes = {
        "fc": (H, 3 * H),
        "embed": (V, H),
        "wqkv": (qkv_rows(cfg), 2 * H),
        "wo": (H, nqd),
        "w_gate_up": (2 * I, H),
        "w_down": (H, I),
        "lm_head": (V if cfg["cand_rank"] else Vd, H),
    }
    if cfg["cand_rank"]:
        r = cfg["cand_rank"]
        shapes["cand_down"] = (r, H)
        shapes["cand_up"] = (V, r)
    return shapes


def make_weights(cfg: dict, seed: int) -> dict:
    """Draft weights as float32 arrays (bf16-valued for bf16 workloads)."""
    dt = cfg["dtype"]
    w = {}
    for name, shape in weight_shapes(cfg).items():
        w[name] = _normal(seed, "w/" + name, shape, WEIGHT_STD, dt, parallel=True)
    H = cfg["hidden"]
    for name in ("input_norm", "hidden_norm", "post_attn_norm", "final_norm"):
        w[name] = np.ones(H, dtype=np.float32)
    if cfg.get("fc_norm"):
        w["fc_norm"] = np.ones(H, dtype=np.float32)
    w["d2t"] = make_d2t(cfg, seed)
    return w


def make_d2t(cfg: dict, seed: int):
    """Draft id -> target id for a trimmed draft vocabulary, else None."""
    V, Vd = cfg["vocab"], cfg["draft_vocab"]
    if Vd == V or cfg["cand_rank"]:
        return None
    ids = _rng(seed, "d2t").choice(V, size=Vd, replace=False)
    return np.sort(ids).astype(np.int32)


def make_step_inputs(cfg: dict, seed: int, ctx_len=None) -> dict:
    """Aux states, root tokens, context lengths and the draft KV cache."""
    B, n_new, H = cfg["batch"], cfg["n_new"], cfg["hidden"]
    nkv, hd, S = cfg["n_kv_heads"], cfg["head_dim"], cfg["kv_capacity"]
    dt = cfg["dtype"]
    if ctx_len is None:
        ctx_len = np.full(B, cfg["ctx"], dtype=np.int32)
    ctx_len = np.asarray(ctx_len, dtype=np.int32)
    L = int(min(cfg["ctx"], S))
    out = {
        "aux": _normal(seed, "aux", (B, n_new, 3 * H), 1.0, dt),
        "in_tokens": _rng(seed, "tokens").integers(0, cfg["vocab"], size=(B, n_new)).astype(np.int32),
        "ctx_len": ctx_len,
    }
    for name in ("k", "v"):
        cache = np.zeros((B, nkv, S, hd), dtype=np.float32)
        cache[:, :, :L, :] = _normal(seed, "kv/" + name, (B, nkv, L, hd), 1.0, dt, parallel=True)
        out[name + "_cache"] = cache
    return out


def make_target_kv(cfg: dict, seed: int, slots: int, layers: int | None = None) -> dict:
    """A target-shaped KV cache [layers, B, nkv, slots, hd] of N(0,1) values,
    used by the compaction step."""
    B, nkv, hd = cfg["batch"], cfg["n_kv_heads"], cfg["head_dim"]
    layers = cfg["target_layers"] if layers is None else layers
    shape = (layers, B, nkv, slots, hd)
    return {"k": _normal(seed, "tkv/k", shape, 1.0, cfg["dtype"]),
            "v": _normal(seed, "tkv/v", shape, 1.0, cfg["dtype"])}


def _first_child_tokens(tokens: np.ndarray, parent: np.ndarray, num_nodes: np.ndarray):
    """For every node, the token of its first child in node order (-1 if none).
    Pure indexing over the given tree arrays."""
    B, n1 = tokens.shape
    first = np.full((B, n1), -1, dtype=np.int64)
    for b in range(B):
        for c in range(int(num_nodes[b]), 0, -1):
            first[b, parent[b, c]] = tokens[b, c]
    return first


def plant_target_logits(cfg: dict, tree: dict, seed: int, std: float = 2.0) -> np.ndarray:
    """Target logits [B, N+1, V] ~ N(0, std); at each node with a drafted
    child, with probability plant_p the first child's token is made the argmax
    by swapping two values."""
    B = tree["tokens"].shape[0]
    n1 = cfg["total_tokens"] + 1
    V = cfg["vocab"]
    logits = _normal(seed, "target_logits", (B, n1, V), std, "f32")
    coin = _rng(seed, "plant").random(size=(B, n1))
    first = _first_child_tokens(tree["tokens"], tree["parent"], tree["num_nodes"])
    for b in range(B):
        for n in range(n1):
            t = first[b, n]
            if t < 0 or coin[b, n] >= cfg["plant_p"]:
                continue
            row = logits[b, n]
            a = int(np.argmax(row))
            row[a], row[t] = row[t], row[a]
    return logits


def add_noise_logits(draft_logits: np.ndarray, seed: int, std: float = 1.0) -> np.ndarray:
    """Target logits = given per-node draft logits + N(0, std) noise."""
    noise = _rng(seed, "target_noise").standard_normal(size=draft_logits.shape, dtype=np.float32)
    if std != 1.0:
        noise *= np.float32(std)
    noise += draft_logits.astype(np.float32)
    return noise


def make_accept_u(cfg: dict, seed: int, batch: int | None = None) -> np.ndarray:
    B = cfg["batch"] if batch is None else batch
    shape = (B, cfg["total_tokens"] + 1, cfg["top_k"])
    return _rng(seed, "accept_u").random(size=shape, dtype=np.float32)


def philox_seed(seed: int) -> int:
    return int(_rng(seed, "philox").integers(0, 2**63 - 1))


def random_logits(seed: int, tag: str, shape, std: float = 2.0) -> np.ndarray:
    return _normal(seed, tag, shape, std, "f32")


def random_states(seed: int, tag: str, shape, dtype: str) -> np.ndarray:
    """N(0, 1) rows in the workload's storage type (synthetic recurrent states)."""
    return _normal(seed, tag, shape, 1.0, dtype)


def random_tree(cfg: dict, seed: int, batch: int | None = None) -> dict:
    """A random valid tree in the output layout (node 0 = root; nodes in
    depth-major order so parents precede children; sibling tokens distinct).
    Used to drive the verify and compaction steps independently of drafting."""
    rng = _rng(seed, "random_tree")
    B = cfg["batch"] if batch is None else batch
    N, k, D, V = cfg["total_tokens"], cfg["top_k"], cfg["depth"], cfg["vocab"]
    n1 = N + 1
    tokens = np.full((B, n1), -1, dtype=np.int32)
    parent = np.full((B, n1), -1, dtype=np.int32)
    depth = np.zeros((B, n1), dtype=np.int32)
    num_nodes = np.zeros(B, dtype=np.int32)
    for b in range(B):
        tokens[b, 0] = rng.integers(0, V)
        nodes = 1
        frontier = [0]
        while nodes <= N and frontier:
            nxt = []
            for p in frontier:
                if depth[b, p] >= D:
                    continue
                nch = int(rng.integers(0, k + 1)) if p else max(1, int(rng.integers(0, k + 1)))
                toks = rng.choice(V, size=min(nch, N + 1 - nodes), replace=False)
                for t in toks:
                    tokens[b, nodes] = t
                    parent[b, nodes] = p
                    depth[b, nodes] = depth[b, p] + 1
                    nxt.append(nodes)
                    nodes += 1
                if nodes > N:
                    break
            frontier = nxt
        num_nodes[b] = nodes - 1
    return {"tokens": tokens, "parent": parent, "depth": depth, "num_nodes": num_nodes}


def flat_batch(seed: int, B: int, max_spec_len: int, V: int, *, plant=(6.0, 14.0), p_right=0.8,
               greedy_frac=0.25, ties=False, crowded=False) -> dict:
    """A flat batch of variable-length draft chains with per-request sampling
    parameters.  Draft counts are uniform in [0, max_spec_len]; request r
    schedules 1 + its drafts + a random number of earlier tokens, so
    ``cu_num_scheduled_tokens`` is increasing.  The logits rows (one per draft
    and one bonus row per request, in request order) are N(0, 2) with one
    planted token per row raised by U(plant) (integer-valued draws from
    [-4, 4] when ``ties``; U(1, 1.1) when ``crowded``, so that almost every
    logit shares its sign, exponent and leading mantissa bits); the draft at a row is the planted token with
    probability ``p_right``, else a uniform id.  A fraction of the requests is
    greedy (temperature 0); the others draw T from [0.3, 1.5], top-k from
    {0, 1, 5, 50, 1000} and top-p from {1.0, 0.5, 0.9, 0.97}.  Uniforms ~ U(0, 1)."""
    rng = _rng(seed, "flat_batch")
    nd = rng.integers(0, max_spec_len + 1, B).astype(np.int32)
    sched = nd + 1 + rng.integers(0, 5, B)
    cu_sched = np.cumsum(sched).astype(np.int32)
    rows = int(nd.sum()) + B
    if ties:
        logits = rng.integers(-4, 5, (rows, V)).astype(np.float32)
    elif crowded:
        logits = rng.uniform(1.0, 1.1, (rows, V)).astype(np.float32)
    else:
        logits = _normal(seed, "flat_logits", (rows, V), 2.0, "f32")
    planted = rng.integers(0, V, rows)
    logits[np.arange(rows), planted] += rng.uniform(*plant, rows).astype(np.float32)
    drafts = []
    row = 0
    for r in range(B):
        for j in range(nd[r]):
            drafts.append(int(planted[row]) if rng.random() < p_right else int(rng.integers(0, V)))
            row += 1
        row += 1
    greedy = rng.random(B) < greedy_frac
    temp = np.where(greedy, 0.0, rng.uniform(0.3, 1.5, B)).astype(np.float32)
    top_k = rng.choice(np.array([0, 1, 5, 50, 1000], np.int32), B).astype(np.int32)
    top_p = rng.choice(np.array([1.0, 0.5, 0.9, 0.97], np.float32), B).astype(np.float32)
    u = rng.random(int(nd.sum()), dtype=np.float32)
    return {"num_draft_tokens": nd, "cu_num_scheduled_tokens": cu_sched, "logits": logits,
            "draft_token_ids": np.array(drafts, np.int32), "temperature": temp, "top_k": top_k,
            "top_p": top_p, "uniform": u, "seed": philox_seed(seed)}


def make_target_weights(cfg: dict, seed: int, layers: int) -> dict:
    """Synthetic weights of an L-layer Llama-style target with the draft's
    shapes: embed, lm_head [V, H]; per layer wqkv [(nq+2nkv)hd, H], wo, the
    SwiGLU pair and down; matrices N(0, 0.02), norm gains 1."""
    dt, H, I = cfg["dtype"], cfg["hidden"], cfg["intermediate"]
    V, nqd = cfg["vocab"], cfg["n_q_heads"] * cfg["head_dim"]
    w = {"embed": _normal(seed, "t/embed", (V, H), WEIGHT_STD, dt, parallel=True),
         "lm_head": _normal(seed, "t/lm_head", (V, H), WEIGHT_STD, dt, parallel=True),
         "final_norm": np.ones(H, dtype=np.float32), "layers": []}
    for l in range(layers):
        w["layers"].append({
            "attn_norm": np.ones(H, dtype=np.float32),
            "wqkv": _normal(seed, f"t/{l}/wqkv", (qkv_rows(cfg), H), WEIGHT_STD, dt, parallel=True),
            "wo": _normal(seed, f"t/{l}/wo", (H, nqd), WEIGHT_STD, dt, parallel=True),
            "mlp_norm": np.ones(H, dtype=np.float32),
            "w_gate_up": _normal(seed, f"t/{l}/w_gate_up", (2 * I, H), WEIGHT_STD, dt, parallel=True),
            "w_down": _normal(seed, f"t/{l}/w_down", (H, I), WEIGHT_STD, dt, parallel=True),
        })
    return w


def chain_tree(B: int, K: int, V: int, ctx_len, seed: int) -> dict:
    """A chain of K random draft tokens per sequence in the tree layout
    (node n at depth n, parent n - 1, position ctx + n, ancestors 0..n)."""
    rng = _rng(seed, "chain_tree")
    n1 = K + 1
    ctx = np.asarray(ctx_len, dtype=np.int64)
    tokens = rng.integers(0, V, size=(B, n1)).astype(np.int32)
    parent = np.tile(np.arange(-1, K, dtype=np.int32), (B, 1))
    depth = np.tile(np.arange(n1, dtype=np.int32), (B, 1))
    position = (ctx[:, None] + np.arange(n1)[None, :]).astype(np.int32)
    anc = np.array([(1 << (n + 1)) - 1 for n in range(n1)], dtype=np.uint64)
    return {"tokens": tokens, "parent": parent, "depth": depth, "position": position,
            "num_nodes": np.full(B, K, np.int32), "anc_mask": np.tile(anc, (B, 1))}


def with_positions(tree: dict, ctx_len) -> dict:
    """Fill a tree's position (ctx + depth) and ancestor mask (bit j set for
    every node j on the path from the root to the node, itself included)."""
    B, n1 = tree["tokens"].shape
    ctx = np.asarray(ctx_len, dtype=np.int64)
    pos = np.full((B, n1), -1, np.int32)
    anc = np.zeros((B, n1), np.uint64)
    for b in range(B):
        for n in range(int(tree["num_nodes"][b]) + 1):
            pos[b, n] = ctx[b] + tree["depth"][b, n]
            m, j = 0, n
            while j >= 0:
                m |= 1 << j
                j = int(tree["parent"][b, j])
            anc[b, n] = np.uint64(m)
    return dict(tree, position=pos, anc_mask=anc)
