"""Workload shapes for the speculation step.

Plain data only: the draft shapes, tree parameters and run sizes of the five
synthetic workloads.  Both the oracle and the HIP path read these tables; no
arithmetic of the method lives here.

Sources (page titles as printed on each page):
  * "Speculative Decoding (EAGLE3) in the vLLM Neuron Framework", section
    "Enabling EAGLE3 Speculative Decoding": Llama-3.1-8B target, 4 sequences,
    256-token model length, 5 speculative tokens, greedy sampling
    -> ``llama8b_chain``.
  * "Eaglet", sections "Approach 1: YAML Recipe" and "Block Efficiency (BE)
    Evaluation": Qwen3-4B, draft_top_k 8 / draft_depth 5 / total_draft_tokens
    31, trimmed vocabulary, context length 4096 -> ``qwen4b_tree``.
  * "EAGLE-3" (AMD Quark), sections "Quickstart: Python API": Qwen3-8B,
    ttt_length 7, draft_vocab_size 32000, concurrency up to 32
    -> ``qwen8b_tree``.
  * "nemo_automodel ... eagle4", class Eagle4CandidateHeadConfig (rank 128,
    num_candidates 128) and Eagle4Config.sliding_window -> ``eagle4_llama8b``.
"""

from __future__ import annotations

import copy

# Common defaults: RMSNorm eps and the RoPE base are not printed on the pages;
# 1e-6 and 10000 are the readings taken for every workload.
_BASE = dict(
    cand_rank=0,
    num_candidates=0,
    sliding_window=0,
    rope_base=10000.0,
    rms_eps=1e-6,
    n_new=1,
    verify="greedy",
    temperature=1.0,
    target_logits="planted",  # or "draft_plus_noise"
    plant_p=0.7,
    target_layers=1,          # layers of the target-shaped KV compacted after verify
    fc_norm=0,                # EAGLE-3.1 normalisation flags (off)
    norm_output=0,
)

CONFIGS = {
    # tiny chain, fp32: the correctness-scale workload
    "tiny_chain": dict(
        _BASE, hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, intermediate=688,
        vocab=4096, draft_vocab=4096, top_k=1, depth=3, total_tokens=3,
        dtype="f32", batch=1, ctx=128, target_layers=1,
    ),
    # Llama-3.1-8B-shaped EAGLE-3 chain
    "llama8b_chain": dict(
        _BASE, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=14336,
        vocab=128256, draft_vocab=128256, top_k=1, depth=5, total_tokens=5,
        dtype="bf16", batch=4, ctx=256, target_layers=32,
    ),
    # Qwen3-4B-shaped tree with a trimmed 32000-entry draft vocabulary
    "qwen4b_tree": dict(
        _BASE, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=9728,
        vocab=151936, draft_vocab=32000, top_k=8, depth=5, total_tokens=31,
        dtype="bf16", batch=1, ctx=4096, target_layers=36,
    ),
    # Qwen3-8B-shaped tree, stochastic verification at temperature 1
    "qwen8b_tree": dict(
        _BASE, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=12288,
        vocab=151936, draft_vocab=151936, top_k=8, depth=7, total_tokens=63,
        dtype="bf16", batch=32, ctx=2048, verify="stochastic", temperature=1.0,
        target_logits="draft_plus_noise", target_layers=36,
    ),
    # EAGLE-4 draft on Llama-3-8B shapes: sliding window + low-rank candidate head
    "eagle4_llama8b": dict(
        _BASE, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=14336,
        vocab=128256, draft_vocab=128256, top_k=8, depth=5, total_tokens=31,
        cand_rank=128, num_candidates=128, sliding_window=1024,
        dtype="bf16", batch=64, ctx=8192, target_layers=32,
    ),
}

# Order matches the workload list the measurements are quoted on.
ORDER = ["tiny_chain", "llama8b_chain", "qwen4b_tree", "qwen8b_tree", "eagle4_llama8b"]
SEEDS = {name: 1000 + i for i, name in enumerate(ORDER)}


def kv_capacity(cfg: dict) -> int:
    """Draft-KV slots per sequence: the context plus the tree region, rounded
    up to a multiple of 64 (the tree needs ctx + n_new + (depth-1)*top_k)."""
    need = cfg["ctx"] + cfg["n_new"] + (cfg["depth"] - 1) * cfg["top_k"]
    return (need + 63) // 64 * 64


def get(name: str, **overrides) -> dict:
    """A copy of one workload's table, with overrides applied."""
    cfg = copy.deepcopy(CONFIGS[name])
    cfg.update(overrides)
    cfg["name"] = name
    cfg.setdefault("kv_capacity", kv_capacity(cfg))
    if "kv_capacity" not in overrides:
        cfg["kv_capacity"] = kv_capacity(cfg)
    return cfg


def small(name: str = "tiny_chain", **overrides) -> dict:
    """A reduced workload for tests that must finish in seconds."""
    return get(name, **overrides)
