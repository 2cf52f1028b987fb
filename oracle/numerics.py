"""Scalar numerics of the draft layer, written out in float64.

Pinned by tests/test_oracle_draft.py (an independent torch formulation and
special cases: RoPE at position 0 is the identity, RMSNorm of a constant
vector, rounding of known bit patterns).
"""

from __future__ import annotations

import numpy as np


def to_storage(x, dtype: str) -> np.ndarray:
    """Round to the workload's storage type.  Values are first rounded to
    float32 (as a float32 register would hold them), then, for bf16 workloads,
    to the nearest bfloat16 with ties to even."""
    a = np.array(x, dtype=np.float32, copy=True)
    if dtype == "f32":
        return a
    assert dtype == "bf16"
    bits = a.reshape(-1).view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32).reshape(a.shape)


def rmsnorm(x, gain, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gain, float64.
    ("input_layernorm", "hidden_norm", "post_attention_layernorm" and the final
    "norm" of the EAGLE3 draft; vLLM Neuron design page, "Eagle3 Draft Model
    Architecture".)"""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def rope(x, pos, base: float) -> np.ndarray:
    """Rotary embedding, rotate-half form, float64.

    For head dimension hd and i < hd/2 the pair (x[i], x[i + hd/2]) is rotated
    by the angle pos * base**(-2i/hd).  x has shape [..., hd]; pos broadcasts
    against x[..., 0].  (The draft's shared "rotary_emb"; the rotation style is
    a reading, the pages do not print it.)"""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(float(base), -2.0 * i / hd)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))

