"""Host -> device marshalling of seeded numpy inputs (no arithmetic of the
method): float32 arrays holding bfloat16 values become torch.bfloat16
tensors by keeping their upper 16 bits, which is exact for such values."""

from __future__ import annotations

import numpy as np
import torch

from .spec import KVCache, TargetWeights, Weights


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        return torch.from_numpy(a).to(device)
    if dtype == "f32":
        return torch.from_numpy(a).to(device)
    hi = (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return torch.from_numpy(hi.view(np.int16)).to(device).view(torch.bfloat16)


def upload_weights(cfg: dict, W: dict, device="cuda") -> Weights:
    t = {}
    for name, arr in W.items():
        if arr is None:
            continue
        if name == "d2t":
            t[name] = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).to(device)
        else:
            t[name] = to_device(arr, cfg["dtype"], device)
    return Weights(t)


def upload_kv(cfg: dict, k: np.ndarray, v: np.ndarray, device="cuda") -> KVCache:
    """[B, nkv, S, hd] (one layer) or [L, B, nkv, S, hd] arrays."""
    if k.ndim == 4:
        k, v = k[None], v[None]
    return KVCache(to_device(k, cfg["dtype"], device), to_device(v, cfg["dtype"], device))


def from_device(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def upload_target_weights(cfg: dict, W: dict, device="cuda") -> TargetWeights:
    t = {n: to_device(W[n], cfg["dtype"], device) for n in ("embed", "final_norm", "lm_head")}
    t["layers"] = [{n: to_device(lw[n], cfg["dtype"], device) for n in TargetWeights.LAYER}
                   for lw in W["layers"]]
    return TargetWeights(t)
