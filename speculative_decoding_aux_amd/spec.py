"""Python binding of the speculation-step library.

Argument marshalling only: every function below passes device pointers and
sizes to the C ABI of the same name (include/spec.h) and allocates its output
tensors with torch.  Every step of the path runs in the HIP kernels of
libspec_mi355x.so; there is no CPU or torch fallback.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib as L

_DT = {"f32": (L.SPEC_F32, torch.float32), "bf16": (L.SPEC_BF16, torch.bfloat16)}


class SpecError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"spec error {code}: {msg}")
        self.code = code


def _p(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _i32(x, device):
    if isinstance(x, torch.Tensor):
        assert x.dtype == torch.int32 and x.is_cuda and x.is_contiguous()
        return x
    return torch.as_tensor(x, dtype=torch.int32, device=device).contiguous()


class Weights:
    """Draft weights resident on the GPU, in the workload's storage type."""

    NAMES = ("fc", "embed", "input_norm", "hidden_norm", "post_attn_norm", "final_norm", "wqkv", "wo",
             "w_gate_up", "w_down", "lm_head", "cand_down", "cand_up", "fc_norm")

    def __init__(self, tensors: dict):
        self.t = tensors
        s = L.SpecWeights()
        for n in self.NAMES + ("d2t",):
            v = tensors.get(n)
            setattr(s, n, None if v is None else v.data_ptr())
        self.struct = s


class KVCache:
    """K and V tensors [layers, B, n_kv, slots, head_dim] (contiguous)."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor):
        assert k.shape == v.shape and k.dim() == 5 and k.is_contiguous() and v.is_contiguous()
        self.k, self.v = k, v
        Lr, B, H, S, D = k.shape
        self.struct = L.SpecKV(k.data_ptr(), v.data_ptr(), Lr, B, H, S, D,
                               k.stride(0), k.stride(1), k.stride(2), None, 0, 0, 0)


class PagedKVCache:
    """K and V block pools [layers, num_blocks, n_kv, block_size, head_dim]
    (contiguous) and a block table [B, max_blocks] int32: logical slot s of
    sequence b lives in block block_table[b, s // block_size] at offset
    s % block_size."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, block_table: torch.Tensor):
        assert k.shape == v.shape and k.dim() == 5 and k.is_contiguous() and v.is_contiguous()
        assert block_table.dtype == torch.int32 and block_table.is_contiguous() and block_table.dim() == 2
        self.k, self.v, self.block_table = k, v, block_table
        Lr, NB, H, BS, D = k.shape
        B, MB = block_table.shape
        self.struct = L.SpecKV(k.data_ptr(), v.data_ptr(), Lr, B, H, MB * BS, D,
                               k.stride(0), k.stride(1), k.stride(2), block_table.data_ptr(), BS, MB, NB)


class Tree:
    FIELDS = ("tokens", "parent", "depth", "position", "draft_slot", "num_nodes", "score", "anc_mask")

    def __init__(self, B, n1, device):
        z = lambda dt, *shape: torch.empty(*shape, dtype=dt, device=device)
        self.tokens = z(torch.int32, B, n1)
        self.parent = z(torch.int32, B, n1)
        self.depth = z(torch.int32, B, n1)
        self.position = z(torch.int32, B, n1)
        self.draft_slot = z(torch.int32, B, n1)
        self.num_nodes = z(torch.int32, B)
        self.score = z(torch.float32, B, n1)
        self.anc_mask = z(torch.int64, B, n1)  # uint64 bit pattern
        self.struct = L.SpecTree(*[getattr(self, f).data_ptr() for f in self.FIELDS])

    def numpy(self) -> dict:
        out = {f: getattr(self, f).cpu().numpy() for f in self.FIELDS}
        out["anc_mask"] = out["anc_mask"].view("uint64")
        return out


class SpecContext:
    """One spec_ctx (workspace) bound to the workload's shapes."""

    def __init__(self, cfg: dict, max_batch: int, max_new: int = 1, device="cuda"):
        self.lib = L.load()
        self.cfg = dict(cfg)
        self.device = torch.device(device)
        code, self.tdtype = _DT[cfg["dtype"]]
        c = L.SpecConfig(hidden=cfg["hidden"], n_q_heads=cfg["n_q_heads"], n_kv_heads=cfg["n_kv_heads"],
                         head_dim=cfg["head_dim"], intermediate=cfg["intermediate"], vocab=cfg["vocab"],
                         draft_vocab=cfg["draft_vocab"], cand_rank=cfg.get("cand_rank", 0),
                         num_candidates=cfg.get("num_candidates", 0),
                         sliding_window=cfg.get("sliding_window", 0), rope_base=cfg["rope_base"],
                         rms_eps=cfg["rms_eps"], top_k=cfg["top_k"], depth=cfg["depth"],
                         total_tokens=cfg["total_tokens"], max_batch=max_batch, max_new=max_new,
                         kv_capacity=cfg["kv_capacity"], dtype=code, fc_norm=int(cfg.get("fc_norm", 0)),
                         norm_output=int(cfg.get("norm_output", 0)))
        h = ctypes.c_void_p()
        st = self.lib.spec_create(ctypes.byref(c), ctypes.byref(h))
        if st != L.SPEC_OK:
            raise SpecError(st, "spec_create rejected the configuration")
        self.h = h
        self.max_batch, self.max_new = max_batch, max_new

    def close(self):
        if getattr(self, "h", None):
            self.lib.spec_destroy(self.h)
            self.h = None

    __del__ = close

    def _check(self, st):
        if st != L.SPEC_OK:
            raise SpecError(st, self.lib.spec_last_error(self.h).decode())

    @property
    def workspace_bytes(self) -> int:
        return int(self.lib.spec_workspace_bytes(self.h))

    def profile(self, enable: bool, reset: bool = True):
        self._check(self.lib.spec_profile_enable(self.h, (1 if reset else 2) if enable else 0))

    def profile_read(self, label: int):
        n, ms = ctypes.c_int32(), ctypes.c_double()
        self._check(self.lib.spec_profile_read(self.h, label, ctypes.byref(n), ctypes.byref(ms)))
        return int(n.value), float(ms.value)


# --------------------------------------------------------------- entry points
def spec_draft_step(ctx: SpecContext, w: Weights, kv: KVCache, B, rows_per_seq, mode, hidden_in,
                    tokens, positions, kv_slot, ctx_len, anc_slots, k_out, want_logits=False,
                    want_candidates=False):
    cfg, dev = ctx.cfg, ctx.device
    M = B * rows_per_seq
    tokens, positions, kv_slot, ctx_len = (_i32(x, dev) for x in (tokens, positions, kv_slot, ctx_len))
    anc = _i32(anc_slots, dev).reshape(M, -1)
    ids = torch.empty(M, k_out, dtype=torch.int32, device=dev)
    logp = torch.empty(M, k_out, dtype=torch.float32, device=dev)
    hid = torch.empty(M, cfg["hidden"], dtype=ctx.tdtype, device=dev)
    width = cfg["vocab"] if cfg.get("cand_rank") else cfg["draft_vocab"]
    logits = torch.empty(M, width, dtype=torch.float32, device=dev) if want_logits else None
    K = cfg.get("num_candidates", 0)
    cids = torch.empty(M, K, dtype=torch.int32, device=dev) if want_candidates else None
    cz = torch.empty(M, K, dtype=torch.float32, device=dev) if want_candidates else None
    st = ctx.lib.spec_draft_step(ctx.h, ctypes.byref(w.struct), ctypes.byref(kv.struct), B, rows_per_seq,
                                 mode, _p(hidden_in), _p(tokens), _p(positions), _p(kv_slot), _p(ctx_len),
                                 _p(anc), anc.shape[1], k_out, _p(ids), _p(logp), _p(hid), _p(logits),
                                 _p(cids), _p(cz), _stream())
    ctx._check(st)
    return {"ids": ids, "logp": logp, "h_out": hid, "logits": logits, "cand_ids": cids, "cand_logits": cz}


def spec_topk_logprobs(ctx: SpecContext, logits: torch.Tensor, k: int, id_map=None):
    M, n = logits.shape
    ids = torch.empty(M, k, dtype=torch.int32, device=logits.device)
    logp = torch.empty(M, k, dtype=torch.float32, device=logits.device)
    st = ctx.lib.spec_topk_logprobs(ctx.h, M, n, _p(logits), k, _p(id_map), _p(ids), _p(logp), _stream())
    ctx._check(st)
    return ids, logp


def spec_retrieve_candidates(ctx: SpecContext, scores: torch.Tensor, K: int):
    M, n = scores.shape
    ids = torch.empty(M, K, dtype=torch.int32, device=scores.device)
    st = ctx.lib.spec_retrieve_candidates(ctx.h, M, n, _p(scores), K, _p(ids), _stream())
    ctx._check(st)
    return ids


def spec_tree_candidates(ctx: SpecContext, B: int) -> dict:
    """The candidate table of the context's last tree build: tokens, parent,
    slot and score, each [B, C] (C = top_k + (depth - 1) * top_k^2)."""
    cfg, dev = ctx.cfg, ctx.device
    k, D = cfg["top_k"], cfg["depth"]
    C = k + (D - 1) * k * k
    out = {f: torch.empty(B, C, dtype=torch.int32, device=dev) for f in ("tokens", "parent", "slot")}
    out["score"] = torch.empty(B, C, dtype=torch.float32, device=dev)
    st = ctx.lib.spec_tree_candidates(ctx.h, B, _p(out["tokens"]), _p(out["parent"]), _p(out["slot"]),
                                      _p(out["score"]), _stream())
    ctx._check(st)
    return out


def spec_tree_from_topk(ctx: SpecContext, B, n_new, in_tokens, ctx_len, ids_tab, lp_tab) -> Tree:
    dev = ctx.device
    tree = Tree(B, ctx.cfg["total_tokens"] + 1, dev)
    in_tokens, ctx_len, ids_tab = (_i32(x, dev) for x in (in_tokens, ctx_len, ids_tab))
    lp_tab = lp_tab.contiguous()
    st = ctx.lib.spec_tree_from_topk(ctx.h, B, n_new, _p(in_tokens), _p(ctx_len), _p(ids_tab),
                                     _p(lp_tab), ctypes.byref(tree.struct), _stream())
    ctx._check(st)
    return tree


def spec_build_tree(ctx: SpecContext, w: Weights, kv: KVCache, aux, in_tokens, ctx_len, tree=None) -> Tree:
    dev = ctx.device
    B, n_new = in_tokens.shape
    if tree is None:
        tree = Tree(B, ctx.cfg["total_tokens"] + 1, dev)
    in_tokens, ctx_len = _i32(in_tokens, dev), _i32(ctx_len, dev)
    st = ctx.lib.spec_build_tree(ctx.h, ctypes.byref(w.struct), ctypes.byref(kv.struct), B, n_new,
                                 _p(aux), _p(in_tokens), _p(ctx_len), ctypes.byref(tree.struct), _stream())
    ctx._check(st)
    return tree


def spec_verify_tree(ctx: SpecContext, tree: Tree, target_logits, mode, temperature=1.0, accept_u=None,
                     seed=0, out=None):
    B = tree.tokens.shape[0]
    D = ctx.cfg["depth"]
    dev = target_logits.device
    if out is None:
        out = (torch.empty(B, D + 1, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, D, dtype=torch.int32, device=dev))
    st = ctx.lib.spec_verify_tree(ctx.h, B, ctypes.byref(tree.struct), _p(target_logits), mode,
                                  float(temperature), _p(accept_u), int(seed) & (2**64 - 1), _p(out[0]),
                                  _p(out[1]), _p(out[2]), _stream())
    ctx._check(st)
    return out


def spec_verify_tree_static(tree: Tree, target_logits, mode, total_tokens, depth, top_k, temperature=1.0,
                            accept_u=None, seed=0, out=None):
    """spec_verify_tree without a context: its scratch is the library's fixed
    per-GPU array, so the call allocates no device memory (``out`` may be
    passed preallocated as well)."""
    lib = L.load()
    B = tree.tokens.shape[0]
    V = target_logits.shape[-1]
    dev = target_logits.device
    if out is None:
        out = (torch.empty(B, depth + 1, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, depth, dtype=torch.int32, device=dev))
    st = lib.spec_verify_tree_static(B, total_tokens, depth, top_k, V, ctypes.byref(tree.struct),
                                     _p(target_logits), mode, float(temperature), _p(accept_u),
                                     int(seed) & (2**64 - 1), _p(out[0]), _p(out[1]), _p(out[2]), _stream())
    if st != L.SPEC_OK:
        raise SpecError(st, lib.spec_last_error(None).decode())
    return out


def spec_compact_kv(ctx: SpecContext, kv: KVCache, tree_base, accepted_nodes, accepted_len):
    B, max_accept = accepted_nodes.shape
    dev = ctx.device
    tree_base = _i32(tree_base, dev)
    st = ctx.lib.spec_compact_kv(ctx.h, ctypes.byref(kv.struct), B, _p(tree_base), _p(accepted_nodes),
                                 _p(accepted_len), max_accept, _stream())
    ctx._check(st)


def spec_decode_metadata(ctx: SpecContext, cu_num_scheduled_tokens, num_draft_tokens, total_drafts: int):
    """Index bookkeeping of a flat batch; ``total_drafts`` (the sum of the
    draft counts) sizes the outputs.  Returns (cu_num_draft_tokens,
    logits_indices, target_logits_indices, bonus_logits_indices)."""
    dev = ctx.device
    cu_s = _i32(cu_num_scheduled_tokens, dev)
    nd = _i32(num_draft_tokens, dev)
    B = nd.shape[0]
    out = (torch.empty(B, dtype=torch.int32, device=dev),
           torch.empty(total_drafts + B, dtype=torch.int32, device=dev),
           torch.empty(max(total_drafts, 1), dtype=torch.int32, device=dev),
           torch.empty(B, dtype=torch.int32, device=dev))
    st = ctx.lib.spec_decode_metadata(ctx.h, B, _p(cu_s), _p(nd), _p(out[0]), _p(out[1]), _p(out[2]),
                                      _p(out[3]), _stream())
    ctx._check(st)
    return out[0], out[1], out[2][:total_drafts], out[3]


def spec_rejection_sample(ctx: SpecContext, cu_num_draft_tokens, draft_token_ids, logits,
                          target_logits_indices, bonus_logits_indices, temperature, top_k=None, top_p=None,
                          uniform=None, seed=0, max_spec_len=None, out=None):
    """Flat-batch rejection sampling; returns (out_tokens [B, L+1], num_accepted [B])."""
    dev = logits.device
    cu = _i32(cu_num_draft_tokens, dev)
    B = cu.shape[0]
    L = ctx.cfg["total_tokens"] if max_spec_len is None else int(max_spec_len)
    drafts = _i32(draft_token_ids, dev)
    tgt = _i32(target_logits_indices, dev)
    if drafts.numel() == 0:  # no drafts in the batch: any valid pointer will do
        drafts = torch.zeros(1, dtype=torch.int32, device=dev)
        tgt = torch.zeros(1, dtype=torch.int32, device=dev)
    bonus = _i32(bonus_logits_indices, dev)
    temp = torch.as_tensor(temperature, dtype=torch.float32).to(dev)
    tk = None if top_k is None else _i32(top_k, dev)
    tp = None if top_p is None else torch.as_tensor(top_p, dtype=torch.float32).to(dev)
    u = None if uniform is None else torch.as_tensor(uniform, dtype=torch.float32).to(dev)
    if out is None:
        out = (torch.empty(B, L + 1, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    st = ctx.lib.spec_rejection_sample(ctx.h, B, L, _p(cu), _p(drafts), _p(logits), logits.shape[0], _p(tgt),
                                       _p(bonus), _p(temp), _p(tk), _p(tp), _p(u), int(seed) & (2**64 - 1),
                                       _p(out[0]), _p(out[1]), _stream())
    ctx._check(st)
    return out


class TargetWeights:
    """Weights of a Llama-style target on the GPU: embed, final_norm, lm_head
    and a list of per-layer dicts (attn_norm, wqkv, wo, mlp_norm, w_gate_up,
    w_down) of device tensors."""

    LAYER = ("attn_norm", "wqkv", "wo", "mlp_norm", "w_gate_up", "w_down")

    def __init__(self, tensors: dict):
        self.t = tensors
        L_ = len(tensors["layers"])
        self._layers = (L.SpecTargetLayer * L_)()
        for i, lw in enumerate(tensors["layers"]):
            for n in self.LAYER:
                setattr(self._layers[i], n, lw[n].data_ptr())
        self.struct = L.SpecTargetWeights(tensors["embed"].data_ptr(), tensors["final_norm"].data_ptr(),
                                          tensors["lm_head"].data_ptr(), L_, self._layers)


def spec_target_forward(ctx: SpecContext, tw: TargetWeights, kv, tree: Tree, ctx_len):
    """The target's forward over the trees: (logits [B, N+1, V] float32,
    aux_hidden [B, N+1, 3H])."""
    cfg, dev = ctx.cfg, ctx.device
    B, n1 = tree.tokens.shape
    ctx_len = _i32(ctx_len, dev)
    logits = torch.empty(B, n1, cfg["vocab"], dtype=torch.float32, device=dev)
    aux = torch.empty(B, n1, 3 * cfg["hidden"], dtype=ctx.tdtype, device=dev)
    st = ctx.lib.spec_target_forward(ctx.h, ctypes.byref(tw.struct), ctypes.byref(kv.struct), B,
                                     ctypes.byref(tree.struct), _p(ctx_len), _p(logits), _p(aux), _stream())
    ctx._check(st)
    return logits, aux
