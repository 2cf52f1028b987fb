"""ctypes view of include/spec.h.  Loads the in-tree libspec_mi355x.so and
fails loudly when it is missing: there is no fallback path."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspec_mi355x.so")

SPEC_OK, SPEC_EINVAL, SPEC_EUNSUPPORTED, SPEC_EHIP, SPEC_ENOMEM = 0, -1, -2, -3, -4
SPEC_F32, SPEC_BF16 = 0, 1
SPEC_VERIFY_GREEDY, SPEC_VERIFY_STOCHASTIC = 0, 1

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p


class SpecConfig(ctypes.Structure):
    _fields_ = [(n, c_i32) for n in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "intermediate",
                                     "vocab", "draft_vocab", "cand_rank", "num_candidates",
                                     "sliding_window")] + \
               [("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float)] + \
               [(n, c_i32) for n in ("top_k", "depth", "total_tokens", "max_batch", "max_new",
                                     "kv_capacity", "dtype", "fc_norm", "norm_output")]


class SpecWeights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ("fc", "embed", "input_norm", "hidden_norm", "post_attn_norm",
                                    "final_norm", "wqkv", "wo", "w_gate_up", "w_down", "lm_head",
                                    "d2t", "cand_down", "cand_up", "fc_norm")]


class SpecKV(ctypes.Structure):
    _fields_ = [("k", c_vp), ("v", c_vp)] + \
               [(n, c_i32) for n in ("num_layers", "batch", "n_kv_heads", "slots", "head_dim")] + \
               [(n, ctypes.c_int64) for n in ("stride_layer", "stride_seq", "stride_head")] + \
               [("block_table", c_vp)] + \
               [(n, c_i32) for n in ("block_size", "max_blocks", "num_blocks")]


class SpecTree(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ("tokens", "parent", "depth", "position", "draft_slot",
                                    "num_nodes", "score", "anc_mask")]


class SpecTargetLayer(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ("attn_norm", "wqkv", "wo", "mlp_norm", "w_gate_up", "w_down")]


class SpecTargetWeights(ctypes.Structure):
    _fields_ = [("embed", c_vp), ("final_norm", c_vp), ("lm_head", c_vp), ("num_layers", c_i32),
                ("layers", ctypes.POINTER(SpecTargetLayer))]


EXPORTS = ["spec_create", "spec_destroy", "spec_last_error", "spec_workspace_bytes", "spec_version",
           "spec_draft_step", "spec_topk_logprobs", "spec_retrieve_candidates", "spec_tree_from_topk", "spec_tree_candidates", "spec_build_tree",
           "spec_verify_tree", "spec_verify_tree_static", "spec_compact_kv", "spec_decode_metadata", "spec_rejection_sample",
           "spec_target_forward",
           "spec_profile_enable", "spec_profile_read"]
SPEC_PROF_LM_HEAD, SPEC_PROF_ATTENTION, SPEC_PROF_VERIFY, SPEC_PROF_TOPK, SPEC_PROF_LM_HEAD_TILED = 0, 1, 2, 3, 4

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m speculative_decoding_aux_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.spec_create.argtypes = [P(SpecConfig), P(c_vp)]
    lib.spec_create.restype = c_i32
    lib.spec_destroy.argtypes = [c_vp]
    lib.spec_destroy.restype = None
    lib.spec_last_error.argtypes = [c_vp]
    lib.spec_last_error.restype = ctypes.c_char_p
    lib.spec_workspace_bytes.argtypes = [c_vp]
    lib.spec_workspace_bytes.restype = ctypes.c_int64
    lib.spec_version.argtypes = []
    lib.spec_version.restype = ctypes.c_char_p
    lib.spec_draft_step.argtypes = [c_vp, P(SpecWeights), P(SpecKV), c_i32, c_i32, c_i32, c_vp,
                                    c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp,
                                    c_vp, c_vp, c_vp, c_vp]
    lib.spec_draft_step.restype = c_i32
    lib.spec_topk_logprobs.argtypes = [c_vp, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp]
    lib.spec_topk_logprobs.restype = c_i32
    lib.spec_retrieve_candidates.argtypes = [c_vp, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp]
    lib.spec_retrieve_candidates.restype = c_i32
    lib.spec_tree_from_topk.argtypes = [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, P(SpecTree), c_vp]
    lib.spec_tree_from_topk.restype = c_i32
    lib.spec_tree_candidates.argtypes = [c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]
    lib.spec_tree_candidates.restype = c_i32
    lib.spec_build_tree.argtypes = [c_vp, P(SpecWeights), P(SpecKV), c_i32, c_i32, c_vp, c_vp, c_vp,
                                    P(SpecTree), c_vp]
    lib.spec_build_tree.restype = c_i32
    lib.spec_verify_tree.argtypes = [c_vp, c_i32, P(SpecTree), c_vp, c_i32, ctypes.c_float, c_vp,
                                     ctypes.c_uint64, c_vp, c_vp, c_vp, c_vp]
    lib.spec_verify_tree.restype = c_i32
    lib.spec_verify_tree_static.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32, P(SpecTree), c_vp, c_i32,
                                            ctypes.c_float, c_vp, ctypes.c_uint64, c_vp, c_vp, c_vp, c_vp]
    lib.spec_verify_tree_static.restype = c_i32
    lib.spec_compact_kv.argtypes = [c_vp, P(SpecKV), c_i32, c_vp, c_vp, c_vp, c_i32, c_vp]
    lib.spec_compact_kv.restype = c_i32
    lib.spec_decode_metadata.argtypes = [c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]
    lib.spec_decode_metadata.restype = c_i32
    lib.spec_rejection_sample.argtypes = [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp,
                                          c_vp, c_vp, c_vp, c_vp, ctypes.c_uint64, c_vp, c_vp, c_vp]
    lib.spec_rejection_sample.restype = c_i32
    lib.spec_target_forward.argtypes = [c_vp, P(SpecTargetWeights), P(SpecKV), c_i32, P(SpecTree), c_vp,
                                        c_vp, c_vp, c_vp]
    lib.spec_target_forward.restype = c_i32
    lib.spec_profile_enable.argtypes = [c_vp, c_i32]
    lib.spec_profile_enable.restype = c_i32
    lib.spec_profile_read.argtypes = [c_vp, c_i32, P(c_i32), P(ctypes.c_double)]
    lib.spec_profile_read.restype = c_i32
    _lib = lib
    return lib
