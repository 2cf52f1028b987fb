"""The C-ABI libraries load on the CPU and export every function their headers
declare (include/spec.h: the speculation library; include/spec_peaks.h: the
peak probes), and the speculation library rejects bad configurations before
touching the GPU."""

import ctypes
import os
import re

import pytest

from conftest import ROOT
from speculative_decoding_aux_amd import _lib as L


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from speculative_decoding_aux_amd import build
        build.build()
    return L.load()


def _declared(header="spec.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


def test_every_include_header_is_covered():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["spec.h", "spec_peaks.h"]


def test_peak_probes_export_their_header():
    from speculative_decoding_aux_amd import peaks as PK

    if not os.path.exists(PK.LIB_PATH):
        from speculative_decoding_aux_amd import build
        build.build()
    plib = PK.load()
    names = _declared("spec_peaks.h")
    assert set(names) == set(PK.EXPORTS)
    for n in names:
        assert hasattr(plib, n), n
    assert plib.spec_peak_mfma_flops(10, 4) == 4 * 4 * 10 * 8 * 16 * 16 * 32 * 2
    # argument checks return before any launch
    assert plib.spec_peak_read(None, 16, None, 1, None) == -1
    assert plib.spec_peak_copy(ctypes.c_void_p(16), ctypes.c_void_p(16), 16, 1, None) == -1
    assert plib.spec_peak_mfma(0, ctypes.c_void_p(16), 1, None) == -1


def test_version_string(lib):
    assert b"gfx950" in lib.spec_version()


def _cfg(**kw):
    base = dict(hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, intermediate=688, vocab=4096,
                draft_vocab=4096, cand_rank=0, num_candidates=0, sliding_window=0, rope_base=10000.0,
                rms_eps=1e-6, top_k=1, depth=3, total_tokens=3, max_batch=1, max_new=1,
                kv_capacity=192, dtype=L.SPEC_F32)
    base.update(kw)
    return L.SpecConfig(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), L.SPEC_EUNSUPPORTED),
    (dict(top_k=17, total_tokens=40, depth=3), L.SPEC_EUNSUPPORTED),
    (dict(total_tokens=64, depth=3), L.SPEC_EUNSUPPORTED),
    (dict(depth=5, total_tokens=3), L.SPEC_EUNSUPPORTED),
    (dict(n_q_heads=6, n_kv_heads=4), L.SPEC_EINVAL),
    (dict(draft_vocab=5000), L.SPEC_EINVAL),
    (dict(dtype=7), L.SPEC_EINVAL),
    (dict(hidden=250, dtype=L.SPEC_BF16), L.SPEC_EUNSUPPORTED),
    (dict(cand_rank=16, num_candidates=300), L.SPEC_EUNSUPPORTED),
    (dict(max_batch=0), L.SPEC_EINVAL),
])
def test_create_rejects_bad_configs_before_any_gpu_call(lib, kw, code):
    h = ctypes.c_void_p()
    assert lib.spec_create(ctypes.byref(_cfg(**kw)), ctypes.byref(h)) == code
    assert not h.value


def test_null_context_is_rejected(lib):
    assert lib.spec_verify_tree(None, 1, None, None, 0, 1.0, None, 0, None, None, None, None) == L.SPEC_EINVAL



def test_static_verify_rejects_bad_arguments_before_any_launch(lib):
    """The context-free verification refuses null arrays and shapes beyond
    its fixed scratch on the host (no GPU needed) and reports why through
    spec_last_error(NULL)."""
    tree = L.SpecTree()
    assert lib.spec_verify_tree_static(4, 63, 7, 8, 1000, ctypes.byref(tree), None, 0, 1.0, None, 0,
                                       None, None, None, None) == L.SPEC_EINVAL
    assert b"null argument" in lib.spec_last_error(None)
    assert lib.spec_verify_tree_static(4, 64, 7, 8, 1000, None, None, 0, 1.0, None, 0,
                                       None, None, None, None) == L.SPEC_EUNSUPPORTED
    p = ctypes.c_void_p(16)  # never dereferenced: the call is refused first
    big = L.SpecTree(p, p, p, p, p, p, p, p)
    assert lib.spec_verify_tree_static(40000, 63, 7, 8, 1000, ctypes.byref(big), p, 0, 1.0, None, 0,
                                       p, p, p, None) == L.SPEC_EUNSUPPORTED
    assert b"scratch bytes" in lib.spec_last_error(None)
