"""ctypes view of include/spec_peaks.h plus the timing loop around it: the
HBM read and copy bandwidth and the dense bf16 MFMA rate that this GPU
attains, measured with the probe kernels of libspec_peaks.so."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspec_peaks.so")
EXPORTS = ["spec_peak_read", "spec_peak_copy", "spec_peak_mfma", "spec_peak_mfma_flops"]

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.spec_peak_read.argtypes = [vp, i64, vp, i32, vp]
    lib.spec_peak_copy.argtypes = [vp, vp, i64, i32, vp]
    lib.spec_peak_mfma.argtypes = [i32, vp, i32, vp]
    lib.spec_peak_mfma_flops.argtypes = [i32, i32]
    lib.spec_peak_mfma_flops.restype = ctypes.c_double
    for f in ("spec_peak_read", "spec_peak_copy", "spec_peak_mfma"):
        getattr(lib, f).restype = i32
    _lib = lib
    return lib


def _best_ms(launch, reps: int) -> float:
    import torch

    s = torch.cuda.current_stream()
    best = float("inf")
    for _ in range(reps + 1):  # the first launch warms up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        rc = launch(ctypes.c_void_p(s.cuda_stream))
        e1.record(s)
        if rc != 0:
            raise RuntimeError(f"peak probe launch failed with code {rc}")
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    return best


def measure(read_gib: int = 4, reps: int = 5) -> dict:
    """Best of `reps` launches of each probe on cuda's current device:
    read and copy stream bandwidth in GB/s (buffers far beyond the 256 MB
    last-level cache) and the bf16 MFMA rate in TFLOP/s."""
    import torch

    lib = load()
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    cus = props.multi_processor_count
    n = read_gib << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(cus * 4 * 256, dtype=torch.float32, device="cuda")
    blocks = cus * 8
    ms_read = _best_ms(lambda st: lib.spec_peak_read(ctypes.c_void_p(buf.data_ptr()), n,
                                                     ctypes.c_void_p(sink.data_ptr()), blocks, st), reps)
    half = n // 2
    src, dst = buf.data_ptr(), buf.data_ptr() + half
    ms_copy = _best_ms(lambda st: lib.spec_peak_copy(ctypes.c_void_p(dst), ctypes.c_void_p(src), half,
                                                     blocks, st), reps)
    del buf
    iters, mblocks = 4096, cus * 4
    ms_mfma = _best_ms(lambda st: lib.spec_peak_mfma(iters, ctypes.c_void_p(sink.data_ptr()), mblocks, st), reps)
    torch.cuda.synchronize()
    flops = lib.spec_peak_mfma_flops(iters, mblocks)
    return {"hbm_read_gbs": round(n / (ms_read * 1e-3) / 1e9, 1),
            "hbm_copy_gbs": round(2 * half / (ms_copy * 1e-3) / 1e9, 1),
            "mfma_bf16_tflops": round(flops / (ms_mfma * 1e-3) / 1e12, 1),
            "probe": f"{read_gib} GiB read, {read_gib // 2} GiB copy (read + write counted), "
                     f"{mblocks} x 256-thread MFMA loop; best of {reps}"}
