"""Device calibration for the benchmark harness: the bf16 MFMA rate of a pure matrix-core loop and
the HBM rate of a streaming read, measured on the device in use (ctypes over libmla_calib.so)."""
from __future__ import annotations

import ctypes
import os

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_calib.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is missing: build it with `python -m mla_varlen_prefill_amd._build`")
        lib = ctypes.CDLL(_PATH)
        lib.mla_calib_mfma_loop.restype = ctypes.c_int
        lib.mla_calib_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.mla_calib_mfma_flop.restype = ctypes.c_double
        lib.mla_calib_mfma_flop.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.mla_calib_stream_read.restype = ctypes.c_int
        lib.mla_calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_void_p]
        _lib = lib
    return _lib


def _timed(launch, reps: int, settle_ms: float = 100.0) -> float:
    """Best milliseconds of `reps` launches, after launching for `settle_ms` untimed so that the
    device's clocks have settled under load (the first tens of milliseconds after idle run at
    transient clocks)."""
    import time
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        launch()
        torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        launch()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    return min(times)


def mfma_tflops(reps: int = 5) -> float:
    """Sustained TFLOP/s of 32x32x16 bf16 MFMA chains: 4 work-groups of 4 waves per CU."""
    import torch
    lib = _load()
    blocks = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    iters = 8192
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        if lib.mla_calib_mfma_loop(ctypes.c_void_p(out.data_ptr()), blocks, iters, stream) != 0:
            raise RuntimeError("mla_calib_mfma_loop failed")

    ms = _timed(launch, reps)
    return lib.mla_calib_mfma_flop(blocks, iters) / (ms * 1e-3) / 1e12


def stream_read_gbps(nbytes: int = 4 << 30, reps: int = 5) -> float:
    """Sustained GB/s of a streaming read of `nbytes` (far beyond the caches); `nbytes` must be a
    multiple of 4 work-groups per CU x 16 KiB."""
    import torch
    lib = _load()
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    blocks = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        if lib.mla_calib_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                     blocks, stream) != 0:
            raise RuntimeError("mla_calib_stream_read failed")

    ms = _timed(launch, reps)
    del src, out
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9
