"""Helpers for the GPU parity tests: device copies of the seeded inputs and the parity checks.

Tolerances (fixed by the method's accuracy target): O max-abs error <= 2e-2 against the fp64
oracle, LSE max-abs error <= 1e-3 on finite entries, and -inf entries must match exactly.
"""
import sys

import numpy as np
import pytest

O_TOL = 2e-2
LSE_TOL = 1e-3


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_parity(o_gpu: np.ndarray, lse_gpu, o_ref: np.ndarray, lse_ref, tag: str,
                 o_tol: float = O_TOL, lse_tol: float = LSE_TOL) -> float:
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{tag}: non-finite O"
    err = float(np.max(np.abs(o_gpu - o_ref))) if o_gpu.size else 0.0
    assert err <= o_tol, f"{tag}: O max-abs error {err:.3e} > {o_tol}"
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
        ninf_ref = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(lse_gpu), ninf_ref), f"{tag}: -inf LSE pattern differs"
        fin = ~ninf_ref
        assert np.all(np.isfinite(lse_gpu[fin])), f"{tag}: non-finite LSE"
        lerr = float(np.max(np.abs(lse_gpu[fin] - lse_ref[fin]))) if fin.any() else 0.0
        assert lerr <= lse_tol, f"{tag}: LSE max-abs error {lerr:.3e} > {lse_tol}"
    return err


requires_gpu = pytest.mark.skipif(not gpu_available(), reason="needs a GPU")
