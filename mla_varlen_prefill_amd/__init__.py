"""MI355X (gfx950) MLA prefill: thin Python binding over the C ABI of libmla_prefill.so.

Every step of the computation runs in the HIP kernels behind the C ABI (see ``include/mla_prefill.h``).
This module only marshals arguments: it takes PyTorch tensors (device memory and the current
stream are PyTorch's), checks shapes/dtypes, allocates outputs and the workspace with PyTorch,
and passes raw pointers. There is no fallback: if the library is missing or the device is not a
gfx950 GPU, every call raises.

Entry points (same names as the C ABI):
  mla_prefill_varlen  dense varlen prefill, q/k 192 = 128 nope + 64 rope, v 128, causal or not
                      (also the other MLA layouts: q/k 128 with v 128, q/k 256 with v 256)
  mla_prefill_varlen_noalloc  the same without a workspace or any allocation (static scratch)
  mla_prefill_varlen_window  the same with a (left, right) sliding-window band mask
  mla_prefill_varlen_fp8  the same with FP8 e4m3 output under a static per-tensor scale
  mla_prefill_sparse  sparse top-k prefill over one shared 576-wide latent KV (v = first 512)
  mla_prefill_sparse_paged  the same over a paged latent cache with logical indices
  mla_prefill_chunked_context  new tokens over an up-projected latent context, chunk by chunk
  mla_latent_upproject  one chunk of cached latent rows -> per-head K/V
  mla_combine         merge split partial results through their LSEs
  mla_prefill_plan    the varlen tile plan (test hook for the bit-exact plan checks)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; MLA_PREFILL_LIBRARY may name another build of the same sources (the
# host-AddressSanitizer build the CPU tests load).
LIB_PATH = os.environ.get("MLA_PREFILL_LIBRARY") or os.path.join(_PKG_DIR, "libmla_prefill.so")

MLA_OK = 0
STATUS_NAMES = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED",
                3: "MLA_ERR_ALIGNMENT", 4: "MLA_ERR_WORKSPACE", 5: "MLA_ERR_HIP"}

EXPORTED_SYMBOLS = (
    "mla_status_string", "mla_abi_version", "mla_dense_tile_shape", "mla_prefill_plan",
    "mla_prefill_varlen_workspace_size", "mla_prefill_varlen", "mla_prefill_varlen_noalloc",
    "mla_prefill_varlen_window",
    "mla_prefill_varlen_fp8", "mla_prefill_varlen_num_splits",
    "mla_prefill_sparse_workspace_size", "mla_prefill_sparse", "mla_prefill_sparse_paged",
    "mla_prefill_chunked_context_workspace_size", "mla_prefill_chunked_context", "mla_latent_upproject",
    "mla_combine",
    "mla_profile_enable", "mla_profile_select", "mla_profile_read",
)
KERNEL_IDS = {"plan": 0, "dense": 1, "combine": 2, "sparse": 3, "upproj": 4}

_c_i32, _c_i64, _c_f32, _c_sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla_prefill.so (built in-tree by ``mla_varlen_prefill_amd._build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m mla_varlen_prefill_amd._build`")
    lib = ctypes.CDLL(path)
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_abi_version.restype = _c_i32
    lib.mla_dense_tile_shape.restype = None
    lib.mla_dense_tile_shape.argtypes = [ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i32)]
    lib.mla_prefill_plan.restype = ctypes.c_int
    lib.mla_prefill_plan.argtypes = [_vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                     _vp, _c_i32, _vp, _vp]
    lib.mla_prefill_varlen_workspace_size.restype = _c_sz
    lib.mla_prefill_varlen_workspace_size.argtypes = [_c_i32] * 8
    lib.mla_prefill_varlen_num_splits.restype = _c_i32
    lib.mla_prefill_varlen_num_splits.argtypes = [_c_i32] * 8
    lib.mla_prefill_varlen.restype = ctypes.c_int
    lib.mla_prefill_varlen.argtypes = [
        _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _vp,
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
        _c_f32, _c_i32, _c_i32, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _c_sz, _vp]
    lib.mla_prefill_varlen_noalloc.restype = ctypes.c_int
    lib.mla_prefill_varlen_noalloc.argtypes = [
        _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _vp,
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
        _c_f32, _c_i32, _c_i32, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp]
    lib.mla_prefill_varlen_window.restype = ctypes.c_int
    lib.mla_prefill_varlen_window.argtypes = [
        _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _vp,
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
        _c_f32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp,
        _c_sz, _vp]
    lib.mla_prefill_varlen_fp8.restype = ctypes.c_int
    lib.mla_prefill_varlen_fp8.argtypes = [
        _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _vp,
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
        _c_f32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp,
        _c_sz, _vp]
    lib.mla_prefill_sparse_workspace_size.restype = _c_sz
    lib.mla_prefill_sparse_workspace_size.argtypes = [_c_i32] * 4
    lib.mla_prefill_sparse.restype = ctypes.c_int
    lib.mla_prefill_sparse.argtypes = [
        _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i32, _vp,
        _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64,
        _vp, _c_sz, _vp]
    lib.mla_prefill_sparse_paged.restype = ctypes.c_int
    lib.mla_prefill_sparse_paged.argtypes = [
        _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i32, _c_i32, _vp, _c_i64, _c_i32, _vp, _c_i32, _vp, _vp,
        _vp, _c_i64, _c_i32, _vp,
        _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64,
        _vp, _c_sz, _vp]
    lib.mla_prefill_chunked_context_workspace_size.restype = _c_sz
    lib.mla_prefill_chunked_context_workspace_size.argtypes = [_c_i32] * 5
    lib.mla_prefill_chunked_context.restype = ctypes.c_int
    lib.mla_prefill_chunked_context.argtypes = [
        _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp, _vp, _c_i64, _vp, _vp, _c_i64,
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64,
        _vp, _c_sz, _vp]
    lib.mla_latent_upproject.restype = ctypes.c_int
    lib.mla_latent_upproject.argtypes = [_vp, _c_i64, _vp, _c_i32, _c_i32, _c_i32, _vp, _c_i64, _c_i32, _vp,
                                         _vp, _vp, _vp]
    lib.mla_combine.restype = ctypes.c_int
    lib.mla_combine.argtypes = [_vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _c_i64, _c_i64,
                                _vp, _c_i64, _c_i64, _vp]
    lib.mla_profile_enable.restype = ctypes.c_int
    lib.mla_profile_enable.argtypes = [_c_i32]
    lib.mla_profile_select.restype = ctypes.c_int
    lib.mla_profile_select.argtypes = [ctypes.c_uint32]
    lib.mla_profile_read.restype = ctypes.c_int
    lib.mla_profile_read.argtypes = [_c_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_c_i64)]
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != MLA_OK:
        raise MLAError(fn, status)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _require_cuda(*ts) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


# Shape and dtype checks, run before anything touches the device: every tensor the kernels read
# is checked against the sizes passed to the C ABI, so that a short or mistyped tensor is an
# error here rather than an out-of-bounds read on the GPU.
def _int32_vec(name: str, t: Optional[torch.Tensor], n: int) -> None:
    if t is None:
        return
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 vector")
    if t.numel() != n:
        raise ValueError(f"{name} must have {n} elements, got {t.numel()}")


def _f32_vec(name: str, t: Optional[torch.Tensor], n: int) -> None:
    if t is None:
        return
    if t.dtype != torch.float32 or t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 vector")
    if t.numel() != n:
        raise ValueError(f"{name} must have {n} elements, got {t.numel()}")


def _bf16(name: str, t: torch.Tensor, dims: int) -> None:
    if t.dtype != torch.bfloat16 or t.dim() != dims or t.stride(-1) != 1:
        raise ValueError(f"{name} must be a bf16 tensor of {dims} dims with a contiguous last dim")


def _cu_batch(name: str, t: torch.Tensor) -> int:
    """Batch size B of a cu_seqlens tensor (int32 [B + 1])."""
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or t.numel() < 1:
        raise ValueError(f"{name} must be a contiguous int32 [batch + 1] tensor")
    return t.numel() - 1


def dense_tile_shape() -> Tuple[int, int]:
    lib = load_library()
    bm, bn = _c_i32(), _c_i32()
    lib.mla_dense_tile_shape(ctypes.byref(bm), ctypes.byref(bn))
    return bm.value, bn.value


def mla_prefill_plan(cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
                     causal: bool, block_m: Optional[int] = None, block_n: Optional[int] = None,
                     capacity: Optional[int] = None,
                     window: Tuple[int, int] = (-1, -1)) -> Tuple[torch.Tensor, torch.Tensor]:
    """Run the GPU planner; returns (plan int32 [capacity, 4], num_items int32 [1])."""
    lib = load_library()
    batch = _cu_batch("cu_seqlens_q", cu_seqlens_q)
    _int32_vec("cu_seqlens_k", cu_seqlens_k, batch + 1)
    _require_cuda(cu_seqlens_q, cu_seqlens_k)
    bm0, bn0 = dense_tile_shape()
    bm = bm0 if block_m is None else block_m
    bn = bn0 if block_n is None else block_n
    mt = -(-max_seqlen_q // bm) if max_seqlen_q > 0 else 0
    cap = batch * mt if capacity is None else capacity
    plan = torch.empty((max(cap, 1), 4), dtype=torch.int32, device=cu_seqlens_q.device)
    n = torch.empty(1, dtype=torch.int32, device=cu_seqlens_q.device)
    _check("mla_prefill_plan", lib.mla_prefill_plan(
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch, max_seqlen_q, bm, bn, int(bool(causal)),
        int(window[0]), int(window[1]), _ptr(plan), cap, _ptr(n), _stream()))
    return plan[:cap], n


def varlen_workspace_bytes(batch: int, total_q: int, max_seqlen_q: int, max_seqlen_k: int,
                           num_heads: int, causal: bool, num_splits: int, head_dim_v: int = 128) -> int:
    return load_library().mla_prefill_varlen_workspace_size(
        batch, total_q, max_seqlen_q, max_seqlen_k, num_heads, head_dim_v, int(bool(causal)), num_splits)


def varlen_num_splits(batch: int, max_seqlen_q: int, max_seqlen_k: int, num_heads: int,
                      causal: bool, num_splits: int = 0, head_dim_qk: int = 192, head_dim_v: int = 128) -> int:
    """The key-split count mla_prefill_varlen uses for these arguments and head layout."""
    return load_library().mla_prefill_varlen_num_splits(batch, max_seqlen_q, max_seqlen_k, num_heads,
                                                        head_dim_qk, head_dim_v, int(bool(causal)), num_splits)


def _check_out_lse(out, lse, rows: int, heads: int, dv: int, elem: int = 2) -> None:
    """A caller-supplied output must be [rows, heads, dv] with a contiguous last dim (elements of
    `elem` bytes) and a caller-supplied LSE float32 [rows, heads]; any other strides are passed on."""
    if tuple(out.shape) != (rows, heads, dv) or out.stride(-1) != 1 or out.element_size() != elem:
        raise ValueError(f"out must be a [{rows}, {heads}, {dv}] tensor of {elem}-byte elements with a "
                         "contiguous last dim")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (rows, heads)):
        raise ValueError(f"lse must be a float32 [{rows}, {heads}] tensor")


def mla_prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                       max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float,
                       causal: bool = True, num_splits: int = 0,
                       sink: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       return_lse: bool = True, lse: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       window: Optional[Tuple[int, int]] = None,
                       out_scale: Optional[torch.Tensor] = None):
    """Dense varlen MLA prefill. q [Tq,H,Dqk], k [Tk,H,Dqk], v [Tk,H,Dv] bf16 with (Dqk, Dv) one
    of (192, 128), (128, 128), (256, 256) (last dim contiguous; V may be strided); cu_seqlens
    int32 [B+1]. With ``window`` = (left, right) (-1 = unlimited) the sliding-window entry point
    mla_prefill_varlen_window is called; with ``out_scale`` (float32 [1] on the device) the
    output is FP8 e4m3 of O / out_scale through mla_prefill_varlen_fp8. Returns out [Tq,H,Dv]
    (bf16, or float8_e4m3fn) and, when ``return_lse``, lse float32 [Tq,H]."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _bf16(name, t, 3)
    total_q, heads, dqk = q.shape
    dv = v.shape[2]
    if tuple(k.shape[1:]) != (heads, dqk):
        raise ValueError(f"k must be [tokens, {heads}, {dqk}] like q, got {tuple(k.shape)}")
    if v.shape[0] != k.shape[0] or v.shape[1] != heads:
        raise ValueError(f"v must be [{k.shape[0]}, {heads}, dv] like k, got {tuple(v.shape)}")
    batch = _cu_batch("cu_seqlens_q", cu_seqlens_q)
    _int32_vec("cu_seqlens_k", cu_seqlens_k, batch + 1)
    _f32_vec("sink", sink, heads)
    fp8 = out_scale is not None
    if fp8:
        _f32_vec("out_scale", out_scale, 1)
    _require_cuda(q, k, v, cu_seqlens_q, cu_seqlens_k, sink, out, lse, workspace, out_scale)
    if out is None:
        out = torch.empty((total_q, heads, dv), dtype=torch.float8_e4m3fn if fp8 else torch.bfloat16,
                          device=q.device)
    elif out.element_size() != (1 if fp8 else 2):
        raise ValueError("out must be float8_e4m3fn with out_scale, else bf16")
    if return_lse and lse is None:
        lse = torch.empty((total_q, heads), dtype=torch.float32, device=q.device)
    _check_out_lse(out, lse, total_q, heads, dv, 1 if fp8 else 2)
    ws_bytes = lib.mla_prefill_varlen_workspace_size(batch, total_q, max_seqlen_q, max_seqlen_k,
                                                     heads, dv, int(bool(causal)), num_splits)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    head = (_ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1),
            _ptr(v), v.stride(0), v.stride(1), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
            batch, total_q, max_seqlen_q, max_seqlen_k, heads, dqk, dv,
            float(softmax_scale), int(bool(causal)))
    tail = (num_splits, _ptr(sink), _ptr(out), out.stride(0), out.stride(1),
            _ptr(lse), lse.stride(0) if lse is not None else 0, lse.stride(1) if lse is not None else 0,
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    if fp8:
        left, right = window if window is not None else (-1, -1)
        _check("mla_prefill_varlen_fp8",
               lib.mla_prefill_varlen_fp8(*head, int(left), int(right), num_splits, _ptr(sink), _ptr(out_scale),
                                          *tail[2:]))
    elif window is None:
        _check("mla_prefill_varlen", lib.mla_prefill_varlen(*head, *tail))
    else:
        _check("mla_prefill_varlen_window",
               lib.mla_prefill_varlen_window(*head, int(window[0]), int(window[1]), *tail))
    return (out, lse) if return_lse else out


NOALLOC_SCRATCH_BYTES = 64 << 20   # MLA_NOALLOC_SCRATCH_BYTES of include/mla_prefill.h


def mla_prefill_varlen_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                               max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float,
                               out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                               causal: bool = True, num_splits: int = 0,
                               sink: Optional[torch.Tensor] = None) -> None:
    """The allocation-free dense entry point (mla_prefill_varlen_noalloc): the caller passes the
    output (bf16 [Tq, H, Dv]) and, optionally, the LSE (float32 [Tq, H]); nothing is allocated
    here or in the library (the plan and partials use the library's static device scratch, so
    calls that overlap in time on one GPU race). Results are those of mla_prefill_varlen."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _bf16(name, t, 3)
    total_q, heads, dqk = q.shape
    dv = v.shape[2]
    if tuple(k.shape[1:]) != (heads, dqk):
        raise ValueError(f"k must be [tokens, {heads}, {dqk}] like q, got {tuple(k.shape)}")
    if v.shape[0] != k.shape[0] or v.shape[1] != heads:
        raise ValueError(f"v must be [{k.shape[0]}, {heads}, dv] like k, got {tuple(v.shape)}")
    batch = _cu_batch("cu_seqlens_q", cu_seqlens_q)
    _int32_vec("cu_seqlens_k", cu_seqlens_k, batch + 1)
    _f32_vec("sink", sink, heads)
    _check_out_lse(out, lse, total_q, heads, dv)
    _require_cuda(q, k, v, cu_seqlens_q, cu_seqlens_k, sink, out, lse)
    _check("mla_prefill_varlen_noalloc", lib.mla_prefill_varlen_noalloc(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1), _ptr(v), v.stride(0), v.stride(1),
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch, total_q, max_seqlen_q, max_seqlen_k, heads, dqk, dv,
        float(softmax_scale), int(bool(causal)), num_splits, _ptr(sink), _ptr(out), out.stride(0), out.stride(1),
        _ptr(lse), lse.stride(0) if lse is not None else 0, lse.stride(1) if lse is not None else 0, _stream()))


def mla_prefill_varlen_window(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                              cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                              max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float,
                              causal: bool, window_left: int, window_right: int, **kw):
    """Dense varlen MLA prefill with a (left, right) sliding window, -1 = unlimited."""
    return mla_prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                              softmax_scale, causal=causal, window=(window_left, window_right), **kw)


def mla_prefill_varlen_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                           max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float,
                           out_scale: torch.Tensor, causal: bool = True, **kw):
    """Dense varlen MLA prefill with FP8 e4m3 output of O / out_scale (static per-tensor scale,
    float32 [1] on the device); the LSE stays float32."""
    return mla_prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                              softmax_scale, causal=causal, out_scale=out_scale, **kw)


def mla_prefill_sparse(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor,
                       softmax_scale: float, topk_length: Optional[torch.Tensor] = None,
                       sink: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       return_lse: bool = True, lse: Optional[torch.Tensor] = None, dv: int = 512):
    """Sparse top-k MLA prefill. q [T,H,576] bf16, kv [N,576] bf16, indices int32 [T, topk]
    (physical rows, -1 = padded). Returns out [T,H,512] bf16 (and lse float32 [T,H])."""
    lib = load_library()
    _bf16("q", q, 3)
    _bf16("kv", kv, 2)
    t, heads, dqk = q.shape
    if kv.shape[1] != dqk:
        raise ValueError(f"kv must be [n_kv, {dqk}] like q's head, got {tuple(kv.shape)}")
    if indices.dtype != torch.int32 or indices.dim() != 2 or indices.stride(-1) != 1 or indices.shape[0] != t:
        raise ValueError(f"indices must be int32 [{t}, topk] with a contiguous last dim")
    topk = indices.shape[1]
    _int32_vec("topk_length", topk_length, t)
    _f32_vec("sink", sink, heads)
    _require_cuda(q, kv, indices, topk_length, sink, out, lse)
    if out is None:
        out = torch.empty((t, heads, dv), dtype=torch.bfloat16, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((t, heads), dtype=torch.float32, device=q.device)
    _check_out_lse(out, lse, t, heads, dv)
    ws_bytes = lib.mla_prefill_sparse_workspace_size(t, heads, topk, dv)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    _check("mla_prefill_sparse", lib.mla_prefill_sparse(
        _ptr(q), q.stride(0), q.stride(1), _ptr(kv), kv.stride(0), kv.shape[0],
        _ptr(indices), indices.stride(0), topk, _ptr(topk_length),
        t, heads, dqk, dv, float(softmax_scale), _ptr(sink),
        _ptr(out), out.stride(0), out.stride(1),
        _ptr(lse), lse.stride(0) if lse is not None else 0, lse.stride(1) if lse is not None else 0,
        _ptr(ws), ws_bytes, _stream()))
    return (out, lse) if return_lse else out


def mla_prefill_sparse_paged(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                             cu_seqlens_q: torch.Tensor, indices: torch.Tensor, softmax_scale: float,
                             seqused_kv: Optional[torch.Tensor] = None,
                             topk_length: Optional[torch.Tensor] = None,
                             sink: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                             return_lse: bool = True, lse: Optional[torch.Tensor] = None,
                             dv: int = 512, seqused_q: Optional[torch.Tensor] = None):
    """Sparse top-k MLA prefill over a paged latent cache. kv_cache bf16 [num_blocks, block_size,
    576] (contiguous rows), block_table int32 [B, max_blocks], cu_seqlens_q int32 [B+1], indices
    int32 [T, topk] logical positions of each token's sequence (-1 = padded), seqused_kv int32
    [B] or None (valid KV positions per sequence), seqused_q int32 [B] or None (query tokens in
    use per sequence). Returns out [T,H,512] bf16 (and lse float32 [T,H])."""
    lib = load_library()
    _bf16("q", q, 3)
    _bf16("kv_cache", kv_cache, 3)
    t, heads, dqk = q.shape
    if kv_cache.shape[2] != dqk or kv_cache.stride(0) != kv_cache.shape[1] * kv_cache.stride(1):
        raise ValueError(f"kv_cache must be [num_blocks, block_size, {dqk}] with rows of one stride")
    if indices.dtype != torch.int32 or indices.dim() != 2 or indices.stride(-1) != 1 or indices.shape[0] != t:
        raise ValueError(f"indices must be int32 [{t}, topk] with a contiguous last dim")
    batch = _cu_batch("cu_seqlens_q", cu_seqlens_q)
    if (block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(-1) != 1
            or block_table.shape[0] != batch):
        raise ValueError(f"block_table must be int32 [{batch}, max_blocks] with a contiguous last dim")
    _int32_vec("seqused_kv", seqused_kv, batch)
    _int32_vec("seqused_q", seqused_q, batch)
    _int32_vec("topk_length", topk_length, t)
    _f32_vec("sink", sink, heads)
    _require_cuda(q, kv_cache, block_table, cu_seqlens_q, indices, seqused_kv, seqused_q, topk_length, sink,
                  out, lse)
    topk = indices.shape[1]
    num_blocks, block_size = kv_cache.shape[0], kv_cache.shape[1]
    if out is None:
        out = torch.empty((t, heads, dv), dtype=torch.bfloat16, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((t, heads), dtype=torch.float32, device=q.device)
    _check_out_lse(out, lse, t, heads, dv)
    ws_bytes = lib.mla_prefill_sparse_workspace_size(t, heads, topk, dv)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    _check("mla_prefill_sparse_paged", lib.mla_prefill_sparse_paged(
        _ptr(q), q.stride(0), q.stride(1), _ptr(kv_cache), kv_cache.stride(1), num_blocks, block_size,
        _ptr(block_table), block_table.stride(0), block_table.shape[1], _ptr(cu_seqlens_q), batch,
        _ptr(seqused_kv), _ptr(seqused_q), _ptr(indices), indices.stride(0), topk, _ptr(topk_length),
        t, heads, dqk, dv, float(softmax_scale), _ptr(sink),
        _ptr(out), out.stride(0), out.stride(1),
        _ptr(lse), lse.stride(0) if lse is not None else 0, lse.stride(1) if lse is not None else 0,
        _ptr(ws), ws_bytes, _stream()))
    return (out, lse) if return_lse else out


def chunked_context_workspace_bytes(batch: int, total_q: int, max_seqlen_q: int, num_heads: int,
                                    chunk_tokens: int) -> int:
    return load_library().mla_prefill_chunked_context_workspace_size(batch, total_q, max_seqlen_q, num_heads,
                                                                      chunk_tokens)


def _check_latent_weights(latent: torch.Tensor, w_kv: torch.Tensor, heads: int) -> None:
    """latent rows [N, 576] (512 latent + 64 rope); W_KV [>= H * 256, 512]."""
    if latent.shape[1] != 576:
        raise ValueError(f"latent must be [rows, 576], got {tuple(latent.shape)}")
    if w_kv.shape[1] != 512 or w_kv.shape[0] < heads * 256:
        raise ValueError(f"w_kv must be [>= {heads * 256}, 512], got {tuple(w_kv.shape)}")


def mla_prefill_chunked_context(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                                latent: torch.Tensor, cu_seqlens_ctx: torch.Tensor, w_kv: torch.Tensor,
                                max_seqlen_q: int, max_seqlen_ctx: int, softmax_scale: float,
                                chunk_tokens: int = 4096, sink: Optional[torch.Tensor] = None,
                                out: Optional[torch.Tensor] = None, return_lse: bool = True,
                                lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """New tokens (q/k/v [T,H,192/192/128] bf16, cu_seqlens_q) over their cached latent context
    (latent [N,576] bf16 rows, cu_seqlens_ctx int32 [B+1]) up-projected by w_kv [H*256, 512] bf16,
    chunk_tokens context positions per sequence at a time. Returns out [T,H,128] bf16 (and lse)."""
    lib = load_library()
    for name, t, d in (("q", q, 3), ("k", k, 3), ("v", v, 3), ("latent", latent, 2), ("w_kv", w_kv, 2)):
        _bf16(name, t, d)
    total_q, heads, _ = q.shape
    for name, t, width in (("q", q, 192), ("k", k, 192), ("v", v, 128)):
        if tuple(t.shape) != (total_q, heads, width):
            raise ValueError(f"{name} must be [{total_q}, {heads}, {width}], got {tuple(t.shape)}")
    batch = _cu_batch("cu_seqlens_q", cu_seqlens_q)
    _int32_vec("cu_seqlens_ctx", cu_seqlens_ctx, batch + 1)
    _check_latent_weights(latent, w_kv, heads)
    _f32_vec("sink", sink, heads)
    _require_cuda(q, k, v, cu_seqlens_q, latent, cu_seqlens_ctx, w_kv, sink, out, lse, workspace)
    if out is None:
        out = torch.empty((total_q, heads, 128), dtype=torch.bfloat16, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((total_q, heads), dtype=torch.float32, device=q.device)
    _check_out_lse(out, lse, total_q, heads, 128)
    ws_bytes = lib.mla_prefill_chunked_context_workspace_size(batch, total_q, max_seqlen_q, heads, chunk_tokens)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    _check("mla_prefill_chunked_context", lib.mla_prefill_chunked_context(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1), _ptr(v), v.stride(0), v.stride(1),
        _ptr(cu_seqlens_q), _ptr(latent), latent.stride(0), _ptr(cu_seqlens_ctx), _ptr(w_kv), w_kv.stride(0),
        batch, total_q, max_seqlen_q, max_seqlen_ctx, heads, chunk_tokens, float(softmax_scale), _ptr(sink),
        _ptr(out), out.stride(0), out.stride(1),
        _ptr(lse), lse.stride(0) if lse is not None else 0, lse.stride(1) if lse is not None else 0,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return (out, lse) if return_lse else out


def mla_latent_upproject(latent: torch.Tensor, cu_seqlens_ctx: torch.Tensor, w_kv: torch.Tensor, num_heads: int,
                         ctx_start: int, chunk_tokens: int):
    """One chunk of cached latent rows -> (k [B*chunk, H, 192], v [B*chunk, H, 128], cu_chunk [B+1])."""
    lib = load_library()
    _bf16("latent", latent, 2)
    _bf16("w_kv", w_kv, 2)
    batch = _cu_batch("cu_seqlens_ctx", cu_seqlens_ctx)
    _check_latent_weights(latent, w_kv, num_heads)
    _require_cuda(latent, cu_seqlens_ctx, w_kv)
    rows = max(batch * chunk_tokens, 1)
    k = torch.empty((rows, num_heads, 192), dtype=torch.bfloat16, device=latent.device)
    v = torch.empty((rows, num_heads, 128), dtype=torch.bfloat16, device=latent.device)
    cu = torch.empty(batch + 1, dtype=torch.int32, device=latent.device)
    _check("mla_latent_upproject", lib.mla_latent_upproject(
        _ptr(latent), latent.stride(0), _ptr(cu_seqlens_ctx), batch, ctx_start, chunk_tokens, _ptr(w_kv),
        w_kv.stride(0), num_heads, _ptr(cu), _ptr(k), _ptr(v), _stream()))
    return k, v, cu


def mla_combine(o_part: torch.Tensor, lse_part: torch.Tensor, num_heads: int,
                sink: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                return_lse: bool = True, lse: Optional[torch.Tensor] = None):
    """Merge partials o_part float32 [S, T*H, Dv] / lse_part float32 [S, T*H] into out bf16
    [T, H, Dv] (and lse float32 [T, H])."""
    lib = load_library()
    if (o_part.dtype != torch.float32 or lse_part.dtype != torch.float32 or o_part.dim() != 3
            or not (o_part.is_contiguous() and lse_part.is_contiguous())):
        raise ValueError("o_part and lse_part must be contiguous float32 tensors")
    s, rows, dv = o_part.shape
    if tuple(lse_part.shape) != (s, rows):
        raise ValueError(f"lse_part must be [{s}, {rows}], got {tuple(lse_part.shape)}")
    if num_heads <= 0 or rows % num_heads != 0:
        raise ValueError(f"the {rows} partial rows are not a whole number of tokens of {num_heads} heads")
    _f32_vec("sink", sink, num_heads)
    _require_cuda(o_part, lse_part, sink, out, lse)
    t = rows // num_heads
    if out is None:
        out = torch.empty((t, num_heads, dv), dtype=torch.bfloat16, device=o_part.device)
    if return_lse and lse is None:
        lse = torch.empty((t, num_heads), dtype=torch.float32, device=o_part.device)
    _check_out_lse(out, lse, t, num_heads, dv)
    _check("mla_combine", lib.mla_combine(
        _ptr(o_part), _ptr(lse_part), s, t, num_heads, dv, _ptr(sink),
        _ptr(out), out.stride(0), out.stride(1),
        _ptr(lse), lse.stride(0) if lse is not None else 0, lse.stride(1) if lse is not None else 0,
        _stream()))
    return (out, lse) if return_lse else out


def profile_enable(enable: bool = True, kinds=None) -> None:
    """Bracket library kernel launches with HIP events on their stream (clears totals): every
    kind, or only the named ones (e.g. ["dense"])."""
    lib = load_library()
    mask = 0xFFFFFFFF if kinds is None else sum(1 << KERNEL_IDS[k] for k in kinds)
    _check("mla_profile_select", lib.mla_profile_select(mask))
    _check("mla_profile_enable", lib.mla_profile_enable(int(bool(enable))))


def profile_read(kernel: str) -> Tuple[float, int]:
    """(total device ms, launches) of one kernel kind since profile_enable(): plan, dense,
    combine, sparse or upproj. Waits for the recorded events."""
    ms, n = ctypes.c_double(), _c_i64()
    _check("mla_profile_read", load_library().mla_profile_read(KERNEL_IDS[kernel], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
