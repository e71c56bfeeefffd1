"""Seeded synthetic inputs for MLA prefill, shared by the tests, the bench and the oracle's callers.

This module only draws random numbers and lays them out. It holds none of the attention
arithmetic: no scores, no masks, no softmax. Both the HIP path and the CPU oracle consume the
exact bf16 bit patterns produced here (stored as ``uint16``), so the two sides see identical
inputs.

Recipe (one generator per (config, stream)): ``numpy.random.default_rng([config_id, stream])``
with stream 0 = sequence lengths / indices, 1 = Q, 2 = K (or the latent KV pool), 3 = V,
4 = sink logits, 5 = the -1 pad mask of the sparse indices. Normal values are drawn as float32
``standard_normal`` and rounded to bf16 with round-to-nearest-even.

The workloads follow the shapes the pages describe: the vLLM MLA-prefill backend expands K/V to
all heads with a 192-wide q/k head (128 "nope" + 64 rope) and a 128-wide v head, indexed by
``cu_seqlens`` (page "FlashAttention backend for MLA prefill", ``dispatch``); the sparse path reads
one shared latent KV of 576 columns through int32 top-k indices where -1 marks a padded slot
(page "SparseFlashMla", Parameters table, ``ori_sparse_indices``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

DQK_DENSE = 192
DV_DENSE = 128
DQK_SPARSE = 576
DV_SPARSE = 512

STREAM_LENS, STREAM_Q, STREAM_K, STREAM_V, STREAM_SINK, STREAM_PAD = 0, 1, 2, 3, 4, 5


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def randn_bf16(rng: np.random.Generator, shape: Sequence[int], chunk: int = 1 << 26) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16 bits, generated in chunks to bound host memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def cu_from_lens(lens: Sequence[int]) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)


@dataclass
class DenseCase:
    name: str
    q: np.ndarray          # uint16 bf16 bits [total_q, H, 192]
    k: np.ndarray          # uint16 bf16 bits [total_k, H, 192]
    v: np.ndarray          # uint16 bf16 bits [total_k, H, 128]
    cu_q: np.ndarray       # int32 [B+1]
    cu_k: np.ndarray       # int32 [B+1]
    scale: float
    causal: bool
    sink: Optional[np.ndarray] = None   # float32 [H]
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.cu_q) - 1

    @property
    def heads(self) -> int:
        return self.q.shape[1]

    @property
    def max_q(self) -> int:
        return int(np.max(np.diff(self.cu_q))) if self.batch else 0

    @property
    def max_k(self) -> int:
        return int(np.max(np.diff(self.cu_k))) if self.batch else 0


@dataclass
class SparseCase:
    name: str
    q: np.ndarray          # uint16 bf16 bits [T, H, 576]
    kv: np.ndarray         # uint16 bf16 bits [N_kv, 576]  (V = first 512 columns)
    indices: np.ndarray    # int32 [T, topk]
    scale: float
    topk_length: Optional[np.ndarray] = None  # int32 [T]
    sink: Optional[np.ndarray] = None         # float32 [H]
    meta: dict = field(default_factory=dict)


def make_dense(name: str, lens_q: Sequence[int], lens_k: Sequence[int], heads: int, causal: bool,
               seed: int, with_sink: bool = False, scale: Optional[float] = None,
               dqk: int = DQK_DENSE, dv: int = DV_DENSE) -> DenseCase:
    """Dense varlen case: Q/K/V ~ N(0,1) rounded to bf16, contiguous [tokens, heads, dim]."""
    cu_q, cu_k = cu_from_lens(lens_q), cu_from_lens(lens_k)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = randn_bf16(np.random.default_rng([seed, STREAM_Q]), (tq, heads, dqk))
    k = randn_bf16(np.random.default_rng([seed, STREAM_K]), (tk, heads, dqk))
    v = randn_bf16(np.random.default_rng([seed, STREAM_V]), (tk, heads, dv))
    sink = None
    if with_sink:
        sink = np.random.default_rng([seed, STREAM_SINK]).standard_normal(heads, dtype=np.float32)
    if scale is None:
        scale = float(dqk) ** -0.5
    return DenseCase(name, q, k, v, cu_q, cu_k, float(np.float32(scale)), causal, sink)


def varlen_lens(seed: int, batch: int, lo: int, hi: int) -> list:
    """Sequence lengths uniform in [lo, hi] (inclusive), from the lengths stream."""
    rng = np.random.default_rng([seed, STREAM_LENS])
    return [int(x) for x in rng.integers(lo, hi + 1, size=batch)]


def sparse_indices(seed: int, num_tokens: int, n_kv: int, topk: int, pad_p: float) -> np.ndarray:
    """Causal-valid top-k indices for one sequence whose last ``num_tokens`` positions are queries.

    Token t sits at absolute position p_t = n_kv - num_tokens + t and draws ``topk`` distinct rows
    uniformly from [0, p_t] (unsorted). Each slot then independently becomes -1 with probability
    ``pad_p``.
    """
    rng = np.random.default_rng([seed, STREAM_LENS])
    out = np.empty((num_tokens, topk), dtype=np.int32)
    for t in range(num_tokens):
        p = n_kv - num_tokens + t
        if p + 1 <= topk:
            row = rng.permutation(p + 1)
            row = np.concatenate([row, -np.ones(topk - row.size, dtype=np.int64)])
        else:
            picked = np.unique(rng.integers(0, p + 1, size=topk + topk // 8 + 16))
            while picked.size < topk:
                picked = np.unique(np.concatenate([picked, rng.integers(0, p + 1, size=topk)]))
            row = rng.permutation(picked)[:topk]
        out[t] = row
    if pad_p > 0:
        pad = np.random.default_rng([seed, STREAM_PAD]).random((num_tokens, topk)) < pad_p
        out[pad] = -1
    return out


def make_sparse(name: str, num_tokens: int, heads: int, n_kv: int, topk: int, seed: int,
                pad_p: float = 0.05, with_sink: bool = True, with_topk_length: bool = False,
                scale: Optional[float] = None, dqk: int = DQK_SPARSE) -> SparseCase:
    q = randn_bf16(np.random.default_rng([seed, STREAM_Q]), (num_tokens, heads, dqk))
    kv = randn_bf16(np.random.default_rng([seed, STREAM_K]), (n_kv, dqk))
    idx = sparse_indices(seed, num_tokens, n_kv, topk, pad_p)
    sink = None
    if with_sink:
        sink = np.random.default_rng([seed, STREAM_SINK]).standard_normal(heads, dtype=np.float32)
    tl = None
    if with_topk_length:
        tl = np.random.default_rng([seed, STREAM_PAD + 1]).integers(0, topk + 1, size=num_tokens).astype(np.int32)
    if scale is None:
        scale = float(dqk) ** -0.5
    return SparseCase(name, q, kv, idx, float(np.float32(scale)), tl, sink)


@dataclass
class PagedSparseCase:
    name: str
    q: np.ndarray            # uint16 bf16 bits [T, H, 576]
    kv_cache: np.ndarray     # uint16 bf16 bits [num_blocks, block_size, 576]
    block_table: np.ndarray  # int32 [B, max_blocks]
    cu_q: np.ndarray         # int32 [B+1]
    indices: np.ndarray      # int32 [T, topk] logical positions of each token's sequence
    scale: float
    seqused: Optional[np.ndarray] = None      # int32 [B]
    topk_length: Optional[np.ndarray] = None  # int32 [T]
    sink: Optional[np.ndarray] = None         # float32 [H]
    meta: dict = field(default_factory=dict)


def make_sparse_paged(name: str, lens_kv: Sequence[int], n_tok: Sequence[int], heads: int, topk: int,
                      block_size: int, seed: int, pad_p: float = 0.05, spare_blocks: int = 3,
                      with_seqused: bool = True, with_sink: bool = True,
                      with_topk_length: bool = False) -> PagedSparseCase:
    """Paged latent cache: sequence b owns ceil(lens_kv[b] / block_size) blocks drawn from a
    shuffled pool that also holds `spare_blocks` never-referenced blocks; unused table entries are
    -1. Token rows of sequence b draw logical positions uniformly from [-1, lens_kv[b] + 2] (so
    some are padded or past the used length), then each slot is padded with probability pad_p."""
    rng = np.random.default_rng([seed, STREAM_LENS])
    blocks = [(n + block_size - 1) // block_size for n in lens_kv]
    max_blocks = max(1, max(blocks))
    nb = sum(blocks) + spare_blocks
    perm = rng.permutation(nb)
    table = np.full((len(lens_kv), max_blocks), -1, dtype=np.int32)
    used = 0
    for b, nblk in enumerate(blocks):
        table[b, :nblk] = perm[used:used + nblk]
        used += nblk
    cache = randn_bf16(np.random.default_rng([seed, STREAM_K]), (nb, block_size, DQK_SPARSE))
    cu_q = cu_from_lens(n_tok)
    t = int(cu_q[-1])
    idx = np.empty((t, topk), dtype=np.int32)
    for b, n in enumerate(lens_kv):
        for ti in range(int(cu_q[b]), int(cu_q[b + 1])):
            idx[ti] = rng.integers(-1, n + 3, size=topk)
    if pad_p > 0:
        idx[np.random.default_rng([seed, STREAM_PAD]).random(idx.shape) < pad_p] = -1
    q = randn_bf16(np.random.default_rng([seed, STREAM_Q]), (t, heads, DQK_SPARSE))
    sink = None
    if with_sink:
        sink = np.random.default_rng([seed, STREAM_SINK]).standard_normal(heads, dtype=np.float32)
    tl = None
    if with_topk_length:
        tl = np.random.default_rng([seed, STREAM_PAD + 1]).integers(0, topk + 1, size=t).astype(np.int32)
    seqused = np.asarray(lens_kv, dtype=np.int32) if with_seqused else None
    return PagedSparseCase(name, q, cache, table, cu_q, idx, float(np.float32(DQK_SPARSE ** -0.5)),
                           seqused, tl, sink)


# --------------------------------------------------------------------------------------------
# The five workloads (shapes from the pages' serving use: vLLM MLA prefill with K/V expanded to
# 128 heads; absorbed sparse MLA over one latent head). Each is generated on demand.
# --------------------------------------------------------------------------------------------
CHUNKED_SK = (16384, 12345, 8191, 4097)


def dense_small(seed: int = 1) -> DenseCase:
    """B=1, Sq=Sk=128, 16 heads, causal, O+LSE."""
    return make_dense("dense_small_1x128_h16", [128], [128], 16, True, seed)


def dense_varlen(seed: int = 2, heads: int = 128) -> DenseCase:
    """B=8 sequences with lengths uniform in [64, 2048], Sq=Sk, 128 heads, causal."""
    lens = varlen_lens(seed, 8, 64, 2048)
    c = make_dense("dense_varlen_b8_h128", lens, lens, heads, True, seed)
    c.meta["lens"] = lens
    return c


def dense_long(seed: int = 3, heads: int = 128, seqlen: int = 32768) -> DenseCase:
    """B=1, Sq=Sk=32768, 128 heads, causal."""
    return make_dense(f"dense_long_1x{seqlen}_h{heads}", [seqlen], [seqlen], heads, True, seed)


def dense_chunked(seed: int = 4, heads: int = 128) -> DenseCase:
    """B=4, 2048 new query tokens each against Sk = 16384/12345/8191/4097 keys, bottom-right causal."""
    return make_dense("dense_chunked_b4_q2048", [2048] * 4, list(CHUNKED_SK), heads, True, seed)


def sparse_topk(seed: int = 5, num_tokens: int = 4096, heads: int = 128, n_kv: int = 65536,
                topk: int = 2048) -> SparseCase:
    """4096 query tokens x 128 heads over a 65536-row latent pool, top-k 2048, ~5% -1, fp32 sink."""
    return make_sparse(f"sparse_t{num_tokens}_h{heads}_k{topk}", num_tokens, heads, n_kv, topk, seed)


# --------------------------------------------------------------------------------------------
# On-device generation for the full-size workloads (hundreds of millions of values). Same value
# distribution (N(0,1) rounded to bf16 by round-to-nearest-even), drawn by a seeded PyTorch
# generator on the GPU; the oracle receives copies of exactly the rows it evaluates.
# --------------------------------------------------------------------------------------------
def device_randn_bf16(shape, seed: int, stream: int, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(stream))
    out = torch.empty(tuple(shape), dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    chunk = 1 << 27
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        flat[s:e] = torch.randn(e - s, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
    return out


def device_dense(lens_q, lens_k, heads: int, seed: int, device="cuda",
                 dqk: int = DQK_DENSE, dv: int = DV_DENSE):
    """Full-size dense inputs on the device: (q, k, v, cu_q, cu_k) as torch tensors."""
    import torch
    cu_q, cu_k = cu_from_lens(lens_q), cu_from_lens(lens_k)
    q = device_randn_bf16((int(cu_q[-1]), heads, dqk), seed, STREAM_Q, device)
    k = device_randn_bf16((int(cu_k[-1]), heads, dqk), seed, STREAM_K, device)
    v = device_randn_bf16((int(cu_k[-1]), heads, dv), seed, STREAM_V, device)
    return q, k, v, torch.from_numpy(cu_q).to(device), torch.from_numpy(cu_k).to(device)


def device_sparse(num_tokens: int, heads: int, n_kv: int, topk: int, seed: int, pad_p: float = 0.05,
                  device="cuda", dqk: int = DQK_SPARSE):
    """Full-size sparse inputs: q/kv drawn on the device, indices from ``sparse_indices`` (host,
    numpy, seeded) copied over, sink float32 [H]. Returns (q, kv, idx, sink, idx_host)."""
    import torch
    q = device_randn_bf16((num_tokens, heads, dqk), seed, STREAM_Q, device)
    kv = device_randn_bf16((n_kv, dqk), seed, STREAM_K, device)
    idx_host = sparse_indices(seed, num_tokens, n_kv, topk, pad_p)
    sink = np.random.default_rng([seed, STREAM_SINK]).standard_normal(heads, dtype=np.float32)
    return q, kv, torch.from_numpy(idx_host).to(device), torch.from_numpy(sink).to(device), idx_host


def device_sparse_paged(num_tokens: int, heads: int, n_kv: int, topk: int, block_size: int, seed: int,
                        pad_p: float = 0.05, device="cuda"):
    """The full-size sparse workload laid out as a paged cache: the latent rows of
    ``device_sparse`` (one sequence of n_kv positions) scattered over n_kv / block_size blocks in
    a seeded random order, with the block table of that order; the indices of ``device_sparse``
    become logical positions. Returns (q, kv_rows, cache, block_table, cu_q, idx, sink, idx_host):
    kv_rows are the unpaged rows, so the paged call must reproduce the physical-row call."""
    import torch
    assert n_kv % block_size == 0
    q, kv, idx, sink, idx_host = device_sparse(num_tokens, heads, n_kv, topk, seed, pad_p, device)
    nb = n_kv // block_size
    perm = np.random.default_rng([seed, STREAM_LENS + 7]).permutation(nb).astype(np.int32)
    cache = torch.empty((nb, block_size, kv.shape[1]), dtype=kv.dtype, device=device)
    cache[torch.from_numpy(perm).to(device).long()] = kv.view(nb, block_size, kv.shape[1])
    table = torch.from_numpy(perm[None, :].copy()).to(device)
    cu_q = torch.tensor([0, num_tokens], dtype=torch.int32, device=device)
    return q, kv, cache, table, cu_q, idx, sink, idx_host


def bf16_tensor_to_bits(t) -> np.ndarray:
    """Copy a torch bf16 tensor to the host as uint16 bit patterns (for the oracle)."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
