"""Full-size parity of the dense and sparse paths at the workloads' real shapes, in the launch
configuration the benchmark times (num_splits = 0, default persistent grid), plus forced splits.

Two checks per run:
  * every output row is written: O and LSE are filled with NaN before the call and no NaN may
    survive (every row of these workloads sees at least one key, so every LSE is also finite);
  * every work item is right: for each (query tile, head) item of the checked heads, one row of
    each 32-row wave slab of the tile (the tile's last row always among them, so the diagonal is
    covered) is compared with the fp64 oracle.
The workloads are those of page "FlashAttention backend for MLA prefill": new tokens attending
causally to themselves (run_prefill_new_tokens, cu_seqlens_q = cu_seqlens_k) over a batch of
ragged sequences and over one 32K sequence, and new tokens over a longer prefix (bottom-right
causal); and the sparse top-k workload of page "SparseFlashMla" (formula; -1 = padded slot).
"""
import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import (device_dense, device_sparse, bf16_tensor_to_bits, cu_from_lens, varlen_lens,
                       CHUNKED_SK)
from tests.gpu_util import announce, host_f64, check_parity

pytestmark = pytest.mark.gpu

SLAB = 32  # query rows per wave


def item_rows(lens_q, bm, seed):
    """Global query rows: per sequence and query tile, one row in each 32-row wave slab of the tile
    that holds rows of the sequence (the tile's last row for the last slab). Tiles are aligned to
    the sequence end: local row r of tile m is sequence row m*bm - pad + r, pad = ceil(sq/bm)*bm - sq."""
    rng = np.random.default_rng(seed)
    cu = cu_from_lens(lens_q)
    rows = []
    for b, sq in enumerate(lens_q):
        pad = -(-sq // bm) * bm - sq
        for m in range(-(-sq // bm)):
            row0 = m * bm - pad
            for w in range(bm // SLAB):
                lo, hi = max(w * SLAB, -row0), (w + 1) * SLAB
                if lo >= hi:
                    continue
                r = hi - 1 if hi == bm else int(rng.integers(lo, hi))
                rows.append(int(cu[b]) + row0 + r)
    return np.asarray(sorted(set(rows)), dtype=np.int64)


def _nan_outputs(t, h, dv):
    import torch
    out = torch.full((t, h, dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((t, h), float("nan"), dtype=torch.float32, device="cuda")
    return out, lse


def _assert_all_written(out, lse, tag):
    import torch
    n_o = int(torch.isnan(out).sum())
    n_l = int(torch.isnan(lse).sum())
    assert n_o == 0 and n_l == 0, f"{tag}: {n_o} O values and {n_l} LSE values never written"
    assert bool(torch.isfinite(lse).all()), f"{tag}: non-finite LSE"


def dense_full_size(lens_q, lens_k, heads, seed, num_splits, check_heads, head_group=16):
    import torch
    import mla_varlen_prefill_amd as mla
    bm, _ = mla.dense_tile_shape()
    q, k, v, cu_q, cu_k = device_dense(lens_q, lens_k, heads, seed)
    scale = float(np.float32(192 ** -0.5))
    out, lse = _nan_outputs(q.shape[0], heads, 128)
    mla.mla_prefill_varlen(q, k, v, cu_q, cu_k, max(lens_q), max(lens_k), scale, causal=True,
                           num_splits=num_splits, out=out, lse=lse)
    torch.cuda.synchronize()
    tag = f"full-size {lens_q[:2]}.. H={heads} splits={num_splits}"
    _assert_all_written(out, lse, tag)
    rows = item_rows(lens_q, bm, seed)
    rows_dev = torch.from_numpy(rows).cuda()
    cq, ck = cu_from_lens(lens_q), cu_from_lens(lens_k)
    worst = 0.0
    for g in range(0, len(check_heads), head_group):
        hs = list(check_heads[g:g + head_group])
        hs_dev = torch.tensor(hs, device="cuda")
        qb = np.zeros((q.shape[0], len(hs), 192), dtype=np.uint16)
        qb[rows] = bf16_tensor_to_bits(q[rows_dev][:, hs_dev])
        kb = bf16_tensor_to_bits(k[:, hs_dev])
        vb = bf16_tensor_to_bits(v[:, hs_dev])
        ro, rl = O.dense_mla_prefill_rows(qb, kb, vb, cq, ck, scale, True, rows, list(range(len(hs))))
        og = host_f64(out[rows_dev][:, hs_dev])
        lg = host_f64(lse[rows_dev][:, hs_dev])
        worst = max(worst, check_parity(og, lg, ro, rl, f"{tag} heads {hs[0]}..{hs[-1]}"))
    announce(f"{tag}: {rows.size} rows x {len(check_heads)} heads checked, O max-abs {worst:.2e}")
    del q, k, v, out, lse
    torch.cuda.empty_cache()


def test_full_size_headline_batch_every_item():
    """8 ragged sequences (lengths uniform in [64, 2048]), 128 heads: every item of every head."""
    lens = varlen_lens(2, 8, 64, 2048)
    announce(f"dense full size varlen b8 h128 lens={lens}")
    dense_full_size(lens, lens, 128, 2, 0, list(range(128)))


def test_full_size_long_context_every_item():
    """One 32768-token sequence, 128 heads, the launch the benchmark times: every item of 17 heads
    spread over all eight XCDs' head ranges (two per XCD plus the last head)."""
    announce("dense full size 1x32768 h128 splits=auto")
    dense_full_size([32768], [32768], 128, 3, 0, list(range(0, 128, 8)) + [127])


@pytest.mark.parametrize("num_splits", [2, 4])
def test_full_size_long_context_forced_splits(num_splits):
    """The same sequence with the keys split and combined: all rows written, every item of 4 heads."""
    announce(f"dense full size 1x32768 h128 splits={num_splits}")
    dense_full_size([32768], [32768], 128, 3, num_splits, [0, 45, 90, 127])


def test_full_size_chunked_prefill_every_item():
    """4 x 2048 new tokens over 16384 / 12345 / 8191 / 4097 keys (bottom-right causal): every item
    of all 128 heads."""
    announce("dense full size chunked b4 q2048 h128")
    dense_full_size([2048] * 4, list(CHUNKED_SK), 128, 4, 0, list(range(128)))


def test_full_size_sparse_all_rows_written_and_sampled_tokens():
    """4096 tokens x 128 heads, top-2048 of a 65536-row pool (~5 % padded), sink: every row written,
    and 512 tokens spread over the batch (all heads each) against the oracle."""
    import torch
    import mla_varlen_prefill_amd as mla
    announce("sparse full size t4096 h128 topk2048 pool65536")
    t, h, n_kv, topk = 4096, 128, 65536, 2048
    q, kv, idx, sink, idx_host = device_sparse(t, h, n_kv, topk, seed=5)
    scale = float(np.float32(576 ** -0.5))
    out = torch.full((t, h, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((t, h), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_prefill_sparse(q, kv, idx, scale, sink=sink, out=out, lse=lse)
    torch.cuda.synchronize()
    _assert_all_written(out, lse, "sparse full size")
    toks = np.unique(np.concatenate([np.arange(0, t, 8), [1, 2, t - 1]]))
    kv_bits = bf16_tensor_to_bits(kv)
    q_bits = bf16_tensor_to_bits(q[torch.from_numpy(toks).cuda()])
    ro, rl = O.sparse_mla_prefill(q_bits, kv_bits, idx_host[toks], scale, dv=512, sink=sink.cpu().numpy())
    err = check_parity(host_f64(out[torch.from_numpy(toks).cuda()]), host_f64(lse[torch.from_numpy(toks).cuda()]),
                       ro, rl, "sparse full size sampled")
    announce(f"sparse full size: {toks.size} tokens x {h} heads checked, O max-abs {err:.2e}")
    del q, kv, idx, out, lse
    torch.cuda.empty_cache()
