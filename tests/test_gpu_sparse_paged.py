"""GPU parity of the sparse top-k MLA prefill over a paged latent cache (HIP path through the C ABI)
against the fp64 oracle (logical indices through a block table, seqused, cu_seqlens_q)."""
import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import make_sparse_paged, device_sparse_paged, bf16_tensor_to_bits
from tests.gpu_util import announce, dev_bf16, dev, host_f64, check_parity

pytestmark = pytest.mark.gpu


def run_paged(c, seqused_q=None):
    import torch
    import mla_varlen_prefill_amd as mla
    q, cache = dev_bf16(c.q), dev_bf16(c.kv_cache)
    res = mla.mla_prefill_sparse_paged(
        q, cache, dev(c.block_table), dev(c.cu_q), dev(c.indices), c.scale,
        seqused_kv=dev(c.seqused) if c.seqused is not None else None,
        topk_length=dev(c.topk_length) if c.topk_length is not None else None,
        sink=dev(c.sink) if c.sink is not None else None,
        seqused_q=dev(np.asarray(seqused_q, dtype=np.int32)) if seqused_q is not None else None)
    torch.cuda.synchronize()
    return host_f64(res[0]), host_f64(res[1])


def oracle(c, seqused_q=None):
    return O.sparse_mla_prefill_paged(c.q, c.kv_cache, c.block_table, c.cu_q, c.indices, c.scale,
                                      dv=512, seqused=c.seqused, topk_length=c.topk_length, sink=c.sink,
                                      seqused_q=seqused_q)


@pytest.mark.parametrize("block_size", [1, 16, 64, 100])
def test_paged_ragged_sequences(block_size):
    """Three sequences of ragged KV length (one of a single position), shuffled blocks, seqused,
    topk_length, sink, logical positions past the used length and -1 pads; 2048-slot rows so the
    index window is restaged."""
    c = make_sparse_paged(f"paged_bs{block_size}", [1300, 1, 3000], [3, 2, 4], 128, 2100, block_size,
                          seed=60 + block_size, with_topk_length=True)
    announce(f"sparse paged {c.name}")
    o, lse = run_paged(c)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


def test_paged_many_tokens_per_work_group():
    """More tokens than the device has CUs over 9 sequences (one empty, one with a single cached
    position), so a persistent work-group's consecutive tokens can belong to different sequences:
    each token finds its own block-table row, used length and seqused_q state; seqused_q drops
    part of three sequences. Checked in full against the oracle."""
    lens_kv = [900, 1, 2500, 0, 64, 1700, 333, 4000, 128]
    n_tok = [120, 30, 150, 0, 45, 140, 99, 190, 86]
    c = make_sparse_paged("paged_persist", lens_kv, n_tok, 32, 160, 16, seed=90, with_topk_length=True)
    used_q = [120, 30, 100, 0, 0, 140, 99, 37, 86]
    announce(f"sparse paged {c.name}")
    o, lse = run_paged(c, used_q)
    ro, rl = oracle(c, used_q)
    check_parity(o, lse, ro, rl, c.name)


@pytest.mark.parametrize("with_sink", [False, True])
def test_paged_seqused_q(with_sink):
    """seqused_q: only the first seqused_q[b] tokens of each sequence are in use; the others are
    written as rows without keys (O = 0, LSE = -inf or the sink). Counts of 0, partial and full."""
    c = make_sparse_paged("paged_seqused_q", [700, 40, 300], [5, 3, 4], 128, 300, 16, seed=80,
                          with_sink=with_sink)
    used_q = [2, 0, 4]
    announce(f"sparse paged seqused_q sink={with_sink}")
    o, lse = run_paged(c, used_q)
    ro, rl = oracle(c, used_q)
    check_parity(o, lse, ro, rl, "paged seqused_q")
    for b in range(3):
        drop = slice(int(c.cu_q[b]) + used_q[b], int(c.cu_q[b + 1]))
        assert np.all(o[drop] == 0)


def test_paged_edges_bad_table_entries_empty_sequence_and_stray_token():
    """No seqused (whole allocated blocks count), table entries of -1 and past num_blocks, an empty
    sequence in the middle, 40 heads, and one token past cu_seqlens_q[-1] (no valid slot)."""
    c = make_sparse_paged("paged_edges", [200, 0, 90], [3, 0, 2], 40, 64, 16, seed=70,
                          with_seqused=False, with_sink=False)
    c.block_table[0, 2] = -1
    c.block_table[2, 1] = c.kv_cache.shape[0] + 3
    # one stray token past the last sequence, with in-range positions
    extra_q = np.random.default_rng(71).standard_normal((1, 40, 576)).astype(np.float32)
    from workloads import f32_to_bf16_bits
    c.q = np.concatenate([c.q, f32_to_bf16_bits(extra_q)])
    c.indices = np.concatenate([c.indices, np.arange(64, dtype=np.int32)[None, :]])
    announce(f"sparse paged {c.name}")
    o, lse = run_paged(c)
    ro, rl = oracle(c)
    assert np.isneginf(rl[-1]).all()
    check_parity(o, lse, ro, rl, c.name)


def test_paged_full_size_matches_physical_rows_and_oracle():
    """The 4096-token, top-2048 workload over a 65536-row pool split into 1024 shuffled pages of 64:
    bit-identical to the physical-row call on the unpaged rows (same rows, same slot order), and
    within tolerance of the oracle on sampled tokens."""
    import torch
    import mla_varlen_prefill_amd as mla
    announce("sparse paged full size t4096 h128 topk2048 pool65536 bs64")
    t, h, n_kv, topk, bs = 4096, 128, 65536, 2048, 64
    q, kv, cache, table, cu_q, idx, sink, idx_host = device_sparse_paged(t, h, n_kv, topk, bs, seed=5)
    scale = 576 ** -0.5
    o_p = torch.full((t, h, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    l_p = torch.full((t, h), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_prefill_sparse_paged(q, cache, table, cu_q, idx, scale, sink=sink, out=o_p, lse=l_p)
    o_r, l_r = mla.mla_prefill_sparse(q, kv, idx, scale, sink=sink)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(o_p).any()) and not bool(torch.isnan(l_p).any()), "rows never written"
    assert torch.equal(o_p.view(torch.int16), o_r.view(torch.int16))
    assert torch.equal(l_p, l_r)
    toks = [0, 1, 2047, 4095]
    q_bits = bf16_tensor_to_bits(q[toks])
    rows = np.unique(idx_host[toks][(idx_host[toks] >= 0)])
    kv_bits = np.zeros((n_kv, 576), dtype=np.uint16)
    kv_bits[rows] = bf16_tensor_to_bits(kv[torch.from_numpy(rows).cuda().long()])
    ro, rl = O.sparse_mla_prefill(q_bits, kv_bits, idx_host[toks], scale, dv=512, sink=sink.cpu().numpy())
    check_parity(host_f64(o_p[toks]), host_f64(l_p[toks]), ro, rl, "paged full size sampled")
    del q, kv, cache, o_p, o_r
    torch.cuda.empty_cache()
