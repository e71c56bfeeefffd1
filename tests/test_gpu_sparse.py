"""GPU parity of the sparse top-k MLA prefill (HIP path through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import make_sparse, f32_to_bf16_bits
from tests.gpu_util import announce, dev_bf16, dev, host_f64, check_parity

pytestmark = pytest.mark.gpu


def run_sparse(c, return_lse=True):
    import torch
    import mla_varlen_prefill_amd as mla
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    idx = dev(c.indices)
    tl = dev(c.topk_length) if c.topk_length is not None else None
    sink = dev(c.sink) if c.sink is not None else None
    res = mla.mla_prefill_sparse(q, kv, idx, c.scale, topk_length=tl, sink=sink, return_lse=return_lse)
    torch.cuda.synchronize()
    if return_lse:
        return host_f64(res[0]), host_f64(res[1])
    return host_f64(res), None


def oracle(c):
    return O.sparse_mla_prefill(c.q, c.kv, c.indices, c.scale, dv=512, topk_length=c.topk_length,
                                sink=c.sink)


@pytest.mark.parametrize("heads", [128, 40, 16, 1])
def test_sparse_small_ragged_topk(heads):
    c = make_sparse(f"sparse_h{heads}", num_tokens=6, heads=heads, n_kv=777, topk=100, seed=41,
                    pad_p=0.1, with_sink=True)
    announce(f"sparse {c.name}")
    o, lse = run_sparse(c)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


def test_sparse_many_tokens_per_work_group():
    """More tokens than the device has CUs, so each persistent work-group computes several tokens
    one after the other (1000 tokens: 3 or 4 per work-group, ranges per XCD that do not divide
    evenly), with token lengths from 0 to the full top-k: each token's softmax state, index window
    and ring start from scratch whatever the previous token of the work-group left. 40 heads
    leave part of a wave and whole waves without a head. Checked in full against the oracle."""
    c = make_sparse("sparse_persist", num_tokens=1000, heads=40, n_kv=5000, topk=192, seed=51,
                    pad_p=0.05, with_sink=True, with_topk_length=True)
    tl = c.topk_length.copy()
    tl[::7] = 0                          # some tokens with no block at all
    tl[3::11] = 192                      # some with every slot
    c.topk_length = tl
    announce(f"sparse {c.name}")
    o, lse = run_sparse(c)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


def test_sparse_many_tokens_two_index_windows():
    """As above with a top-k past one staged index window (2100 slots: a second window is
    staged part-way through each token), 300 tokens over 16 heads."""
    c = make_sparse("sparse_persist_win", num_tokens=300, heads=16, n_kv=20000, topk=2100, seed=52,
                    pad_p=0.05, with_sink=False, with_topk_length=True)
    tl = c.topk_length.copy()
    tl[::5] = 2100
    c.topk_length = tl
    announce(f"sparse {c.name}")
    o, lse = run_sparse(c)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


def test_sparse_topk_length_out_of_range_and_duplicates():
    c = make_sparse("sparse_edges", num_tokens=7, heads=128, n_kv=500, topk=96, seed=42, pad_p=0.05,
                    with_sink=False, with_topk_length=True)
    idx = c.indices.copy()
    idx[0, :] = -1                    # every slot padded
    idx[1, 5] = 500                   # out of range -> skipped
    idx[1, 6] = -7
    idx[2, :10] = idx[2, 10]          # duplicates count once per slot
    c.indices = idx
    c.topk_length = np.array([96, 96, 50, 0, 1, 33, 64], dtype=np.int32)
    announce(f"sparse {c.name}")
    o, lse = run_sparse(c)
    ro, rl = oracle(c)
    assert np.isneginf(rl[0]).all() and np.isneginf(rl[3]).all()
    check_parity(o, lse, ro, rl, c.name)


def test_sparse_all_padded_with_sink():
    c = make_sparse("sparse_allpad", num_tokens=3, heads=128, n_kv=64, topk=64, seed=43, pad_p=0.0,
                    with_sink=True)
    c.indices[:] = -1
    announce(f"sparse {c.name}")
    o, lse = run_sparse(c)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


def test_sparse_wide_logit_range_redoes_the_block():
    """Logits spanning far more than 2^64 in probability: the first block sets a low reference
    logit and a later key exceeds it by 80 nats, so that block's sum would overflow the bound and
    is redone against its exact maximum (the accumulated O and l rescaled): the result must still
    be the definition's."""
    c = make_sparse("sparse_wide", num_tokens=2, heads=128, n_kv=300, topk=128, seed=44, pad_p=0.0,
                    with_sink=True)
    kv = np.zeros((300, 576), dtype=np.float32)
    kv[:, :512] = np.random.default_rng(1).standard_normal((300, 512))
    kv[:, 512] = 1.0
    q = np.zeros((2, 128, 576), dtype=np.float32)
    q[:, :, 512] = 2.0
    c.indices = np.tile(np.arange(128, dtype=np.int32), (2, 1))
    big = c.indices[0, 100]
    kv[big, 512] = 41.0               # logit 82 vs 2 for the others (scale 1)
    c.kv = f32_to_bf16_bits(kv)
    c.q = f32_to_bf16_bits(q)
    c.scale = 1.0
    announce(f"sparse {c.name}")
    o, lse = run_sparse(c)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


def test_sparse_invalid_slots_read_no_pool_bytes():
    """Padded (-1), negative and out-of-range indices contribute nothing, whatever the pool holds:
    here row 0 and every unreferenced row are NaN, and the pool is a strided view whose gap
    columns are NaN too. The result is the oracle's over the valid slots only."""
    import torch
    import mla_varlen_prefill_amd as mla
    c = make_sparse("sparse_nan_pool", num_tokens=5, heads=128, n_kv=600, topk=160, seed=49, pad_p=0.2,
                    with_sink=True)
    n = c.kv.shape[0]
    idx = c.indices.copy()
    idx[idx == 0] = 1                      # row 0 is never a valid slot
    idx[0, 3], idx[1, 7], idx[2, 11], idx[3, 0] = n, n + 100, 2 ** 31 - 1, -5
    c.indices = idx
    used = np.unique(idx[(idx >= 0) & (idx < n)])
    wide = torch.full((n, 640), float("nan"), dtype=torch.bfloat16, device="cuda")
    wide[torch.from_numpy(used).cuda(), :576] = dev_bf16(c.kv)[torch.from_numpy(used).cuda()]
    pool = wide[:, :576]
    announce(f"sparse {c.name}")
    o, lse = mla.mla_prefill_sparse(dev_bf16(c.q), pool, dev(c.indices), c.scale, sink=dev(c.sink))
    torch.cuda.synchronize()
    ro, rl = oracle(c)
    check_parity(host_f64(o), host_f64(lse), ro, rl, c.name)


def test_sparse_deterministic_no_lse():
    c = make_sparse("sparse_det", num_tokens=4, heads=128, n_kv=2000, topk=256, seed=45)
    announce(f"sparse {c.name}")
    o1, l1 = run_sparse(c)
    o2, _ = run_sparse(c, return_lse=False)
    assert np.array_equal(o1, o2)
    ro, rl = oracle(c)
    check_parity(o1, l1, ro, rl, c.name)


@pytest.mark.parametrize("topk", [200, 2500])
def test_sparse_slot_permutation_invariance(topk):
    """Each index slot counts independently (page "SparseFlashMla", formula over the participating
    KV; -1 = padded slot), so permuting the slots of every token's row, pads included, leaves the
    result unchanged up to summation order: the permuted call agrees with the oracle of the
    original rows and with the unpermuted call within the tolerances. topk 2500 crosses the
    kernel's staged index windows, so slots move between windows."""
    import torch
    c = make_sparse(f"sparse_perm_k{topk}", num_tokens=6, heads=128, n_kv=4000, topk=topk, seed=48,
                    pad_p=0.1, with_sink=True)
    announce(f"sparse {c.name}")
    o1, l1 = run_sparse(c)
    ro, rl = oracle(c)
    rng = np.random.default_rng(49)
    perm = c.indices.copy()
    for t in range(perm.shape[0]):
        perm[t] = perm[t][rng.permutation(topk)]
    assert not np.array_equal(perm, c.indices)
    c.indices = perm
    o2, l2 = run_sparse(c)
    check_parity(o2, l2, ro, rl, f"{c.name} permuted vs oracle of the original rows")
    check_parity(o2, l2, o1, l1, f"{c.name} permuted vs unpermuted")


def test_sparse_strided_views():
    """Q, the latent pool, the index rows, the output and the LSE as strided views into larger
    buffers: the result matches the oracle and no byte outside the output view changes."""
    import torch
    import mla_varlen_prefill_amd as mla
    c = make_sparse("sparse_views", num_tokens=5, heads=24, n_kv=500, topk=96, seed=47, pad_p=0.1,
                    with_sink=True)
    announce(f"sparse {c.name}")
    t, h, _ = c.q.shape
    n = c.kv.shape[0]
    qb = torch.full((t, h, 640), 2.0, dtype=torch.bfloat16, device="cuda")
    qb[:, :, 64:] = dev_bf16(c.q)
    kvb = torch.full((n, 640), -4.0, dtype=torch.bfloat16, device="cuda")
    kvb[:, :576] = dev_bf16(c.kv)
    ib = torch.full((t, 104), 0, dtype=torch.int32, device="cuda")
    ib[:, :96] = dev(c.indices)
    ob = torch.full((t, h, 520), 9.0, dtype=torch.bfloat16, device="cuda")
    lb = torch.full((h, t), 1.5, dtype=torch.float32, device="cuda")
    q, kv, idx, out, lse = qb[:, :, 64:], kvb[:, :576], ib[:, :96], ob[:, :, 8:], lb.t()
    mla.mla_prefill_sparse(q, kv, idx, c.scale, sink=dev(c.sink), out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle(c)
    check_parity(host_f64(out), host_f64(lse), ro, rl, c.name)
    assert torch.all(ob[:, :, :8] == 9.0)
