"""GPU parity of the sparse top-k MLA prefill (HIP path through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import make_sparse, device_sparse, bf16_tensor_to_bits, f32_to_bf16_bits
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


def test_sparse_wide_logit_range_takes_second_pass():
    """Logits spanning far more than 2^32 in probability: the first block sets a low reference
    max and a later key exceeds it by ~40 nats, which the kernel must handle exactly."""
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


def test_sparse_deterministic_no_lse():
    c = make_sparse("sparse_det", num_tokens=4, heads=128, n_kv=2000, topk=256, seed=45)
    announce(f"sparse {c.name}")
    o1, l1 = run_sparse(c)
    o2, _ = run_sparse(c, return_lse=False)
    assert np.array_equal(o1, o2)
    ro, rl = oracle(c)
    check_parity(o1, l1, ro, rl, c.name)


def test_sparse_full_size_sampled_tokens():
    import torch
    import mla_varlen_prefill_amd as mla
    announce("sparse full size t4096 h128 topk2048 pool65536")
    q, kv, idx, sink, idx_host = device_sparse(4096, 128, 65536, 2048, seed=5)
    scale = 576 ** -0.5
    out, lse = mla.mla_prefill_sparse(q, kv, idx, scale, sink=sink)
    torch.cuda.synchronize()
    toks = [0, 1, 2047, 4094, 4095]
    qb = bf16_tensor_to_bits(q[toks])
    kvb = bf16_tensor_to_bits(kv)
    ro, rl = O.sparse_mla_prefill(qb, kvb, idx_host[toks], float(np.float32(scale)), dv=512,
                                  sink=sink.cpu().numpy())
    check_parity(host_f64(out[toks]), host_f64(lse[toks]), ro, rl, "sparse full size")


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
