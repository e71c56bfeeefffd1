"""GPU parity at the size limits of the HIP path (through the C ABI, against the fp64 oracle):
sparse top-k past one staged index window up to the largest top-k (8192), with and without
topk_length; latent pools near and beyond 4 GiB; dense sequences far longer than the tile and
split sizes; and the largest head count of the sparse path (128) with a single query token."""
import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import make_sparse, make_dense
from tests.gpu_util import announce, dev_bf16, dev, host_f64, check_parity

pytestmark = pytest.mark.gpu


def _sparse(c):
    import torch
    import mla_varlen_prefill_amd as mla
    tl = dev(c.topk_length) if c.topk_length is not None else None
    sink = dev(c.sink) if c.sink is not None else None
    o, lse = mla.mla_prefill_sparse(dev_bf16(c.q), dev_bf16(c.kv), dev(c.indices), c.scale, topk_length=tl,
                                    sink=sink)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(lse)


@pytest.mark.parametrize("topk,with_tl", [(2049, False), (4113, True), (8192, False), (8192, True)])
def test_sparse_topk_across_index_windows(topk, with_tl):
    """The token's index slots are staged 2048 at a time: top-k values that cross one, two and
    three window boundaries (8192 is the largest supported), with topk_length cutting inside a
    later window."""
    c = make_sparse(f"sparse_topk{topk}", num_tokens=3, heads=16, n_kv=12000, topk=topk, seed=91, pad_p=0.05,
                    with_topk_length=with_tl)
    if with_tl:
        c.topk_length = np.array([topk, 2048 + 5, 4096 + 31], dtype=np.int32)
    announce(f"sparse {c.name} tl={with_tl}")
    o, lse = _sparse(c)
    ro, rl = O.sparse_mla_prefill(c.q, c.kv, c.indices, c.scale, dv=512, topk_length=c.topk_length, sink=c.sink)
    check_parity(o, lse, ro, rl, c.name)


@pytest.mark.parametrize("n_kv", [(2 ** 32 - 3 * 1152) // 1152, 5 * 2 ** 30 // 1152])
def test_sparse_pool_near_and_beyond_4_gib(n_kv):
    """Latent pools of just under 4 GiB (copies at 32-bit byte offsets near 2^32) and of 5 GiB
    (each lane forms a 64-bit address): rows at the far end of the pool and on both sides of the
    4 GiB mark are gathered correctly, and padded or out-of-range slots read none of the pool's
    bytes (row 0 holds NaN). Only the rows the indices name are written; the oracle sees them as
    a compact pool."""
    import torch
    import mla_varlen_prefill_amd as mla
    from workloads import randn_bf16
    announce(f"sparse pool of {n_kv} rows ({n_kv * 1152 / 2 ** 30:.2f} GiB)")
    pool = torch.empty((n_kv, 576), dtype=torch.bfloat16, device="cuda")
    pool[0] = float("nan")
    t, h, topk = 3, 16, 192
    rng = np.random.default_rng(94)
    idx = rng.integers(1, n_kv, size=(t, topk), dtype=np.int64)
    mark = 2 ** 32 // 1152
    marks = [m for m in (mark - 1, mark, mark + 1) if m < n_kv] + [n_kv - 2, n_kv - 1]
    idx[:, :len(marks)] = marks
    idx[1, len(marks) + 3] = -1            # padded
    idx[2, len(marks) + 4] = n_kv          # past the pool
    valid = (idx >= 0) & (idx < n_kv)
    uniq = np.unique(idx[valid])
    rows = randn_bf16(rng, (len(uniq), 576))
    pool[torch.from_numpy(uniq).cuda()] = dev_bf16(rows)
    local = np.full(idx.shape, -1, dtype=np.int32)
    local[valid] = np.searchsorted(uniq, idx[valid])
    q = randn_bf16(np.random.default_rng(95), (t, h, 576))
    scale = float(np.float32(576 ** -0.5))
    o, lse = mla.mla_prefill_sparse(dev_bf16(q), pool, dev(idx.astype(np.int32)), scale)
    torch.cuda.synchronize()
    ro, rl = O.sparse_mla_prefill(q, rows, local, scale, dv=512)
    check_parity(host_f64(o), host_f64(lse), ro, rl, f"sparse pool {n_kv} rows")
    del pool, o, lse
    torch.cuda.empty_cache()


def test_sparse_single_token_all_heads():
    c = make_sparse("sparse_t1", num_tokens=1, heads=128, n_kv=3000, topk=1000, seed=92)
    announce(f"sparse {c.name}")
    o, lse = _sparse(c)
    ro, rl = O.sparse_mla_prefill(c.q, c.kv, c.indices, c.scale, dv=512, sink=c.sink)
    check_parity(o, lse, ro, rl, c.name)


@pytest.mark.parametrize("splits", [0, 1, 7])
@pytest.mark.parametrize("causal", [True, False])
def test_dense_very_long_keys_few_queries(causal, splits):
    """Three sequences of a few query rows over 131072 + ragged keys (the split heuristic splits
    such calls heavily; 1 and 7 are forced), two heads, with a sink."""
    lens_q, lens_k = [3, 1, 130], [131072 + 17, 65536, 4000]
    c = make_dense(f"dense_longk_c{int(causal)}_s{splits}", lens_q, lens_k, heads=2, causal=causal, seed=93,
                   with_sink=True)
    announce(f"dense {c.name}")
    import torch
    import mla_varlen_prefill_amd as mla
    out, lse = mla.mla_prefill_varlen(dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v), dev(c.cu_q), dev(c.cu_k),
                                      c.max_q, c.max_k, c.scale, causal=causal, num_splits=splits,
                                      sink=dev(c.sink))
    torch.cuda.synchronize()
    ro, rl = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal, sink=c.sink)
    check_parity(host_f64(out), host_f64(lse), ro, rl, c.name)
