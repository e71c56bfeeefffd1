"""GPU parity of the dense varlen MLA prefill (HIP path through the C ABI) against the fp64 oracle."""
import math

import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import make_dense, dense_small, dense_varlen, f32_to_bf16_bits
from tests.gpu_util import announce, dev_bf16, dev, host_f64, check_parity

pytestmark = pytest.mark.gpu


def run_case(c, num_splits=1, strided_v=False, return_lse=True):
    import torch
    import mla_varlen_prefill_amd as mla
    q, k = dev_bf16(c.q), dev_bf16(c.k)
    if strided_v:
        # vLLM layout: V is a view into a packed [T, H, 128 nope + 128 v] buffer
        tk, h, dv = c.v.shape
        packed = torch.zeros((tk, h, 256), dtype=torch.bfloat16, device="cuda")
        packed[:, :, 128:] = dev_bf16(c.v)
        packed[:, :, :128] = 7.0
        v = packed[:, :, 128:]
        assert v.stride() == (h * 256, 256, 1)
    else:
        v = dev_bf16(c.v)
    sink = dev(c.sink) if c.sink is not None else None
    res = mla.mla_prefill_varlen(q, k, v, dev(c.cu_q), dev(c.cu_k), c.max_q, c.max_k, c.scale,
                                 causal=c.causal, num_splits=num_splits, sink=sink, return_lse=return_lse)
    torch.cuda.synchronize()
    if return_lse:
        return host_f64(res[0]), host_f64(res[1])
    return host_f64(res), None


def oracle(c, heads=None):
    return O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, c.causal, sink=c.sink, heads=heads)


def test_dense_small_config():
    c = dense_small()
    announce(f"dense {c.name}")
    o, lse = run_case(c)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


# The warm-up shape probes of page "FlashAttention backend for MLA prefill" (get_warmup_keys:
# (max_seqlen_q, max_seqlen_k) in (1, 128), (129, 512), (1, 4096), (129, 4096), (1, 8192),
# (129, 8192)), plus two ragged tile tails.
PROBES = [(1, 128), (129, 512), (1, 4096), (129, 4096), (1, 8192), (129, 8192), (257, 300), (64, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,sk", PROBES)
def test_dense_probe_shapes(sq, sk, causal):
    c = make_dense(f"probe_{sq}x{sk}_c{int(causal)}", [sq], [sk], heads=2, causal=causal, seed=31)
    announce(f"dense {c.name}")
    o, lse = run_case(c)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


@pytest.mark.parametrize("causal", [False, True])
def test_dense_ragged_batch_with_sink(causal):
    lens_q = [0, 5, 129, 1, 300, 64, 200]
    lens_k = [7, 0, 129, 4096, 100, 64, 700]
    c = make_dense(f"ragged_c{int(causal)}", lens_q, lens_k, heads=3, causal=causal, seed=32,
                   with_sink=True)
    announce(f"dense {c.name}")
    o, lse = run_case(c)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


def test_dense_more_queries_than_keys_bottom_right():
    c = make_dense("sq_gt_sk", [300, 70], [100, 70], heads=2, causal=True, seed=33)
    announce(f"dense {c.name}")
    o, lse = run_case(c)
    ro, rl = oracle(c)
    assert np.isneginf(rl[:200]).all()
    check_parity(o, lse, ro, rl, c.name)


def test_dense_strided_v_and_no_lse():
    c = make_dense("strided_v", [333, 90], [333, 90], heads=4, causal=True, seed=34)
    announce(f"dense {c.name}")
    o, _ = run_case(c, strided_v=True, return_lse=False)
    ro, rl = oracle(c)
    check_parity(o, None, ro, rl, c.name)


@pytest.mark.parametrize("splits", [1, 3])
def test_dense_strided_views(splits):
    """Q, K, the output and the LSE as strided views into larger buffers (Q inside a wider
    per-head row, K every other head of an interleaved buffer, O inside padded rows, LSE
    head-major): the result matches the oracle and no byte outside the views changes."""
    import torch
    import mla_varlen_prefill_amd as mla
    c = make_dense(f"views_s{splits}", [200, 77, 513], [260, 77, 513], heads=4, causal=True, seed=35,
                   with_sink=True)
    announce(f"dense {c.name}")
    tq, h, _ = c.q.shape
    tk = c.k.shape[0]
    qb = torch.full((tq, h, 256), 5.0, dtype=torch.bfloat16, device="cuda")
    qb[:, :, 64:] = dev_bf16(c.q)
    kb = torch.full((tk, 2 * h, 192), -3.0, dtype=torch.bfloat16, device="cuda")
    kb[:, 1::2] = dev_bf16(c.k)
    ob = torch.full((tq, h, 160), 9.0, dtype=torch.bfloat16, device="cuda")
    lb = torch.full((h, tq), 1.5, dtype=torch.float32, device="cuda")
    q, k, out, lse = qb[:, :, 64:], kb[:, 1::2], ob[:, :, 16:144], lb.t()
    assert q.stride() == (h * 256, 256, 1) and k.stride() == (2 * h * 192, 384, 1)
    assert out.stride() == (h * 160, 160, 1) and lse.stride() == (1, tq)
    mla.mla_prefill_varlen(q, k, dev_bf16(c.v), dev(c.cu_q), dev(c.cu_k), c.max_q, c.max_k, c.scale,
                           causal=True, num_splits=splits, sink=dev(c.sink), out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle(c)
    check_parity(host_f64(out), host_f64(lse), ro, rl, c.name)
    assert torch.all(ob[:, :, :16] == 9.0) and torch.all(ob[:, :, 144:] == 9.0)
    with pytest.raises(ValueError):
        mla.mla_prefill_varlen(q, k, dev_bf16(c.v), dev(c.cu_q), dev(c.cu_k), c.max_q, c.max_k, c.scale,
                               causal=True, out=ob[:, :, :120])


@pytest.mark.parametrize("splits", [2, 3, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_forced_splits(splits, causal):
    c = make_dense(f"split{splits}_c{int(causal)}", [1000, 37], [1000, 1500], heads=4, causal=causal,
                   seed=35, with_sink=True)
    announce(f"dense {c.name}")
    o, lse = run_case(c, num_splits=splits)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_long_key_bound_tiles(causal, splits):
    """With at least 256 query rows the (192, 128) layout runs 256-row query tiles (eight-wave
    work-groups) from max_seqlen_k = 2048 on (8192 with the causal mask), 128-row tiles below; the
    bound is only a bound, so the same ragged batch (tiles cut by sequence ends, a one-row
    sequence with many keys) goes through both and each matches the oracle."""
    import torch
    import mla_varlen_prefill_amd as mla
    c = make_dense(f"bound_tiles_c{int(causal)}_s{splits}", [700, 129, 1, 513, 256, 40],
                   [700, 300, 2000, 513, 260, 0], heads=3, causal=causal, seed=37, with_sink=True)
    ro, rl = oracle(c)
    for bound in (c.max_k, 4096, 8192):
        announce(f"dense {c.name} max_seqlen_k={bound}")
        o, lse = mla.mla_prefill_varlen(dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v), dev(c.cu_q), dev(c.cu_k),
                                        c.max_q, bound, c.scale, causal=causal, num_splits=splits,
                                        sink=dev(c.sink))
        torch.cuda.synchronize()
        check_parity(host_f64(o), host_f64(lse), ro, rl, f"{c.name} max_seqlen_k={bound}")


@pytest.mark.parametrize("causal", [False, True])
def test_dense_wide_logit_range_redoes_tiles(causal):
    """Logits far beyond the 2^64 sum bound: each row's reference logit comes from its first keys
    (about 5), then a key 77 nats above it arrives in the first 32-key tile of an unmasked block
    and a key 82 nats above that one in the second tile of a later block, and a third such key
    sits in the diagonal (masked) region. Each forces the redo of its tile against the exact
    maximum, with O and l rescaled; the result must still be the definition's, in both the
    128-row and the 256-row tiles."""
    import torch
    import mla_varlen_prefill_amd as mla
    n = 1000
    c = make_dense(f"wide_c{int(causal)}", [n], [n], heads=2, causal=causal, seed=38, scale=1.0)
    rng = np.random.default_rng(7)
    q = np.zeros((n, 2, 192), dtype=np.float32)
    q[:, :, 0] = 2.0
    k = np.zeros((n, 2, 192), dtype=np.float32)
    k[:, :, 0] = rng.standard_normal((n, 2))
    k[330, :, 0] = 41.0    # block 5, first tile: logit 82
    k[616, :, 0] = 82.0    # block 9, second tile: logit 164
    k[950, :, 0] = 123.0   # block 14, the last tile's diagonal region: logit 246
    c.q, c.k = f32_to_bf16_bits(q), f32_to_bf16_bits(k)
    ro, rl = oracle(c)
    for bound in (n, 8192):
        announce(f"dense {c.name} max_seqlen_k={bound}")
        o, lse = mla.mla_prefill_varlen(dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v), dev(c.cu_q), dev(c.cu_k),
                                        n, bound, c.scale, causal=causal, num_splits=1)
        torch.cuda.synchronize()
        check_parity(host_f64(o), host_f64(lse), ro, rl, f"{c.name} max_seqlen_k={bound}")


def test_dense_auto_splits_small_grid():
    import mla_varlen_prefill_amd as mla
    c = make_dense("auto_split", [4096], [4096], heads=2, causal=True, seed=36)
    s = mla.varlen_num_splits(1, 4096, 4096, 2, True, 0)
    assert s > 1
    announce(f"dense {c.name} splits={s}")
    o, lse = run_case(c, num_splits=0)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


def test_dense_varlen_config_sampled_heads():
    c = dense_varlen()
    announce(f"dense {c.name} lens={c.meta['lens']}")
    o, lse = run_case(c, num_splits=0)
    heads = [0, 37, 90, 127]
    ro, rl = oracle(c, heads=heads)
    check_parity(o[:, heads], lse[:, heads], ro[:, heads], rl[:, heads], c.name)


def test_dense_deterministic_and_batch_invariant():
    import torch
    import mla_varlen_prefill_amd as mla
    lens = [700, 129, 1500]
    c = make_dense("invariance", lens, lens, heads=8, causal=True, seed=37)
    announce(f"dense {c.name}")
    o1, l1 = run_case(c)
    o2, l2 = run_case(c)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # the middle sequence alone gives the same bits as inside the batch
    a, b = int(c.cu_q[1]), int(c.cu_q[2])
    alone = make_dense("alone", [129], [129], heads=8, causal=True, seed=37)
    alone.q, alone.k, alone.v = c.q[a:b], c.k[a:b], c.v[a:b]
    o3, l3 = run_case(alone)
    assert np.array_equal(o3, o1[a:b]) and np.array_equal(l3, l1[a:b])


# The dense kernel keeps a fixed grid of work-groups that each run many work items in turn, handing
# over from one item to the next inside the last key blocks. A tiny grid makes every work-group run
# a long chain of items: items with zero, one, two and many key blocks, tail tiles, ties in the
# longest-first order and split keys all follow one another.
MANY_LENS_Q = [1, 64, 128, 129, 300, 700, 33, 256, 0, 190]
MANY_LENS_K = [1, 64, 128, 129, 300, 1500, 20, 256, 9, 100]


@pytest.mark.parametrize("wgs_per_xcd", [1, 3])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("num_splits", [1, 3])
def test_dense_persistent_item_chains(wgs_per_xcd, causal, num_splits, monkeypatch):
    monkeypatch.setenv("MLA_DENSE_WGS_PER_XCD", str(wgs_per_xcd))
    c = make_dense(f"chains_w{wgs_per_xcd}_c{int(causal)}_s{num_splits}", MANY_LENS_Q, MANY_LENS_K,
                   heads=5, causal=causal, seed=41, with_sink=(num_splits == 1))
    announce(f"dense {c.name}")
    o, lse = run_case(c, num_splits=num_splits)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)


def test_dense_persistent_item_chains_repeat_identical(monkeypatch):
    # the work a work-group picks up depends on timing; the result must not
    monkeypatch.setenv("MLA_DENSE_WGS_PER_XCD", "2")
    c = make_dense("chains_repeat", MANY_LENS_Q, MANY_LENS_K, heads=7, causal=True, seed=42)
    announce(f"dense {c.name}")
    first = run_case(c)
    for _ in range(3):
        again = run_case(c)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1], equal_nan=True)


@pytest.mark.parametrize("heads", [16, 32])
@pytest.mark.parametrize("wgs_per_xcd", [1, 3])
@pytest.mark.parametrize("num_splits", [1, 3])
def test_dense_contiguous_xcd_units_item_chains(heads, wgs_per_xcd, num_splits, monkeypatch):
    """Head counts whose (head, split) units divide over the 8 XCDs take the contiguous per-XCD
    lists (the path every 128-head call takes: several units per XCD, the shortest eighth of the
    items last, stealing from other XCDs' lists once a list is used up). A tiny grid makes every
    work-group run long chains of ragged items; every head is checked in full."""
    monkeypatch.setenv("MLA_DENSE_WGS_PER_XCD", str(wgs_per_xcd))
    c = make_dense(f"xcd_units_h{heads}_w{wgs_per_xcd}_s{num_splits}", MANY_LENS_Q, MANY_LENS_K,
                   heads=heads, causal=True, seed=43, with_sink=True)
    announce(f"dense {c.name}")
    o, lse = run_case(c, num_splits=num_splits)
    ro, rl = oracle(c)
    check_parity(o, lse, ro, rl, c.name)
