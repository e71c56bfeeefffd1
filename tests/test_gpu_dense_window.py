"""GPU parity of the dense varlen MLA prefill with a sliding-window (band) mask (HIP path through
the C ABI) against the fp64 oracle, and bit-exact plans with windows."""
import numpy as np
import pytest

from oracle import mla_oracle as O, plan_ref
from workloads import make_dense, device_dense, bf16_tensor_to_bits, cu_from_lens
from tests.gpu_util import announce, dev_bf16, dev, host_f64, check_parity

pytestmark = pytest.mark.gpu

LENS_Q = [0, 5, 129, 1, 300, 64, 200, 2000]
LENS_K = [7, 0, 129, 4096, 100, 64, 700, 2000]


def run_window(c, window, num_splits=1):
    import torch
    import mla_varlen_prefill_amd as mla
    sink = dev(c.sink) if c.sink is not None else None
    res = mla.mla_prefill_varlen(dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v), dev(c.cu_q), dev(c.cu_k),
                                 c.max_q, c.max_k, c.scale, causal=c.causal, num_splits=num_splits,
                                 sink=sink, window=window)
    torch.cuda.synchronize()
    return host_f64(res[0]), host_f64(res[1])


def oracle(c, window):
    return O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, c.causal, sink=c.sink, window=window)


@pytest.mark.parametrize("causal,window", [
    (True, (256, -1)), (False, (100, 30)), (False, (0, 0)), (False, (-1, 17)), (True, (10, -1)),
    (False, (64, 64)), (True, (1000, 5)), (False, (-1, -1)),
])
@pytest.mark.parametrize("num_splits", [1, 3])
def test_window_ragged_batch(causal, window, num_splits):
    c = make_dense(f"win_{window[0]}_{window[1]}_c{int(causal)}_s{num_splits}", LENS_Q, LENS_K, heads=3,
                   causal=causal, seed=51, with_sink=(num_splits == 1))
    announce(f"dense window {c.name}")
    o, lse = run_window(c, window, num_splits)
    ro, rl = oracle(c, window)
    check_parity(o, lse, ro, rl, c.name)


def test_window_unlimited_equals_plain_call():
    """(-1, -1) through the window entry point is bit-identical to mla_prefill_varlen."""
    import torch
    import mla_varlen_prefill_amd as mla
    c = make_dense("win_plain", [300, 129], [700, 129], heads=4, causal=True, seed=52)
    announce(f"dense window {c.name}")
    args = (dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v), dev(c.cu_q), dev(c.cu_k), c.max_q, c.max_k, c.scale)
    a = mla.mla_prefill_varlen(*args, causal=True)
    b = mla.mla_prefill_varlen(*args, causal=True, window=(-1, -1))
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("wgs_per_xcd", [1, 3])
def test_window_persistent_item_chains(wgs_per_xcd, monkeypatch):
    """A tiny persistent grid runs long chains of windowed items (left-edge masked blocks, items
    with no block, tail tiles) back to back."""
    monkeypatch.setenv("MLA_DENSE_WGS_PER_XCD", str(wgs_per_xcd))
    lens_q = [1, 64, 128, 129, 300, 700, 33, 256, 0, 190]
    lens_k = [1, 64, 128, 129, 300, 1500, 20, 256, 9, 100]
    c = make_dense(f"win_chains_w{wgs_per_xcd}", lens_q, lens_k, heads=5, causal=True, seed=53, with_sink=True)
    announce(f"dense window {c.name}")
    o, lse = run_window(c, (150, -1))
    ro, rl = oracle(c, (150, -1))
    check_parity(o, lse, ro, rl, c.name)


@pytest.mark.parametrize("lens_q,lens_k,causal,window,bm,bn", [
    ([1726, 583, 280, 656], None, True, (256, -1), 128, 64),
    ([0, 5, 129, 1, 300], [7, 0, 129, 4096, 100], False, (100, 30), 64, 32),
    ([32768], None, True, (4096, -1), 128, 64),
    ([200], [50], True, (10, -1), 64, 64),
    ([3] * 20000, None, False, (1, 1), 128, 64),     # unsorted path
])
def test_window_plan_bit_exact(lens_q, lens_k, causal, window, bm, bn):
    import torch
    import mla_varlen_prefill_amd as mla
    lens_k = lens_q if lens_k is None else lens_k
    cu_q, cu_k = cu_from_lens(lens_q), cu_from_lens(lens_k)
    max_q = max(lens_q)
    announce(f"plan window {window} B={len(lens_q)} causal={causal}")
    plan, n = mla.mla_prefill_plan(dev(cu_q), dev(cu_k), max_q, causal, block_m=bm, block_n=bn, window=window)
    torch.cuda.synchronize()
    want, want_n = plan_ref.plan_buffer(cu_q, cu_k, max_q, bm, bn, causal, plan.shape[0], window)
    assert int(n.item()) == want_n
    assert np.array_equal(plan.cpu().numpy(), want)


def test_window_long_context_sampled():
    """One causal sequence of 32768 tokens with a 4096-key window, 128 heads, at sampled rows
    (including rows whose window starts inside a key block and the first rows, which see fewer
    than 4096 keys)."""
    import torch
    import mla_varlen_prefill_amd as mla
    announce("dense window long 1x32768 h128 (4096, 0)")
    lens = [32768]
    q, k, v, cu_q, cu_k = device_dense(lens, lens, 128, 3)
    window = (4096, -1)
    out, lse = mla.mla_prefill_varlen(q, k, v, cu_q, cu_k, 32768, 32768, 192 ** -0.5, causal=True, window=window)
    torch.cuda.synchronize()
    tokens = [0, 1, 4095, 4096, 4097, 10000, 32766, 32767]
    hs = [0, 63, 127]
    qfull = np.zeros((32768, len(hs), 192), dtype=np.uint16)
    qfull[tokens] = bf16_tensor_to_bits(q[tokens][:, hs])
    kb = bf16_tensor_to_bits(k[:, hs])
    vb = bf16_tensor_to_bits(v[:, hs])
    ro, rl = O.dense_mla_prefill_rows(qfull, kb, vb, [0, 32768], [0, 32768], float(np.float32(192 ** -0.5)),
                                      True, tokens, list(range(len(hs))), window=window)
    check_parity(host_f64(out[tokens][:, hs]), host_f64(lse[tokens][:, hs]), ro, rl, "window long sampled")
    del q, k, v, out, lse
    torch.cuda.empty_cache()
