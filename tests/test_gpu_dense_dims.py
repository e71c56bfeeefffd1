"""GPU parity of the dense varlen MLA prefill for the other MLA head layouts, (Dqk, Dv) =
(128, 128) and (256, 256), and for FP8 output under a static scale (HIP path through the C ABI)
against the fp64 oracle (readings R21, R22)."""
import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import make_dense, device_dense, bf16_tensor_to_bits, f32_to_bf16_bits, varlen_lens
from tests.gpu_util import announce, dev_bf16, dev, host_f64, check_parity

pytestmark = pytest.mark.gpu

OTHER_DIMS = [(128, 128), (256, 256)]
ALL_DIMS = [(192, 128), (128, 128), (256, 256)]


def _run(c, num_splits=1, window=None, out_scale=None, max_k=None):
    """Runs a DenseCase through the library (max_seqlen_k = max_k, else the case's longest
    sequence); returns (out tensor, lse as float64 numpy)."""
    import torch
    import mla_varlen_prefill_amd as mla
    sink = dev(c.sink) if c.sink is not None else None
    scale_t = None if out_scale is None else torch.tensor([out_scale], dtype=torch.float32, device="cuda")
    out, lse = mla.mla_prefill_varlen(dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v), dev(c.cu_q), dev(c.cu_k),
                                      c.max_q, c.max_k if max_k is None else max_k, c.scale, causal=c.causal,
                                      num_splits=num_splits,
                                      sink=sink, window=window, out_scale=scale_t)
    torch.cuda.synchronize()
    return out, host_f64(lse)


def _codes(t) -> np.ndarray:
    import torch
    return t.view(torch.uint8).cpu().numpy()


def _half_step(y: np.ndarray) -> np.ndarray:
    """Half the spacing of the E4M3 values around |y| (subnormal spacing below 2^-6)."""
    e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
    return np.exp2(e - 3) / 2


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dims", OTHER_DIMS)
def test_other_dims_ragged_match_oracle(dims, causal, splits):
    """Ragged batch with an empty query sequence, an empty key sequence, Sk > Sq and Sk < Sq;
    a sink on the causal cases; forced key splits go through the combine kernel."""
    dqk, dv = dims
    c = make_dense(f"dims{dqk}x{dv}_c{int(causal)}_s{splits}", [5, 129, 1, 300, 0, 77], [7, 0, 129, 700, 3, 40],
                   heads=4, causal=causal, seed=71, with_sink=causal, dqk=dqk, dv=dv)
    announce(f"dense {c.name}")
    out, lse = _run(c, num_splits=splits)
    ro, rl = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, c.causal, sink=c.sink)
    check_parity(host_f64(out), lse, ro, rl, c.name)


@pytest.mark.parametrize("window,causal", [((64, 0), True), ((100, 30), False)])
@pytest.mark.parametrize("dims", OTHER_DIMS)
def test_other_dims_window(dims, window, causal):
    dqk, dv = dims
    c = make_dense(f"dims{dqk}x{dv}_w{window[0]}_{window[1]}", [300, 129], [300, 257], heads=2, causal=causal,
                   seed=72, dqk=dqk, dv=dv)
    announce(f"dense {c.name}")
    out, lse = _run(c, window=window)
    ro, rl = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, c.causal, window=window)
    check_parity(host_f64(out), lse, ro, rl, c.name)


@pytest.mark.parametrize("dims", OTHER_DIMS)
def test_other_dims_full_size_sampled(dims):
    """The varlen batch of eight sequences (7015 tokens) at 128 heads, causal, in the bench's
    launch configuration; sampled (token, head) rows against the oracle."""
    import torch
    import mla_varlen_prefill_amd as mla
    dqk, dv = dims
    lens = varlen_lens(2, 8, 64, 2048)
    q, k, v, cu_q, cu_k = device_dense(lens, lens, 128, seed=73, dqk=dqk, dv=dv)
    announce(f"dense dims{dqk}x{dv} full size {lens}")
    out, lse = mla.mla_prefill_varlen(q, k, v, cu_q, cu_k, max(lens), max(lens), dqk ** -0.5, causal=True)
    torch.cuda.synchronize()
    heads = [0, 63, 127]
    cu = np.concatenate([[0], np.cumsum(lens)])
    rng = np.random.default_rng(74)
    toks = sorted(set([int(x) for x in cu[:-1]] + [int(x) - 1 for x in cu[1:]] +
                      rng.integers(0, int(cu[-1]), 12).tolist()))
    qs, ks, vs = (bf16_tensor_to_bits(t[:, heads]) for t in (q, k, v))
    ro, rl = O.dense_mla_prefill_rows(qs, ks, vs, cu, cu, float(np.float32(dqk ** -0.5)), True, toks,
                                      list(range(len(heads))))
    check_parity(host_f64(out[toks][:, heads]), host_f64(lse[toks][:, heads]), ro, rl, f"dims{dqk}x{dv} sampled")


@pytest.mark.parametrize("splits", [1, 2])
@pytest.mark.parametrize("dims", ALL_DIMS)
def test_fp8_output_is_exact_when_o_is_v(dims, splits):
    """One query and one key per sequence, K = 0: every score is 0, so the softmax weight and its
    normaliser are exactly 1 and O is that key's V row exactly (a nonzero score leaves the
    normaliser a rounding step away from 1, which moves values sitting on a rounding tie). With a
    power-of-two scale the FP8 codes must then equal the oracle's encoding of V / scale bit for
    bit. V spans magnitudes from below the smallest subnormal to past the saturation point, and
    about one value in sixteen sits exactly on a tie."""
    import torch
    import mla_varlen_prefill_amd as mla
    dqk, dv = dims
    n, heads, s = 96, 8, 2.0 ** -3
    rng = np.random.default_rng([75, dqk])
    mag = np.exp2(rng.uniform(-15, 7, (n, heads, dv))) * rng.choice([-1.0, 1.0], (n, heads, dv))
    v = f32_to_bf16_bits(mag.astype(np.float32))
    c = make_dense(f"fp8 exact {dqk}x{dv}", [1] * n, [1] * n, heads=heads, causal=True, seed=76, dqk=dqk, dv=dv)
    c.v = v
    c.k = np.zeros_like(c.k)
    announce(f"dense {c.name} splits={splits}")
    out, lse = _run(c, num_splits=splits, out_scale=s)
    want = O.quantize_output_fp8(O.widen_bf16(v), s)
    got = _codes(out)
    bad = np.flatnonzero(got != want)
    y = (O.widen_bf16(v) / s).ravel()
    detail = [(float(y[i]), int(got.ravel()[i]), int(want.ravel()[i])) for i in bad[:12]]
    assert bad.size == 0, f"{bad.size} codes differ (value / scale, got, want): {detail}"
    ties = np.isin(np.abs(y), (O.fp8_e4m3_decode(np.arange(0x7E)) + O.fp8_e4m3_decode(np.arange(1, 0x7F))) / 2)
    assert ties.sum() > 1000
    assert np.all(lse == 0.0)   # log of the single weight 1


@pytest.mark.parametrize("splits", [1, 2])
@pytest.mark.parametrize("dims,max_k", [(d, None) for d in ALL_DIMS] + [((192, 128), 8192)])
def test_fp8_output_within_a_rounding_step(dims, max_k, splits):
    """General ragged causal case: every decoded code is within half an E4M3 step of the oracle's
    O / scale plus the fp32 accumulation error, no code is NaN, and the LSE is that of the bf16
    output path bit for bit (also in the 256-row tiles a causal max_seqlen_k of 8192 selects)."""
    dqk, dv = dims
    s = 2.0 ** -8
    c = make_dense(f"fp8 {dqk}x{dv}", [5, 129, 1, 300, 77], [7, 0, 129, 700, 77], heads=4, causal=True,
                   seed=77, with_sink=True, dqk=dqk, dv=dv)
    announce(f"dense {c.name} splits={splits} max_seqlen_k={max_k}")
    out, lse = _run(c, num_splits=splits, out_scale=s, max_k=max_k)
    _, lse_bf16 = _run(c, num_splits=splits, max_k=max_k)
    ro, rl = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, c.causal, sink=c.sink)
    codes = _codes(out)
    assert not np.any((codes & 0x7F) == 0x7F), "NaN code"
    y = np.clip(ro / s, -448, 448)
    err = np.abs(O.fp8_e4m3_decode(codes) - y)
    assert np.all(err <= _half_step(y) + 2e-3 / s), float(np.max(err - _half_step(y)))
    check_parity(np.zeros_like(ro), lse, np.zeros_like(ro), rl, c.name)
    assert np.array_equal(lse, lse_bf16)


@pytest.mark.parametrize("dims", ALL_DIMS)
def test_fp8_output_saturates(dims):
    """A scale far below the output's size: values past 448 become the largest finite code of
    their sign, never NaN."""
    dqk, dv = dims
    s = 1e-5
    c = make_dense(f"fp8 sat {dqk}x{dv}", [200], [200], heads=2, causal=True, seed=78, dqk=dqk, dv=dv)
    announce(f"dense {c.name}")
    out, _ = _run(c, out_scale=s)
    ro, _ = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, True)
    codes = _codes(out)
    assert not np.any((codes & 0x7F) == 0x7F)
    big = np.abs(ro) / s > 448 + 4e-3 / s      # past 448 by more than the fp32 accumulation error
    assert big.sum() > 1000
    assert np.all(codes[big & (ro > 0)] == 0x7E) and np.all(codes[big & (ro < 0)] == 0xFE)
