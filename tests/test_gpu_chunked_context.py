"""GPU parity of the latent up-projection and of new tokens over a cached latent context processed
chunk by chunk through a bounded buffer (HIP path through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import randn_bf16, f32_to_bf16_bits, bf16_tensor_to_bits, cu_from_lens
from tests.gpu_util import announce, dev_bf16, dev, host_f64, check_parity

pytestmark = pytest.mark.gpu


def _inputs(ctx, new, heads, seed):
    """Seeded bf16 inputs: latent rows N(0,1), weights N(0, 1/512) (so K/V are of unit size), new
    tokens' q/k/v N(0,1)."""
    rng = np.random.default_rng(seed)
    cu_c, cu_q = cu_from_lens(ctx), cu_from_lens(new)
    lat = randn_bf16(np.random.default_rng([seed, 1]), (max(int(cu_c[-1]), 1), 576))
    w = f32_to_bf16_bits((rng.standard_normal((heads * 256, 512)) / np.sqrt(512)).astype(np.float32))
    q = randn_bf16(np.random.default_rng([seed, 2]), (int(cu_q[-1]), heads, 192))
    k = randn_bf16(np.random.default_rng([seed, 3]), (int(cu_q[-1]), heads, 192))
    v = randn_bf16(np.random.default_rng([seed, 4]), (int(cu_q[-1]), heads, 128))
    sink = rng.standard_normal(heads).astype(np.float32)
    return cu_c, cu_q, lat, w, q, k, v, sink


@pytest.mark.parametrize("heads", [4, 5, 128])
@pytest.mark.parametrize("ctx_start,chunk", [(0, 128), (100, 64), (0, 1000)])
def test_upproject_chunk_matches_oracle(ctx_start, chunk, heads):
    """Rows of several sequences (one empty, one of a single row, tails of 128-row tiles), an odd
    head count (a half-filled head pair) and 128 heads (every XCD's head pairs)."""
    import torch
    import mla_varlen_prefill_amd as mla
    ctx = [300, 0, 129, 1]
    cu_c, _, lat, w, *_ = _inputs(ctx, [1] * 4, heads, 61)
    announce(f"upproject start={ctx_start} chunk={chunk} heads={heads}")
    k, v, cu = mla.mla_latent_upproject(dev_bf16(lat), dev(cu_c), dev_bf16(w), heads, ctx_start, chunk)
    torch.cuda.synchronize()
    lens = [min(max(n - ctx_start, 0), chunk) for n in ctx]
    assert cu.cpu().numpy().tolist() == cu_from_lens(lens).tolist()
    row = 0
    for b, n in enumerate(lens):
        if n == 0:
            continue
        rows = O.widen_bf16(lat[cu_c[b] + ctx_start: cu_c[b] + ctx_start + n])
        kr, vr = O.upproject_latent(rows, O.widen_bf16(w), heads)
        kg, vg = host_f64(k[row:row + n]), host_f64(v[row:row + n])
        assert np.max(np.abs(kg - kr)) < 2e-2 and np.max(np.abs(vg - vr)) < 2e-2
        assert np.array_equal(kg[:, :, 128:], kr[:, :, 128:])          # rope copied exactly
        row += n


@pytest.mark.parametrize("chunk", [64, 100, 4096])
@pytest.mark.parametrize("heads", [4, 128])
def test_chunked_context_matches_oracle(chunk, heads):
    """Ragged contexts (one empty, one shorter than a chunk, one spanning many chunks) and ragged
    new-token counts, with a sink: every chunk width gives the oracle's result."""
    import torch
    import mla_varlen_prefill_amd as mla
    ctx, new = [300, 0, 1000, 64], [3, 5, 1, 129]
    cu_c, cu_q, lat, w, q, k, v, sink = _inputs(ctx, new, heads, 62)
    announce(f"chunked context heads={heads} chunk={chunk}")
    o, lse = mla.mla_prefill_chunked_context(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(cu_q), dev_bf16(lat),
                                             dev(cu_c), dev_bf16(w), max(new), max(ctx), 192 ** -0.5,
                                             chunk_tokens=chunk, sink=dev(sink))
    torch.cuda.synchronize()
    hs = list(range(heads)) if heads <= 8 else [0, 1, 63, 127]
    ro, rl = O.mla_prefill_with_latent_context(q, k, v, cu_q, lat, cu_c, w, float(np.float32(192 ** -0.5)),
                                               sink=sink, heads=hs, round_kv_bf16=True)
    check_parity(host_f64(o)[:, hs], host_f64(lse)[:, hs], ro[:, hs], rl[:, hs], f"chunked h{heads} c{chunk}")


def test_chunked_context_empty_context_equals_causal_prefill():
    """Without context the result is the plain causal prefill of the new tokens: bit-identical to
    the unsplit varlen call (the same planner and kernel launches), and within rounding of a
    2-split call."""
    import torch
    import mla_varlen_prefill_amd as mla
    ctx, new = [0, 0], [200, 77]
    cu_c, cu_q, lat, w, q, k, v, sink = _inputs(ctx, new, 8, 63)
    announce("chunked context empty")
    o, lse = mla.mla_prefill_chunked_context(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(cu_q), dev_bf16(lat),
                                             dev(cu_c), dev_bf16(w), max(new), 0, 192 ** -0.5, chunk_tokens=64)
    o1, lse1 = mla.mla_prefill_varlen(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(cu_q), dev(cu_q), max(new), max(new),
                                      192 ** -0.5, causal=True, num_splits=1)
    o2, lse2 = mla.mla_prefill_varlen(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(cu_q), dev(cu_q), max(new), max(new),
                                      192 ** -0.5, causal=True, num_splits=2)
    torch.cuda.synchronize()
    ro, rl = O.dense_mla_prefill(q, k, v, cu_q, cu_q, float(np.float32(192 ** -0.5)), True)
    check_parity(host_f64(o), host_f64(lse), ro, rl, "chunked empty")
    assert torch.equal(o.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse1.view(torch.int32))
    assert torch.allclose(o.float(), o2.float(), atol=1e-2)


def test_chunked_context_strided_views():
    """New-token Q/K/V, the latent cache, the output and the LSE as strided views into larger
    buffers: the result matches the oracle and no byte outside the output view changes."""
    import torch
    import mla_varlen_prefill_amd as mla
    ctx, new, heads = [150, 0, 70], [4, 9, 33], 4
    cu_c, cu_q, lat, w, q, k, v, sink = _inputs(ctx, new, heads, 63)
    announce("chunked context strided views")
    t, n = int(cu_q[-1]), lat.shape[0]
    qb = torch.full((t, heads, 256), 3.0, dtype=torch.bfloat16, device="cuda")
    qb[:, :, 64:] = dev_bf16(q)
    kb = torch.full((t, 2 * heads, 192), -2.0, dtype=torch.bfloat16, device="cuda")
    kb[:, ::2] = dev_bf16(k)
    vb = torch.full((t, heads, 256), 4.0, dtype=torch.bfloat16, device="cuda")
    vb[:, :, 128:] = dev_bf16(v)
    lb = torch.full((n, 640), -1.0, dtype=torch.bfloat16, device="cuda")
    lb[:, 64:] = dev_bf16(lat)
    ob = torch.full((t, heads, 144), 9.0, dtype=torch.bfloat16, device="cuda")
    eb = torch.full((heads, t), 1.5, dtype=torch.float32, device="cuda")
    out, lse = ob[:, :, 16:], eb.t()
    mla.mla_prefill_chunked_context(qb[:, :, 64:], kb[:, ::2], vb[:, :, 128:], dev(cu_q), lb[:, 64:], dev(cu_c),
                                    dev_bf16(w), max(new), max(ctx), 192 ** -0.5, chunk_tokens=64,
                                    sink=dev(sink), out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = O.mla_prefill_with_latent_context(q, k, v, cu_q, lat, cu_c, w, float(np.float32(192 ** -0.5)),
                                               sink=sink, heads=list(range(heads)), round_kv_bf16=True)
    check_parity(host_f64(out), host_f64(lse), ro, rl, "chunked views")
    assert torch.all(ob[:, :, :16] == 9.0)
