"""GPU check of the allocation-free dense entry point (mla_prefill_varlen_noalloc), through the C
ABI: its output and LSE must equal those of mla_prefill_varlen (same planner and kernels; only
where the plan, ticket counters and split partials live differs) on two calls in a row, the
second with a smaller input, so that the second call cannot lean on what the first left in the
library's static scratch. Unsplit and split calls are both covered, and the result is also
checked against the fp64 oracle."""
import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import make_dense
from tests.gpu_util import announce, dev_bf16, dev, host_f64, check_parity

pytestmark = pytest.mark.gpu


def _both(c, num_splits):
    import torch
    import mla_varlen_prefill_amd as mla
    q, k, v = dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v)
    cu_q, cu_k = dev(c.cu_q), dev(c.cu_k)
    sink = dev(c.sink) if c.sink is not None else None
    ref_o, ref_l = mla.mla_prefill_varlen(q, k, v, cu_q, cu_k, c.max_q, c.max_k, c.scale, causal=c.causal,
                                          num_splits=num_splits, sink=sink)
    out = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    mla.mla_prefill_varlen_noalloc(q, k, v, cu_q, cu_k, c.max_q, c.max_k, c.scale, out, lse, causal=c.causal,
                                   num_splits=num_splits, sink=sink)
    torch.cuda.synchronize()
    return out, lse, ref_o, ref_l


@pytest.mark.parametrize("num_splits", [1, 0, 3])
def test_noalloc_matches_workspace_entry_point_on_two_calls(num_splits):
    import torch
    big = make_dense(f"noalloc_big_s{num_splits}", [700, 129, 1500, 1], [700, 300, 1500, 9], heads=8,
                     causal=True, seed=91, with_sink=True)
    small = make_dense(f"noalloc_small_s{num_splits}", [65, 3], [65, 40], heads=4, causal=True, seed=92)
    for c in (big, small):
        announce(f"noalloc {c.name}")
        out, lse, ref_o, ref_l = _both(c, num_splits)
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"{c.name}: O differs"
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), f"{c.name}: LSE differs"
        ro, rl = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, c.causal, sink=c.sink)
        check_parity(host_f64(out), host_f64(lse), ro, rl, c.name)


def test_noalloc_rejects_calls_beyond_its_scratch():
    import torch
    import mla_varlen_prefill_amd as mla
    c = make_dense("noalloc_too_big", [1000], [1000], heads=8, causal=True, seed=93)
    q, k, v = dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v)
    out = torch.empty((1000, 8, 128), dtype=torch.bfloat16, device="cuda")
    announce("noalloc too big")
    with pytest.raises(mla.MLAError, match="WORKSPACE"):
        mla.mla_prefill_varlen_noalloc(q, k, v, dev(c.cu_q), dev(c.cu_k), 1000, 1000, c.scale, out,
                                       num_splits=64)
