"""GPU planner bit-exactness against the CPU plan specification, and the combine kernel's parity."""
import numpy as np
import pytest

from oracle import plan_ref
from oracle import mla_oracle as O
from workloads import cu_from_lens
from tests.gpu_util import announce, dev, host_f64, check_parity

pytestmark = pytest.mark.gpu

PLAN_CASES = [
    ([128], None, True, 128, 64),
    ([1726, 583, 280, 656, 885, 1680, 959, 246], None, True, 128, 64),
    ([2048] * 4, [16384, 12345, 8191, 4097], True, 128, 64),
    ([0, 5, 129, 1, 300], [7, 0, 129, 4096, 100], True, 64, 32),
    ([0, 5, 129, 1, 300], [7, 0, 129, 4096, 100], False, 256, 64),
    ([32768], None, True, 128, 64),
    ([3] * 20000, None, True, 128, 64),          # more slots than the sort capacity
    ([1, 2, 3] * 3000, None, False, 16, 16),     # sorted path, many ties
    # sequence-order path (no window, up to 1024 sequences): ragged lengths with empty sequences
    # and ties in key blocks, exactly 1024 sequences, and 1025 (the slot sort again)
    ([int(x) for x in np.random.default_rng(7).integers(0, 700, 300)],
     [int(x) for x in np.random.default_rng(8).integers(0, 2000, 300)], True, 64, 64),
    ([(i % 129) + 1 for i in range(1024)], None, True, 128, 64),
    ([(i % 129) + 1 for i in range(1025)], None, False, 128, 64),
]


@pytest.mark.parametrize("lens_q,lens_k,causal,bm,bn", PLAN_CASES)
def test_plan_bit_exact(lens_q, lens_k, causal, bm, bn):
    import torch
    import mla_varlen_prefill_amd as mla
    lens_k = lens_q if lens_k is None else lens_k
    cu_q, cu_k = cu_from_lens(lens_q), cu_from_lens(lens_k)
    max_q = max(lens_q)
    announce(f"plan B={len(lens_q)} max_q={max_q} causal={causal} bm={bm} bn={bn}")
    plan, n = mla.mla_prefill_plan(dev(cu_q), dev(cu_k), max_q, causal, block_m=bm, block_n=bn)
    torch.cuda.synchronize()
    cap = plan.shape[0]
    want, want_n = plan_ref.plan_buffer(cu_q, cu_k, max_q, bm, bn, causal, cap)
    assert int(n.item()) == want_n
    assert np.array_equal(plan.cpu().numpy(), want)


@pytest.mark.parametrize("dv,with_sink", [(128, False), (512, True), (128, True)])
def test_combine_matches_oracle(dv, with_sink):
    import torch
    import mla_varlen_prefill_amd as mla
    rng = np.random.default_rng(7)
    s, t, h = 3, 9, 4
    o_part = rng.standard_normal((s, t * h, dv)).astype(np.float32)
    lse_part = (rng.standard_normal((s, t * h)) * 3).astype(np.float32)
    lse_part[0, :5] = -np.inf
    lse_part[:, 7] = -np.inf           # a row with no mass at all
    o_part[lse_part == -np.inf] = 0.0
    sink = rng.standard_normal(h).astype(np.float32) if with_sink else None
    announce(f"combine dv={dv} sink={with_sink}")
    out, lse = mla.mla_combine(dev(o_part), dev(lse_part), h, sink=dev(sink) if with_sink else None)
    torch.cuda.synchronize()
    ro, rl = O.combine_partials(o_part, lse_part, None if sink is None else np.tile(sink, t))
    check_parity(host_f64(out).reshape(t * h, dv), host_f64(lse).reshape(-1), ro, rl, "combine")
