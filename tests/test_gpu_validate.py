"""GPU checks of the MLA_VALIDATE mode: malformed cu_seqlens are rejected on the host, before any
launch, with MLA_ERR_INVALID_ARG; well-formed ones give the unvalidated result bit for bit."""
import numpy as np
import pytest

from workloads import make_dense, cu_from_lens
from tests.gpu_util import announce, dev_bf16, dev

pytestmark = pytest.mark.gpu


def _call(c, cu_q, cu_k, max_q=None, max_k=None):
    import torch
    import mla_varlen_prefill_amd as mla
    out, lse = mla.mla_prefill_varlen(dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v), dev(cu_q), dev(cu_k),
                                      max_q or c.max_q, max_k or c.max_k, c.scale, causal=c.causal)
    torch.cuda.synchronize()
    return out, lse


BAD_CU = {
    "starts_above_zero": lambda cu: np.concatenate([[1], cu[1:]]).astype(np.int32),
    "decreasing": lambda cu: cu[[0, 2, 1, 3]].astype(np.int32),
    "last_below_total": lambda cu: np.concatenate([cu[:-1], [cu[-1] - 1]]).astype(np.int32),
}


@pytest.mark.parametrize("which", ["q", "k"])
@pytest.mark.parametrize("bad", list(BAD_CU))
def test_malformed_cu_seqlens_rejected(monkeypatch, which, bad):
    import mla_varlen_prefill_amd as mla
    monkeypatch.setenv("MLA_VALIDATE", "1")
    c = make_dense("validate", [40, 70, 30], [40, 70, 30], heads=2, causal=True, seed=81)
    cu_q, cu_k = c.cu_q.copy(), c.cu_k.copy()
    if which == "q":
        cu_q = BAD_CU[bad](cu_q)
    else:
        if bad == "last_below_total":
            pytest.skip("the total key count is not an argument of the call")
        cu_k = BAD_CU[bad](cu_k)
    announce(f"validate {which} {bad}")
    with pytest.raises(mla.MLAError) as e:
        _call(c, cu_q, cu_k)
    assert e.value.status == 1


def test_length_above_max_rejected(monkeypatch):
    import mla_varlen_prefill_amd as mla
    monkeypatch.setenv("MLA_VALIDATE", "1")
    c = make_dense("validate max", [40, 70], [40, 70], heads=2, causal=True, seed=82)
    announce("validate max_seqlen")
    with pytest.raises(mla.MLAError) as e:
        _call(c, c.cu_q, c.cu_k, max_q=69, max_k=70)
    assert e.value.status == 1
    with pytest.raises(mla.MLAError):
        _call(c, c.cu_q, c.cu_k, max_q=70, max_k=69)


def test_well_formed_inputs_pass_and_match(monkeypatch):
    import torch
    c = make_dense("validate ok", [0, 40, 70, 1], [5, 40, 90, 0], heads=3, causal=True, seed=83)
    announce("validate ok")
    o1, l1 = _call(c, c.cu_q, c.cu_k)
    monkeypatch.setenv("MLA_VALIDATE", "1")
    o2, l2 = _call(c, c.cu_q, c.cu_k)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_chunked_context_and_paged_validation(monkeypatch):
    """The chunked-context entry point checks its new-token and context cu_seqlens; the paged
    sparse one checks that cu_seqlens_q is well formed and ends at most at the token count."""
    import torch
    import mla_varlen_prefill_amd as mla
    from workloads import randn_bf16, device_sparse_paged
    monkeypatch.setenv("MLA_VALIDATE", "1")
    heads = 2
    rng = np.random.default_rng(84)
    new, ctx = [3, 5], [10, 7]
    cu_q, cu_c = cu_from_lens(new), cu_from_lens(ctx)
    q = randn_bf16(rng, (8, heads, 192)); k = randn_bf16(rng, (8, heads, 192)); v = randn_bf16(rng, (8, heads, 128))
    lat = randn_bf16(rng, (17, 576)); w = randn_bf16(rng, (heads * 256, 512))
    announce("validate chunked context")
    args = (dev_bf16(q), dev_bf16(k), dev_bf16(v))
    bad_c = np.array([0, 10, 9], dtype=np.int32)
    with pytest.raises(mla.MLAError) as e:
        mla.mla_prefill_chunked_context(*args, dev(cu_q), dev_bf16(lat), dev(bad_c), dev_bf16(w), 5, 10, 0.07,
                                        chunk_tokens=4)
    assert e.value.status == 1
    o, l = mla.mla_prefill_chunked_context(*args, dev(cu_q), dev_bf16(lat), dev(cu_c), dev_bf16(w), 5, 10, 0.07,
                                           chunk_tokens=4)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    announce("validate paged sparse")
    qs, kv, cache, table, cu_t, idx, sink, _ = device_sparse_paged(64, 16, 4096, 64, 64, seed=85)
    bad_t = torch.tensor([0, 65], dtype=torch.int32, device="cuda")   # ends past the 64 tokens
    with pytest.raises(mla.MLAError) as e:
        mla.mla_prefill_sparse_paged(qs, cache, table, bad_t, idx, 576 ** -0.5, sink=sink)
    assert e.value.status == 1
    mla.mla_prefill_sparse_paged(qs, cache, table, cu_t, idx, 576 ** -0.5, sink=sink)
    torch.cuda.synchronize()
