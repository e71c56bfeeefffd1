"""CPU checks of the Python binding's argument checks: every tensor the kernels read is checked
for dtype and shape against the sizes handed to the C ABI, before anything touches a device.
The tensors here live on the CPU, so a call that passes every shape check stops at the device
check; one that fails a shape check names the offending tensor."""
import os

import pytest
import torch

import mla_varlen_prefill_amd as mla

pytestmark = pytest.mark.skipif(not os.path.exists(mla.LIB_PATH), reason="libmla_prefill.so not built")

BF = torch.bfloat16
I32 = torch.int32
F32 = torch.float32


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def _dense(t=10, h=4, dqk=192, dv=128, tk=None):
    tk = t if tk is None else tk
    return (torch.zeros(t, h, dqk, dtype=BF), torch.zeros(tk, h, dqk, dtype=BF),
            torch.zeros(tk, h, dv, dtype=BF), torch.tensor([0, 4, t], dtype=I32), torch.tensor([0, 4, tk], dtype=I32))


def test_varlen_checks():
    q, k, v, cq, ck = _dense()
    f = mla.mla_prefill_varlen
    _raises("GPU", f, q, k, v, cq, ck, 6, 6, 0.1)                                    # well-formed
    _raises("cu_seqlens_q", f, q, k, v, cq.long(), ck, 6, 6, 0.1)                    # int64
    _raises("cu_seqlens_k", f, q, k, v, cq, ck[:2], 6, 6, 0.1)                       # short
    _raises("cu_seqlens_k", f, q, k, v, cq, ck.long(), 6, 6, 0.1)
    _raises("k must be", f, q, k[:, :3], v[:, :3], cq, ck, 6, 6, 0.1)                # head count
    _raises("k must be", f, q, k[..., :128], v, cq, ck, 6, 6, 0.1)                   # q/k width differ
    _raises("v must be", f, q, k, v[:9], cq, ck, 6, 6, 0.1)                          # token count
    _raises("v must be", f, q, k, v[:, :2], cq, ck, 6, 6, 0.1)
    _raises("sink", f, q, k, v, cq, ck, 6, 6, 0.1, sink=torch.zeros(3, dtype=F32))
    _raises("sink", f, q, k, v, cq, ck, 6, 6, 0.1, sink=torch.zeros(4, dtype=BF))
    _raises("out_scale", f, q, k, v, cq, ck, 6, 6, 0.1, out_scale=torch.ones(2, dtype=F32))
    _raises("q must be", f, q.float(), k, v, cq, ck, 6, 6, 0.1)


def test_sparse_checks():
    q = torch.zeros(5, 8, 576, dtype=BF)
    kv = torch.zeros(100, 576, dtype=BF)
    idx = torch.zeros(5, 64, dtype=I32)
    f = mla.mla_prefill_sparse
    _raises("GPU", f, q, kv, idx, 0.04)
    _raises("indices", f, q, kv, idx[:4], 0.04)                                      # fewer rows than tokens
    _raises("indices", f, q, kv, idx.long(), 0.04)
    _raises("indices", f, q, kv, idx[:, 0], 0.04)
    _raises("kv must be", f, q, kv[:, :512], idx, 0.04)
    _raises("topk_length", f, q, kv, idx, 0.04, topk_length=torch.zeros(4, dtype=I32))
    _raises("topk_length", f, q, kv, idx, 0.04, topk_length=torch.zeros(5, dtype=torch.int64))
    _raises("sink", f, q, kv, idx, 0.04, sink=torch.zeros(7, dtype=F32))


def test_sparse_paged_checks():
    q = torch.zeros(5, 8, 576, dtype=BF)
    cache = torch.zeros(10, 16, 576, dtype=BF)
    table = torch.zeros(2, 4, dtype=I32)
    cu = torch.tensor([0, 2, 5], dtype=I32)
    idx = torch.zeros(5, 64, dtype=I32)
    f = mla.mla_prefill_sparse_paged
    _raises("GPU", f, q, cache, table, cu, idx, 0.04)
    _raises("block_table", f, q, cache, table[:1], cu, idx, 0.04)
    _raises("block_table", f, q, cache, table.long(), cu, idx, 0.04)
    _raises("cu_seqlens_q", f, q, cache, table, cu.float(), idx, 0.04)
    _raises("seqused_kv", f, q, cache, table, cu, idx, 0.04, seqused_kv=torch.zeros(3, dtype=I32))
    _raises("seqused_q", f, q, cache, table, cu, idx, 0.04, seqused_q=torch.zeros(1, dtype=I32))
    _raises("indices", f, q, cache, table, cu, idx[:3], 0.04)
    _raises("kv_cache", f, q, cache[..., :512], table, cu, idx, 0.04)
    _raises("sink", f, q, cache, table, cu, idx, 0.04, sink=torch.zeros(9, dtype=F32))


def test_chunked_context_and_upprojection_checks():
    q, k, v, cq, _ = _dense(t=10, h=4)
    lat = torch.zeros(50, 576, dtype=BF)
    cc = torch.tensor([0, 20, 50], dtype=I32)
    w = torch.zeros(4 * 256, 512, dtype=BF)
    f = mla.mla_prefill_chunked_context
    _raises("GPU", f, q, k, v, cq, lat, cc, w, 6, 30, 0.1)
    _raises("cu_seqlens_ctx", f, q, k, v, cq, lat, cc[:2], w, 6, 30, 0.1)
    _raises("cu_seqlens_ctx", f, q, k, v, cq, lat, cc.long(), w, 6, 30, 0.1)
    _raises("w_kv", f, q, k, v, cq, lat, cc, w[:1000], 6, 30, 0.1)                     # fewer than H*256 rows
    _raises("w_kv", f, q, k, v, cq, lat, cc, w[:, :256], 6, 30, 0.1)
    _raises("latent", f, q, k, v, cq, lat[:, :512], cc, w, 6, 30, 0.1)
    _raises("v must be", f, q, k, v[:, :, :64], cq, lat, cc, w, 6, 30, 0.1)
    _raises("k must be", f, q, k[:9], v, cq, lat, cc, w, 6, 30, 0.1)
    u = mla.mla_latent_upproject
    _raises("GPU", u, lat, cc, w, 4, 0, 16)
    _raises("w_kv", u, lat, cc, w, 5, 0, 16)                                            # 5 heads need 1280 rows
    _raises("cu_seqlens_ctx", u, lat, cc.long(), w, 4, 0, 16)


def test_combine_and_plan_checks():
    o = torch.zeros(2, 12, 128, dtype=F32)
    l = torch.zeros(2, 12, dtype=F32)
    f = mla.mla_combine
    _raises("GPU", f, o, l, 4)
    _raises("lse_part", f, o, l[:, :10], 4)
    _raises("whole number", f, o, l, 5)
    _raises("float32", f, o.double(), l, 4)
    _raises("sink", f, o, l, 4, sink=torch.zeros(3, dtype=F32))
    cu = torch.tensor([0, 3, 7], dtype=I32)
    _raises("GPU", mla.mla_prefill_plan, cu, cu, 4, True)
    _raises("cu_seqlens_k", mla.mla_prefill_plan, cu, cu[:2], 4, True)
    _raises("cu_seqlens_q", mla.mla_prefill_plan, cu.long(), cu, 4, True)
