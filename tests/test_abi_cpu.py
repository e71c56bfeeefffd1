"""CPU checks of the C ABI: the library loads, exports every function include/mla_prefill.h
declares, and rejects bad arguments with the documented status codes before touching a GPU
(no compute call is made here)."""
import ctypes
import os
import re

import pytest

import mla_varlen_prefill_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_prefill.h")

pytestmark = pytest.mark.skipif(not os.path.exists(mla.LIB_PATH), reason="libmla_prefill.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = mla.load_library()
    declared = _declared_functions()
    assert set(declared) == set(mla.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = mla.load_library()
    for code, name in mla.STATUS_NAMES.items():
        assert lib.mla_status_string(code).decode() == name
    assert lib.mla_abi_version() == 2
    bm, bn = mla.dense_tile_shape()
    assert bm in (128, 256) and bn == 64


P = 0x10000  # a 16-byte aligned fake device address; never dereferenced by these calls


def _varlen(lib, **kw):
    a = dict(q=P, qst=128 * 192, qsh=192, k=P, kst=128 * 192, ksh=192, v=P, vst=128 * 128, vsh=128,
             cuq=P, cuk=P, batch=1, total_q=16, max_q=16, max_k=16, heads=128, dqk=192, dv=128,
             scale=0.07, causal=1, splits=1, sink=None, out=P, ost=128 * 128, osh=128, lse=None,
             lst=128, lsh=1, ws=P, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.mla_prefill_varlen(a["q"], a["qst"], a["qsh"], a["k"], a["kst"], a["ksh"], a["v"],
                                  a["vst"], a["vsh"], a["cuq"], a["cuk"], a["batch"], a["total_q"],
                                  a["max_q"], a["max_k"], a["heads"], a["dqk"], a["dv"], a["scale"],
                                  a["causal"], a["splits"], a["sink"], a["out"], a["ost"], a["osh"],
                                  a["lse"], a["lst"], a["lsh"], a["ws"], a["ws_bytes"], a["stream"])


def _varlen_window(lib, wl, wr, **kw):
    a = dict(q=P, qst=128 * 192, qsh=192, k=P, kst=128 * 192, ksh=192, v=P, vst=128 * 128, vsh=128,
             cuq=P, cuk=P, batch=1, total_q=16, max_q=16, max_k=16, heads=128, dqk=192, dv=128,
             scale=0.07, causal=0, splits=1, sink=None, out=P, ost=128 * 128, osh=128, lse=None,
             lst=128, lsh=1, ws=P, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.mla_prefill_varlen_window(
        a["q"], a["qst"], a["qsh"], a["k"], a["kst"], a["ksh"], a["v"], a["vst"], a["vsh"], a["cuq"],
        a["cuk"], a["batch"], a["total_q"], a["max_q"], a["max_k"], a["heads"], a["dqk"], a["dv"],
        a["scale"], a["causal"], wl, wr, a["splits"], a["sink"], a["out"], a["ost"], a["osh"], a["lse"],
        a["lst"], a["lsh"], a["ws"], a["ws_bytes"], a["stream"])


def test_varlen_window_argument_errors():
    """Windows below -1 are rejected; the other checks are those of mla_prefill_varlen."""
    lib = mla.load_library()
    assert _varlen_window(lib, -2, 0) == 1
    assert _varlen_window(lib, 256, 0, scale=0.0) == 1
    assert _varlen_window(lib, 5, -3) == 1
    assert _varlen_window(lib, 256, 0, dqk=256) == 2
    assert _varlen_window(lib, 256, 0, q=P + 2) == 3
    assert _varlen_window(lib, 256, 0, batch=0) == 0


def test_varlen_argument_errors():
    lib = mla.load_library()
    assert _varlen(lib, q=None) == 1
    assert _varlen(lib, out=None) == 1
    assert _varlen(lib, heads=0) == 1
    assert _varlen(lib, splits=-1) == 1
    assert _varlen(lib, splits=65) == 1
    assert _varlen(lib, scale=float("nan")) == 1
    assert _varlen(lib, scale=0.0) == 1                    # the scale must be positive
    assert _varlen(lib, scale=-0.07) == 1
    assert _varlen(lib, qsh=100) == 1                      # head stride smaller than the row
    assert _varlen(lib, dqk=256) == 2                      # (256, 128) is not an MLA layout
    assert _varlen(lib, dv=256) == 2                       # nor (192, 256)
    assert _varlen(lib, dv=192) == 2
    assert _varlen(lib, max_k=(1 << 24) + 1) == 2
    assert _varlen(lib, q=P + 8) == 3                      # misaligned base
    assert _varlen(lib, vst=128 * 128 + 4) == 3            # stride not a multiple of 8
    assert _varlen(lib, ws=None) == 4
    assert _varlen(lib, ws_bytes=64) == 4
    assert _varlen(lib, batch=0) == 0                      # nothing to do, nothing launched
    # vLLM-style strided V view (token stride H*256, head stride 256) passes validation up to the
    # workspace check
    assert _varlen(lib, vst=128 * 256, vsh=256, ws_bytes=64) == 4
    # the other layouts pass validation up to the workspace check
    assert _varlen(lib, dqk=128, qst=128 * 128, qsh=128, kst=128 * 128, ksh=128, ws_bytes=64) == 4
    assert _varlen(lib, dqk=256, dv=256, qst=128 * 256, qsh=256, kst=128 * 256, ksh=256,
                   vst=128 * 256, vsh=256, ost=128 * 256, osh=256, ws_bytes=64) == 4
    assert _varlen(lib, dqk=256, dv=256, qst=128 * 256, qsh=256, kst=128 * 256, ksh=256,
                   vst=128 * 256, vsh=256, ost=128 * 128, osh=128) == 1   # output rows overlap


def _varlen_noalloc(lib, **kw):
    a = dict(q=P, qst=128 * 192, qsh=192, k=P, kst=128 * 192, ksh=192, v=P, vst=128 * 128, vsh=128,
             cuq=P, cuk=P, batch=1, total_q=16, max_q=16, max_k=16, heads=128, dqk=192, dv=128,
             scale=0.07, causal=1, splits=1, sink=None, out=P, ost=128 * 128, osh=128, lse=None,
             lst=128, lsh=1, stream=None)
    a.update(kw)
    return lib.mla_prefill_varlen_noalloc(
        a["q"], a["qst"], a["qsh"], a["k"], a["kst"], a["ksh"], a["v"], a["vst"], a["vsh"], a["cuq"],
        a["cuk"], a["batch"], a["total_q"], a["max_q"], a["max_k"], a["heads"], a["dqk"], a["dv"], a["scale"],
        a["causal"], a["splits"], a["sink"], a["out"], a["ost"], a["osh"], a["lse"], a["lst"], a["lsh"],
        a["stream"])


def test_varlen_noalloc_argument_errors_and_size_limit():
    """The allocation-free entry point validates like mla_prefill_varlen, then checks on the host
    that the call's workspace fits the library's static scratch (64 MiB): a call that does not
    fit returns WORKSPACE before anything is resolved or launched; one that fits gets as far as
    the device (HIP on a machine without a GPU)."""
    lib = mla.load_library()
    assert _varlen_noalloc(lib, q=None) == 1
    assert _varlen_noalloc(lib, scale=0.0) == 1
    assert _varlen_noalloc(lib, dqk=256) == 2
    assert _varlen_noalloc(lib, q=P + 8) == 3
    assert _varlen_noalloc(lib, batch=0) == 0
    limit = mla.NOALLOC_SCRATCH_BYTES
    # 64 forced splits of 1000 rows x 8 heads: 64 * 8000 * 129 * 4 bytes of partials
    big = dict(qst=8 * 192, kst=8 * 192, vst=8 * 128, ost=8 * 128, heads=8, total_q=1000, max_q=1000, max_k=1000,
               splits=64)
    assert lib.mla_prefill_varlen_workspace_size(1, 1000, 1000, 1000, 8, 128, 1, 64) > limit
    assert _varlen_noalloc(lib, **big) == 4
    fits = dict(big, splits=2)
    assert lib.mla_prefill_varlen_workspace_size(1, 1000, 1000, 1000, 8, 128, 1, 2) <= limit
    assert _varlen_noalloc(lib, **fits) == 5


def _varlen_fp8(lib, scale_ptr=P, **kw):
    a = dict(q=P, qst=128 * 192, qsh=192, k=P, kst=128 * 192, ksh=192, v=P, vst=128 * 128, vsh=128,
             cuq=P, cuk=P, batch=1, total_q=16, max_q=16, max_k=16, heads=128, dqk=192, dv=128,
             scale=0.07, causal=1, splits=1, sink=None, out=P, ost=128 * 128, osh=128, lse=None,
             lst=128, lsh=1, ws=P, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.mla_prefill_varlen_fp8(
        a["q"], a["qst"], a["qsh"], a["k"], a["kst"], a["ksh"], a["v"], a["vst"], a["vsh"], a["cuq"],
        a["cuk"], a["batch"], a["total_q"], a["max_q"], a["max_k"], a["heads"], a["dqk"], a["dv"],
        a["scale"], a["causal"], -1, -1, a["splits"], a["sink"], scale_ptr, a["out"], a["ost"], a["osh"],
        a["lse"], a["lst"], a["lsh"], a["ws"], a["ws_bytes"], a["stream"])


def test_varlen_fp8_argument_errors():
    """FP8 output needs a scale, 16-element output strides and a 4-byte aligned scale; the rest
    is validated as for bf16 output."""
    lib = mla.load_library()
    assert _varlen_fp8(lib, scale_ptr=None) == 1
    assert _varlen_fp8(lib, scale=-1.0) == 1
    assert _varlen_fp8(lib, ost=128 * 128 + 8) == 3
    assert _varlen_fp8(lib, osh=136, ost=128 * 136) == 3
    assert _varlen_fp8(lib, scale_ptr=P + 2) == 3
    assert _varlen_fp8(lib, dqk=256) == 2
    assert _varlen_fp8(lib, ws_bytes=64) == 4
    assert _varlen_fp8(lib, batch=0) == 0


def test_workspace_size_grows_with_splits():
    lib = mla.load_library()
    w1 = lib.mla_prefill_varlen_workspace_size(2, 300, 200, 200, 8, 128, 1, 1)
    w4 = lib.mla_prefill_varlen_workspace_size(2, 300, 200, 200, 8, 128, 1, 4)
    assert w1 > 0 and w4 >= w1 + 4 * 300 * 8 * 128 * 4
    assert lib.mla_prefill_varlen_workspace_size(2, 300, 200, 200, 8, 128, 1, 99) == 0
    # a 256-column v head: partials twice as wide; other widths are rejected
    w1b = lib.mla_prefill_varlen_workspace_size(2, 300, 200, 200, 8, 256, 1, 1)
    w4b = lib.mla_prefill_varlen_workspace_size(2, 300, 200, 200, 8, 256, 1, 4)
    assert w1b > 0 and w4b >= w1b + 4 * 300 * 8 * 256 * 4
    assert lib.mla_prefill_varlen_workspace_size(2, 300, 200, 200, 8, 64, 1, 1) == 0


def _sparse(lib, **kw):
    a = dict(q=P, qst=128 * 576, qsh=576, kv=P, kvst=576, nkv=1000, idx=P, idxst=64, topk=64,
             tl=None, t=4, heads=128, dqk=576, dv=512, scale=0.04, sink=None, out=P,
             ost=128 * 512, osh=512, lse=None, lst=128, lsh=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.mla_prefill_sparse(a["q"], a["qst"], a["qsh"], a["kv"], a["kvst"], a["nkv"], a["idx"],
                                  a["idxst"], a["topk"], a["tl"], a["t"], a["heads"], a["dqk"], a["dv"],
                                  a["scale"], a["sink"], a["out"], a["ost"], a["osh"], a["lse"],
                                  a["lst"], a["lsh"], a["ws"], a["wsb"], a["stream"])


def test_sparse_argument_errors():
    lib = mla.load_library()
    assert lib.mla_prefill_sparse_workspace_size(4096, 128, 2048, 512) == 0
    assert _sparse(lib, kv=None) == 1
    assert _sparse(lib, topk=0) == 1
    assert _sparse(lib, scale=0.0) == 1
    assert _sparse(lib, scale=-0.04) == 1
    assert _sparse(lib, scale=float("inf")) == 1
    assert _sparse(lib, idxst=32) == 1
    assert _sparse(lib, heads=129) == 2
    assert _sparse(lib, topk=8193, idxst=8193) == 2
    assert _sparse(lib, dqk=512) == 2
    assert _sparse(lib, kvst=2 ** 31) == 2          # row strides of 2^31 elements or more
    assert _sparse(lib, kv=P + 4) == 3
    assert _sparse(lib, idx=P + 2) == 3
    assert _sparse(lib, t=0) == 0


def test_latent_upproject_argument_errors():
    """Checked before any device access: W_KV row strides of 2^23 elements or more are
    unsupported (a head's rows are addressed with 32-bit byte offsets)."""
    lib = mla.load_library()
    cu = P + 64
    assert lib.mla_latent_upproject(P, 576, cu, 2, 0, 128, P, 2 ** 23, 4, cu, P, P, None) == 2
    assert lib.mla_latent_upproject(P, 576, cu, 2, 0, 128, P, 500, 4, cu, P, P, None) == 1
    assert lib.mla_latent_upproject(P, 576, cu, 65536, 0, 128, P, 512, 4, cu, P, P, None) == 2
    assert lib.mla_latent_upproject(P, 576, cu, 0, 0, 128, P, 512, 4, cu, P, P, None) == 0


def _sparse_paged(lib, **kw):
    a = dict(q=P, qst=128 * 576, qsh=576, kv=P, kvst=576, nb=100, bs=64, bt=P, btst=16, maxb=16,
             cu=P, batch=2, used=None, usedq=None, idx=P, idxst=64, topk=64, tl=None, t=4, heads=128, dqk=576,
             dv=512, scale=0.04, sink=None, out=P, ost=128 * 512, osh=512, lse=None, lst=128, lsh=1,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.mla_prefill_sparse_paged(
        a["q"], a["qst"], a["qsh"], a["kv"], a["kvst"], a["nb"], a["bs"], a["bt"], a["btst"],
        a["maxb"], a["cu"], a["batch"], a["used"], a["usedq"], a["idx"], a["idxst"], a["topk"], a["tl"], a["t"],
        a["heads"], a["dqk"], a["dv"], a["scale"], a["sink"], a["out"], a["ost"], a["osh"], a["lse"],
        a["lst"], a["lsh"], a["ws"], a["wsb"], a["stream"])


def test_sparse_paged_argument_errors():
    """The paged entry point rejects bad table/cache geometry before touching a GPU, then applies
    the same checks as the physical-row entry point."""
    lib = mla.load_library()
    assert _sparse_paged(lib, bt=None) == 1
    assert _sparse_paged(lib, cu=None) == 1
    assert _sparse_paged(lib, batch=0) == 1
    assert _sparse_paged(lib, bs=0) == 1
    assert _sparse_paged(lib, nb=0) == 1
    assert _sparse_paged(lib, btst=8) == 1                       # stride below max_blocks
    assert _sparse_paged(lib, bs=1025) == 2                      # page sizes 1..1024
    assert _sparse_paged(lib, nb=1 << 22, bs=1024) == 2          # rows above 2^31 - 1
    assert _sparse_paged(lib, bt=P + 2) == 3
    assert _sparse_paged(lib, used=P + 1) == 3
    assert _sparse_paged(lib, usedq=P + 2) == 3
    assert _sparse_paged(lib, scale=0.0) == 1
    assert _sparse_paged(lib, heads=129) == 2                    # shared sparse checks
    assert _sparse_paged(lib, kv=P + 4) == 3
    assert _sparse_paged(lib, t=0) == 0


def _chunked(lib, **kw):
    a = dict(q=P, qst=128 * 192, qsh=192, k=P, kst=128 * 192, ksh=192, v=P, vst=128 * 128, vsh=128, cuq=P,
             lat=P, latst=576, cuc=P, w=P, wst=512, batch=2, total_q=16, max_q=8, max_c=100, heads=128,
             chunk=64, scale=0.07, sink=None, out=P, ost=128 * 128, osh=128, lse=None, lst=128, lsh=1,
             ws=P, wsb=64, stream=None)
    a.update(kw)
    return lib.mla_prefill_chunked_context(
        a["q"], a["qst"], a["qsh"], a["k"], a["kst"], a["ksh"], a["v"], a["vst"], a["vsh"], a["cuq"],
        a["lat"], a["latst"], a["cuc"], a["w"], a["wst"], a["batch"], a["total_q"], a["max_q"], a["max_c"],
        a["heads"], a["chunk"], a["scale"], a["sink"], a["out"], a["ost"], a["osh"], a["lse"], a["lst"],
        a["lsh"], a["ws"], a["wsb"], a["stream"])


def test_chunked_context_argument_errors():
    lib = mla.load_library()
    assert _chunked(lib, lat=None) == 1
    assert _chunked(lib, chunk=0) == 1
    assert _chunked(lib, scale=0.0) == 1
    assert _chunked(lib, scale=-0.07) == 1
    assert _chunked(lib, latst=512) == 1
    assert _chunked(lib, lat=P + 8) == 3
    assert _chunked(lib) == 4                                     # 64 bytes of workspace
    assert _chunked(lib, batch=0) == 0


@pytest.mark.parametrize("dqk,dv", [(192, 128), (128, 128), (256, 256)])
@pytest.mark.parametrize("batch,max_len,heads", [(1, 4096, 2), (2, 300, 8), (1, 32768, 1), (8, 2048, 128),
                                                 (3, 100, 1)])
def test_num_splits_helper_is_the_split_count_the_call_uses(dqk, dv, batch, max_len, heads):
    """mla_prefill_varlen_num_splits resolves num_splits = 0 with the tile height and residency of
    the (dqk, dv) instance the call runs: a workspace sized for that split count passes the call's
    workspace check (which happens before any device access, so the call then stops at
    MLA_ERR_HIP on a machine without a GPU), and one sized for one split fewer fails it. The
    workspace grows by total_q * H * dv * 4 bytes per split, far more than the plan sizes of the
    instances differ by, so no other split count passes both checks."""
    lib = mla.load_library()
    total_q = batch * max_len
    s = lib.mla_prefill_varlen_num_splits(batch, max_len, max_len, heads, dqk, dv, 1, 0)
    assert 1 <= s <= 64
    ws = lib.mla_prefill_varlen_workspace_size(batch, total_q, max_len, max_len, heads, dv, 1, s)
    if s > 1:
        ws_less = lib.mla_prefill_varlen_workspace_size(batch, total_q, max_len, max_len, heads, dv, 1, s - 1)
        assert ws - ws_less >= total_q * heads * dv * 4
    kw = dict(qst=heads * dqk, qsh=dqk, kst=heads * dqk, ksh=dqk, vst=heads * dv, vsh=dv, ost=heads * dv,
              osh=dv, batch=batch, total_q=total_q, max_q=max_len, max_k=max_len, heads=heads, dqk=dqk, dv=dv,
              splits=0)
    assert _varlen(lib, ws_bytes=ws, **kw) == 5
    if s > 1:
        assert _varlen(lib, ws_bytes=ws_less, **kw) == 4
    assert lib.mla_prefill_varlen_num_splits(batch, max_len, max_len, heads, dqk, dv, 1, 3) == 3
    assert lib.mla_prefill_varlen_num_splits(batch, max_len, max_len, heads, 192, 256, 1, 0) == -1
    assert lib.mla_prefill_varlen_num_splits(batch, max_len, max_len, heads, dqk, dv, 1, 65) == -1


def test_combine_and_plan_argument_errors():
    lib = mla.load_library()
    args = [P, P, 2, 4, 8, 128, None, P, 8 * 128, 128, None, 8, 1, None]
    bad = list(args); bad[2] = 0
    assert lib.mla_combine(*bad) == 1
    bad = list(args); bad[5] = 100
    assert lib.mla_combine(*bad) == 1
    bad = list(args); bad[0] = P + 4
    assert lib.mla_combine(*bad) == 3
    assert lib.mla_prefill_plan(P, P, 2, 300, 100, 64, 1, -1, -1, P, 100, P, None) == 1  # block_m not a power of 2
    assert lib.mla_prefill_plan(P, P, 2, 300, 128, 64, 1, -1, -1, P, 5, P, None) == 1    # capacity < 2*3
    assert lib.mla_prefill_plan(P, P, 2, 300, 128, 64, 1, -2, -1, P, 6, P, None) == 1    # window below -1
    assert lib.mla_prefill_plan(P, P, 2, 300, 128, 64, 1, -1, -1, P + 4, 6, P, None) == 3


def test_calibration_library_exports():
    """The benchmark's calibration kernels (MFMA loop, streaming read) live in their own library;
    it loads without a GPU and exports its three entry points."""
    path = os.path.join(os.path.dirname(mla.LIB_PATH), "libmla_calib.so")
    if not os.path.exists(path):
        pytest.skip("libmla_calib.so not built")
    lib = ctypes.CDLL(path)
    for name in ("mla_calib_mfma_loop", "mla_calib_mfma_flop", "mla_calib_stream_read"):
        assert hasattr(lib, name), name
    lib.mla_calib_mfma_flop.restype = ctypes.c_double
    lib.mla_calib_mfma_flop.argtypes = [ctypes.c_int, ctypes.c_int]
    assert lib.mla_calib_mfma_flop(1, 1) == 4 * 8 * 2 * 32 * 32 * 16
