"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: hand-derived examples, closed
forms, a library routine the oracle does not use (PyTorch's CPU scaled_dot_product_attention and
logsumexp, SciPy's softmax), invariants of the definition and brute force on tiny inputs. Together
they are chosen so that a dropped scale, a wrong mask alignment, a transposed operand, a sink
multiplied by the scale, a log in the wrong base, the wrong value columns or an ignored
``topk_length`` each fail at least one test.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from workloads import f32_to_bf16_bits, bf16_bits_to_f32, make_dense, make_sparse

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dense_hand_examples.json")


def _f(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- hand-derived examples
@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_examples(case):
    q = _f(case["q"])[:, None, :]
    k = _f(case["k"])[:, None, :]
    v = _f(case["v"])[:, None, :]
    sink = None if case["sink"] is None else _f(case["sink"])
    o, lse = O.dense_mla_prefill(q, k, v, [0, q.shape[0]], [0, k.shape[0]], case["scale"],
                                 case["causal"], sink=sink)
    np.testing.assert_allclose(o[:, 0, :], _f(case["O"]), rtol=0, atol=1e-12)
    want_lse = np.array([-math.inf if x == "-inf" else x for x in case["LSE"]], dtype=np.float64)
    assert np.array_equal(np.isinf(lse[:, 0]), np.isinf(want_lse))
    fin = np.isfinite(want_lse)
    np.testing.assert_allclose(lse[fin, 0], want_lse[fin], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- bf16 widening
def _widening_mismatches(widen) -> int:
    """Codes (of all 65536 bf16 bit patterns) where `widen` differs from PyTorch's own bf16 ->
    float64 conversion, NaN codes compared as NaN and zeros by sign."""
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    with np.errstate(invalid="ignore"):   # signalling-NaN codes raise the invalid flag when widened
        got = np.asarray(widen(codes), dtype=np.float64)
    if got.shape != want.shape:
        return codes.size
    same = ((got == want) & (np.signbit(got) == np.signbit(want))) | (np.isnan(got) & np.isnan(want))
    return int((~same).sum())


def test_widen_bf16_matches_torch_on_every_code():
    """The oracle's entry point for every bf16 input (page "SparseFlashMla", Parameters table:
    q and the KV are BFLOAT16) agrees with PyTorch's bf16 -> float64 cast on all 65536 codes:
    normals, subnormals, both zeros, both infinities and every NaN."""
    assert _widening_mismatches(O.widen_bf16) == 0


def test_widen_bf16_pin_rejects_plausible_mistakes():
    """Planted on the CPU: each of these wrong widenings must fail the pin above."""
    def wrong_shift(b):
        return (np.asarray(b, np.uint16).astype(np.uint32) << 15).view(np.float32).astype(np.float64)

    def low_half(b):
        return np.asarray(b, np.uint16).astype(np.uint32).view(np.float32).astype(np.float64)

    def as_half(b):
        return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)

    def truncated_to_int(b):
        return np.trunc(O.widen_bf16(b))

    for bad in (wrong_shift, low_half, as_half, truncated_to_int):
        assert _widening_mismatches(bad) > 1000, bad.__name__


# ---------------------------------------------------------------- library special case
def _torch_reference(q, k, v, cu_q, cu_k, scale, causal):
    """PyTorch fp64 CPU SDPA with an explicit boolean mask, and logsumexp of the masked logits."""
    outs, lses = [], []
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        sq, sk = q1 - q0, k1 - k0
        qt = torch.from_numpy(q[q0:q1]).transpose(0, 1)  # [H, sq, d]
        kt = torch.from_numpy(k[k0:k1]).transpose(0, 1)
        vt = torch.from_numpy(v[k0:k1]).transpose(0, 1)
        i = torch.arange(sq)[:, None]
        j = torch.arange(sk)[None, :]
        mask = (j <= i + (sk - sq)) if causal else torch.ones(sq, sk, dtype=torch.bool)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        logits = torch.matmul(qt, kt.transpose(1, 2)) * scale
        lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
        outs.append(o.transpose(0, 1).numpy())
        lses.append(lse.transpose(0, 1).numpy())
    return np.concatenate(outs), np.concatenate(lses)


@pytest.mark.parametrize("lens_q,lens_k,causal", [
    ([7, 33, 1], [7, 33, 1], True),
    ([7, 33, 1], [7, 33, 1], False),
    ([5, 16], [40, 16], True),      # Sq < Sk: bottom-right aligned
    ([12], [30], False),
])
def test_dense_matches_torch_sdpa(lens_q, lens_k, causal):
    c = make_dense("t", lens_q, lens_k, heads=3, causal=causal, seed=11, dqk=24, dv=16)
    q, k, v = (O.widen_bf16(x) for x in (c.q, c.k, c.v))
    o, lse = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal)
    ro, rl = _torch_reference(q, k, v, list(c.cu_q), list(c.cu_k), c.scale, causal)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_bottom_right_empty_rows_match_definition():
    # Sq > Sk with the bottom-right mask: the first Sq - Sk rows see nothing (reading R4).
    c = make_dense("t", [9], [4], heads=2, causal=True, seed=12, dqk=16, dv=8)
    o, lse = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, True)
    assert np.all(o[:5] == 0) and np.all(np.isneginf(lse[:5]))
    q, k, v = (O.widen_bf16(x) for x in (c.q, c.k, c.v))
    ro, rl = _torch_reference(q[5:], k, v, [0, 4], [0, 4], c.scale, True)
    np.testing.assert_allclose(o[5:], ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[5:], rl, rtol=0, atol=1e-12)


def test_bottom_right_equals_prefix_plus_causal_merge():
    """Chunked prefill decomposition (page "FlashAttention backend for MLA prefill": context chunk
    non-causal with LSE, new tokens causal): the bottom-right causal result over [prefix | new]
    equals the LSE merge of (new tokens vs prefix, unmasked) and (new tokens vs themselves, causal)."""
    sq, prefix = 11, 23
    c = make_dense("t", [sq], [prefix + sq], heads=2, causal=True, seed=13, dqk=32, dv=16)
    full_o, full_l = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, True)
    o1, l1 = O.dense_mla_prefill(c.q, c.k[:prefix], c.v[:prefix], [0, sq], [0, prefix], c.scale, False)
    o2, l2 = O.dense_mla_prefill(c.q, c.k[prefix:], c.v[prefix:], [0, sq], [0, sq], c.scale, True)
    mo, ml = O.combine_partials(np.stack([o1.reshape(-1, 16), o2.reshape(-1, 16)]),
                                np.stack([l1.reshape(-1), l2.reshape(-1)]))
    np.testing.assert_allclose(mo.reshape(full_o.shape), full_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml.reshape(full_l.shape), full_l, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_identical_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(0)
    sq = sk = 6
    q = rng.standard_normal((sq, 1, 8))
    kvec = rng.standard_normal(8)
    k = np.tile(kvec, (sk, 1))[:, None, :]
    v = rng.standard_normal((sk, 1, 5))
    scale = 0.3
    o, lse = O.dense_mla_prefill(q, k, v, [0, sq], [0, sk], scale, True)
    for i in range(sq):
        n = i + 1
        np.testing.assert_allclose(o[i, 0], v[:n, 0].mean(axis=0), atol=1e-12)
        np.testing.assert_allclose(lse[i, 0], math.log(n) + scale * q[i, 0] @ kvec, atol=1e-12)


def test_identical_keys_with_sink_closed_form():
    rng = np.random.default_rng(1)
    n = 5
    q = rng.standard_normal((1, 1, 4))
    kvec = rng.standard_normal(4)
    k = np.tile(kvec, (n, 1))[:, None, :]
    v = rng.standard_normal((n, 1, 3))
    scale, sigma = 0.7, 1.3
    a = scale * float(q[0, 0] @ kvec)
    o, lse = O.dense_mla_prefill(q, k, v, [0, 1], [0, n], scale, False, sink=np.array([sigma]))
    z = n * math.exp(a) + math.exp(sigma)
    np.testing.assert_allclose(o[0, 0], n * math.exp(a) / z * v[:, 0].mean(axis=0), atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], math.log(z), atol=1e-12)


def test_single_visible_key():
    c = make_dense("t", [4], [4], heads=2, causal=True, seed=14, dqk=16, dv=8)
    q, k, v = (O.widen_bf16(x) for x in (c.q, c.k, c.v))
    o, lse = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, True)
    for h in range(2):
        np.testing.assert_array_equal(o[0, h], v[0, h])
        np.testing.assert_allclose(lse[0, h], c.scale * q[0, h] @ k[0, h], atol=1e-12)


def test_sparse_all_padded():
    c = make_sparse("t", 3, 4, 50, 8, seed=15, pad_p=0.0, with_sink=True, dqk=40)
    idx = -np.ones_like(c.indices)
    o, lse = O.sparse_mla_prefill(c.q, c.kv, idx, c.scale, dv=32, sink=c.sink)
    assert np.all(o == 0)
    np.testing.assert_array_equal(lse, np.tile(c.sink.astype(np.float64), (3, 1)))
    o, lse = O.sparse_mla_prefill(c.q, c.kv, idx, c.scale, dv=32, sink=None)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- invariants
def test_rows_sum_to_one_including_sink():
    c = make_sparse("t", 4, 3, 64, 16, seed=16, pad_p=0.2, with_sink=True, dqk=24)
    kv = O.widen_bf16(c.kv)
    kv[:, :8] = 1.0  # value columns all ones: O = total softmax mass on keys
    o, lse = O.sparse_mla_prefill(c.q, kv, c.indices, c.scale, dv=8, sink=c.sink)
    p_sink = np.exp(c.sink[None, :].astype(np.float64) - lse)
    np.testing.assert_allclose(o[..., 0] + p_sink, 1.0, atol=1e-12)


def test_padded_slot_contributes_nothing():
    c = make_sparse("t", 3, 2, 40, 10, seed=17, pad_p=0.0, with_sink=False, dqk=16)
    idx = c.indices.copy()
    idx[:, 3] = -1
    o1, l1 = O.sparse_mla_prefill(c.q, c.kv, idx, c.scale, dv=12)
    o2, l2 = O.sparse_mla_prefill(c.q, c.kv, np.delete(idx, 3, axis=1), c.scale, dv=12)
    idx_oob = idx.copy()
    idx_oob[:, 3] = 40  # out of range is skipped like -1 (reading R8)
    o3, l3 = O.sparse_mla_prefill(c.q, c.kv, idx_oob, c.scale, dv=12)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    np.testing.assert_allclose(o1, o3, atol=1e-13)


def test_sparse_slot_permutation_invariance():
    c = make_sparse("t", 3, 2, 40, 10, seed=18, pad_p=0.3, with_sink=True, dqk=16)
    perm = np.random.default_rng(3).permutation(10)
    o1, l1 = O.sparse_mla_prefill(c.q, c.kv, c.indices, c.scale, dv=12, sink=c.sink)
    o2, l2 = O.sparse_mla_prefill(c.q, c.kv, c.indices[:, perm], c.scale, dv=12, sink=c.sink)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_key_shift_and_scale_transfer():
    c = make_dense("t", [5, 8], [5, 8], heads=2, causal=True, seed=19, dqk=16, dv=8)
    q, k, v = (O.widen_bf16(x) for x in (c.q, c.k, c.v))
    o, lse = O.dense_mla_prefill(q, k, v, c.cu_q, c.cu_k, c.scale, True)
    shift = np.random.default_rng(4).standard_normal(16)
    o2, lse2 = O.dense_mla_prefill(q, k + shift, v, c.cu_q, c.cu_k, c.scale, True)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + c.scale * (q @ shift), atol=1e-12)
    o3, lse3 = O.dense_mla_prefill(2.5 * q, k, v, c.cu_q, c.cu_k, c.scale / 2.5, True)
    np.testing.assert_allclose(o3, o, atol=1e-12)
    np.testing.assert_allclose(lse3, lse, atol=1e-12)


def test_sink_to_minus_infinity_is_no_sink():
    c = make_dense("t", [6], [6], heads=2, causal=True, seed=20, dqk=16, dv=8)
    o1, l1 = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, True)
    o2, l2 = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, True,
                                 sink=np.array([-np.inf, -1e300]))
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1, atol=1e-12)


def test_zero_padded_value_columns():
    """Zero-padding V to the q/k width, as the vLLM backend does for kernels that need equal head
    dims (page "FlashAttention backend for MLA prefill", ``_flash_attn_varlen_diff_headdims``),
    leaves the first Dv output columns unchanged and makes the pad columns zero."""
    c = make_dense("t", [7], [7], heads=2, causal=True, seed=21, dqk=16, dv=8)
    v = O.widen_bf16(c.v)
    vpad = np.concatenate([v, np.zeros((7, 2, 8))], axis=2)
    o1, _ = O.dense_mla_prefill(c.q, c.k, v, c.cu_q, c.cu_k, c.scale, True)
    o2, _ = O.dense_mla_prefill(c.q, c.k, vpad, c.cu_q, c.cu_k, c.scale, True)
    np.testing.assert_array_equal(o2[..., :8], o1)
    assert np.all(o2[..., 8:] == 0)


# ---------------------------------------------------------------- sparse vs dense, brute force
def test_sparse_with_all_causal_indices_equals_dense():
    """Indices [0..p_t] for every token reproduce dense causal attention with the latent row used as
    K for every head and its first dv columns as V (page "SparseFlashMla": K~ = V~)."""
    t, h, n, d, dv = 5, 3, 9, 24, 16
    c = make_sparse("t", t, h, n, n, seed=22, pad_p=0.0, with_sink=True, dqk=d)
    idx = -np.ones((t, n), dtype=np.int32)
    for ti in range(t):
        p = n - t + ti
        idx[ti, : p + 1] = np.random.default_rng(ti).permutation(p + 1)
    o_s, l_s = O.sparse_mla_prefill(c.q, c.kv, idx, c.scale, dv=dv, sink=c.sink)
    kv = O.widen_bf16(c.kv)
    k = np.repeat(kv[:, None, :], h, axis=1)
    v = np.repeat(kv[:, None, :dv], h, axis=1)
    o_d, l_d = O.dense_mla_prefill(c.q, k, v, [0, t], [0, n], c.scale, True, sink=c.sink)
    np.testing.assert_allclose(o_s, o_d, atol=1e-12)
    np.testing.assert_allclose(l_s, l_d, atol=1e-12)


def test_sparse_brute_force_with_topk_length_and_duplicates():
    """Pure-Python loops with math.exp, no max shift, on a tiny case with duplicate indices, -1
    slots, out-of-range slots and a topk_length that cuts valid slots (readings R8, R9)."""
    from scipy.special import softmax, logsumexp
    rng = np.random.default_rng(5)
    t, h, n, d, dv, topk = 3, 2, 7, 6, 4, 6
    q = rng.standard_normal((t, h, d)) * 0.5
    kv = rng.standard_normal((n, d)) * 0.5
    idx = np.array([[2, 2, -1, 5, 0, 9], [1, -1, -1, 3, 3, 3], [6, 4, 0, 1, 2, 5]], dtype=np.int32)
    tl = np.array([6, 5, 3], dtype=np.int32)
    sink = np.array([0.25, -0.5])
    scale = 0.8
    o, lse = O.sparse_mla_prefill(q, kv, idx, scale, dv=dv, topk_length=tl, sink=sink)
    for ti in range(t):
        for hi in range(h):
            logits, vals = [], []
            for s in range(tl[ti]):
                j = int(idx[ti, s])
                if 0 <= j < n:
                    logits.append(scale * sum(q[ti, hi, x] * kv[j, x] for x in range(d)))
                    vals.append(kv[j, :dv])
            z = sum(math.exp(a) for a in logits) + math.exp(sink[hi])
            want = sum(math.exp(a) * vv for a, vv in zip(logits, vals)) / z
            np.testing.assert_allclose(o[ti, hi], want, atol=1e-12)
            np.testing.assert_allclose(lse[ti, hi], math.log(z), atol=1e-12)
            # library cross-check of the same row
            lg = np.array(logits + [sink[hi]])
            np.testing.assert_allclose(lse[ti, hi], logsumexp(lg), atol=1e-12)
            np.testing.assert_allclose(o[ti, hi], softmax(lg)[:-1] @ np.array(vals), atol=1e-12)


# ---------------------------------------------------------------- sliding window (R18)
def test_window_special_cases_reduce_to_causal_and_full():
    """(-1, -1) is the unmasked rule, (-1, 0) the bottom-right causal rule, causal overrides a
    given right window, and a window wider than the sequence changes nothing."""
    for sq, sk in [(5, 9), (9, 9), (7, 3)]:
        full = O.dense_visible(sq, sk, False)
        caus = O.dense_visible(sq, sk, True)
        assert np.array_equal(O.dense_visible(sq, sk, False, window=(-1, -1)), full)
        assert np.array_equal(O.dense_visible(sq, sk, False, window=(-1, 0)), caus)
        assert np.array_equal(O.dense_visible(sq, sk, True, window=(-1, 5)), caus)
        assert np.array_equal(O.dense_visible(sq, sk, False, window=(sk + sq, sk + sq)), full)
        assert np.array_equal(O.dense_visible(sq, sk, True, window=(sk + sq, 3)), caus)


def test_window_brute_force_band_and_sparse_equivalence():
    """A band of left 3 / right 1 by brute force (math.exp over an explicit list of visible keys),
    and the same rows as sparse top-k attention over the enumerated key indices (the sparse
    definition is pinned separately)."""
    rng = np.random.default_rng(91)
    sq, sk, h, d, dv = 6, 9, 2, 5, 3
    q = rng.standard_normal((sq, h, d))
    k = rng.standard_normal((sk, h, d))
    v = rng.standard_normal((sk, h, dv))
    scale, left, right = 0.6, 3, 1
    o, lse = O.dense_mla_prefill(q, k, v, [0, sq], [0, sk], scale, False, window=(left, right))
    off = sk - sq
    for i in range(sq):
        keys = [j for j in range(sk) if i + off - left <= j <= i + off + right]
        for hh in range(h):
            lg = [scale * sum(q[i, hh, x] * k[j, hh, x] for x in range(d)) for j in keys]
            z = sum(math.exp(a) for a in lg)
            want = sum(math.exp(a) * v[j, hh] for a, j in zip(lg, keys)) / z
            np.testing.assert_allclose(o[i, hh], want, atol=1e-12)
            np.testing.assert_allclose(lse[i, hh], math.log(z), atol=1e-12)
        # the same row as sparse attention over the enumerated indices, head by head (one shared
        # "latent" row per key: concatenate k and v of that head)
        for hh in range(h):
            kv = np.concatenate([v[:, hh, :], k[:, hh, :]], axis=1)   # value columns first
            qq = np.concatenate([np.zeros((1, 1, dv)), q[i:i + 1, hh:hh + 1, :]], axis=2)
            idx = np.array([keys + [-1] * (sk - len(keys))], dtype=np.int32)
            so, sl = O.sparse_mla_prefill(qq, kv, idx, scale, dv=dv)
            np.testing.assert_allclose(so[0, 0], o[i, hh], atol=1e-12)
            np.testing.assert_allclose(sl[0, 0], lse[i, hh], atol=1e-12)


def test_window_rows_with_no_key_are_empty():
    """A left window of 0 with right -1 on Sq > Sk leaves the rows before the diagonal with no key."""
    rng = np.random.default_rng(92)
    q = rng.standard_normal((5, 1, 4)); k = rng.standard_normal((2, 1, 4)); v = rng.standard_normal((2, 1, 3))
    o, lse = O.dense_mla_prefill(q, k, v, [0, 5], [0, 2], 1.0, False, window=(0, -1))
    # d = -3: row i sees keys j >= i - 3 -> rows 0..3 see keys, row 4 sees j >= 1 only
    vis = O.dense_visible(5, 2, False, window=(0, -1))
    assert vis.tolist() == [[True, True], [True, True], [True, True], [True, True], [False, True]]
    o2, lse2 = O.dense_mla_prefill(q, k, v, [0, 5], [0, 2], 1.0, False, window=(0, 0))
    # band (0, 0): only j == i - 3 -> rows 3, 4 see one key each, rows 0..2 none
    assert np.isneginf(lse2[:3]).all() and np.all(o2[:3] == 0)
    np.testing.assert_allclose(o2[3, 0], v[0, 0], atol=1e-12)
    np.testing.assert_allclose(o2[4, 0], v[1, 0], atol=1e-12)


# ---------------------------------------------------------------- latent context (R19)
def _latent_case(rng, ctx, new, h):
    cu_q = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    cu_c = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    q = rng.standard_normal((cu_q[-1], h, 192)) * 0.3
    kn = rng.standard_normal((cu_q[-1], h, 192)) * 0.3
    vn = rng.standard_normal((cu_q[-1], h, 128))
    lat = rng.standard_normal((cu_c[-1], 576))
    return q, kn, vn, cu_q, lat, cu_c


def test_latent_context_selector_weights_reduce_to_dense():
    """With W_UK_h selecting latent columns 0..127 and W_UV_h columns 128..255, the context keys
    are [latent[:, :128] || rope] and values latent[:, 128:256]: the result must equal the dense
    definition on those explicitly built keys, with all context keys visible."""
    rng = np.random.default_rng(101)
    h = 2
    q, kn, vn, cu_q, lat, cu_c = _latent_case(rng, [5, 0, 7], [3, 2, 4], h)
    w = np.zeros((h, 256, 512))
    for hh in range(h):
        w[hh, :128, :128] = np.eye(128)
        w[hh, 128:, 128:256] = np.eye(128)
    o, lse = O.mla_prefill_with_latent_context(q, kn, vn, cu_q, lat, cu_c, w.reshape(h * 256, 512), 0.2)
    for b in range(3):
        c = lat[cu_c[b]:cu_c[b + 1]]
        kc = np.repeat(np.concatenate([c[:, :128], c[:, 512:]], axis=1)[:, None, :], h, axis=1)
        vc = np.repeat(c[:, None, 128:256], h, axis=1)
        k_all = np.concatenate([kc, kn[cu_q[b]:cu_q[b + 1]]])
        v_all = np.concatenate([vc, vn[cu_q[b]:cu_q[b + 1]]])
        sq, sk = cu_q[b + 1] - cu_q[b], k_all.shape[0]
        ro, rl = O.dense_mla_prefill(q[cu_q[b]:cu_q[b + 1]], k_all, v_all, [0, sq], [0, sk], 0.2, True)
        np.testing.assert_allclose(o[cu_q[b]:cu_q[b + 1]], ro, atol=1e-12)
        np.testing.assert_allclose(lse[cu_q[b]:cu_q[b + 1]], rl, atol=1e-12)


def test_latent_context_equals_merge_of_context_and_new_token_passes():
    """The pages' decomposition: an unmasked pass over the context keys and a causal pass over
    the new tokens, merged through their LSEs (combine formula, pinned separately), equals the
    single bottom-right causal pass over [context || new]."""
    rng = np.random.default_rng(102)
    h = 3
    q, kn, vn, cu_q, lat, cu_c = _latent_case(rng, [6, 4], [4, 5], h)
    w = rng.standard_normal((h * 256, 512)) * 0.05
    sink = np.array([0.1, -0.4, 0.7])
    o, lse = O.mla_prefill_with_latent_context(q, kn, vn, cu_q, lat, cu_c, w, 0.3, sink=sink)
    for b in range(2):
        kc, vc = O.upproject_latent(lat[cu_c[b]:cu_c[b + 1]], w, h)
        qs = q[cu_q[b]:cu_q[b + 1]]
        sq = qs.shape[0]
        o1, l1 = O.dense_mla_prefill(qs, kc, vc, [0, sq], [0, kc.shape[0]], 0.3, False)
        o2, l2 = O.dense_mla_prefill(qs, kn[cu_q[b]:cu_q[b + 1]], vn[cu_q[b]:cu_q[b + 1]], [0, sq], [0, sq], 0.3, True)
        om, lm = O.combine_partials(np.stack([o1.reshape(-1, 128), o2.reshape(-1, 128)]),
                                    np.stack([l1.reshape(-1), l2.reshape(-1)]), np.tile(sink, sq))
        np.testing.assert_allclose(o[cu_q[b]:cu_q[b + 1]].reshape(-1, 128), om, atol=1e-12)
        np.testing.assert_allclose(lse[cu_q[b]:cu_q[b + 1]].reshape(-1), lm, atol=1e-12)


def test_latent_upprojection_brute_force():
    """Element-wise sums for the up-projection and the rope broadcast on a tiny case."""
    rng = np.random.default_rng(103)
    lat = rng.standard_normal((2, 576))
    w = rng.standard_normal((2 * 256, 512))
    k, v = O.upproject_latent(lat, w, 2)
    for t in range(2):
        for hh in (0, 1):
            for c in (0, 77, 127):
                assert abs(k[t, hh, c] - sum(lat[t, d] * w[hh * 256 + c, d] for d in range(512))) < 1e-9
                assert abs(v[t, hh, c] - sum(lat[t, d] * w[hh * 256 + 128 + c, d] for d in range(512))) < 1e-9
            assert np.array_equal(k[t, hh, 128:], lat[t, 512:])


def test_round_to_bf16_hand_values():
    """Round-to-nearest-even at the 8-bit mantissa: ties go to the even neighbour, values just
    above a tie go up, and representable values are kept."""
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 1.0 + 2 ** -7, 0.0])
    want = np.array([1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, 1.0 + 2 ** -7, 0.0])
    np.testing.assert_array_equal(O.round_to_bf16(x), want)


# ---------------------------------------------------------------- paged latent cache (R17)
def _paged_case(rng, block_size, lens_kv, n_tok_per_seq, topk, d=6, num_blocks_extra=3):
    """Per-sequence contiguous KV scattered into a shuffled block pool, with its block table."""
    max_blocks = max((n + block_size - 1) // block_size for n in lens_kv)
    nb = sum((n + block_size - 1) // block_size for n in lens_kv) + num_blocks_extra
    perm = rng.permutation(nb)
    cache = rng.standard_normal((nb, block_size, d)) * 0.5
    table = np.full((len(lens_kv), max_blocks), -1, dtype=np.int32)
    seq_kv = []
    used = 0
    for b, n in enumerate(lens_kv):
        kv_b = rng.standard_normal((n, d)) * 0.5
        seq_kv.append(kv_b)
        for i in range((n + block_size - 1) // block_size):
            blk = perm[used]
            used += 1
            table[b, i] = blk
            chunk = kv_b[i * block_size:(i + 1) * block_size]
            cache[blk, :len(chunk)] = chunk
    cu_q = np.concatenate([[0], np.cumsum(n_tok_per_seq)]).astype(np.int32)
    t = int(cu_q[-1])
    idx = np.empty((t, topk), dtype=np.int32)
    for b in range(len(lens_kv)):
        for ti in range(cu_q[b], cu_q[b + 1]):
            idx[ti] = rng.integers(-2, lens_kv[b] + 3, size=topk)   # includes -1/-2 and past-the-end
    return cache, table, cu_q, idx, seq_kv


@pytest.mark.parametrize("block_size", [1, 3, 4])
def test_paged_brute_force_against_unpaged_sequences(block_size):
    """Brute force with math.exp over each sequence's own contiguous KV (never paged): with
    seqused = the sequence lengths, the paged oracle must give the same result whatever the block
    size and the order of the blocks."""
    rng = np.random.default_rng(11 + block_size)
    lens_kv, n_tok, topk, h, d, dv = [7, 10], [2, 3], 5, 2, 6, 4
    cache, table, cu_q, idx, seq_kv = _paged_case(rng, block_size, lens_kv, n_tok, topk, d=d)
    q = rng.standard_normal((idx.shape[0], h, d)) * 0.5
    scale = 0.7
    o, lse = O.sparse_mla_prefill_paged(q, cache, table, cu_q, idx, scale, dv=dv, seqused=lens_kv)
    for b in range(len(lens_kv)):
        for ti in range(cu_q[b], cu_q[b + 1]):
            for hi in range(h):
                logits, vals = [], []
                for pos in idx[ti]:
                    if 0 <= pos < lens_kv[b]:
                        row = seq_kv[b][pos]
                        logits.append(scale * sum(q[ti, hi, x] * row[x] for x in range(d)))
                        vals.append(row[:dv])
                if not logits:
                    assert lse[ti, hi] == -math.inf and np.all(o[ti, hi] == 0)
                    continue
                z = sum(math.exp(a) for a in logits)
                want = sum(math.exp(a) * vv for a, vv in zip(logits, vals)) / z
                np.testing.assert_allclose(o[ti, hi], want, atol=1e-12)
                np.testing.assert_allclose(lse[ti, hi], math.log(z), atol=1e-12)


def test_paged_seqused_equals_padding_past_the_used_length():
    """seqused[b] = u drops exactly the logical positions >= u, like writing -1 there."""
    rng = np.random.default_rng(21)
    lens_kv, n_tok, topk, h, d = [9, 6], [2, 2], 6, 2, 6
    cache, table, cu_q, idx, _ = _paged_case(rng, 4, lens_kv, n_tok, topk, d=d)
    q = rng.standard_normal((idx.shape[0], h, d))
    used = [5, 2]
    o1, l1 = O.sparse_mla_prefill_paged(q, cache, table, cu_q, idx, 0.5, dv=4, seqused=used)
    idx2 = idx.copy()
    for b in range(2):
        for ti in range(cu_q[b], cu_q[b + 1]):
            idx2[ti][idx2[ti] >= used[b]] = -1
    o2, l2 = O.sparse_mla_prefill_paged(q, cache, table, cu_q, idx2, 0.5, dv=4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_paged_seqused_q_gives_empty_rows_past_the_used_tokens():
    """seqused_q[b] = u: the first u tokens of sequence b are unchanged, every later token of the
    sequence is a row with no key (O = 0 and LSE = -inf, or LSE = sink with a sink), exactly as if
    all its slots were -1 (page "Sgl project Sglang FA4 Interface", Signature: seqused_q)."""
    rng = np.random.default_rng(41)
    lens_kv, n_tok, topk, h, d = [9, 6, 5], [3, 2, 2], 6, 2, 6
    cache, table, cu_q, idx, _ = _paged_case(rng, 4, lens_kv, n_tok, topk, d=d)
    q = rng.standard_normal((idx.shape[0], h, d))
    used_q = [1, 2, 0]
    sink = np.array([0.25, -0.5])
    for s in (None, sink):
        o0, l0 = O.sparse_mla_prefill_paged(q, cache, table, cu_q, idx, 0.5, dv=4, sink=s)
        o1, l1 = O.sparse_mla_prefill_paged(q, cache, table, cu_q, idx, 0.5, dv=4, sink=s, seqused_q=used_q)
        idx2 = idx.copy()
        for b in range(3):
            idx2[cu_q[b] + used_q[b]:cu_q[b + 1]] = -1
        o2, l2 = O.sparse_mla_prefill_paged(q, cache, table, cu_q, idx2, 0.5, dv=4, sink=s)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)
        for b in range(3):
            keep = slice(cu_q[b], cu_q[b] + used_q[b])
            drop = slice(cu_q[b] + used_q[b], cu_q[b + 1])
            np.testing.assert_array_equal(o1[keep], o0[keep])
            np.testing.assert_array_equal(l1[keep], l0[keep])
            assert np.all(o1[drop] == 0)
            want = np.full((cu_q[b + 1] - cu_q[b] - used_q[b], h), -math.inf) if s is None else \
                np.broadcast_to(s, (cu_q[b + 1] - cu_q[b] - used_q[b], h))
            np.testing.assert_array_equal(l1[drop], want)


def test_paged_bad_table_entry_drops_that_block_only():
    """A table entry outside [0, num_blocks) invalidates exactly the slots in that logical block;
    a token outside every sequence has no valid slot (O = 0, LSE = -inf; sink alone with a sink)."""
    rng = np.random.default_rng(31)
    lens_kv, n_tok, topk, h, d, bs = [8], [3], 8, 2, 6, 4
    cache, table, cu_q, idx, _ = _paged_case(rng, bs, lens_kv, n_tok, topk, d=d)
    q = rng.standard_normal((idx.shape[0] + 1, h, d))       # one token past cu_q[-1]
    idx = np.concatenate([idx, rng.integers(0, 8, size=(1, topk)).astype(np.int32)])
    t2 = table.copy()
    t2[0, 1] = cache.shape[0] + 5                            # logical block 1: positions 4..7
    o1, l1 = O.sparse_mla_prefill_paged(q, cache, t2, cu_q, idx, 0.5, dv=4)
    idx2 = idx.copy()
    idx2[:3][(idx2[:3] >= 4) & (idx2[:3] < 8)] = -1
    o2, l2 = O.sparse_mla_prefill_paged(q, cache, table, cu_q, idx2, 0.5, dv=4)
    np.testing.assert_array_equal(o1[:3], o2[:3])
    np.testing.assert_array_equal(l1[:3], l2[:3])
    assert np.all(o1[3] == 0) and np.all(l1[3] == -math.inf)
    sink = np.array([0.3, -1.0])
    o3, l3 = O.sparse_mla_prefill_paged(q, cache, table, cu_q, idx, 0.5, dv=4, sink=sink)
    assert np.all(o3[3] == 0)
    np.testing.assert_array_equal(l3[3], sink)


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("with_sink", [False, True])
def test_combine_of_disjoint_key_splits_equals_unsplit(with_sink):
    t, h, n, d, dv = 4, 3, 30, 16, 8
    c = make_sparse("t", t, h, n, 20, seed=23, pad_p=0.1, with_sink=with_sink, dqk=d)
    full_o, full_l = O.sparse_mla_prefill(c.q, c.kv, c.indices, c.scale, dv=dv, sink=c.sink)
    cuts = [0, 3, 4, 11, 20]   # includes a 1-slot split
    parts_o, parts_l = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        po, pl = O.sparse_mla_prefill(c.q, c.kv, c.indices[:, a:b], c.scale, dv=dv)
        parts_o.append(po.reshape(-1, dv))
        parts_l.append(pl.reshape(-1))
    sink_rows = None if c.sink is None else np.tile(c.sink.astype(np.float64), t)
    mo, ml = O.combine_partials(np.stack(parts_o), np.stack(parts_l), sink=sink_rows)
    np.testing.assert_allclose(mo.reshape(full_o.shape), full_o, atol=1e-12)
    np.testing.assert_allclose(ml.reshape(full_l.shape), full_l, atol=1e-12)


def test_combine_all_empty_partials():
    o, l = O.combine_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(l))
    o, l = O.combine_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf), sink=np.array([0.5, -2.0]))
    assert np.all(o == 0)
    np.testing.assert_array_equal(l, [0.5, -2.0])


# ---------------------------------------------------------------- rows helper, inputs
def test_rows_helper_matches_full():
    c = make_dense("t", [9, 20, 3], [15, 20, 3], heads=4, causal=True, seed=24, dqk=16, dv=8,
                   with_sink=True)
    o, lse = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, True, sink=c.sink)
    toks, heads = [0, 8, 9, 28, 31], [0, 3]
    ro, rl = O.dense_mla_prefill_rows(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, True, toks, heads,
                                      sink=c.sink)
    np.testing.assert_allclose(ro, o[np.ix_(toks, heads)], atol=1e-13)
    np.testing.assert_allclose(rl, lse[np.ix_(toks, heads)], atol=1e-13)


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (-1, -1)), (False, (4, 2)), (True, (3, -1))])
def test_rows_helper_any_order_and_duplicates(causal, window):
    """Rows requested out of order, repeated and from several sequences (one with Sq > Sk, so some
    rows see no key) give the full evaluation's rows, for every mask rule."""
    c = make_dense("t", [9, 20, 6], [15, 20, 3], heads=3, causal=causal, seed=25, dqk=16, dv=8,
                   with_sink=True)
    o, lse = O.dense_mla_prefill(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal, sink=c.sink, window=window)
    toks, heads = [33, 0, 12, 8, 12, 30, 29, 9], [2, 0]
    ro, rl = O.dense_mla_prefill_rows(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal, toks, heads,
                                      sink=c.sink, window=window)
    np.testing.assert_allclose(ro, o[np.ix_(toks, heads)], atol=1e-13)
    np.testing.assert_array_equal(np.isinf(rl), np.isinf(lse[np.ix_(toks, heads)]))
    fin = np.isfinite(rl)
    np.testing.assert_allclose(rl[fin], lse[np.ix_(toks, heads)][fin], atol=1e-13)


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3.0e38], dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    back = bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0).
    np.testing.assert_array_equal(back[:4], np.array([1.0, 1.0, 1.0 + 2**-6, -2.5], dtype=np.float32))
    np.testing.assert_array_equal(torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), bits)


# ---------------------------------------------------------------- FP8 output (reading R21)
def test_fp8_decode_closed_form_values():
    """Code values fixed by the E4M3 format: bias 7, 3 mantissa bits, subnormals below 2^-6,
    448 the largest finite value, S.1111.111 NaN, sign in the top bit."""
    d = O.fp8_e4m3_decode
    assert d(0x00) == 0.0 and d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9
    assert d(0x08) == 2.0 ** -6 and d(0x38) == 1.0 and d(0x39) == 1.125 and d(0x40) == 2.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0 and d(0xB8) == -1.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    pos = d(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)                              # increasing, no duplicates
    assert np.all(d(np.arange(0x80, 0xFF)) == -pos)


def test_fp8_encode_round_trip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(O.fp8_e4m3_encode(O.fp8_e4m3_decode(codes)), codes)
    e = O.fp8_e4m3_encode
    assert e(1 + 2.0 ** -4) == 0x38            # halfway between 1 and 1.125: to even (1.0)
    assert e(1 + 3 * 2.0 ** -4) == 0x3A        # halfway between 1.125 and 1.25: to even (1.25)
    assert e(2.0 ** -10) == 0x00               # half the smallest subnormal: to even (zero)
    assert e(3 * 2.0 ** -10) == 0x02           # halfway between codes 1 and 2: to 2
    assert e(15 * 2.0 ** -10) == 0x08          # halfway between 7*2^-9 and 2^-6: to even (2^-6)
    assert e(1.0625 + 1e-9) == 0x39            # just above a tie: up
    assert e(464.0) == 0x7E and e(1e9) == 0x7E and e(-500.0) == 0xFE   # saturation at 448
    assert e(-1e-6) == 0x80 and e(0.0) == 0x00


def test_fp8_encode_is_nearest_by_brute_force():
    """Every encoding is a nearest finite value to the clamped input (brute force over all
    codes), carries the input's sign bit, and between two equally near values is the even code."""
    rng = np.random.default_rng(21)
    pos = O.fp8_e4m3_decode(np.arange(0x7F))
    x = rng.standard_normal(4000) * np.exp2(rng.uniform(-12, 9, 4000))
    x = np.concatenate([x, pos[:-1] + np.diff(pos) / 2, -(pos[:-1] + np.diff(pos) / 2)])  # with every tie
    got = O.fp8_e4m3_encode(x)
    grid = O.fp8_e4m3_decode(np.arange(256))
    dist_all = np.abs(grid[None, :] - np.clip(x, -448, 448)[:, None])
    dist_all[:, np.isnan(grid)] = np.inf
    best = dist_all.min(axis=1)
    assert np.array_equal(dist_all[np.arange(x.size), got], best)
    assert np.array_equal(got >> 7, np.signbit(x).astype(np.uint8))
    ties = (np.sort(dist_all, axis=1)[:, 1] == best) & (best > 0)
    n_tie_values = [len({abs(grid[c]) for c in np.flatnonzero(dist_all[i] == best[i])}) for i in np.flatnonzero(ties)]
    tied = np.flatnonzero(ties)[np.array(n_tie_values) > 1]
    assert tied.size > 200 and np.all(got[tied] % 2 == 0)


def test_fp8_encode_matches_torch_cast():
    """In range, the encoding equals PyTorch's CPU float8_e4m3fn cast (a library routine the
    oracle does not call)."""
    rng = np.random.default_rng(22)
    x = (rng.standard_normal(200000) * np.exp2(rng.uniform(-14, 9, 200000))).astype(np.float32)
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.fp8_e4m3_encode(x), ref)


def test_quantize_output_divides_by_the_scale():
    out = np.array([[0.5, -0.25, 3.0, 1000.0]])
    q = O.quantize_output_fp8(out, 2.0 ** -4)
    assert np.array_equal(O.fp8_e4m3_decode(q), [[8.0, -4.0, 48.0, 448.0]])
