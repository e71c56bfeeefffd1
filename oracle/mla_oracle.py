"""Plain fp64 CPU oracle for MLA prefill: the definition of what the HIP path computes.

TEST INFRASTRUCTURE ONLY. This module is imported by ``tests/``, by the entry point's smoke
check and by the bench's ``cpu_baseline`` leg, never by the product path. It shares no code with
the HIP kernels or their host layer; it only reads the bf16 bit patterns the input generators
produce and widens them to float64.

Every function is the plain mathematical definition, written two-pass (scores, then a max, then
the normaliser) with an explicit visibility mask. There is no tiling, no online softmax and no
reordering beyond what the definition states.

What the pages fix:
  * The operation is ``O = softmax(Q K^T * softmax_scale) V`` where the K and V that take part are
    selected by the inputs (page "SparseFlashMla", Description: the formula, with K~ = V~ the
    participating KV).
  * Dense MLA prefill runs with K/V expanded to every query head, q/k head 192 = 128 nope + 64
    rope and v head 128, over ``cu_seqlens`` (page "FlashAttention backend for MLA prefill",
    ``dispatch`` and the "MLA prefill expands K/V" comment); new tokens attend causally to
    themselves (``run_prefill_new_tokens``, causal=True, cu_seqlens_q = cu_seqlens_k) and a
    context chunk attends without a mask and always returns the LSE
    (``run_prefill_context_chunk``).
  * The LSE is float32 log-sum-exp of the softmax (page "Sgl project Sglang FA4 Interface",
    I/O Contract; page "SparseFlashMla", ``softmax_lse``).
  * Sparse indices are int32; -1 marks an invalid or padded slot; ``topk_length`` gives the valid,
    left-aligned prefix of each index row (page "SparseFlashMla", Parameters table and
    Constraints). Sinks are float values per head (same table; page "mla_prefill_branch_sparse_fp8",
    ``attn_sink_ptr``).
  * Split partial results are combined into the final result (page "Mojo module mla",
    ``mla_splitk_reduce``; page "Sgl project Sglang FA4 Interface", Description: split-KV with a
    combine kernel).

Readings taken where the pages are silent (each also listed with the design notes):
  R1 LSE is the natural log of the sum of exp of the *scaled* logits.
  R3 Causal masking is bottom-right aligned: key j is visible to query i of a sequence with
     Sq queries and Sk keys iff j <= i + Sk - Sq ("RightDownCausal", page "SparseFlashMla",
     ``ori_mask_mode``). For Sq == Sk this is the ordinary causal mask.
  R4 A row with no visible key and no sink gets O = 0 and LSE = -inf. With a sink it gets O = 0
     and LSE = sink.
  R6 A sink is one extra logit per head, added as-is (not multiplied by the scale), whose value
     vector is zero. It counts in the normaliser and in the LSE.
  R7 In the sparse path V is the first ``dv`` columns of the same gathered rows as K.
  R8 Indices are physical pool rows; any index outside [0, N_kv) is skipped like -1.
  R9 Slots at or beyond ``topk_length[t]`` are ignored even when they hold a valid row.
  R17 Paged latent cache (page "SparseFlashMla": ``block_table`` for PageAttention, cache shape
     [block_num, block_size, KV_N, D], ``topk_value_mode`` 1 = logical token indices,
     ``seqused`` = valid KV length per sequence, ``cu_seqlens_q``). Token t belongs to sequence b
     with cu_q[b] <= t < cu_q[b+1]; logical index p of its row is cache row
     (block_table[b][p // block_size], p % block_size). A slot is valid iff R9 holds,
     0 <= p < used_b (used_b = seqused[b] if given, else max_blocks * block_size) and the table
     entry lies in [0, num_blocks). A token outside every sequence has no valid slot.
     ``seqused_q`` (page "Sgl project Sglang FA4 Interface", Signature: the query tokens of each
     sequence that are in use): token t of sequence b is in use iff t - cu_q[b] < seqused_q[b];
     a token not in use has no valid slot (so O = 0 and LSE = -inf, or the sink, by R4).
  R18 Sliding window / band mask (page "Sgl project Sglang FA4 Interface", ``window_size`` =
     (left, right), e.g. (256, 0) = causal with a 256-key window; page "SparseFlashMla",
     ``ori_win_left`` / ``ori_win_right``: the number of past / future tokens a query sees, -1 =
     unlimited, Band mask mode). Aligned bottom-right like R3, with d = Sk - Sq: key j is visible
     to query i iff j >= i + d - left (when left >= 0) and j <= i + d + right (when right >= 0).
     ``causal`` is the case right = 0 and overrides a given right.
  R19 Context from the latent cache (page "FlashAttention backend for MLA prefill",
     ``run_prefill_new_tokens`` / ``run_prefill_context_chunk``: new tokens attend causally to
     themselves, context keys without a mask, the LSE merges the parts; page
     "mla_prefill_branch_sparse_fp8": latent rows of 512 + 64 rope, ``w_uk`` / ``w_uv``
     up-projections). The context key of head h at cached token t is
     [c_t W_UK_h^T (128) || rope_t (64)] and its value is c_t W_UV_h^T (128), where c_t is the
     512-wide latent and rope_t the last 64 columns of the cached row; W_KV is laid out like a
     linear layer's weight, [H * 256, 512], rows h*256 + 0..127 for W_UK_h and h*256 + 128..255
     for W_UV_h. The result for a new query is attention over [context keys || new keys] with
     the bottom-right causal mask (R3), i.e. every context key plus the causal new keys.
  R20 The up-projected context K/V are materialised in bf16 (round-to-nearest-even of the fp32
     products), the type the attention takes its K/V in; the parity tests compare with the
     oracle evaluated on the same rounded K/V, so that the attention is what is measured.
  R21 FP8 output (page "FlashAttention backend for MLA prefill": ``supports_quant_output`` with
     a static, symmetric per-tensor FP8 key, kFp8StaticTensorSym). The stored value is the OCP
     FP8 E4M3 encoding (the finite-only variant: bias 7, no infinities, S.1111.111 = NaN, largest
     magnitude 448) of O / scale, rounded to the nearest representable value with ties to the
     even code, after clamping to [-448, 448] (saturation, as static FP8 quantisation does; the
     pages do not say). The LSE is not quantised.
  R22 Other MLA head layouts (same page, ``supports_mla_dimensions``: (nope, rope, v) =
     (128, 64, 128), (64, 64, 128), (192, 64, 256), (256, 0, 256)). The attention sees q/k heads
     of nope + rope columns, so the layouts are (Dqk, Dv) = (192, 128), (128, 128), (256, 256);
     the definition above is the same for every width.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -math.inf


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (a bf16 is the top half of a float32)."""
    f32 = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return f32.astype(np.float64)


def _softmax_rows(scores: np.ndarray, visible: np.ndarray, values: np.ndarray,
                  sink: Optional[float]) -> Tuple[np.ndarray, np.ndarray]:
    """Two-pass masked softmax-weighted sum for a block of rows.

    scores: [R, N] scaled logits; visible: [R, N] bool; values: [N, Dv]; sink: scalar logit or None.
    Returns O [R, Dv] and LSE [R] in float64.
    """
    masked = np.where(visible, scores, NEG_INF)
    row_max = masked.max(axis=1) if masked.shape[1] else np.full(masked.shape[0], NEG_INF)
    if sink is not None:
        row_max = np.maximum(row_max, sink)
    empty = ~np.isfinite(row_max)
    shift = np.where(empty, 0.0, row_max)
    weights = np.where(visible, np.exp(masked - shift[:, None]), 0.0)
    z = weights.sum(axis=1)
    if sink is not None:
        z = z + np.exp(sink - shift)
    out = np.zeros((scores.shape[0], values.shape[1]), dtype=np.float64)
    ok = ~empty
    if ok.any():
        out[ok] = (weights[ok] @ values) / z[ok, None]
    lse = np.full(scores.shape[0], NEG_INF, dtype=np.float64)
    lse[ok] = shift[ok] + np.log(z[ok])
    return out, lse


def dense_visible(sq: int, sk: int, causal: bool, rows: Optional[np.ndarray] = None,
                  window: Tuple[int, int] = (-1, -1)) -> np.ndarray:
    """Visibility mask [len(rows), sk] for one sequence (readings R3 and R18: bottom-right
    causal, optional (left, right) window with -1 = unlimited)."""
    i = np.arange(sq) if rows is None else np.asarray(rows)
    j = np.arange(sk)
    left, right = int(window[0]), int(window[1])
    if causal:
        right = 0
    vis = np.ones((i.size, sk), dtype=bool)
    if right >= 0:
        vis &= j[None, :] <= (i[:, None] + (sk - sq) + right)
    if left >= 0:
        vis &= j[None, :] >= (i[:, None] + (sk - sq) - left)
    return vis


def dense_mla_prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q: Sequence[int],
                      cu_k: Sequence[int], scale: float, causal: bool,
                      sink: Optional[np.ndarray] = None,
                      heads: Optional[Iterable[int]] = None,
                      window: Tuple[int, int] = (-1, -1)) -> Tuple[np.ndarray, np.ndarray]:
    """Dense varlen attention, per sequence and head, straight from the definition.

    q [Tq, H, Dqk], k [Tk, H, Dqk], v [Tk, H, Dv] (float64 or bf16 bits). Sequence b owns query
    rows cu_q[b]:cu_q[b+1] and key rows cu_k[b]:cu_k[b+1]. For query i of sequence b and head h:
    s_j = scale * <q_i, k_j> over all Dqk columns, visible keys per R3/R18, softmax with the optional
    sink (R6), O = sum_j p_j v_j, LSE = log(sum exp). Returns O [Tq, H, Dv] and LSE [Tq, H]
    (rows of heads not requested stay NaN).
    """
    q, k, v = (_as_f64(x) for x in (q, k, v))
    tq, h_all, _ = q.shape
    dv = v.shape[2]
    heads = list(range(h_all)) if heads is None else list(heads)
    out = np.full((tq, h_all, dv), np.nan)
    lse = np.full((tq, h_all), np.nan)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        sq, sk = q1 - q0, k1 - k0
        if sq == 0:
            continue
        vis = dense_visible(sq, sk, causal, window=window)
        for h in heads:
            scores = scale * (q[q0:q1, h, :] @ k[k0:k1, h, :].T)
            s = None if sink is None else float(sink[h])
            o, l = _softmax_rows(scores, vis, v[k0:k1, h, :], s)
            out[q0:q1, h, :] = o
            lse[q0:q1, h] = l
    return out, lse


def dense_mla_prefill_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q: Sequence[int],
                           cu_k: Sequence[int], scale: float, causal: bool,
                           tokens: Sequence[int], heads: Sequence[int],
                           sink: Optional[np.ndarray] = None,
                           window: Tuple[int, int] = (-1, -1)) -> Tuple[np.ndarray, np.ndarray]:
    """The same definition evaluated only at the given (token, head) grid: O [n_tok, n_head, Dv],
    LSE [n_tok, n_head]. Used to check large problems at sampled rows. The requested rows of one
    sequence are scored in one product against that sequence's keys, exactly as
    ``dense_mla_prefill`` scores a whole sequence; each head's K/V rows of the sequence are
    widened once."""
    cu_q = np.asarray(cu_q)
    tokens = np.asarray(tokens, dtype=np.int64)
    dv = v.shape[2]
    out = np.zeros((tokens.size, len(heads), dv))
    lse = np.zeros((tokens.size, len(heads)))
    seq = np.searchsorted(cu_q, tokens, side="right") - 1
    for b in np.unique(seq):
        sel = np.nonzero(seq == b)[0]
        q0, k0, k1 = int(cu_q[b]), int(cu_k[b]), int(cu_k[b + 1])
        sq, sk = int(cu_q[b + 1]) - q0, k1 - k0
        local = tokens[sel] - q0
        vis = dense_visible(sq, sk, causal, rows=local, window=window)
        for hi, h in enumerate(heads):
            qrows = _as_f64(q[tokens[sel], h, :])
            scores = scale * (qrows @ _as_f64(k[k0:k1, h, :]).T)
            s = None if sink is None else float(sink[h])
            o, l = _softmax_rows(scores, vis, _as_f64(v[k0:k1, h, :]), s)
            out[sel, hi] = o
            lse[sel, hi] = l
    return out, lse


def sparse_valid_slots(indices_row: np.ndarray, n_kv: int, length: Optional[int]) -> np.ndarray:
    """Valid slots of one token's index row (page "SparseFlashMla": -1 = padded; readings R8, R9)."""
    idx = np.asarray(indices_row, dtype=np.int64)
    ok = (idx >= 0) & (idx < n_kv)
    if length is not None:
        ok &= np.arange(idx.size) < int(length)
    return ok


def sparse_mla_prefill(q: np.ndarray, kv: np.ndarray, indices: np.ndarray, scale: float,
                       dv: int = 512, topk_length: Optional[np.ndarray] = None,
                       sink: Optional[np.ndarray] = None,
                       tokens: Optional[Iterable[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Sparse top-k attention over one shared latent KV (page "SparseFlashMla" formula, KV_N = 1).

    q [T, H, D], kv [N_kv, D], indices [T, topk] int32. For token t and head h, every valid slot
    contributes the logit scale * <q[t,h,:], kv[idx,:]> and the value kv[idx, :dv] (R7); each slot
    counts once, so a duplicated index counts once per slot. Returns O [T, H, dv] and LSE [T, H]
    (tokens not requested stay NaN).
    """
    q = _as_f64(q)
    kvf = _as_f64(kv)
    t_all, h_all, _ = q.shape
    n_kv = kvf.shape[0]
    toks = range(t_all) if tokens is None else tokens
    out = np.full((t_all, h_all, dv), np.nan)
    lse = np.full((t_all, h_all), np.nan)
    for t in toks:
        length = None if topk_length is None else int(topk_length[t])
        ok = sparse_valid_slots(indices[t], n_kv, length)
        rows = kvf[np.asarray(indices[t], dtype=np.int64)[ok]]
        scores = scale * (q[t] @ rows.T)                      # [H, n_valid]
        vis = np.ones(scores.shape, dtype=bool)
        for h in range(h_all):
            s = None if sink is None else float(sink[h])
            o, l = _softmax_rows(scores[h:h + 1], vis[h:h + 1], rows[:, :dv], s)
            out[t, h] = o[0]
            lse[t, h] = l[0]
    return out, lse


def paged_physical_indices(indices: np.ndarray, block_table: np.ndarray, block_size: int,
                           num_blocks: int, cu_q: Sequence[int],
                           seqused: Optional[Sequence[int]] = None,
                           seqused_q: Optional[Sequence[int]] = None) -> np.ndarray:
    """Logical index rows -> physical cache rows of [num_blocks * block_size] (reading R17);
    invalid slots, and every slot of a token not in use under seqused_q, become -1. block_table
    is [B, max_blocks] int32."""
    idx = np.asarray(indices, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    n_tok = idx.shape[0]
    out = np.full(idx.shape, -1, dtype=np.int64)
    max_blocks = bt.shape[1]
    for b in range(len(cu_q) - 1):
        used = max_blocks * block_size if seqused is None else min(int(seqused[b]), max_blocks * block_size)
        t_end = min(int(cu_q[b + 1]), n_tok)
        if seqused_q is not None:
            t_end = min(t_end, int(cu_q[b]) + max(int(seqused_q[b]), 0))
        for t in range(int(cu_q[b]), t_end):
            for k, pos in enumerate(idx[t]):
                if 0 <= pos < used:
                    entry = bt[b, pos // block_size]
                    if 0 <= entry < num_blocks:
                        out[t, k] = entry * block_size + pos % block_size
    return out


def sparse_mla_prefill_paged(q: np.ndarray, kv_cache: np.ndarray, block_table: np.ndarray,
                             cu_q: Sequence[int], indices: np.ndarray, scale: float, dv: int = 512,
                             seqused: Optional[Sequence[int]] = None,
                             topk_length: Optional[np.ndarray] = None,
                             sink: Optional[np.ndarray] = None,
                             tokens: Optional[Iterable[int]] = None,
                             seqused_q: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Sparse top-k attention over a paged latent cache kv_cache [num_blocks, block_size, D]
    with logical indices (reading R17): the indices are mapped to cache rows, then the sparse
    definition applies unchanged."""
    num_blocks, block_size, d = kv_cache.shape
    phys = paged_physical_indices(indices, block_table, block_size, num_blocks, cu_q, seqused, seqused_q)
    rows = np.asarray(kv_cache).reshape(num_blocks * block_size, d)
    return sparse_mla_prefill(q, rows, phys, scale, dv=dv, topk_length=topk_length, sink=sink, tokens=tokens)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Values rounded to bfloat16 through float32, round-to-nearest-even at each step (the
    precision in which K/V are materialised for the attention), returned as float64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def upproject_latent(latent_rows: np.ndarray, w_kv: np.ndarray, heads: int,
                     round_bf16: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Context K [n, H, 192] and V [n, H, 128] from cached latent rows [n, 576] (reading R19);
    with round_bf16 the up-projected columns are rounded to bf16 (R20)."""
    c = _as_f64(latent_rows)
    w = _as_f64(w_kv).reshape(heads * 256, 512)
    kv = (c[:, :512] @ w.T).reshape(c.shape[0], heads, 256)   # row h*256 + j of W gives column (h, j)
    if round_bf16:
        kv = round_to_bf16(kv)
    rope = np.broadcast_to(c[:, None, 512:576], (c.shape[0], heads, 64))
    return np.concatenate([kv[:, :, :128], rope], axis=2), kv[:, :, 128:]


def mla_prefill_with_latent_context(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                                    cu_q: Sequence[int], latent: np.ndarray, cu_ctx: Sequence[int],
                                    w_kv: np.ndarray, scale: float,
                                    sink: Optional[np.ndarray] = None,
                                    heads: Optional[Iterable[int]] = None,
                                    round_kv_bf16: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """New tokens q [T, H, 192] (with their k_new [T, H, 192], v_new [T, H, 128]) attending to
    their sequence's cached context (latent rows [cu_ctx[b]:cu_ctx[b+1]] of latent [N, 576],
    up-projected by w_kv) and causally to themselves (reading R19). Returns O [T, H, 128] and
    LSE [T, H]."""
    h_all = np.asarray(q).shape[1]
    k_parts, v_parts, cu_k = [], [], [0]
    for b in range(len(cu_q) - 1):
        kc, vc = upproject_latent(np.asarray(latent)[int(cu_ctx[b]):int(cu_ctx[b + 1])], w_kv, h_all,
                                  round_bf16=round_kv_bf16)
        k_parts += [kc, _as_f64(np.asarray(k_new)[int(cu_q[b]):int(cu_q[b + 1])])]
        v_parts += [vc, _as_f64(np.asarray(v_new)[int(cu_q[b]):int(cu_q[b + 1])])]
        cu_k.append(cu_k[-1] + kc.shape[0] + int(cu_q[b + 1]) - int(cu_q[b]))
    k_all = np.concatenate(k_parts) if k_parts else np.zeros((0, h_all, 192))
    v_all = np.concatenate(v_parts) if v_parts else np.zeros((0, h_all, 128))
    return dense_mla_prefill(q, k_all, v_all, cu_q, cu_k, scale, True, sink=sink, heads=heads)


def combine_partials(o_parts: np.ndarray, lse_parts: np.ndarray,
                     sink: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Merge S normalised partial results of disjoint key sets (page "Mojo module mla",
    ``mla_splitk_reduce``; page "Sgl project Sglang FA4 Interface", split-KV combine).

    o_parts [S, R, Dv], lse_parts [S, R]; sink [R] or None (an extra logit with a zero value).
    LSE = log(sum_s exp(LSE_s) [+ exp(sink)]), O = sum_s exp(LSE_s - LSE) O_s. Rows whose partials
    are all -inf (and no sink) give O = 0, LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    terms = lse_parts if sink is None else np.concatenate([lse_parts, np.asarray(sink, np.float64)[None, :]])
    m = terms.max(axis=0)
    empty = ~np.isfinite(m)
    shift = np.where(empty, 0.0, m)
    total = np.exp(terms - shift[None, :]).sum(axis=0)
    lse = np.where(empty, NEG_INF, shift + np.log(np.where(empty, 1.0, total)))
    w = np.where(empty[None, :], 0.0, np.exp(lse_parts - np.where(empty, 0.0, lse)[None, :]))
    out = (w[:, :, None] * o_parts).sum(axis=0)
    return out, lse


FP8_E4M3_MAX = 448.0


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (reading R21): bit 7 sign, bits 6..3 exponent e (bias 7),
    bits 2..0 mantissa m; e = 0 gives m * 2^-9, otherwise (1 + m/8) * 2^(e-7); e = 15 with m = 7
    is NaN. Returns float64."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def fp8_e4m3_encode(x) -> np.ndarray:
    """Saturating round-to-nearest-even into OCP FP8 E4M3 (reading R21): |x| is clamped to 448,
    then the nearest of the 127 non-negative finite values is taken, a tie going to the even
    code (the one whose mantissa ends in 0); the sign bit is x's (so -0.0 and negatives that
    round to zero give 0x80). NaN inputs are not allowed. Returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no saturating encoding here")
    grid = fp8_e4m3_decode(np.arange(0x7F))          # increasing with the code
    a = np.minimum(np.abs(x), FP8_E4M3_MAX)
    hi = np.minimum(np.searchsorted(grid, a, side="left"), 0x7E)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    code = np.where(d_hi < d_lo, hi, np.where(d_lo < d_hi, lo, np.where(hi % 2 == 0, hi, lo)))
    code = np.where(a == grid[hi], hi, code)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def quantize_output_fp8(out: np.ndarray, scale: float) -> np.ndarray:
    """FP8 output of an attention result under a static per-tensor scale (reading R21)."""
    return fp8_e4m3_encode(np.asarray(out, dtype=np.float64) / float(scale))


def _as_f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return widen_bf16(x)
    return x.astype(np.float64, copy=False)
