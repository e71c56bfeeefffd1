/*
 * mla_prefill.h -- C ABI of the MI355X (gfx950) MLA prefill library (libmla_prefill.so).
 *
 * Multi-head Latent Attention prefill, forward only:
 *   O = softmax(Q K^T * softmax_scale + mask) V, with an optional float32 log-sum-exp (LSE).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is caller-owned DEVICE memory on the current HIP device. The library
 *    never allocates or frees memory in these calls and keeps no pointer after a call returns.
 *  - Calls only enqueue work on `hip_stream` (a hipStream_t; NULL = the default stream) and
 *    never synchronise; the caller keeps every buffer alive until the stream has consumed it.
 *    Device-side faults surface at the caller's next synchronisation.
 *  - bf16 tensors are row-major with a contiguous last dimension. Strides are in ELEMENTS,
 *    must be multiples of 8 (16 bytes) and non-negative; base pointers must be 16-byte aligned.
 *  - LSE is the natural-log log-sum-exp of the *scaled* logits, float32. A row that sees no key
 *    gets O = 0 and LSE = -inf (LSE = sink when a sink is given).
 *  - `sink` (nullable) is one float32 logit per head, used as-is (not scaled) as an extra key
 *    whose value vector is zero.
 *  - `softmax_scale` must be finite and > 0 (the kernels track the running maximum of the raw
 *    logits, which is the maximum of the scaled ones only for a positive scale); any other value
 *    returns MLA_ERR_INVALID_ARG.
 *  - Errors are returned as mla_status_t; nothing is launched when a call returns an error.
 *    Per-element contents (cu_seqlens values, index values) are not validated by default:
 *    out-of-range sparse indices are skipped, which is memory-safe; malformed cu_seqlens are the
 *    caller's bug. With the environment variable MLA_VALIDATE set to a nonzero integer (read at
 *    every call), the dense and chunked-context entry points and the paged sparse entry point
 *    first copy their cu_seqlens to the host, SYNCHRONISING the stream, and return
 *    MLA_ERR_INVALID_ARG unless every array starts at 0 and is non-decreasing with no length
 *    above its max_seqlen, cu_seqlens_q ends at total_q (dense, chunked context) or at most at
 *    num_tokens (paged sparse); MLA_ERR_HIP if the copy fails. It is a debugging aid, not for
 *    graph capture.
 *  - `out`/`lse` must not alias any input or the workspace.
 */
#ifndef MLA_PREFILL_H
#define MLA_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,  /* null required pointer, bad size, bad stride, bad num_splits     */
  MLA_ERR_UNSUPPORTED = 2,  /* head dims, head count, top-k or device outside what is built    */
  MLA_ERR_ALIGNMENT = 3,    /* base pointer not 16-byte aligned or stride not a multiple of 8  */
  MLA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the *_workspace_size result   */
  MLA_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed                      */
} mla_status_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* mla_status_string(int status);

/* Library ABI version (increments on any signature change). */
int32_t mla_abi_version(void);

/* Query-tile rows (BM) and key-block size (BN) of the dense kernel's default instances; the
 * plan uses the same values by default. The (192, 128) layout runs tiles of 2 * BM rows instead
 * when max_seqlen_q >= 256 and max_seqlen_k >= 2048 (8192 with the causal mask); see
 * mla_prefill_varlen. */
void mla_dense_tile_shape(int32_t* block_m, int32_t* block_n);

/* ------------------------------------------------------------------------------------------
 * Varlen tile plan (GPU kernel, no host synchronisation).
 *
 * Prior art: a device-side planner for ragged batches with a helper that clears its counters
 * (page "Mojo module mla", mla_prefill_plan_kernel, set_buffer_lengths_to_zero), and a metadata
 * call run before the attention operator that fills a fixed-size int32 task table (page
 * "SparseFlashMla", Description and Constraints, SparseFlashMlaMetadata).
 *
 * It is the planner mla_prefill_varlen itself runs, exposed so that its bytes can be checked.
 * It takes the tile sizes and the window instead of max_seqlen_k and num_splits: the items
 * depend on the tile height, the key block and the mask (a window changes n_blocks and the
 * order), not on the key-length bound or the split count. The split is not a planned field:
 * the attention kernel divides an item's n_blocks key blocks into the call's S contiguous
 * ranges itself (split s takes blocks [s*n/S, (s+1)*n/S)), so one plan serves every split
 * count.
 *
 * Slots are (b, m) for b < batch and m < Mt = ceil(max_seqlen_q / block_m); slot (b, m) is an
 * item iff m < T_b = ceil(Sq_b / block_m). Query tiles are aligned to the end of the sequence:
 * tile m holds the existing rows of [m * block_m - pad_b, (m + 1) * block_m - pad_b), pad_b =
 * T_b * block_m - Sq_b (the Sq_b mod block_m leftover rows form tile 0, where causal rows see the
 * fewest keys). Each item is four int32 words (b, m, n_blocks, kv_end): kv_end is the count of
 * leading keys any row of the tile may see (Sk_b without a right limit, else the bottom-right
 * bound clamp(i_last + Sk_b - Sq_b + r + 1, 0, Sk_b) with i_last the tile's last row and r the
 * right window, 0 when causal). With a left window l >= 0 the first key any row may see is
 * kv_start = clamp(i_first + Sk_b - Sq_b - l, 0, Sk_b) with i_first the tile's first row, else 0;
 * n_blocks counts the blocks from kv_start / block_n to ceil(kv_end / block_n) (0 when
 * kv_end <= kv_start).
 * Items are ordered sequence by sequence, sequences with more key blocks first
 * (min(ceil(Sk_b / block_n), 0x3FFFE) descending, ties by b ascending), and within a sequence
 * from its last query tile to its first (m descending); with a left window (window_left >= 0)
 * by n_blocks descending, then slot (b * Mt + m) ascending. With more than 16384 slots they stay
 * in slot order. Words of unused items up to plan_capacity are set to -1.
 *
 *   cu_seqlens_q, cu_seqlens_k : device int32 [batch + 1], non-decreasing, starting at 0.
 *   causal, window_left, window_right : the mask rule of mla_prefill_varlen_window.
 *   plan                       : device int32 [plan_capacity * 4], written.
 *   num_items                  : device int32 [1], written.
 * Errors: INVALID_ARG for null pointers, batch < 0, max_seqlen_q < 0, block sizes that are not
 * powers of two in [16, 1024], plan_capacity < batch * Mt, or a window below -1.
 * ------------------------------------------------------------------------------------------ */
mla_status_t mla_prefill_plan(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t batch, int32_t max_seqlen_q, int32_t block_m,
                              int32_t block_n, int32_t causal, int32_t window_left,
                              int32_t window_right, int32_t* plan, int32_t plan_capacity,
                              int32_t* num_items, void* hip_stream);

/* ------------------------------------------------------------------------------------------
 * Dense varlen MLA prefill.
 *
 * The vLLM MLA prefill backend expands K/V to every query head and calls a varlen attention
 * kernel with q/k head 192 (128 nope + 64 rope), v head 128, int32 cu_seqlens [B+1], an explicit
 * softmax scale, causal on for new tokens and off for context chunks, optional LSE and a
 * caller-owned `out` (page "FlashAttention backend for MLA prefill": dispatch,
 * _flash_attn_varlen_diff_headdims, run_prefill_new_tokens, run_prefill_context_chunk); the
 * varlen API's I/O contract and num_splits (0 = heuristic, 1 = no split) follow page
 * "Sgl project Sglang FA4 Interface" (Signature, I/O Contract).
 *
 * Head dimensions (head_dim_qk, head_dim_v): (192, 128), the layout above, and the other MLA
 * layouts the same backend lists (supports_mla_dimensions): nope 64 + rope 64 with v 128 =
 * (128, 128); nope 192 + rope 64 and nope 256 + rope 0, both with v 256 = (256, 256). Written
 * below for (192, 128); Dqk / Dv stand for the pair in use.
 *
 *   q   : bf16 [total_q, H, 192], strides (q_stride_tok, q_stride_head)
 *   k   : bf16 [total_k, H, 192], strides (k_stride_tok, k_stride_head)
 *   v   : bf16 [total_k, H, 128], strides (v_stride_tok, v_stride_head); V may be a strided view
 *         (e.g. token stride H*256, head stride 256 inside a packed K/V buffer)
 *   cu_seqlens_q/k : device int32 [batch + 1]; sequence b owns query rows [cu_q[b], cu_q[b+1])
 *         and key rows [cu_k[b], cu_k[b+1]); max_seqlen_q/k bound every Sq_b / Sk_b.
 *   causal : 0 = no mask; 1 = bottom-right aligned causal (key j visible to query i iff
 *         j <= i + Sk_b - Sq_b), which is the usual causal mask when Sq_b == Sk_b.
 *   num_splits : 0 = library heuristic, 1 = no split, n in [2, 64] = split each row's keys into n
 *         parts merged by the combine kernel (results agree within rounding, not bitwise).
 *   sink : nullable float32 [H].
 *   out  : bf16 [total_q, H, 128], strides (o_stride_tok, o_stride_head), written.
 *   lse  : nullable float32 [total_q, H], strides (lse_stride_tok, lse_stride_head), written.
 *   workspace : device memory of at least mla_prefill_varlen_workspace_size(...) bytes with the
 *         same batch/total_q/max_seqlen/H/head_dim_v/causal/num_splits (it returns 0 for arguments it
 *         rejects, a head_dim_v other than 128 or 256 included); scratch only, contents undefined
 *         after.
 *         It holds the plan and the work-ticket counters of the call: calls that may overlap in
 *         time (other streams) must not share a workspace.
 * Work items are query tiles of 128 rows (four-wave work-groups, two per CU). For (192, 128),
 * when max_seqlen_q >= 256 and max_seqlen_k >= 2048 (8192 with causal != 0), they are tiles of
 * 256 rows (eight-wave work-groups, one per CU), which halve the key/value copies per query row
 * where the rows see many keys; the bounds pick the instance, so a call with looser bounds may
 * run the other one (results agree within rounding).
 * Tuning (environment, read by the library): MLA_DENSE_GROUP=n schedules n (head, split) units
 * per XCD at a time (default 1); MLA_DENSE_WGS_PER_XCD=n caps the persistent grid at 8*n
 * work-groups (default: all resident slots). Both leave results bitwise unchanged (each work item
 * is computed the same way whichever work-group runs it). MLA_DENSE_WAVES=4 or 8 forces the
 * (192, 128) tile height (read once per process; the workspace size and split helpers follow it).
 * With num_splits == 1 a sequence's result does not depend on the other sequences in the batch,
 * and repeated calls are bitwise identical.
 * Errors: INVALID_ARG (null q/k/v/cu/out, sizes <= 0 where a count is required, strides smaller
 * than the row they hold, num_splits outside [0, 64]); UNSUPPORTED (head dims other than the
 * three pairs above, H > 65535, max_seqlen_k beyond 2^24, K or V token stride of 2^23 elements or more);
 * ALIGNMENT; WORKSPACE; HIP.
 * ------------------------------------------------------------------------------------------ */
size_t mla_prefill_varlen_workspace_size(int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                         int32_t max_seqlen_k, int32_t num_heads,
                                         int32_t head_dim_v, int32_t causal, int32_t num_splits);

mla_status_t mla_prefill_varlen(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, int32_t causal, int32_t num_splits, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------------------------
 * Allocation-free variant of mla_prefill_varlen.
 *
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. Same operation, arguments (without the workspace),
 * kernels and results as mla_prefill_varlen; the plan, the work-ticket counters and the split
 * partials live in a static device array of MLA_NOALLOC_SCRATCH_BYTES bytes inside the library
 * (one per GPU, held from library load until the process ends). The call allocates nothing and
 * clears what must start at zero itself (the planner kernel zeroes the counters), so it may be
 * captured into a HIP graph.
 *   - Every call on one GPU uses that GPU's single array: calls that may overlap in time on the
 *     same GPU (different streams, or concurrent host threads) RACE and must be serialised by
 *     the caller. Sequential calls on one stream are safe.
 *   - MLA_VALIDATE is ignored here (its host copy allocates and synchronises).
 * Size limit: the call runs iff mla_prefill_varlen_workspace_size(...) for the same arguments is
 * at most MLA_NOALLOC_SCRATCH_BYTES (64 MiB). Unsplit, that is about 1.3 KB plus 32 bytes per
 * query-tile slot (batch * ceil(max_seqlen_q / 128)), so every call below two million slots
 * fits; each split adds total_q * H * (head_dim_v + 1) * 4 bytes of partials, so a split call
 * (forced, or chosen by the heuristic for small grids) fits only while those partials do.
 * Errors: those of mla_prefill_varlen, where WORKSPACE means the size limit above is exceeded
 * (checked on the host before anything is launched); HIP if the array's device address cannot
 * be resolved.
 * ------------------------------------------------------------------------------------------ */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

mla_status_t mla_prefill_varlen_noalloc(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, int32_t causal, int32_t num_splits, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head, void* hip_stream);

/* ------------------------------------------------------------------------------------------
 * Dense varlen MLA prefill with a sliding-window (band) mask.
 *
 * mla_prefill_varlen with a window (page "Sgl project Sglang FA4 Interface", window_size =
 * (left, right), e.g. (256, 0) = causal with a 256-key window; page "SparseFlashMla",
 * ori_win_left / ori_win_right: past / future tokens a query sees, -1 = unlimited). Aligned
 * bottom-right like the causal mask: with d = Sk_b - Sq_b, key j is visible to local query i iff
 * j >= i + d - window_left (when window_left >= 0) and j <= i + d + window_right (when
 * window_right >= 0); causal != 0 sets window_right to 0. (-1, -1) without causal is the
 * unmasked rule and equals mla_prefill_varlen. Rows with no visible key get O = 0 and
 * LSE = -inf (or the sink). Key blocks outside every row's window are not read. Arguments,
 * workspace (mla_prefill_varlen_workspace_size), outputs and errors as for mla_prefill_varlen,
 * plus INVALID_ARG for a window below -1.
 * ------------------------------------------------------------------------------------------ */
mla_status_t mla_prefill_varlen_window(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, int32_t causal, int32_t window_left, int32_t window_right,
    int32_t num_splits, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------------------------
 * Dense varlen MLA prefill with FP8 output under a static per-tensor scale.
 *
 * The FA4 path of the MLA prefill backend can emit its output already quantised to FP8 with a
 * static, symmetric per-tensor scale (page "FlashAttention backend for MLA prefill",
 * supports_quant_output with kFp8StaticTensorSym). Reading: the stored value is the OCP FP8
 * E4M3 (finite-only, bias 7, max 448) encoding, rounded to nearest even, of O / out_scale, where
 * O is the fp32 normalised attention output; values beyond +-448 saturate to +-448. The LSE
 * stays float32 and unscaled.
 *
 * Arguments are those of mla_prefill_varlen_window, except:
 *   out_scale : device float32 [1], > 0 (read on the device; not validated).
 *   out       : fp8 e4m3 bytes [total_q, H, Dv], strides in elements (bytes) that are multiples
 *               of 16; 16-byte aligned.
 * The workspace is sized by mla_prefill_varlen_workspace_size with the same head_dim_v.
 * Errors: as mla_prefill_varlen_window; INVALID_ARG also for a null out_scale; ALIGNMENT for an
 * output stride that is not a multiple of 16 or an out_scale not 4-byte aligned.
 * ------------------------------------------------------------------------------------------ */
mla_status_t mla_prefill_varlen_fp8(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, int32_t causal, int32_t window_left, int32_t window_right,
    int32_t num_splits, const float* sink, const float* out_scale,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream);

/* The number of key splits mla_prefill_varlen (and its window and FP8 variants) uses for these
 * arguments: num_splits itself when >= 1, else the library heuristic's choice for the kernel
 * instance of (head_dim_qk, head_dim_v), with the same tile height and residency the call uses.
 * Returns -1 for num_splits outside [0, 64] or head dims that are not built. */
int32_t mla_prefill_varlen_num_splits(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
                                      int32_t causal, int32_t num_splits);

/* ------------------------------------------------------------------------------------------
 * Sparse top-k MLA prefill over one shared latent KV (absorbed MLA, KV_N = 1).
 *
 * Formula O = softmax(Q K~^T * softmax_scale) V~ with K~ = V~ the gathered rows; int32 indices
 * with -1 marking an invalid/padded slot; optional topk_length (valid, left-aligned prefix of
 * each index row, in [0, topk]); optional float sinks; nullable LSE (page "SparseFlashMla",
 * Description: formula; Parameters table; Constraints). Indices are physical pool rows, already
 * remapped by the caller (page "mla_prefill_branch_sparse_fp8", description of d_indices).
 * The 576-column rows hold 512 latent columns then 64 rope columns; V is the first 512 columns.
 *
 *   q       : bf16 [num_tokens, H, 576], strides (q_stride_tok, q_stride_head)
 *   kv      : bf16 [n_kv, 576], row stride kv_stride_row
 *   indices : int32 [num_tokens, topk], row stride idx_stride_tok (>= topk). Slot s of token t
 *             takes part iff s < topk_length[t] (when given) and 0 <= indices[t][s] < n_kv.
 *             Each slot counts once, so a repeated index counts once per slot.
 *   topk_length : nullable int32 [num_tokens]
 *   sink    : nullable float32 [H]
 *   out     : bf16 [num_tokens, H, 512], strides (o_stride_tok, o_stride_head), written.
 *   lse     : nullable float32 [num_tokens, H], strides (lse_stride_tok, lse_stride_head).
 *   workspace : may be NULL when mla_prefill_sparse_workspace_size(...) returns 0.
 * Errors: INVALID_ARG; UNSUPPORTED (head dims other than 576/512, H outside [1, 128], topk
 * outside [1, 8192], n_kv or kv_stride_row above 2^31 - 1); ALIGNMENT; WORKSPACE; HIP.
 * ------------------------------------------------------------------------------------------ */
size_t mla_prefill_sparse_workspace_size(int32_t num_tokens, int32_t num_heads, int32_t topk,
                                         int32_t head_dim_v);

mla_status_t mla_prefill_sparse(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* kv, int64_t kv_stride_row, int64_t n_kv,
    const int32_t* indices, int64_t idx_stride_tok, int32_t topk,
    const int32_t* topk_length,
    int32_t num_tokens, int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------------------------
 * Sparse top-k MLA prefill over a paged latent cache with logical indices.
 *
 * The same operation as mla_prefill_sparse, with the latent cache laid out in pages and the
 * indices given as logical token positions of each query's own sequence (page "SparseFlashMla",
 * Parameters table: block_table for PageAttention, cu_seqlens_q, seqused, topk_value_mode 1 =
 * logical token indices; Constraints: PA_BBND cache [block_num, block_size, KV_N = 1, D],
 * block_size 1..1024, block table [B, >= ceil(max KV length / block_size)]).
 *
 *   kv_cache    : bf16 [num_blocks * block_size, 576] rows, row stride kv_stride_row; block e
 *                 holds rows [e * block_size, (e + 1) * block_size). Read only.
 *   block_table : device int32 [batch, bt_stride_seq >= max_blocks_per_seq]; entry [b][i] is the
 *                 cache block of logical positions [i * block_size, (i + 1) * block_size) of
 *                 sequence b.
 *   cu_seqlens_q: device int32 [batch + 1], non-decreasing, cu[0] = 0; token t belongs to the
 *                 sequence b with cu[b] <= t < cu[b + 1].
 *   seqused_kv  : nullable device int32 [batch]; the number of valid logical positions of each
 *                 sequence (default: max_blocks_per_seq * block_size).
 *   seqused_q   : nullable device int32 [batch]; the number of query tokens of each sequence
 *                 that are in use (page "Sgl project Sglang FA4 Interface", Signature:
 *                 seqused_q). Token t of sequence b is in use iff t - cu[b] < seqused_q[b];
 *                 a token not in use is written as a row without keys (O = 0, LSE = -inf, or
 *                 the sink). Default: every token of [cu[b], cu[b + 1]).
 *   indices     : int32 [num_tokens, topk] logical positions, row stride idx_stride_tok.
 * Slot s of token t takes part iff s < topk_length[t] (when given), 0 <= pos < min(seqused[b],
 * max_blocks_per_seq * block_size) and 0 <= block_table[b][pos / block_size] < num_blocks; it
 * then reads cache row block_table[b][pos / block_size] * block_size + pos % block_size. Any
 * other slot (-1, past the used length, a bad table entry) is skipped, which is memory-safe.
 * A token outside every sequence, or not in use under seqused_q, gets O = 0 and LSE = -inf
 * (or the sink). Other arguments,
 * outputs and ownership as for mla_prefill_sparse.
 * Errors: INVALID_ARG (null block_table or cu_seqlens_q, batch, num_blocks, block_size or
 * max_blocks_per_seq <= 0, bt_stride_seq < max_blocks_per_seq, and the mla_prefill_sparse
 * checks); UNSUPPORTED (block_size > 1024, num_blocks * block_size or max_blocks_per_seq *
 * block_size above 2^31 - 1, and the mla_prefill_sparse cases); ALIGNMENT (also int32 arrays
 * not 4-byte aligned); HIP. Sequence boundaries and table contents are not validated on the host
 * (they are device memory); the kernel only reads table entries [0, max_blocks_per_seq).
 * ------------------------------------------------------------------------------------------ */
mla_status_t mla_prefill_sparse_paged(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* kv_cache, int64_t kv_stride_row, int32_t num_blocks, int32_t block_size,
    const int32_t* block_table, int64_t bt_stride_seq, int32_t max_blocks_per_seq,
    const int32_t* cu_seqlens_q, int32_t batch, const int32_t* seqused_kv,
    const int32_t* seqused_q,
    const int32_t* indices, int64_t idx_stride_tok, int32_t topk,
    const int32_t* topk_length,
    int32_t num_tokens, int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------------------------
 * Dense MLA prefill of new tokens over a cached latent context, chunk by chunk.
 *
 * The new tokens of each sequence attend causally to themselves and, without a mask, to the
 * sequence's cached context; the parts are merged through their LSEs (page "FlashAttention
 * backend for MLA prefill", run_prefill_new_tokens, run_prefill_context_chunk with causal=False
 * and the LSE always returned). The context is cached as latent rows of 512 columns + 64 rope
 * columns and turned into per-head K/V by the W_UK / W_UV up-projections (page
 * "mla_prefill_branch_sparse_fp8", w_uk / w_uv): head h's key of cached row c is
 * [c[0:512] W_UK_h^T (128) || c[512:576] (64)] and its value c[0:512] W_UV_h^T (128).
 * Equivalently: attention over [context keys || new keys] with the bottom-right causal mask.
 *
 * The context is processed in chunks of chunk_tokens positions per sequence through a bounded
 * buffer (batch * chunk_tokens rows of K and V, in the workspace): per chunk, the rows are
 * up-projected (mla_latent_upproject) and attended without a mask, and the chunk's result is
 * merged into the running fp32 result by the attention kernel as it writes it; the sink is
 * folded in once at the end.
 *
 *   q, k, v        : the new tokens, bf16 [total_q, H, 192] / [total_q, H, 192] / [total_q, H, 128].
 *   cu_seqlens_q   : device int32 [batch + 1] (new tokens of each sequence).
 *   latent         : bf16 [N, 576] cached rows, row stride latent_stride_row; sequence b's context
 *                    is rows [cu_seqlens_ctx[b], cu_seqlens_ctx[b + 1]) in position order.
 *   cu_seqlens_ctx : device int32 [batch + 1]; max_seqlen_ctx >= every context length (the number
 *                    of chunks is ceil(max_seqlen_ctx / chunk_tokens)).
 *   w_kv           : bf16 [H * 256, 512], row stride w_stride_row: rows h*256 + 0..127 = W_UK_h,
 *                    h*256 + 128..255 = W_UV_h (a linear layer's weight layout).
 *   sink, out, lse : as for mla_prefill_varlen.
 *   workspace      : mla_prefill_chunked_context_workspace_size(...) bytes, 16-byte aligned.
 * Errors: INVALID_ARG, UNSUPPORTED (batch > 65535, chunk buffer above 2^31 - 1 rows, w_stride_row
 * of 2^23 elements or more), ALIGNMENT, WORKSPACE, HIP, and those of mla_prefill_varlen for the
 * new-token tensors.
 * ------------------------------------------------------------------------------------------ */
size_t mla_prefill_chunked_context_workspace_size(int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                                  int32_t num_heads, int32_t chunk_tokens);

mla_status_t mla_prefill_chunked_context(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    const int32_t* cu_seqlens_q, const void* latent, int64_t latent_stride_row,
    const int32_t* cu_seqlens_ctx, const void* w_kv, int64_t w_stride_row,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_ctx,
    int32_t num_heads, int32_t chunk_tokens, float softmax_scale, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------------------------
 * Up-projection of one chunk of cached latent rows into per-head K/V (the building block of
 * mla_prefill_chunked_context; same reading of the pages).
 *
 * For each sequence b, the context positions [ctx_start, ctx_start + chunk_tokens) that exist
 * (clamped to its length) are written to consecutive rows of k_out / v_out, sequence after
 * sequence; cu_chunk (device int32 [batch + 1], written) receives the row offsets, so k_out /
 * v_out with cu_chunk are directly the keys of a varlen call.
 *   k_out : bf16 [batch * chunk_tokens, H, 192] (token stride H * 192), written: key columns
 *           0..127 = c W_UK_h^T, 128..191 = the rope columns.
 *   v_out : bf16 [batch * chunk_tokens, H, 128] (token stride H * 128), written.
 * Errors: INVALID_ARG, UNSUPPORTED (batch > 65535, w_stride_row of 2^23 elements or more),
 * ALIGNMENT, HIP.
 * ------------------------------------------------------------------------------------------ */
mla_status_t mla_latent_upproject(const void* latent, int64_t latent_stride_row,
                                  const int32_t* cu_seqlens_ctx, int32_t batch, int32_t ctx_start,
                                  int32_t chunk_tokens, const void* w_kv, int64_t w_stride_row,
                                  int32_t num_heads, int32_t* cu_chunk, void* k_out, void* v_out,
                                  void* hip_stream);

/* ------------------------------------------------------------------------------------------
 * Combine S partial results of disjoint key sets into the final result (split-KV reduction;
 * also merges a context-chunk result with a new-token result through their LSEs).
 *
 * Prior art: per-partition partial outputs reduced into the final result (page "Mojo module
 * mla", mla_splitk_reduce; page "Sgl project Sglang FA4 Interface", Description: split-KV with a
 * combine kernel); the LSE-returning context-chunk call exists to allow this merge (page
 * "FlashAttention backend for MLA prefill", run_prefill_context_chunk).
 *
 *   o_part   : float32 [num_splits, num_rows, head_dim_v] contiguous, each partial normalised
 *   lse_part : float32 [num_splits, num_rows] contiguous; -inf marks an empty partial
 *   num_rows = num_tokens * num_heads with row r = t * num_heads + h
 *   sink     : nullable float32 [num_heads], merged as one more partial with a zero value
 *   out      : bf16 [num_tokens, num_heads, head_dim_v], strides (o_stride_tok, o_stride_head)
 *   lse      : nullable float32 [num_tokens, num_heads], strides (lse_stride_tok, lse_stride_head)
 * LSE = log(sum_s exp(LSE_s) [+ exp(sink)]); O = sum_s exp(LSE_s - LSE) O_s.
 * Errors: INVALID_ARG (nulls, num_splits outside [1, 256], head_dim_v not a multiple of 8 or
 * above 1024); ALIGNMENT; HIP.
 * ------------------------------------------------------------------------------------------ */
mla_status_t mla_combine(const float* o_part, const float* lse_part, int32_t num_splits,
                         int32_t num_tokens, int32_t num_heads, int32_t head_dim_v,
                         const float* sink, void* out, int64_t o_stride_tok,
                         int64_t o_stride_head, float* lse, int64_t lse_stride_tok,
                         int64_t lse_stride_head, void* hip_stream);

/* ------------------------------------------------------------------------------------------
 * Measurement aid (not part of the computation). While enabled, every kernel the library
 * launches is bracketed by a pair of HIP events recorded on the launch stream; reading waits
 * for the recorded events and accumulates per-kernel launch counts and total device time.
 * Enabling clears the totals. Events are created on first use and reused; at most 65536
 * launches are held between two reads (later ones are not timed).
 *   kernel: MLA_KERNEL_PLAN, MLA_KERNEL_DENSE, MLA_KERNEL_COMBINE, MLA_KERNEL_SPARSE,
 *           or MLA_KERNEL_UPPROJ (latent up-projection).
 * Errors: INVALID_ARG (unknown kernel, null outputs); HIP (event calls failed).
 * ------------------------------------------------------------------------------------------ */
enum { MLA_KERNEL_PLAN = 0, MLA_KERNEL_DENSE = 1, MLA_KERNEL_COMBINE = 2, MLA_KERNEL_SPARSE = 3,
       MLA_KERNEL_UPPROJ = 4 };
mla_status_t mla_profile_enable(int32_t enable);
/* Restricts the timing to the kernel kinds whose bit (1 << MLA_KERNEL_x) is set in `kinds`
 * (default: all); kinds left out are launched without events. Never fails. */
mla_status_t mla_profile_select(uint32_t kinds);
mla_status_t mla_profile_read(int32_t kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PREFILL_H */
