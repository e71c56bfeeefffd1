// Internal launch interface between the C-ABI host layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPlanSortCapacity = 16384;  // slots sorted longest-first; beyond: slot order
constexpr int kPlanMaxBlocks = 0x3FFFE;   // largest n_blocks the sort key can hold

struct PlanParams {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  int32_t mt;        // query tiles per sequence slot = ceil(max_seqlen_q / bm)
  int32_t bm, bn;
  int32_t causal;    // right-limited: keys past the bottom-right diagonal + win_right are hidden
  int32_t win_right; // >= 0 (0 when causal)
  int32_t win_left;  // -1: unlimited; else keys before the diagonal - win_left are hidden
  int32_t* plan;     // [capacity][4]
  int32_t capacity;
  int32_t* num_items;
  int32_t* counters;  // nullable [8][32]: element 0 of each line zeroed (dense work tickets)
  int32_t* plan_ext;  // nullable [capacity][4]: (cu_q[b], Sq, cu_k[b], Sk) of each valid entry
};

struct DenseParams {
  const __bf16* q; int64_t q_st, q_sh;
  const __bf16* k; int64_t k_st, k_sh;
  const __bf16* v; int64_t v_st, v_sh;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* plan;
  const int32_t* plan_ext;   // [n_slots][4] (cu_q[b], Sq, cu_k[b], Sk) per valid plan entry
  const int32_t* num_items;
  int32_t n_slots;       // plan capacity (batch * Mt)
  int32_t num_heads;
  int32_t num_splits;
  int32_t causal;        // right-limited (causal, or a right window of win_right keys)
  int32_t win_right;     // >= 0: keys up to diagonal + win_right are visible (0 when causal)
  int32_t win_left;      // -1: unlimited; else keys from diagonal - win_left are visible
  float scale;           // softmax scale
  float scale_log2;      // softmax scale * log2(e)
  const float* sink;     // nullable [H]; applied here only when unsplit
  void* out; int64_t o_st, o_sh;  // bf16, or fp8 e4m3 for the fp8-output instances (element strides)
  const float* out_scale;         // fp8 output: device [1], stored value = O / out_scale
  float* lse; int64_t l_st, l_sh;
  float* o_part;         // split mode: [S][total_q][H][DV] fp32, else null
  float* lse_part;       // split mode: [S][total_q][H]
  int32_t accumulate;    // with one split: 1 = merge into o_part / lse_part (running result) in
                         // place; 2 = merge with it and write out / lse (with the sink) instead
  int32_t total_q;
  int32_t wgs_per_xcd;   // persistent grid: 8 * wgs_per_xcd work-groups
  int32_t group_units;   // (head, split) units per scheduling group
  int32_t xcd_units;     // > 0: units owned by each XCD (contiguous); 0: interleaved lists
  int32_t* counters;     // [8][32] work ticket counter per XCD list (element 0 of each
                         // 128-byte line), zero at launch
};

struct SparseParams {
  const __bf16* q; int64_t q_st, q_sh;
  const __bf16* kv; int64_t kv_st; int64_t n_kv;
  const int32_t* idx; int64_t idx_st; int32_t topk;
  const int32_t* topk_length;
  int32_t num_tokens, num_heads;
  float scale, scale_log2;
  const float* sink;
  __bf16* out; int64_t o_st, o_sh;
  float* lse; int64_t l_st, l_sh;
  // Paged latent cache (null block_table: indices are physical rows). Token t belongs to the
  // sequence b with cu_q[b] <= t < cu_q[b+1]; logical position pos of its index row is cache row
  // block_table[b * bt_st + pos / block_size] * block_size + pos % block_size, valid only for
  // 0 <= pos < min(seqused[b] (if given), max_blocks * block_size) and a table entry in
  // [0, num_blocks).
  const int32_t* block_table; int64_t bt_st;
  int32_t max_blocks, block_size, num_blocks;
  const int32_t* cu_q; int32_t batch;
  const int32_t* seqused;
  const int32_t* seqused_q;  // nullable [batch]: tokens of sequence b at or past cu_q[b] + seqused_q[b] see no key
  int32_t max_wgs;           // persistent grid: at most this many work-groups (the CU count)
};

struct CombineParams {
  const float* o_part;
  const float* lse_part;
  int32_t num_splits;
  int32_t rows;          // tokens * heads
  int32_t num_heads;
  int32_t dv;
  const float* sink;
  void* out; int64_t o_st, o_sh;   // bf16, or fp8 e4m3 when out_scale is set (element strides)
  const float* out_scale;          // nullable device [1]: fp8 output of O / out_scale
  float* lse; int64_t l_st, l_sh;
};

// Up-projection of a chunk of cached latent rows into per-head K/V (see latent_ctx.hip).
struct UpprojParams {
  const __bf16* latent; int64_t lat_st;   // [N, 576] rows: 512 latent + 64 rope
  const int32_t* cu_ctx;                   // [batch + 1] cached rows of each sequence
  const int32_t* cu_chunk;                 // [batch + 1] buffer rows of each sequence in the chunk
  int32_t batch, c0, w;                    // chunk: context positions [c0, c0 + w) of each sequence
  const __bf16* w_kv; int64_t w_st;        // [H * 256, 512]
  int32_t num_heads;
  __bf16* kbuf; int64_t k_st, k_sh;        // [rows, H, 192]
  __bf16* vbuf; int64_t v_st, v_sh;        // [rows, H, 128]
};

hipError_t launch_plan(const PlanParams& p, hipStream_t stream);
hipError_t launch_chunk_cu(const int32_t* cu_ctx, int32_t batch, int32_t c0, int32_t w, int32_t* cu_chunk,
                           hipStream_t stream);
hipError_t launch_upproj(const UpprojParams& p, hipStream_t stream);
// Dense kernel instances: (dqk, dv) in {(192, 128), (128, 128), (256, 256)}, bf16 or fp8 output,
// nw waves (32 query rows each) per work-group: 4 or 8 for (192, 128), dense_default_waves for
// the others. An unsupported combination launches nothing and returns hipErrorInvalidValue.
hipError_t launch_dense_fwd(const DenseParams& p, int nw, int dqk, int dv, bool fp8_out, hipStream_t stream);
bool dense_waves_ok(int nw, int dqk, int dv);
int dense_default_waves(int dqk, int dv);
// Resident work-groups per CU of the instance.
int dense_occupancy_of(int nw, int dqk, int dv);
// Query rows per work item (tile height) of the instance.
int dense_rows_per_tile(int nw, int dqk, int dv);
hipError_t launch_sparse_fwd(const SparseParams& p, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);

}  // namespace mla
