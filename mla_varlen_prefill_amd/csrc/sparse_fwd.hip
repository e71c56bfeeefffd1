// Sparse top-k MLA prefill forward for gfx950 over one shared latent KV (absorbed MLA):
//   O[t,h] = softmax_k(scale * q[t,h] . kv[idx[t,k]]) kv[idx[t,k], :512]  (+ optional sink)
//
// The formula with K~ = V~ the gathered rows, int32 indices with -1 as the padded slot, the
// optional topk_length prefix and the sinks are those of page "SparseFlashMla" (Description:
// formula; Parameters table; Constraints); the indices are physical rows of the latent cache
// as in page "mla_prefill_branch_sparse_fp8". The 576 columns are 512 latent then 64 rope; the
// value vector is the first 512 columns of the same row.
//
// Work decomposition: one work-group (4 waves, one per SIMD) per query token. All heads of a
// token read the same gathered rows, so the heads form the matrix-core N dimension (wave w owns
// heads [32w, 32w+32)) and every latent row is gathered once per token:
//   1. Q is split along its 576 columns: columns [0, 288) of all heads are staged in LDS once,
//      columns [288, 576) stay in registers (72 per lane), which leaves room for the 256-register
//      O^T accumulator without spilling;
//   2. blocks of 32 index slots are processed in slot order: their latent rows are copied
//      global -> LDS directly (double-buffered) and a 32-bit validity mask (-1, out of range, or
//      at/after topk_length) is kept next to them;
//   3. S^T (32 keys x 32 heads) = K~ (A, LDS) * Q^T (B, LDS then registers), 576 deep;
//   4. online softmax per head (one lane pair per head) against a reference max fixed by the
//      first block with a visible key, so the O^T accumulator is never rescaled (P may reach
//      2^32, well inside fp32/bf16 range). The exact running max is tracked as well; if any
//      head's max exceeds its reference by more than 2^32, the work-group runs the slots a
//      second time with the exact max as the reference (rare; never for data whose logits span
//      less than about 22 nats within a row);
//   5. O^T (512 x 32 heads) += V~^T (A, transposed LDS reads of the same rows) * P^T (B).
// Gathered rows are 72 chunks of 16 bytes; chunk c of row r sits at c ^ f(r) with
// f(r) = ((r & 3) << 1) | ((r >> 2) & 1), which keeps both the row-wise K~ reads (8 consecutive
// rows) and the transposed V~ reads (4 consecutive rows, 32 bytes each) free of bank conflicts.
// Q rows in LDS are padded to 592 bytes so 8 consecutive heads start on distinct banks.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int D = 576;
constexpr int DVS = 512;
constexpr int BNS = 32;
constexpr int ROW_BYTES = D * 2;                        // 1152
constexpr int CHUNKS = D / 8;                           // 72
constexpr int STAGE_BYTES = BNS * ROW_BYTES;            // 36864
constexpr int CHUNKS_PER_WAVE = BNS * CHUNKS / 256;     // 9 wave-wide 1 KiB copies per block
constexpr int MAX_HEADS = 128;
constexpr int KK_LDS = 18;                              // 16-deep steps of Q staged in LDS
constexpr int KK_REG = D / 16 - KK_LDS;                 // 18 steps held in registers
constexpr int QROW_BYTES = KK_LDS * 32 + 16;            // 592: 288 columns + 16-byte pad
constexpr float kFlushLog2 = 32.f;                      // P may grow to 2^32 before a flush

__device__ __forceinline__ int row_swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

struct SparseCtx {
  int lane, wave, l32, hl;
  int len;                 // slots considered: [0, len)
  const int32_t* irow;     // this token's index row
  bool hok;                // this lane's head exists
  float scale;
  __bf16* orow;            // this lane's head row of the output
};

// Copy the latent rows of slots [32j, 32j+32) into `stage`; invalid slots copy row 0 (finite,
// in bounds) and are masked. Wave 0 also publishes the block's validity mask.
__device__ __forceinline__ void issue_gather(const SparseParams& p, const SparseCtx& c, int j,
                                             char* stage, uint32_t* mask_slot) {
#pragma unroll
  for (int i = 0; i < CHUNKS_PER_WAVE; ++i) {
    const int pch = (c.wave * CHUNKS_PER_WAVE + i) * 64 + c.lane;
    const int row = pch / CHUNKS;
    const int pc = pch - row * CHUNKS;
    const int lc = pc ^ row_swz(row);
    const int slot = j * BNS + row;
    int rid = (slot < c.len) ? c.irow[slot] : -1;
    rid = (rid >= 0 && (int64_t)rid < p.n_kv) ? rid : 0;
    g2lds16(p.kv + (int64_t)rid * p.kv_st + lc * 8, stage + (c.wave * CHUNKS_PER_WAVE + i) * 1024);
  }
  if (c.wave == 0) {
    const int slot = j * BNS + c.l32;
    const int rid = (slot < c.len) ? c.irow[slot] : -1;
    const bool ok = c.hl == 0 && rid >= 0 && (int64_t)rid < p.n_kv;
    const uint64_t b = __ballot(ok);
    if (c.lane == 0) *mask_slot = (uint32_t)b;
  }
}

__device__ __forceinline__ void compute_block(const SparseCtx& c, const char* stage,
                                              uint32_t valid, const char* qlds,
                                              const bf16x8 (&qf)[KK_REG], float& m_ref,
                                              float& l_run, f32x16 (&o)[DVS / 32],
                                              float scale_log2, float flush_raw, float& m_true,
                                              bool& overflow) {
  // ---- S^T = K~ * Q^T
  f32x16 s = f32x16{};
  {
    const int row = c.l32;
    const char* rb = stage + row * ROW_BYTES;
    const int sw = row_swz(row);
    const char* qb = qlds + (c.wave * 32 + c.l32) * QROW_BYTES + c.hl * 16;
#pragma unroll
    for (int kk = 0; kk < KK_LDS; ++kk) {
      bf16x8 a = lds_read_b128(rb + (((kk * 2 + c.hl) ^ sw) * 16));
      bf16x8 b = lds_read_b128(qb + kk * 32);
      s = mfma32(a, b, s);
    }
#pragma unroll
    for (int kk = KK_LDS; kk < D / 16; ++kk) {
      bf16x8 a = lds_read_b128(rb + (((kk * 2 + c.hl) ^ sw) * 16));
      s = mfma32(a, qf[kk - KK_LDS], s);
    }
  }
  // ---- invalid slots
  if (valid != 0xFFFFFFFFu) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 8 * (i >> 2) + 4 * c.hl + (i & 3);
      if (((valid >> key) & 1u) == 0u) s[i] = -INFINITY;
    }
  }
  // ---- online softmax against the reference max (fixed once the head holds any mass)
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
  mx = xhalf_max(mx);
  m_true = fmaxf(m_true, mx);
  if (m_ref == -INFINITY) m_ref = mx;  // first visible key of this head (same in both halves)
  overflow = overflow || (mx > m_ref + flush_raw);
  const float mc = ((m_ref == -INFINITY) ? 0.f : m_ref) * scale_log2;
  bf16x8 pf[2];
  float rs = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float pv = fast_exp2(fmaf(s[i], scale_log2, -mc));
    rs += pv;
    pf[i >> 3][i & 7] = (__bf16)pv;
  }
  l_run += rs;
  // ---- O^T += V~^T * P^T (V~ = first 512 columns of the same LDS rows, read transposed)
  const int g = c.lane >> 4;
  const int r = c.lane & 15;
  const int dv_lane = (g & 1) * 16 + 4 * (r & 3);
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int k0 = cc * 16 + 4 * c.hl + (r >> 2);
    const int k1 = k0 + 8;
    const char* r0 = stage + k0 * ROW_BYTES;
    const char* r1 = stage + k1 * ROW_BYTES;
    const int sw0 = row_swz(k0), sw1 = row_swz(k1);
#pragma unroll
    for (int dt = 0; dt < DVS / 32; ++dt) {
      const int dv = dt * 32 + dv_lane;
      const int ch = dv >> 3, sub = (dv & 7) * 2;
      bf16x8 a = join(lds_read_tr16(r0 + ((ch ^ sw0) * 16) + sub),
                      lds_read_tr16(r1 + ((ch ^ sw1) * 16) + sub));
      o[dt] = mfma32(a, pf[cc], o[dt]);
    }
  }
}

}  // namespace

__global__ __launch_bounds__(256, 1) void sparse_fwd_kernel(SparseParams p) {
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char qlds[MAX_HEADS * QROW_BYTES];
  __shared__ uint32_t valid_mask[2];
  __shared__ int redo_flag;

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  SparseCtx c;
  c.lane = tid & 63;
  c.wave = tid >> 6;
  c.l32 = c.lane & 31;
  c.hl = c.lane >> 5;
  c.len = p.topk;
  if (p.topk_length != nullptr) c.len = min(max(p.topk_length[t], 0), p.topk);
  if (p.n_kv <= 0) c.len = 0;  // an empty pool has no valid slot (and no row to read)
  c.irow = p.idx + (int64_t)t * p.idx_st;

  const int nblk = (c.len + BNS - 1) / BNS;
  if (nblk > 0) issue_gather(p, c, 0, stage0, &valid_mask[0]);

  // ---- Q columns [0, 288) of every head -> LDS (zero rows for heads >= H)
  const __bf16* qt = p.q + (int64_t)t * p.q_st;
  for (int e = tid; e < MAX_HEADS * (KK_LDS * 2); e += 256) {
    const int hrow = e / (KK_LDS * 2);
    const int ch = e - hrow * (KK_LDS * 2);
    bf16x8 v = bf16x8{};
    if (hrow < p.num_heads) v = *reinterpret_cast<const bf16x8*>(qt + (int64_t)hrow * p.q_sh + ch * 8);
    *reinterpret_cast<bf16x8*>(qlds + hrow * QROW_BYTES + ch * 16) = v;
  }
  // ---- Q columns [288, 576) of this lane's head -> registers
  const int head = c.wave * 32 + c.l32;
  c.hok = head < p.num_heads;
  c.scale = p.scale;
  c.orow = p.out + (int64_t)t * p.o_st + (int64_t)(c.hok ? head : 0) * p.o_sh;
  const bool wave_active = c.wave * 32 < p.num_heads;
  bf16x8 qf[KK_REG];
  {
    const __bf16* qp = qt + (int64_t)(c.hok ? head : 0) * p.q_sh + c.hl * 8;
#pragma unroll
    for (int kk = 0; kk < KK_REG; ++kk) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + (KK_LDS + kk) * 16);
      qf[kk] = c.hok ? v : bf16x8{};
    }
  }
  f32x16 o[DVS / 32];
  float m_ref = -INFINITY, l_run = 0.f, m_true = -INFINITY;
  const float flush_raw = kFlushLog2 / p.scale_log2;

  wait_vmem();
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int dt = 0; dt < DVS / 32; ++dt) o[dt] = f32x16{};
    l_run = 0.f;
    if (pass == 1) m_ref = m_true;  // exact max: P <= 1 everywhere
    bool overflow = false;
    for (int j = 0; j < nblk; j += 2) {
      if (j + 1 < nblk) issue_gather(p, c, j + 1, stage1, &valid_mask[1]);
      if (wave_active)
        compute_block(c, stage0, valid_mask[0], qlds, qf, m_ref, l_run, o, p.scale_log2, flush_raw,
                      m_true, overflow);
      wait_vmem();
      __syncthreads();
      if (j + 1 >= nblk) break;
      if (j + 2 < nblk) issue_gather(p, c, j + 2, stage0, &valid_mask[0]);
      if (wave_active)
        compute_block(c, stage1, valid_mask[1], qlds, qf, m_ref, l_run, o, p.scale_log2, flush_raw,
                      m_true, overflow);
      wait_vmem();
      __syncthreads();
    }
    if (pass == 1) break;
    if (tid == 0) redo_flag = 0;
    __syncthreads();
    if (__ballot(overflow) != 0ull && c.lane == 0) redo_flag = 1;
    __syncthreads();
    if (redo_flag == 0) break;
    if (nblk > 0) issue_gather(p, c, 0, stage0, &valid_mask[0]);
    wait_vmem();
    __syncthreads();
  }

  // ---- epilogue: normalise, fold in the sink logit, write O and LSE
  const float l_tot = xhalf_sum(l_run);
  const float sink_v = (p.sink != nullptr && c.hok) ? p.sink[head] : -INFINITY;
  float inv, lse_v;
  if (l_tot == 0.f) {
    inv = 0.f;
    lse_v = sink_v;
  } else {
    const float mm = m_ref * p.scale;
    if (sink_v == -INFINITY) {
      inv = 1.f / l_tot;
      lse_v = mm + __logf(l_tot);
    } else {
      const float mxs = fmaxf(mm, sink_v);
      const float a = __expf(mm - mxs);
      const float z = l_tot * a + __expf(sink_v - mxs);
      inv = a / z;
      lse_v = mxs + __logf(z);
    }
  }
  if (c.hok) {
    __bf16* op = c.orow;
#pragma unroll
    for (int dt = 0; dt < DVS / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dv = dt * 32 + 8 * g4 + 4 * c.hl;
        u32x2 v = {pack_bf16x2(o[dt][g4 * 4 + 0] * inv, o[dt][g4 * 4 + 1] * inv),
                   pack_bf16x2(o[dt][g4 * 4 + 2] * inv, o[dt][g4 * 4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + dv) = v;
      }
    if (p.lse != nullptr && c.hl == 0) p.lse[(int64_t)t * p.l_st + (int64_t)head * p.l_sh] = lse_v;
  }
}

hipError_t launch_sparse_fwd(const SparseParams& p, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(sparse_fwd_kernel, dim3(p.num_tokens), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
