// Sparse top-k MLA prefill forward for gfx950 over one shared latent KV (absorbed MLA):
//   O[t,h] = softmax_k(scale * q[t,h] . kv[idx[t,k]]) kv[idx[t,k], :512]  (+ optional sink)
//
// The formula with K~ = V~ the gathered rows, int32 indices with -1 as the padded slot, the
// optional topk_length prefix and the sinks are those of page "SparseFlashMla" (Description:
// formula; Parameters table; Constraints); the indices are physical rows of the latent cache
// as in page "mla_prefill_branch_sparse_fp8". The 576 columns are 512 latent then 64 rope; the
// value vector is the first 512 columns of the same row.
//
// Work decomposition: a token is computed by one work-group of 8 waves (two per SIMD); the
// work-groups are persistent, one per CU, each going through a range of tokens. All heads of a
// token read the same gathered rows, so the heads form the matrix-core N dimension: wave w owns
// heads [16w, 16w+16) and every latent row is gathered once per token.
//   * Q^T of the wave's 16 heads (576 deep) stays in registers (72 per lane); the 16x16 O^T tiles
//     (512 x 16 heads) take 128.
//   * The token's index slots are staged in LDS (2048 at a time), so gather addresses never wait
//     on a global load. Blocks of 32 slots are processed in slot order; their latent rows are
//     copied global -> LDS directly into a 4-deep ring, three blocks ahead of the compute, with a
//     32-bit validity mask per block (-1, out of range, or at/after topk_length).
//   * Per block: S^T (32 keys x 16 heads) = K~ (A, LDS) * Q^T (B, registers) with 16x16x32 bf16
//     MFMA (two 16-key tiles, 18 steps each); online softmax per head across the four lanes that
//     hold a head column; O^T (512 x 16) += V~^T (A, transposed LDS reads of the same rows) * P^T
//     (B, the S^T registers converted to bf16 in place).
//   * A head's reference logit is the largest logit of the first block in which it sees a key, so
//     the block maximum is only computed while some head of the wave has no reference yet, and
//     the accumulator is not rescaled in the steady state. A block whose running sum would pass
//     2^64 (a logit some 44 nats above the reference) is redone against its exact maximum, with
//     the accumulated O and l rescaled.
// LDS layout of a gathered block: rows padded to 73 chunks of 16 bytes (1168 B), so row r
// starts on 16-byte bank group 9r mod 16 of the 256-byte (64-bank) window. The LDS serves a
// 16-byte read in four cycles of 16 lanes, each cycle taking the 4-lane quads of one half-wave
// whose quad index has a given parity, and an 8-byte transposed read in two cycles of 32 lanes.
// Two free choices make both reads conflict-free without an XOR swizzle:
//   * key k of each 16-key group sits in row pi(k) = 4 (k & 3) + f((k >> 2) & 3), f = (2,0,1,3):
//     the 8 keys a transposed half-wave reads land on rows of one parity (their 32-byte segments
//     tile the window) and the keys of each 16-byte read cycle on complementary bank groups;
//   * the contraction order inside each 64-byte step is permuted per lane group: group g reads
//     chunk 8 (kk >> 1) + 2 (kk & 1) + sigma(g), sigma = (0,4,1,5), and Q^T uses the same order,
//     so the two lane groups of a half-wave sit 64 bytes apart.
// Every operand read is then a per-lane base plus an immediate offset.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int D = 576;
constexpr int DVS = 512;
constexpr int BNS = 32;
constexpr int CHUNKS = D / 8;                           // 72 data chunks of 16 bytes per row
constexpr int ROW_CHUNKS = CHUNKS + 1;                  // 73: one pad chunk per row
constexpr int ROW_BYTES = ROW_CHUNKS * 16;              // 1168
constexpr int COPIES = (BNS * ROW_CHUNKS + 63) / 64;    // 37 wave-wide 1 KiB copies per block
constexpr int STAGE_BYTES = COPIES * 1024;              // 37888 (whole copies; the tail is scratch)
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr int COPIES_PER_WAVE = (COPIES + NWAVES - 1) / NWAVES;  // 5 (extra slots repeat copy 36)
constexpr int KSTEPS = D / 32;                          // 18 MFMA steps of depth 32
constexpr int DTILES = DVS / 16;                        // 32 output tiles of 16 columns
constexpr int IDX_WIN = 2048;                           // index slots staged in LDS at a time
// A head's probabilities are taken against a reference logit (see compute_block); a block whose
// running sum would pass 2^64 is redone against its exact maximum (P stays far inside bf16 / fp32
// range, and O = sum P V inside fp32 range for any bf16 V).
constexpr float kOverflowSum = 18446744073709551616.f;  // 2^64

// LDS row of key k within a block, and its inverse.
__device__ __forceinline__ int key_row(int k) {
  return (k & ~15) | ((k & 3) << 2) | ((0x3102 >> (4 * ((k >> 2) & 3))) & 3);
}
__device__ __forceinline__ int row_key(int r) {
  return (r & ~15) | (((0x3021 >> (4 * (r & 3))) & 3) << 2) | ((r >> 2) & 3);
}
// Chunk (16 bytes = 8 columns) of the 576 that lane group g contracts in step kk, split into a
// per-lane part and a per-step part.
__device__ __forceinline__ int chunk_lane(int g) { return ((g & 1) << 2) | (g >> 1); }
__host__ __device__ constexpr int chunk_step(int kk) { return 8 * (kk >> 1) + 2 * (kk & 1); }

struct SparseCtx {
  int lane, wave, l16, g;  // g = lane / 16
  int len;                 // slots considered: [0, len)
  const int32_t* irow;     // this token's index row
  int win0;                // first slot of the staged index window
  int* idx;                // LDS index window
  const int32_t* bt_row;   // paged cache: block-table row of the token's sequence (else null)
  int used;                // paged cache: logical positions [0, used) may be valid
  int bs, nblocks;         // paged cache: block size, number of blocks
  // Gather map of this lane's copies (two per word, 16 bits each: row_key of the slot's row in
  // bits 0-4, its 16-byte chunk in bits 5-11): the same for every block, so computed once.
  uint32_t gmap[(COPIES_PER_WAVE + 1) / 2];
  // The latent pool as a buffer of its exact byte extent (pools under 4 GiB): a copy whose offset
  // lies past the end loads zeros.
  __amdgpu_buffer_rsrc_t kvrs;
};

// Bytes of the pool: rows of kv_st elements, the last row's 576 columns.
__host__ __device__ __forceinline__ int64_t pool_extent(const SparseParams& p) {
  return p.n_kv <= 0 ? 0 : (p.n_kv - 1) * p.kv_st * 2 + D * 2;
}

// The source of the copies of invalid slots in pools of 4 GiB or more.
__device__ const uint4 kZero16 = {0u, 0u, 0u, 0u};

// Row-key index and chunk of copy i of this lane (see SparseCtx::gmap).
__device__ __forceinline__ uint32_t gather_map_entry(int wave, int lane, int i) {
  const int q = min(wave + NWAVES * i, COPIES - 1);
  const int slot = q * 64 + lane;
  const int row = min(slot / ROW_CHUNKS, BNS - 1);
  const int ch = slot - (slot / ROW_CHUNKS) * ROW_CHUNKS;
  const int chunk = (slot / ROW_CHUNKS >= BNS || ch >= CHUNKS) ? 0 : ch;
  return (uint32_t)row_key(row) | ((uint32_t)chunk << 5);
}

// Stage index slots [win0, win0 + IDX_WIN) of this token in LDS (entries past `len` read as -1).
// All loads are issued before any is used (slots past the row's end read its slot 0, which
// exists since topk >= 1), so the staging costs one memory round trip, not one per load. With a
// paged cache the logical positions are turned into cache rows here (-1 when invalid), with one
// more round trip for the block-table entries, so the gather itself is the same in both modes.
__device__ __forceinline__ void stage_indices(const SparseCtx& c, int tid) {
  asm volatile("" : "+v"(tid));  // addresses are formed here, not hoisted into long-lived registers
  constexpr int PER = IDX_WIN / NTHREADS;
  static_assert(IDX_WIN % NTHREADS == 0, "whole rounds");
  int v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int slot = c.win0 + tid + i * NTHREADS;
    v[i] = c.irow[slot < c.len ? slot : 0];
  }
  if (c.bt_row != nullptr) {
    int e[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool ok = v[i] >= 0 && v[i] < c.used;
      e[i] = c.bt_row[ok ? v[i] / c.bs : 0];  // entry 0 exists (max_blocks >= 1)
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int pos = v[i];
      const bool ok = pos >= 0 && pos < c.used && e[i] >= 0 && e[i] < c.nblocks;
      const int blk = ok ? pos / c.bs : 0;
      v[i] = ok ? e[i] * c.bs + (pos - blk * c.bs) : -1;
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int slot = c.win0 + tid + i * NTHREADS;
    c.idx[tid + i * NTHREADS] = slot < c.len ? v[i] : -1;
  }
}

// Copy the latent rows of slots [32j, 32j+32) into `stage`; invalid slots copy row 0 (finite,
// in bounds) and are masked. Every wave issues exactly COPIES_PER_WAVE copies (slots past the
// last copy repeat it; identical bytes), so the vector-memory counter advances uniformly per
// block. Pad chunks and the stage tail receive harmless copies of chunk 0 of a valid row.
// Wave 0 also publishes the block's validity mask (bit k = key k).
// Slots that are padded (-1) or name no row of the pool get zeros, never another row's bytes: their
// logits are masked, and a zero value keeps a non-finite number elsewhere in the pool from
// reaching the output through 0 * x. BUF: the pool spans less than 4 GiB (less two rows), so a
// copy is a buffer load at the 32-bit byte offset row * stride + chunk, and an invalid row is
// replaced by n_kv, which lies past the buffer's end (loads there return zeros). Otherwise each
// lane forms its 64-bit address and invalid slots read a zero constant.
template <bool BUF>
__device__ __forceinline__ void issue_gather(const SparseParams& p, const SparseCtx& c, int j,
                                             char* stage, uint32_t* mask_slot) {
  const int base = j * BNS - c.win0;
  // All index reads first, then all copies: the copies write LDS, so the compiler would otherwise
  // keep each index read behind the previous copy and wait for it on its own (one LDS round trip
  // per copy instead of one per block).
  int rid[COPIES_PER_WAVE], chunk[COPIES_PER_WAVE];
#pragma unroll
  for (int i = 0; i < COPIES_PER_WAVE; ++i) {
    const uint32_t e = c.gmap[i >> 1] >> (16 * (i & 1));
    chunk[i] = (int)((e >> 5) & 127u);
    rid[i] = c.idx[base + (int)(e & 31u)];
  }
#pragma unroll
  for (int i = 0; i < COPIES_PER_WAVE; ++i) {
    const int q = min(c.wave + NWAVES * i, COPIES - 1);
    if (BUF) {
      // an invalid row becomes n_kv, whose bytes start at or past the buffer's end
      const uint32_t r = min((uint32_t)rid[i], (uint32_t)p.n_kv);
      const uint32_t off = r * (uint32_t)(p.kv_st * 2) + (uint32_t)chunk[i] * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.kvrs, LDS_PTR(void, stage + q * 1024), 16, off, 0, 0, 0);
    } else {
      // one 32 x 32 -> 64-bit product per copy (row strides are below 2^31 elements)
      const bool ok = (uint32_t)rid[i] < (uint32_t)p.n_kv;
      const uint64_t off = (uint64_t)(uint32_t)rid[i] * (uint32_t)(p.kv_st * 2) + (uint32_t)chunk[i] * 16u;
      g2lds16(ok ? reinterpret_cast<const char*>(p.kv) + off : reinterpret_cast<const char*>(&kZero16), stage + q * 1024);
    }
  }
  if (c.wave == 0) {
    int ln = c.lane;
    asm volatile("" : "+v"(ln));  // the address is formed here, not kept in a register across the loop
    const int rid = c.idx[base + (ln & 31)];
    const bool ok = c.lane < 32 && rid >= 0 && (int64_t)rid < p.n_kv;
    const uint64_t b = __ballot(ok);
    if (c.lane == 0) *mask_slot = (uint32_t)b;
  }
}

// Wait until this wave's copies of the next block have landed, leaving `newer` later blocks'
// copies in flight.
__device__ __forceinline__ void wait_gather(int newer) {
  if (newer >= 2) {
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  } else if (newer == 1) {
    asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

__device__ __forceinline__ void compute_block(const SparseCtx& c, const char* stage, uint32_t valid,
                                              const bf16x8 (&qf)[KSTEPS], float& m_ref,
                                              float& l_run, f32x4 (&o)[DTILES], float scale_log2) {
  // ---- S^T = K~ * Q^T: two 16-key tiles (independent chains), K~ fragments read from LDS a
  // few steps ahead of their MFMA.
  constexpr int NST = 2 * KSTEPS;  // (kk, mt)
  constexpr int PF = 3;
  // lane reads key 16*mt + l16 (row key_row of it), chunk chunk_step(kk) + chunk_lane(g)
  const char* rb = stage + key_row(c.l16) * ROW_BYTES + chunk_lane(c.g) * 16;
  f32x4 s[2] = {f32x4{}, f32x4{}};
  bf16x8 ka[NST];
  auto rd = [&](int st) {
    const int kk = st >> 1, mt = st & 1;
    ka[st] = lds_read_b128(rb + mt * 16 * ROW_BYTES + chunk_step(kk) * 16);
  };
#pragma unroll
  for (int st = 0; st < PF; ++st) rd(st);
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    if (st + PF < NST) rd(st + PF);
    s[st & 1] = mfma16(ka[st], qf[st >> 1], s[st & 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- invalid slots: this lane holds keys 16*mt + 4*g + i
  if (valid != 0xFFFFFFFFu) {
    // the lane's bits, shifted once per block; the tests below then take constant bit positions
    // (per-lane bit masks hoisted out of the loop would cost registers the loop does not have, and
    // a reload from scratch here would wait for every gather in flight)
    uint32_t vl = valid >> (4 * c.g);
    asm volatile("" : "+v"(vl));
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (((vl >> (16 * mt + i)) & 1u) == 0u) s[mt][i] = -INFINITY;
  }
  // ---- online softmax against the head's reference logit (per head = per 4-lane column)
  auto block_max = [&]() {
    const float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                           fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    return xquad_max(mx);  // the same in the 4 lanes of a head
  };
  u32x4 packed;
  auto exps = [&](float ref) {
    const float mc = ((ref == -INFINITY) ? 0.f : ref) * scale_log2;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = fast_exp2(fmaf(s[e >> 1][2 * (e & 1)], scale_log2, -mc));
      const float p1 = fast_exp2(fmaf(s[e >> 1][2 * (e & 1) + 1], scale_log2, -mc));
      packed[e] = pack_bf16x2(p0, p1);
      rs += p0 + p1;
    }
    return rs;
  };
  if (__ballot(m_ref == -INFINITY) != 0ull) {  // some head of the wave has no reference yet
    const float mx = block_max();
    if (m_ref == -INFINITY) m_ref = mx;
  }
  float rs = exps(m_ref);
  if (__ballot(!(l_run + rs <= kOverflowSum)) != 0ull) {  // rare: redo against the exact maximum
    const float m_new = fmaxf(m_ref, block_max());
    const float alpha = (m_new == m_ref) ? 1.f : fast_exp2((m_ref - m_new) * scale_log2);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) o[dt] *= alpha;
    m_ref = m_new;
    rs = exps(m_ref);
  }
  l_run += rs;
  // P^T operand: k-slot 8*g + j holds key 4g + j (j < 4) or 16 + 4g + (j - 4) (j >= 4).
  const bf16x8 pf = __builtin_bit_cast(bf16x8, packed);
  // ---- O^T += V~^T * P^T: V~ = first 512 columns of the same rows, read transposed with the
  // same key order; 32 independent 16-column tiles, reads a few tiles ahead.
  {
    // group lane r supplies row key 4g + r/4 (and +16), columns 16*dt + 4*(r & 3)
    const int k0 = 4 * c.g + (c.l16 >> 2);
    const char* r0 = stage + key_row(k0) * ROW_BYTES + 8 * (c.l16 & 3);
    const char* r1 = r0 + 16 * ROW_BYTES;  // key k0 + 16 sits 16 rows further
    constexpr int PFV = 4;  // (5 spills)
    bf16x8 va[DTILES];
    auto vr = [&](int dt) { va[dt] = join(lds_read_tr16(r0 + dt * 32), lds_read_tr16(r1 + dt * 32)); };
#pragma unroll
    for (int dt = 0; dt < PFV; ++dt) vr(dt);
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      if (dt + PFV < DTILES) vr(dt + PFV);
      o[dt] = mfma16(va[dt], pf, o[dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace

template <bool BUF>
__global__ __launch_bounds__(NTHREADS, 1) void sparse_fwd_kernel(SparseParams p) {
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char stage2[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char stage3[STAGE_BYTES];
  __shared__ int idx_lds[IDX_WIN];
  __shared__ uint32_t valid_mask[4];

  const int tid = threadIdx.x;
  SparseCtx c;
  c.lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.l16 = c.lane & 15;
  c.g = c.lane >> 4;
  c.idx = idx_lds;
  c.bs = p.block_size;
  c.nblocks = p.num_blocks;
#pragma unroll
  for (int i = 0; i < (COPIES_PER_WAVE + 1) / 2; ++i) {
    c.gmap[i] = gather_map_entry(c.wave, c.lane, 2 * i);
    if (2 * i + 1 < COPIES_PER_WAVE) c.gmap[i] |= gather_map_entry(c.wave, c.lane, 2 * i + 1) << 16;
  }
  // word 3: the buffer format the gfx9 family expects for untyped loads
  c.kvrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(p.kv), (short)0, (int)(uint32_t)pool_extent(p),
                                             0x00020000);

  // Persistent: one work-group per CU goes through tokens one after the other (no work-group
  // launch and teardown per token). The tokens are split into 8 contiguous ranges, one per XCD
  // (work-group i runs on XCD i % 8), dealt round-robin to that XCD's work-groups, so tokens close
  // in the sequence (which share many gathered rows in practice) run on the same L2.
  const int xcd = blockIdx.x & 7;
  const int per_xcd = (p.num_tokens + 7) / 8;
  const int t_end = min(p.num_tokens, (xcd + 1) * per_xcd);
  const int wg_x = ((int)gridDim.x - xcd + 7) / 8;  // work-groups on this XCD
  for (int t = xcd * per_xcd + (int)(blockIdx.x >> 3); t < t_end; t += wg_x) {
  c.len = p.topk;
  if (p.topk_length != nullptr) c.len = min(max(p.topk_length[t], 0), p.topk);
  if (p.n_kv <= 0) c.len = 0;  // an empty pool has no valid slot (and no row to read)
  c.irow = p.idx + (int64_t)t * p.idx_st;
  c.win0 = 0;
  c.bt_row = nullptr;
  c.used = 0;
  if (p.block_table != nullptr) {
    // sequence of token t: the last b with cu_q[b] <= t (empty sequences are skipped over)
    int lo = 0, hi = p.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cu_q[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const bool in_use = p.seqused_q == nullptr || t - p.cu_q[lo] < p.seqused_q[lo];
    if (p.cu_q[lo] <= t && t < p.cu_q[lo + 1] && in_use) {
      c.bt_row = p.block_table + (int64_t)lo * p.bt_st;
      int64_t used = (int64_t)p.max_blocks * p.block_size;
      if (p.seqused != nullptr) used = min(used, (int64_t)max(p.seqused[lo], 0));
      c.used = (int)used;
    } else {
      c.len = 0;  // a token outside every sequence, or not in use, has no valid slot
    }
  }
  const int nblk = (c.len + BNS - 1) / BNS;

  // ---- Q^T of this lane's head: the 8 columns of the chunk its lane group contracts per step.
  // The lane's head and chunk are formed again from the thread index for each token (a per-lane
  // address kept from one token to the next would be spilled: the block loop needs every register).
  const bool wave_active = c.wave * 16 < p.num_heads;
  bf16x8 qf[KSTEPS];
  {
    int tid_q = (int)threadIdx.x;
    asm volatile("" : "+v"(tid_q));
    const int head = c.wave * 16 + (tid_q & 15);
    const bool hok = head < p.num_heads;
    const __bf16* qp = p.q + (int64_t)t * p.q_st + (int64_t)(hok ? head : 0) * p.q_sh +
                       chunk_lane((tid_q >> 4) & 3) * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + chunk_step(kk) * 8);
      qf[kk] = hok ? v : bf16x8{};
    }
  }

  f32x4 o[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) o[dt] = f32x4{};
  float m_ref = -INFINITY, l_run = 0.f;
  char* stages[4] = {stage0, stage1, stage2, stage3};

  {
    // prologue: index window 0, then the first three blocks in flight
    c.win0 = 0;
    stage_indices(c, tid);
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 3; ++b)
      if (b < nblk) issue_gather<BUF>(p, c, b, stages[b], &valid_mask[b]);
    wait_gather(min(nblk, 3) - 1);
    lds_barrier();

    // Steady state, unrolled by four so that each ring slot is a distinct LDS object.
#define MLA_SPARSE_STEP(K, CUR, NEXT)                                                            \
    {                                                                                             \
      const int jj = j + (K);                                                                     \
      if (jj >= nblk) break;                                                                      \
      if (jj + 3 < nblk) {                                                                        \
        if ((jj + 3) * BNS - c.win0 >= IDX_WIN) {                                                 \
          /* every copy from the old window has been issued and its indices consumed */          \
          c.win0 += IDX_WIN;                                                                      \
          stage_indices(c, tid);                                                                  \
          __syncthreads();                                                                        \
        }                                                                                         \
        issue_gather<BUF>(p, c, jj + 3, NEXT, &valid_mask[((K) + 3) & 3]);                     \
      }                                                                                           \
      if (wave_active)                                                                            \
        compute_block(c, CUR, valid_mask[(K)], qf, m_ref, l_run, o, p.scale_log2);                \
      wait_gather(min(nblk - 1, jj + 3) - (jj + 1));                                              \
      lds_barrier(); /* the later blocks' copies stay in flight */                                \
    }
    for (int j = 0; j < nblk; j += 4) {
      MLA_SPARSE_STEP(0, stage0, stage3)
      MLA_SPARSE_STEP(1, stage1, stage0)
      MLA_SPARSE_STEP(2, stage2, stage1)
      MLA_SPARSE_STEP(3, stage3, stage2)
    }
#undef MLA_SPARSE_STEP
  }

  // ---- epilogue: normalise, fold in the sink logit, write O and LSE. The head index is formed
  // again here rather than kept in a register through the block loop.
  int tid_e = (int)threadIdx.x;
  asm volatile("" : "+v"(tid_e));
  const int head_e = c.wave * 16 + (tid_e & 15);
  const bool hok_e = head_e < p.num_heads;
  const float l_tot = xquad_sum(l_run);
  const float sink_v = (p.sink != nullptr && hok_e) ? p.sink[head_e] : -INFINITY;
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
  if (hok_e && p.lse != nullptr && (tid_e & 48) == 0) p.lse[(int64_t)t * p.l_st + (int64_t)head_e * p.l_sh] = lse_v;
  // O through LDS: the ring is free (every wave passed the barrier after its last block). Wave w
  // turns its 16 heads x 512 columns (16 KiB) around in half of ring slot w / 2 (row = head,
  // 16-byte chunk c of a row at c ^ head, so the 16 heads of a write land on 16 bank groups),
  // then stores whole 1 KiB head rows, 16 bytes per lane. (Each lane holds 4 columns per output
  // tile, so direct stores would cover 16 rows x 32 bytes per instruction.)
  {
    const int w2 = c.wave >> 1;
    char* tb = (w2 == 0 ? stage0 : w2 == 1 ? stage1 : w2 == 2 ? stage2 : stage3) + (c.wave & 1) * 16384;
    // lane-derived values formed again from the thread index (not kept through the block loop)
    const int l16 = tid_e & 15, g = (tid_e >> 4) & 3, lane = tid_e & 63;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      const u32x2 v = {pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv), pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
      *reinterpret_cast<u32x2*>(tb + l16 * 1024 + (((2 * dt + (g >> 1)) ^ l16) << 4) + (g & 1) * 8) = v;
    }
    __bf16* orow = p.out + (int64_t)t * p.o_st + (int64_t)(c.wave * 16) * p.o_sh + lane * 8;
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(tb + r * 1024 + ((lane ^ r) << 4));
      if (c.wave * 16 + r < p.num_heads) *reinterpret_cast<u32x4*>(orow + (int64_t)r * p.o_sh) = x;
    }
  }
  }
}

hipError_t launch_sparse_fwd(const SparseParams& p, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  // one work-group per CU (their LDS allows no more), no more than tokens
  const int grid = std::max(1, std::min(p.num_tokens, p.max_wgs > 0 ? p.max_wgs : 256));
  // byte offsets of an invalid row must still land past a buffer of the pool's extent
  if (pool_extent(p) <= (int64_t)UINT32_MAX - 2 * p.kv_st * 2)
    hipLaunchKernelGGL(sparse_fwd_kernel<true>, dim3(grid), dim3(NTHREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(sparse_fwd_kernel<false>, dim3(grid), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
