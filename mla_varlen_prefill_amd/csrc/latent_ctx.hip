// Context from the latent cache, chunk by chunk: the kernels that turn a window of cached latent
// rows into per-head K/V in a bounded buffer. (A chunk's partial result is merged into the running
// one by the attention kernel's epilogue.)
//
// The pages run the new tokens causally against themselves and every context chunk without a
// mask, always returning the LSE, and merge the parts (page "FlashAttention backend for MLA
// prefill", run_prefill_new_tokens and run_prefill_context_chunk). The cached rows are the
// 512-wide latent followed by 64 rope columns, turned into per-head keys and values by the W_UK /
// W_UV up-projections (page "mla_prefill_branch_sparse_fp8", w_uk / w_uv). Reading: head h's key
// is [c W_UK_h^T (128) || rope (64)] and its value c W_UV_h^T (128), with W_KV laid out like a
// linear layer's weight, [H * 256, 512]: rows h*256 + 0..127 are W_UK_h, h*256 + 128..255 W_UV_h.
//
// Up-projection: a bf16 GEMM, out = W_KV * C_latent^T on 32x32x16 MFMA, with both operands
// contiguous along the 512-deep contraction. A work-group (4 waves, one per SIMD) owns 128 cached
// rows of one sequence and goes through a group of heads one after the other. Each wave keeps its
// 32 latent rows resident in registers as the MFMA B operand (128 per lane, loaded once for all
// the group's heads) and accumulates a head's 32 rows x 256 columns (its 128 key and 128 value
// columns) in 128 accumulation registers. The heads' W_KV rows stream through a 4-deep LDS ring,
// 64 of the 512 contraction columns per stage (32 KiB), copied straight from global memory
// (global_load_lds) three stages ahead, across head boundaries. Two accumulator sets alternate:
// while a head's products run, the previous head's result leaves in direct 8-byte stores placed
// between them (and the head's rope columns, held in registers for the whole group), so no
// epilogue stands between the products of consecutive heads. A 128-byte operand row keeps its
// 16-byte chunk c at c ^ ((r >> 1) & 7), which makes the operand reads conflict-free under
// gfx950's 16-byte read grouping. Work-groups are dealt to the XCDs by head group, so the ones
// running together on an XCD stream the same W_KV rows through its L2; the groups are small
// enough that every chunk gives the chip about four work-groups per CU.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int UP_ROWS = 128;               // cached rows per work-group (32 per wave)
constexpr int KV_COLS = 256;               // per head: 128 key + 128 value columns
constexpr int UP_KS = 64;                  // contraction columns per stage
constexpr int UP_STAGE = KV_COLS * UP_KS * 2;  // 32 KiB of W_KV per stage
constexpr int UP_NBUF = 4;                 // ring slots: copies run three stages ahead
constexpr int UP_THREADS = 256;
constexpr int LAT_D = 512;
constexpr int UP_NSTAGE = LAT_D / UP_KS;   // 8 stages per head
constexpr int UP_COPIES = UP_STAGE / 1024 / (UP_THREADS / 64);  // 8 wave copies per wave per stage
constexpr int UP_CT = KV_COLS / 32;        // 32-column output tiles per head (4 key, 4 value)
constexpr int UP_WG_PER_CU = 4;            // work-groups per CU the head groups aim at

// Direct global -> LDS copy of 16 bytes per lane (lane l's bytes land at lds_base + 16 l) from
// the scalar base plus the lane's 32-bit byte offset, issued from asm so that the compiler's
// wait-count bookkeeping does not track it: the copies are waited for explicitly (vmcnt) before the
// barrier that precedes their use. The instruction writes no vector register; M0 is set in the
// same statement (the compiler emits no other use of M0 in this file's kernels).
__device__ __forceinline__ void g2lds16_untracked(const void* sbase, uint32_t voff, const void* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0v)
               : "memory", "m0");
}

// An accumulator value read where it is used: the operand is pinned to an accumulation register,
// so the compiler keeps the product results there instead of copying them to vector registers at
// the top of the loop that stores them.
__device__ __forceinline__ float acc_read(float x) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}

// Wait until at most N of this wave's vector memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace

// cu_chunk[b] = sum over b' < b of clamp(ctx_{b'} - c0, 0, W): the buffer rows of each sequence's
// slice [c0, c0 + W) of its context. One work-group; each thread owns a run of sequences.
__global__ __launch_bounds__(1024) void chunk_cu_kernel(const int32_t* cu_ctx, int32_t batch, int32_t c0,
                                                        int32_t w, int32_t* cu_chunk) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (batch + 1023) / 1024;
  const int b0 = tid * per, b1 = min(batch, b0 + per);
  int sum = 0;
  for (int b = b0; b < b1; ++b) sum += min(max(cu_ctx[b + 1] - cu_ctx[b] - c0, 0), w);
  part[tid] = sum;
  __syncthreads();
  // inclusive scan of the per-thread sums (Hillis-Steele)
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tid == 0 ? 0 : part[tid - 1];
  if (tid == 0) cu_chunk[0] = 0;
  for (int b = b0; b < b1; ++b) {
    run += min(max(cu_ctx[b + 1] - cu_ctx[b] - c0, 0), w);
    cu_chunk[b + 1] = run;
  }
}

// Grid: 8 * ceil(groups / 8) * row_tiles work-groups, row_tiles = batch * ceil(w / 128). Work-group
// i runs on XCD i % 8; it takes head group (i % 8) + 8 * (j / row_tiles) (heads [g * hpg, (g + 1) *
// hpg)) and row tile j % row_tiles with j = i / 8, so the XCDs split the head groups and each goes
// through all row tiles of one group before the next.
__global__ __launch_bounds__(UP_THREADS, 1) void upproj_kernel(UpprojParams p, int32_t row_tiles,
                                                                int32_t tiles_per_seq, int32_t hpg) {
  __shared__ __attribute__((aligned(1024))) char ring[UP_NBUF * UP_STAGE];
  __shared__ __attribute__((aligned(16))) u32x2 rope_lds[UP_NSTAGE * UP_THREADS];
  __shared__ __attribute__((aligned(1024))) char obuf[UP_THREADS / 64 * 4096];   // 4 KiB per wave
  const int xcd = blockIdx.x & 7;
  const int j = blockIdx.x >> 3;
  const int grp = xcd + 8 * (j / row_tiles);
  const int rt = j - (j / row_tiles) * row_tiles;
  const int b = rt / tiles_per_seq;
  const int tile = rt - b * tiles_per_seq;
  const int h_begin = grp * hpg;
  const int h_end = min(p.num_heads, h_begin + hpg);
  if (h_begin >= h_end) return;
  const int ctx_b = p.cu_ctx[b + 1] - p.cu_ctx[b];
  const int len = min(max(ctx_b - p.c0, 0), p.w);   // this sequence's rows in the chunk
  const int r0 = tile * UP_ROWS;
  if (r0 >= len) return;
  const int rows = min(UP_ROWS, len - r0);
  const int64_t lat_row0 = (int64_t)p.cu_ctx[b] + p.c0 + r0;    // first cached row of the tile
  const int64_t buf_row0 = (int64_t)p.cu_chunk[b] + r0;          // first buffer row of the tile
  const int total = (h_end - h_begin) * UP_NSTAGE;               // stages of the whole group

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;

  // Stage copies: wave copy q = UP_COPIES * wave + i covers operand rows 8 q .. 8 q + 7 (a head's
  // output columns; operand row r of head h is W_KV row h * 256 + r). Lane l fills row
  // 8 q + l / 8, slot l % 8, with the chunk stored there: (l % 8) ^ ((row >> 1) & 7), which is
  // c0 for even i and c0 ^ 4 for odd i. Byte offsets from the head's first W_KV row, copy i adding
  // the scalar 8 i rows.
  const uint32_t w_st_b = (uint32_t)(p.w_st * 2);
  const uint32_t c0 = (uint32_t)((lane & 7) ^ (lane >> 4));
  const uint32_t vrow = (uint32_t)(64 * wave + (lane >> 3)) * w_st_b;
  const uint32_t voff[2] = {vrow + c0 * 16u, vrow + (c0 ^ 4u) * 16u};
  auto issue = [&](int gs) {
    const int h = h_begin + gs / UP_NSTAGE, s = gs - (gs / UP_NSTAGE) * UP_NSTAGE;
    const char* src = reinterpret_cast<const char*>(p.w_kv + (int64_t)h * KV_COLS * p.w_st + s * UP_KS);
    char* dst = ring + (gs % UP_NBUF) * UP_STAGE;
#pragma unroll
    for (int i = 0; i < UP_COPIES; ++i)
      g2lds16_untracked(src + (size_t)(8 * i) * w_st_b, voff[i & 1], dst + (wave * UP_COPIES + i) * 1024);
  };
  issue(0);
  if (total > 1) issue(1);
  if (total > 2) issue(2);

  // B operand: this wave's 32 cached rows (tail rows re-read the last one), all 512 columns:
  // cb[kk] = columns 16 kk + 8 hl .. +7 of row 32 wave + l32.
  bf16x8 cb[LAT_D / 16];
  {
    const __bf16* src = p.latent + (lat_row0 + min(wave * 32 + l32, rows - 1)) * p.lat_st + hl * 8;
#pragma unroll
    for (int kk = 0; kk < LAT_D / 16; ++kk) cb[kk] = *reinterpret_cast<const bf16x8*>(src + kk * 16);
  }
  // Rope columns 512..575 of the tile's rows, the same for every head, kept in LDS: thread t's
  // entry s holds 8 bytes of row 16 s + t / 16 (bytes 8 (t % 16) ..), written to each head's key
  // columns 128..191 during stage s of that head.
  const int rope_part = tid & 15;
#pragma unroll
  for (int s = 0; s < UP_NSTAGE; ++s) {
    const int r = 16 * s + (tid >> 4);
    rope_lds[s * UP_THREADS + tid] = *reinterpret_cast<const u32x2*>(
        p.latent + (lat_row0 + min(r, rows - 1)) * p.lat_st + LAT_D + rope_part * 4);
  }
  // The compiler waits for these loads where they are first used; make that here, once, rather
  // than in the stage loop, where its count (which does not know of the copies) would also hold
  // back copies issued since.
#pragma unroll
  for (int kk = 0; kk < LAT_D / 16; ++kk) asm volatile("" ::"v"(cb[kk]));
  // Outputs through buffer descriptors that end after the tile's last valid row: the stores of the
  // rows past it (a sequence's last tile) are dropped by the range check, with no branch between
  // the products.
  __amdgpu_buffer_rsrc_t kd = __builtin_amdgcn_make_buffer_rsrc(
      p.kbuf + buf_row0 * p.k_st, (short)0, (int)((int64_t)rows * p.k_st * 2), 0x00020000);
  __amdgpu_buffer_rsrc_t vd = __builtin_amdgcn_make_buffer_rsrc(
      p.vbuf + buf_row0 * p.v_st, (short)0, (int)((int64_t)rows * p.v_st * 2), 0x00020000);
  // the lane's 16 bytes of a turned-around output piece: row 32 wave + 8 i + lane / 8, bytes
  // 16 (lane % 8) of the piece's 128 (i = 0..3 in the scalar offset)
  const uint32_t kpiece = (uint32_t)((wave * 32 + (lane >> 3)) * p.k_st * 2) + (uint32_t)((lane & 7) * 16);
  const uint32_t vpiece = (uint32_t)((wave * 32 + (lane >> 3)) * p.v_st * 2) + (uint32_t)((lane & 7) * 16);
  const uint32_t rope_off = (uint32_t)((tid >> 4) * p.k_st * 2) + (uint32_t)(256 + rope_part * 8);
  // A operand: operand row 32 ct + l32, chunk 2 kk + hl, stored at chunk ^ ((l32 >> 1) & 7)
  int a_off[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) a_off[kk] = l32 * (UP_KS * 2) + (((2 * kk + hl) ^ ((l32 >> 1) & 7)) << 4);

  // Output piece q (0..3) of a head: output tiles 2q and 2q + 1, i.e. columns 64 q .. 64 q + 63 of
  // its 256 (key columns for q < 2, value columns after). Turned around in the wave's 4 KiB of
  // LDS (32 rows x 128 bytes, 16-byte chunk c of row r at c ^ (r & 7)) so that it leaves in
  // 16-byte stores of whole 128-byte row segments.
  char* ob = obuf + wave * 4096;
  auto piece_write = [&](const f32x16 (&v)[UP_CT], int q) {
#pragma unroll
    for (int ctl = 0; ctl < 2; ++ctl)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& x = v[2 * q + ctl];
        const u32x2 o = {pack_bf16x2(acc_read(x[4 * g]), acc_read(x[4 * g + 1])),
                         pack_bf16x2(acc_read(x[4 * g + 2]), acc_read(x[4 * g + 3]))};
        *reinterpret_cast<u32x2*>(ob + l32 * 128 + (((ctl * 4 + g) ^ (l32 & 7)) << 4) + hl * 8) = o;
      }
  };
  u32x4 pv[4];
  auto piece_read = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + (lane >> 3);
      pv[i] = *reinterpret_cast<const u32x4*>(ob + r * 128 + (((lane & 7) ^ (r & 7)) << 4));
    }
  };
  auto piece_store = [&](int h, int q, int i) {
    if (q < 2)
      __builtin_amdgcn_raw_buffer_store_b128(pv[i], kd, kpiece, (int)(8 * i * p.k_st * 2 + h * p.k_sh * 2 + q * 128), 0);
    else
      __builtin_amdgcn_raw_buffer_store_b128(pv[i], vd, vpiece, (int)(8 * i * p.v_st * 2 + h * p.v_sh * 2 + (q - 2) * 128), 0);
  };

  f32x16 acc0[UP_CT], acc1[UP_CT];
  // One head: its 8 stages of 32 products into `cur`, with the previous head's `prev` stored
  // piecewise (piece s / 2 turned around during stage s, even s, and stored during stage s + 1)
  // and this head's rope columns.
  auto head = [&](auto has_prev, f32x16 (&cur)[UP_CT], const f32x16 (&prev)[UP_CT], int h) {
    constexpr bool HAS_PREV = decltype(has_prev)::value;
    const int gs0 = (h - h_begin) * UP_NSTAGE;
#pragma unroll
    for (int s = 0; s < UP_NSTAGE; ++s) {
      const int gs = gs0 + s;
      // this wave's copies of stage gs have landed: every later vector-memory operation is one of
      // the 2 * UP_COPIES copies of the next two stages or a store, and they retire in order
      // (near the end, where fewer copies follow, all of them); then every wave's have, and the
      // barrier also retires stage gs - 1 for all waves, so its slot may be refilled with gs + 3
      if (gs + 2 < total) wait_vm<2 * UP_COPIES>();
      else wait_vm<0>();
      lds_barrier();
      if (gs + 3 < total) issue(gs + 3);
      const char* st = ring + (gs % UP_NBUF) * UP_STAGE;
      constexpr int NT = 4 * UP_CT;   // products: t = kk * 8 + ct
      constexpr int PF = 4;
      bf16x8 a[NT];
      auto rd = [&](int t) { a[t] = lds_read_b128(st + a_off[t / UP_CT] + (t % UP_CT) * 32 * (UP_KS * 2)); };
#pragma unroll
      for (int t = 0; t < PF; ++t) rd(t);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t + PF < NT) rd(t + PF);
        const int kk = t / UP_CT, ct = t % UP_CT;
        cur[ct] = mfma32(a[t], cb[4 * s + kk], (s == 0 && kk == 0) ? f32x16{} : cur[ct]);
        if (t == 0)
          __builtin_amdgcn_raw_buffer_store_b64(rope_lds[s * UP_THREADS + tid], kd, rope_off,
                                                (int)((16 * s) * p.k_st * 2 + h * p.k_sh * 2), 0);
        if (HAS_PREV && (s & 1) == 0 && t == 4) piece_write(prev, s >> 1);
        if (HAS_PREV && (s & 1) == 0 && t == 20) piece_read();
        if (HAS_PREV && (s & 1) == 1 && (t & 7) == 4) piece_store(h - 1, s >> 1, t >> 3);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads PF steps ahead of their products
      }
    }
  };
  head(std::false_type{}, acc0, acc1, h_begin);
  int h = h_begin + 1;
  for (; h + 1 < h_end; h += 2) {
    head(std::true_type{}, acc1, acc0, h);
    head(std::true_type{}, acc0, acc1, h + 1);
  }
  if (h < h_end) head(std::true_type{}, acc1, acc0, h);
  // the last head's result
  auto store_all = [&](const f32x16 (&v)[UP_CT], int hh) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      piece_write(v, q);
      piece_read();
#pragma unroll
      for (int i = 0; i < 4; ++i) piece_store(hh, q, i);
    }
  };
  if (((h_end - 1 - h_begin) & 1) == 0) store_all(acc0, h_end - 1);
  else store_all(acc1, h_end - 1);
}

hipError_t launch_chunk_cu(const int32_t* cu_ctx, int32_t batch, int32_t c0, int32_t w, int32_t* cu_chunk,
                           hipStream_t stream) {
  hipLaunchKernelGGL(chunk_cu_kernel, dim3(1), dim3(1024), 0, stream, cu_ctx, batch, c0, w, cu_chunk);
  return hipGetLastError();
}

hipError_t launch_upproj(const UpprojParams& p, hipStream_t stream) {
  const int tiles_per_seq = (p.w + UP_ROWS - 1) / UP_ROWS;
  if (tiles_per_seq == 0 || p.batch == 0 || p.num_heads == 0) return hipSuccess;
  // a head's W_KV rows are addressed with 32-bit byte offsets
  if ((int64_t)(KV_COLS - 1) * p.w_st * 2 + LAT_D * 2 > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
  const int64_t row_tiles = (int64_t)p.batch * tiles_per_seq;
  // Head groups: multiples of 8 (one per XCD), as many as bring the grid to about UP_WG_PER_CU
  // work-groups per CU; the fewer, the more heads share one load of the latent rows.
  const int64_t want = (int64_t)256 * UP_WG_PER_CU;
  int64_t k = (want + 8 * row_tiles / 2) / (8 * row_tiles);
  k = std::max<int64_t>(1, std::min<int64_t>(k, (p.num_heads + 7) / 8));
  const int hpg = (int)((p.num_heads + 8 * k - 1) / (8 * k));
  const int64_t groups = (p.num_heads + hpg - 1) / hpg;
  const int64_t grid = 8 * ((groups + 7) / 8) * row_tiles;
  if (grid > INT32_MAX || row_tiles > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(upproj_kernel, dim3((unsigned)grid), dim3(UP_THREADS), 0, stream, p, (int32_t)row_tiles,
                     tiles_per_seq, hpg);
  return hipGetLastError();
}

}  // namespace mla
