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
// contiguous along the 512-deep contraction. A work-group (4 waves, one per SIMD) computes all 512
// output columns of a pair of heads (their keys and values) for 128 cached rows of one sequence.
// Each wave keeps its 32 latent rows resident in registers as the MFMA B operand (128 per lane,
// loaded once) and accumulates 32 rows x 512 columns in the 256 accumulation registers; the
// pair's W_KV rows stream through a 4-deep LDS ring, 32 of the 512 contraction columns per
// stage (32 KiB), copied straight from global memory (global_load_lds) three stages ahead. A
// 64-byte operand row keeps its 16-byte chunk c at c ^ ((r >> 2) & 3), which makes the operand
// reads conflict-free under gfx950's 16-byte read grouping. Work-groups are dealt to the XCDs by
// head pair, so the ones running together on an XCD share the pair's 512 KiB of W_KV in its L2,
// and each latent tile is read once per head pair. The outputs are stored after the last copy
// has landed (stores and the copies' wait counts never mix); the key columns 128..191 take the
// rope columns of the cached rows.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int UP_ROWS = 128;               // cached rows per work-group (32 per wave)
constexpr int UP_HEADS = 2;                // heads per work-group
constexpr int KV_COLS = 256;               // per head: 128 key + 128 value columns
constexpr int UP_COLS = UP_HEADS * KV_COLS;  // 512 output columns per work-group
constexpr int UP_KS = 32;                  // contraction columns per stage
constexpr int UP_STAGE = UP_COLS * UP_KS * 2;  // 32 KiB of W_KV per stage
constexpr int UP_NBUF = 4;                 // ring slots: copies run three stages ahead
constexpr int UP_THREADS = 256;
constexpr int LAT_D = 512;
constexpr int UP_NSTAGE = LAT_D / UP_KS;   // 16
constexpr int UP_COPIES = UP_STAGE / 1024 / (UP_THREADS / 64);  // 8 wave copies per wave per stage

// byte offset of 16-byte chunk c of operand row r (64 bytes per row) within a stage
__host__ __device__ constexpr int swz_pos(int r, int c) { return r * (UP_KS * 2) + ((c ^ ((r >> 2) & 3)) << 4); }

// Direct global -> LDS copy of 16 bytes per lane (lane l's bytes land at lds_base + 16 l), issued
// from asm so that the compiler's wait-count bookkeeping does not track it: the copies are waited
// for explicitly (vmcnt) before the barrier that precedes their use. The instruction writes no
// vector register; M0 is declared clobbered.
__device__ __forceinline__ void g2lds16_untracked(const void* gptr, const void* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m0v) : "memory", "m0");
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

// Grid: 8 * ceil(pairs / 8) * row_tiles work-groups, row_tiles = batch * ceil(w / 128). Work-group
// i runs on XCD i % 8; it takes head pair (i % 8) + 8 * (j / row_tiles) and row tile j % row_tiles
// with j = i / 8, so the XCDs split the head pairs and each goes through all row tiles of one pair
// before the next.
__global__ __launch_bounds__(UP_THREADS, 1) void upproj_kernel(UpprojParams p, int32_t row_tiles, int32_t tiles_per_seq) {
  __shared__ __attribute__((aligned(1024))) char ring[UP_NBUF * UP_STAGE];
  const int xcd = blockIdx.x & 7;
  const int j = blockIdx.x >> 3;
  const int pair = xcd + 8 * (j / row_tiles);
  const int rt = j - (j / row_tiles) * row_tiles;
  const int b = rt / tiles_per_seq;
  const int tile = rt - b * tiles_per_seq;
  const int h0 = pair * UP_HEADS;
  if (h0 >= p.num_heads) return;
  const int ctx_b = p.cu_ctx[b + 1] - p.cu_ctx[b];
  const int len = min(max(ctx_b - p.c0, 0), p.w);   // this sequence's rows in the chunk
  const int r0 = tile * UP_ROWS;
  if (r0 >= len) return;
  const int rows = min(UP_ROWS, len - r0);
  const int nh = min(UP_HEADS, p.num_heads - h0);   // heads of this pair that exist
  const int64_t lat_row0 = (int64_t)p.cu_ctx[b] + p.c0 + r0;    // first cached row of the tile
  const int64_t buf_row0 = (int64_t)p.cu_chunk[b] + r0;          // first buffer row of the tile

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;

  // Stage copies: wave copy q (= UP_COPIES * wave + i) covers operand rows 16 q + lane / 4 (output
  // columns of the pair; row h * 256 + c of the pair is W_KV row (h0 + h) * 256 + c), slot lane % 4.
  const __bf16* wsrc[UP_COPIES];
#pragma unroll
  for (int i = 0; i < UP_COPIES; ++i) {
    const int r = (wave * UP_COPIES + i) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const int wr = min(r, nh * KV_COLS - 1);  // a missing second head re-reads the first one's rows
    wsrc[i] = p.w_kv + (int64_t)(h0 * KV_COLS + wr) * p.w_st + c * 8;
  }
  auto issue = [&](int s) {
    char* dst = ring + (s % UP_NBUF) * UP_STAGE;
#pragma unroll
    for (int i = 0; i < UP_COPIES; ++i) g2lds16_untracked(wsrc[i] + s * UP_KS, dst + (wave * UP_COPIES + i) * 1024);
  };
  issue(0);
  issue(1);
  issue(2);

  // B operand: this wave's 32 cached rows (tail rows re-read the last one), all 512 columns:
  // cb[kk] = columns 16 kk + 8 hl .. +7 of row 32 wave + l32.
  bf16x8 cb[LAT_D / 16];
  {
    const __bf16* src = p.latent + (lat_row0 + min(wave * 32 + l32, rows - 1)) * p.lat_st + hl * 8;
#pragma unroll
    for (int kk = 0; kk < LAT_D / 16; ++kk) cb[kk] = *reinterpret_cast<const bf16x8*>(src + kk * 16);
  }
  f32x16 acc[UP_HEADS][KV_COLS / 32];
#pragma unroll
  for (int h = 0; h < UP_HEADS; ++h)
#pragma unroll
    for (int ct = 0; ct < KV_COLS / 32; ++ct) acc[h][ct] = f32x16{};

  // A operand: operand row 256 h + 32 ct + l32, chunk 2 kk + hl; ((row >> 2) & 3) == ((l32 >> 2) & 3).
  const int a_base[2] = {swz_pos(l32, hl), swz_pos(l32, 2 + hl)};
#pragma unroll
  for (int s = 0; s < UP_NSTAGE; ++s) {
    // this wave's copies of stage s have landed (the later stages' copies stay in flight), then
    // every wave's have; the barrier also retires stage s - 1 for all waves, so its slot may be
    // refilled with stage s + 3
    if (s + 2 < UP_NSTAGE) wait_vm<2 * UP_COPIES>();
    else if (s + 1 < UP_NSTAGE) wait_vm<UP_COPIES>();
    else wait_vm<0>();
    lds_barrier();
    if (s + 3 < UP_NSTAGE) issue(s + 3);
    const char* st = ring + (s % UP_NBUF) * UP_STAGE;
    // 32 products per stage, step t = (kk, h, ct); the operand reads run PF steps ahead of their
    // products (one wave per SIMD: nothing else hides the LDS latency)
    constexpr int NT = (UP_KS / 16) * UP_HEADS * (KV_COLS / 32);
    constexpr int PF = 6;
    bf16x8 a[NT];
    auto rd = [&](int t) {
      const int kk = t / (UP_HEADS * (KV_COLS / 32)), hc = t % (UP_HEADS * (KV_COLS / 32));
      a[t] = lds_read_b128(st + a_base[kk] + hc * 32 * (UP_KS * 2));
    };
#pragma unroll
    for (int t = 0; t < PF; ++t) rd(t);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t + PF < NT) rd(t + PF);
      const int kk = t / (UP_HEADS * (KV_COLS / 32)), hc = t % (UP_HEADS * (KV_COLS / 32));
      acc[hc / (KV_COLS / 32)][hc % (KV_COLS / 32)] =
          mfma32(a[t], cb[2 * s + kk], acc[hc / (KV_COLS / 32)][hc % (KV_COLS / 32)]);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads PF steps ahead of their products
    }
  }

  // Output through LDS (the ring is free once every wave has finished the last stage): wave w's
  // 32 rows x 512 columns go to its own 32 KiB, then leave as whole 256-byte segments (a head's
  // 128 key or 128 value columns of one row). In the wave's region, row r (1 KiB) keeps logical
  // 16-byte chunk c at chunk c ^ (r & 15), and the two 8-byte halves of a chunk swapped when
  // r & 16: the 8-byte writes (lane l: row l % 32, half l / 32) and the 16-byte reads (16 lanes
  // per segment) are then free of bank conflicts. Lane l holds columns 32 ct + 8 g + 4 hl .. +3
  // of head h for row l32, i.e. logical chunk 32 h + 4 ct + g, half hl.
  lds_barrier();
  char* ob = ring + wave * 32768;
#pragma unroll
  for (int h = 0; h < UP_HEADS; ++h)
#pragma unroll
    for (int ct = 0; ct < KV_COLS / 32; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& v = acc[h][ct];
        const u32x2 o = {pack_bf16x2(v[4 * g], v[4 * g + 1]), pack_bf16x2(v[4 * g + 2], v[4 * g + 3])};
        const int c = 32 * h + 4 * ct + g;
        *reinterpret_cast<u32x2*>(ob + l32 * 1024 + ((c ^ (l32 & 15)) << 4) + ((hl ^ (l32 >> 4)) << 3)) = o;
      }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave reads back only its own region
  {
    const int part = lane >> 4, i16 = lane & 15;    // part: head part / 2, key (even) or value (odd)
    const int hp = part >> 1;
    __bf16* base = (part & 1) ? p.vbuf + (int64_t)(h0 + hp) * p.v_sh : p.kbuf + (int64_t)(h0 + hp) * p.k_sh;
    const int64_t rst = (part & 1) ? p.v_st : p.k_st;
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      const int c = 16 * part + i16;
      u32x4 v = *reinterpret_cast<const u32x4*>(ob + r * 1024 + ((c ^ (r & 15)) << 4));
      if (r & 16) v = __builtin_shufflevector(v, v, 2, 3, 0, 1);  // halves were swapped
      const int row = wave * 32 + r;
      if (row < rows && hp < nh) *reinterpret_cast<u32x4*>(base + (buf_row0 + row) * rst + i16 * 8) = v;
    }
  }
  // rope columns 512..575 of the cached rows -> key columns 128..191 of both heads
  {
    const int r = tid >> 1, half = tid & 1;
    if (r < rows) {
      const u32x4* src = reinterpret_cast<const u32x4*>(p.latent + (lat_row0 + r) * p.lat_st + LAT_D + half * 32);
      u32x4 rv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) rv[i] = src[i];
#pragma unroll
      for (int h = 0; h < UP_HEADS; ++h) {
        if (h < nh) {
          u32x4* d = reinterpret_cast<u32x4*>(p.kbuf + (buf_row0 + r) * p.k_st + (int64_t)(h0 + h) * p.k_sh + 128 + half * 32);
#pragma unroll
          for (int i = 0; i < 4; ++i) d[i] = rv[i];
        }
      }
    }
  }
}

hipError_t launch_chunk_cu(const int32_t* cu_ctx, int32_t batch, int32_t c0, int32_t w, int32_t* cu_chunk,
                           hipStream_t stream) {
  hipLaunchKernelGGL(chunk_cu_kernel, dim3(1), dim3(1024), 0, stream, cu_ctx, batch, c0, w, cu_chunk);
  return hipGetLastError();
}

hipError_t launch_upproj(const UpprojParams& p, hipStream_t stream) {
  const int tiles_per_seq = (p.w + UP_ROWS - 1) / UP_ROWS;
  if (tiles_per_seq == 0 || p.batch == 0 || p.num_heads == 0) return hipSuccess;
  const int64_t row_tiles = (int64_t)p.batch * tiles_per_seq;
  const int64_t pairs = (p.num_heads + UP_HEADS - 1) / UP_HEADS;
  const int64_t grid = 8 * ((pairs + 7) / 8) * row_tiles;
  if (grid > INT32_MAX || row_tiles > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(upproj_kernel, dim3((unsigned)grid), dim3(UP_THREADS), 0, stream, p, (int32_t)row_tiles,
                     tiles_per_seq);
  return hipGetLastError();
}

}  // namespace mla
