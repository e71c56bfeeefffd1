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
// Up-projection: a bf16 GEMM C = W_KV * C_latent^T on 32x32x16 MFMA with both operands
// contiguous along the 512-deep contraction. A work-group (4 waves) computes 128 output columns
// (half of one head: its key or its value part) for 128 cached rows of one sequence; each wave
// holds a 64 x 64 block (2 x 2 accumulator tiles); three work-groups share a CU. The contraction runs in 16 stages of 32 through
// a 3-slot LDS ring, copied straight from global memory (global_load_lds, 1 KiB per wave copy)
// two stages ahead of the compute; a 64-byte operand row keeps its 16-byte chunk c at
// c ^ ((r >> 2) & 3), which makes the operand reads conflict-free under gfx950's 16-byte read
// grouping. The output tile is turned around in the (then free) ring and written as whole
// 128-byte row segments. The key work-groups also copy the rope columns into every head's key.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int UP_TILE = 128;               // rows and output columns per work-group
constexpr int UP_KS = 32;                  // contraction per stage
constexpr int UP_STAGE = UP_TILE * UP_KS * 2;  // 8 KiB per operand per stage
constexpr int UP_THREADS = 256;
constexpr int UP_NBUF = 3;                 // ring slots (copies run two stages ahead)
constexpr int LAT_D = 512;
constexpr int KV_COLS = 256;               // per head: 128 key + 128 value columns

__device__ __forceinline__ int swz_pos(int r, int c) { return r * (UP_KS * 2) + ((c ^ ((r >> 2) & 3)) << 4); }

// Direct global -> LDS copy of 16 bytes per lane (lane l's bytes land at lds_base + 16 l), issued
// from asm so that the compiler's wait-count bookkeeping does not track it: the ring slot being
// read is chosen at run time, and a tracked copy into any slot would make every operand read wait
// for all copies in flight. The copies are waited for explicitly (vmcnt) before the barrier that
// precedes their use. The instruction writes no vector register; M0 is declared clobbered.
__device__ __forceinline__ void g2lds16_untracked(const void* gptr, const void* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m0v) : "memory", "m0");
}

// LDS reads done, then the work-group barrier; copies in flight stay in flight.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
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

__global__ __launch_bounds__(UP_THREADS) void upproj_kernel(UpprojParams p) {
  __shared__ __attribute__((aligned(1024))) char lds_w[UP_NBUF * UP_STAGE];
  __shared__ __attribute__((aligned(1024))) char lds_c[UP_NBUF * UP_STAGE];
  const int b = blockIdx.y;
  const int tile = blockIdx.x;
  const int z = blockIdx.z;               // 2h: key columns of head h, 2h + 1: value columns
  const int h = z >> 1;
  const bool is_key = (z & 1) == 0;
  const int ctx_b = p.cu_ctx[b + 1] - p.cu_ctx[b];
  const int len = min(max(ctx_b - p.c0, 0), p.w);   // this sequence's rows in the chunk
  const int r0 = tile * UP_TILE;
  if (r0 >= len) return;
  const int rows = min(UP_TILE, len - r0);
  const int64_t lat_row0 = (int64_t)p.cu_ctx[b] + p.c0 + r0;    // first cached row of the tile
  const int64_t buf_row0 = (int64_t)p.cu_chunk[b] + r0;          // first buffer row of the tile

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  // copy addresses: wave copy q (= 2 wave + i) covers tile rows 16 q + lane / 4, slot lane % 4
  const __bf16* wsrc[2];
  const __bf16* csrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wave * 2 + i) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    wsrc[i] = p.w_kv + (int64_t)(h * KV_COLS + (is_key ? 0 : 128) + r) * p.w_st + c * 8;
    csrc[i] = p.latent + (lat_row0 + min(r, rows - 1)) * p.lat_st + c * 8;  // tail rows re-read the last
  }
  auto issue = [&](int s, int slot) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      g2lds16_untracked(wsrc[i] + s * UP_KS, lds_w + slot * UP_STAGE + (wave * 2 + i) * 1024);
      g2lds16_untracked(csrc[i] + s * UP_KS, lds_c + slot * UP_STAGE + (wave * 2 + i) * 1024);
    }
  };
  // wave (wm, wn) computes output columns [64 wm, 64 wm + 64) x rows [64 wn, 64 wn + 64)
  const int wm = wave & 1, wn = wave >> 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  constexpr int NSTAGE = LAT_D / UP_KS;
  issue(0, 0);
  issue(1, 1);
  asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // this wave's stage-0 copies have landed
  ring_barrier();
  for (int s = 0; s < NSTAGE; ++s) {
    const int slot = s % UP_NBUF;
    if (s + 2 < NSTAGE) issue(s + 2, (s + 2) % UP_NBUF);
    const char* wb = lds_w + slot * UP_STAGE;
    const char* cb = lds_c + slot * UP_STAGE;
#pragma unroll
    for (int kk = 0; kk < UP_KS / 16; ++kk) {
      bf16x8 a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = lds_read_b128(wb + swz_pos(wm * 64 + i * 32 + l32, 2 * kk + hl));
        bb[i] = lds_read_b128(cb + swz_pos(wn * 64 + i * 32 + l32, 2 * kk + hl));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], bb[j], acc[i][j]);
    }
    // stage s + 1 must have landed for the next iteration (stage s + 2 may stay in flight)
    if (s + 2 < NSTAGE) {
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    ring_barrier();
  }
  // Output through LDS (the ring is free now): the wave's 64 x 64 tile goes to its own 8 KiB
  // (64 rows of 128 bytes, 16-byte chunk c of row r at c ^ (r & 7)) and leaves as whole 128-byte
  // row segments.
  __bf16* dst = is_key ? p.kbuf : p.vbuf;
  const int64_t dst_st = is_key ? p.k_st : p.v_st;
  char* ob = ((wave & 1) ? lds_c : lds_w) + (wave >> 1) * 8192;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = j * 32 + l32;
        const f32x16& v = acc[i][j];
        u32x2 o = {pack_bf16x2(v[4 * g], v[4 * g + 1]), pack_bf16x2(v[4 * g + 2], v[4 * g + 3])};
        *reinterpret_cast<u32x2*>(ob + r * 128 + (((4 * i + g) ^ (r & 7)) * 16) + 8 * hl) = o;
      }
  const int cc = lane & 7;
#pragma unroll
  for (int ps = 0; ps < 8; ++ps) {
    const int r = ps * 8 + (lane >> 3);
    const u32x4 v = *reinterpret_cast<const u32x4*>(ob + r * 128 + ((cc ^ (r & 7)) * 16));
    const int tr = wn * 64 + r;
    if (tr < rows)
      *reinterpret_cast<u32x4*>(dst + (buf_row0 + tr) * dst_st + (int64_t)h * (is_key ? p.k_sh : p.v_sh) + wm * 64 + cc * 8) = v;
  }
  if (is_key) {
    // rope columns 512..575 of the cached row -> key columns 128..191 of head h
    const int r = tid >> 1, half = tid & 1;
    if (r < rows) {
      const u32x4* src = reinterpret_cast<const u32x4*>(p.latent + (lat_row0 + r) * p.lat_st + LAT_D + half * 32);
      u32x4* d = reinterpret_cast<u32x4*>(p.kbuf + (buf_row0 + r) * p.k_st + (int64_t)h * p.k_sh + 128 + half * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = src[i];
    }
  }
}

hipError_t launch_chunk_cu(const int32_t* cu_ctx, int32_t batch, int32_t c0, int32_t w, int32_t* cu_chunk,
                           hipStream_t stream) {
  hipLaunchKernelGGL(chunk_cu_kernel, dim3(1), dim3(1024), 0, stream, cu_ctx, batch, c0, w, cu_chunk);
  return hipGetLastError();
}

hipError_t launch_upproj(const UpprojParams& p, hipStream_t stream) {
  const int tiles = (p.w + UP_TILE - 1) / UP_TILE;
  if (tiles == 0 || p.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(upproj_kernel, dim3(tiles, p.batch, 2 * p.num_heads), dim3(UP_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
