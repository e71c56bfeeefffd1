// Calibration kernels for the benchmark harness (not part of the prefill library): the matrix-core
// rate of a pure bf16 32x32x16 MFMA loop and the HBM rate of a streaming read, measured on the
// device the benchmark runs on, so that kernel rates can be quoted as fractions of what this
// device actually sustains as well as of its published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wave

// Every wave runs `iters` rounds of kChains independent 32x32x16 bf16 MFMAs on register operands.
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (lane + j));
    b[j] = (__bf16)(0.002f * (lane - j));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Streaming read: block b reads the contiguous chunk [b*per_block, (b+1)*per_block) of 16-byte
// words, kUnroll non-temporal loads in flight per thread; one XOR per thread is written out.
constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t per_block,
                                                          uint32_t* out) {
  const u32x4* p = src + blockIdx.x * per_block + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (int64_t i = 0; i < per_block; i += 256 * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" {

// FLOP per launch = blocks * 4 waves * iters * kChains * 2*32*32*16. `out` holds blocks*256 floats.
int mla_calib_mfma_loop(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

double mla_calib_mfma_flop(int blocks, int iters) {
  return (double)blocks * 4.0 * iters * kChains * 2.0 * 32 * 32 * 16;
}

// Reads `bytes` from `src`: bytes must be a multiple of blocks * 256 threads * kUnroll * 16 B.
// `out` holds blocks*256 words.
int mla_calib_stream_read(const void* src, int64_t bytes, uint32_t* out, int blocks, void* stream) {
  if (src == nullptr || out == nullptr || bytes <= 0 || blocks <= 0) return 1;
  const int64_t quantum = (int64_t)blocks * 256 * kUnroll * 16;
  if (bytes % quantum != 0) return 2;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(src), bytes / 16 / blocks, out);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
