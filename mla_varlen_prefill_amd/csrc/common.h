// Shared device-side helpers for the gfx950 (CDNA4) MLA prefill kernels.
//
// Lane layouts of the bf16 matrix-core instructions used here (wave64, checked on the device):
//   v_mfma_f32_32x32x16_bf16  A (32x16): lane l holds A[l%32][(l/32)*8 + j], j = 0..7
//                             B (16x32): lane l holds B[(l/32)*8 + j][l%32]
//                             D (32x32): lane l holds D[8*(i/4) + 4*(l/32) + i%4][l%32], i = 0..15
//   ds_read_b64_tr_b16        within each 16-lane group, lane i receives element (i%4) of the
//                             4-element rows addressed by group lanes 4*j + i/4, j = 0..3.
//   v_permlane32_swap(x, x)   returns (x[l], x[l^32]) in some order in its two results;
//   v_permlane16_swap(x, x)   likewise (x[l], x[l^16]).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max / sum of a value and its partner lane l^32 (both halves end up with the result).
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// max / sum over the four lanes l, l^16, l^32, l^48 (one 16x16 MFMA output column).
__device__ __forceinline__ float xquad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return xhalf_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float xquad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return xhalf_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// LDS row swizzle: chunk c (16 bytes) of row r is stored at chunk c ^ row_swz(r), with
// row_swz(r) = 2 * ((r >> 1) & 3) + ((r >> 3) & 1). For a row pitch that is an odd multiple of
// 128 bytes this keeps two read patterns free of bank conflicts on the 64-bank (256-byte) LDS:
//   * 16 consecutive rows read at the same chunk (matrix operand reads);
//   * 8 consecutive rows read at the same 32-byte segment (transposed 16x16 operand reads).
__device__ __forceinline__ int row_swz(int r) { return 2 * ((r >> 1) & 3) + ((r >> 3) & 1); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at lds_base + 16*l.
// lds_base must be wave-uniform.
__device__ __forceinline__ void g2lds16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, LDS_PTR(void, lds_base), 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Work-group barrier for hand-offs through LDS: waits for this wave's own LDS operations, then
// joins the barrier, in one asm statement that the compiler cannot move memory accesses across.
// Unlike __syncthreads(), whose work-group release fence also waits for every global -> LDS copy
// still in flight (vmcnt(0)), it leaves those copies running; the caller waits for the copies it
// needs with an explicit vmcnt before calling it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8 lds_read_b128(const void* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x4 lds_read_tr16(const void* p) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
  return __builtin_bit_cast(bf16x4, t);
}

__device__ __forceinline__ bf16x8 join(const bf16x4& a, const bf16x4& b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace mla
