// Split-KV combine: merges S normalised partial results of disjoint key sets (and optionally a
// sink logit with a zero value vector) into the final output (bf16, or fp8 e4m3 with a static
// scale) and float32 LSE.
//
// Prior art: per-partition partial outputs reduced into the final result (page "Mojo module
// mla", mla_splitk_reduce; page "Sgl project Sglang FA4 Interface", Description: split-KV with
// a combine kernel). LSE = log(sum_s exp(LSE_s) [+ exp(sink)]), O = sum_s exp(LSE_s - LSE) O_s;
// rows whose partials are all empty give O = 0 and LSE = -inf (or the sink).
//
// HBM-bound: each thread owns four consecutive output columns of one row, reads the S partial
// LSEs of its row (shared through L1/L2 by the row's other threads) and streams its columns of
// the S partial outputs once with 16-byte loads.
#include "common.h"
#include "kernels.h"

namespace mla {

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int c4_per_row = p.dv >> 2;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)p.rows * c4_per_row) return;
  const int row = (int)(t / c4_per_row);
  const int c4 = (int)(t - (int64_t)row * c4_per_row);
  const int h = row % p.num_heads;
  const int tok = row / p.num_heads;

  float mx = -INFINITY;
  for (int s = 0; s < p.num_splits; ++s) mx = fmaxf(mx, p.lse_part[(int64_t)s * p.rows + row]);
  const float sink_v = p.sink ? p.sink[h] : -INFINITY;
  mx = fmaxf(mx, sink_v);
  float lse_v;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (mx == -INFINITY) {
    lse_v = -INFINITY;
  } else {
    float tot = __expf(sink_v - mx);
    for (int s = 0; s < p.num_splits; ++s) tot += __expf(p.lse_part[(int64_t)s * p.rows + row] - mx);
    lse_v = mx + __logf(tot);
    for (int s = 0; s < p.num_splits; ++s) {
      const float ls = p.lse_part[(int64_t)s * p.rows + row];
      if (ls == -INFINITY) continue;
      const float wgt = __expf(ls - lse_v);
      const f32x4 v = *reinterpret_cast<const f32x4*>(p.o_part + ((int64_t)s * p.rows + row) * p.dv + c4 * 4);
      acc += wgt * v;
    }
  }
  const int64_t off = (int64_t)tok * p.o_st + (int64_t)h * p.o_sh + c4 * 4;
  if (p.out_scale != nullptr) {
    // fp8 e4m3 (round to nearest even) of O / out_scale, saturated at +-448
    const float w = 1.f / p.out_scale[0];
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = fminf(fmaxf(acc[i] * w, -448.f), 448.f);
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], v, true);
    *reinterpret_cast<int*>(static_cast<uint8_t*>(p.out) + off) = v;
  } else {
    u32x2 ov = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<u32x2*>(static_cast<__bf16*>(p.out) + off) = ov;
  }
  if (p.lse != nullptr && c4 == 0) p.lse[(int64_t)tok * p.l_st + (int64_t)h * p.l_sh] = lse_v;
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.rows * (p.dv >> 2);
  if (threads == 0) return hipSuccess;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
