// Dense varlen MLA prefill forward for gfx950: O = softmax(Q K^T * scale + mask) V, with LSE.
//
// The operation and its conventions (K/V expanded to every head, q/k head 192 = 128 nope + 64
// rope, v head 128, cu_seqlens, causal for new tokens, unmasked context chunks that return the
// LSE) are those of page "FlashAttention backend for MLA prefill" (dispatch,
// run_prefill_new_tokens, run_prefill_context_chunk); the softmax is accumulated online in the
// manner the "Mojo module mla" page names as the Flash attention v2 algorithm.
//
// Work decomposition. One work-group (4 waves) owns one (query tile, head, key split). The
// query tile has BM = 128*NQ rows; wave w owns rows [w*32*NQ, (w+1)*32*NQ). Keys stream in
// blocks of BN = 64 through LDS, double-buffered, copied straight from global memory into LDS
// (no register staging). Per block and wave:
//   S^T (keys x queries) = K_blk (A, from LDS) * Q^T (B, registers)       32x32x16 bf16 MFMA
//   each lane owns one query column, so the row max needs one cross-half swap and the row sum
//   stays lane-local until the end;
//   O^T (dv x queries) += V_blk^T (A, LDS transposed reads) * P^T (B, the S^T registers
//   converted to bf16 in place, no data movement).
// The key order inside every 16-key MFMA step is the one the S^T accumulator layout gives each
// lane (keys {4h..4h+3, 8+4h..8+4h+3} for lane half h); the V^T operand is read in the same
// order with two ds_read_b64_tr_b16 of four consecutive keys each.
//
// LDS layout per stage (16-byte chunks, XOR-swizzled so every MFMA operand read is free of bank
// conflicts while each wave's copy still writes 1 KiB contiguous):
//   K: 64 rows x 24 chunks (384 B/row); chunk c of row r sits at c ^ (r & 7).
//   V: 64 rows x 16 chunks (256 B/row); chunk c of row r sits at c ^ ((r & 3) << 1).
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int BN = 64;
constexpr int DQK = 192;
constexpr int DV = 128;
constexpr int K_STAGE_BYTES = BN * DQK * 2;   // 24576
constexpr int V_STAGE_BYTES = BN * DV * 2;    // 16384
constexpr int K_CHUNKS_PER_WAVE = BN * (DQK / 8) / 256;  // 6 wave-wide 1 KiB copies
constexpr int V_CHUNKS_PER_WAVE = BN * (DV / 8) / 256;   // 4

struct Stage {
  char* k;
  char* v;
};

template <int NQ>
struct DenseCtx {
  // per-lane constants
  int lane, wave, l32, hl;
  // problem
  const __bf16* kbase;   // K of this sequence/head at key 0
  const __bf16* vbase;
  int64_t k_st, v_st;
  int sk, sq, row0;
  int koff[K_CHUNKS_PER_WAVE];  // element offset of this lane's chunk within a block (row*k_st + c*8)
  int krow[K_CHUNKS_PER_WAVE];
  int voff[V_CHUNKS_PER_WAVE];
  int vrow[V_CHUNKS_PER_WAVE];
};

template <int NQ>
__device__ __forceinline__ void issue_block_load(const DenseCtx<NQ>& c, int j, Stage st) {
  const int key0 = j * BN;
  const bool tail = key0 + BN > c.sk;
  const __bf16* kb = c.kbase + (int64_t)key0 * c.k_st;
  const __bf16* vb = c.vbase + (int64_t)key0 * c.v_st;
#pragma unroll
  for (int i = 0; i < K_CHUNKS_PER_WAVE; ++i) {
    int off = c.koff[i];
    if (tail) {
      int r = c.krow[i];
      int rr = min(key0 + r, c.sk - 1) - key0;  // clamp to a real row; masked later
      off += (rr - r) * (int)c.k_st;
    }
    g2lds16(kb + off, st.k + (c.wave * K_CHUNKS_PER_WAVE + i) * 1024);
  }
#pragma unroll
  for (int i = 0; i < V_CHUNKS_PER_WAVE; ++i) {
    int off = c.voff[i];
    if (tail) {
      int r = c.vrow[i];
      int rr = min(key0 + r, c.sk - 1) - key0;
      off += (rr - r) * (int)c.v_st;
    }
    g2lds16(vb + off, st.v + (c.wave * V_CHUNKS_PER_WAVE + i) * 1024);
  }
}

template <int NQ>
__device__ __forceinline__ void compute_block(const DenseCtx<NQ>& c, int j, const char* ks,
                                              const char* vs, const bf16x8 (&qf)[NQ][DQK / 16],
                                              float (&m_run)[NQ], float (&l_run)[NQ],
                                              f32x16 (&o)[NQ][DV / 32], float scale_log2,
                                              bool causal) {
  // ---- S^T = K_blk * Q^T
  f32x16 s[NQ][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) s[nq][mt] = f32x16{};
    const int row = mt * 32 + c.l32;
    const char* rbase = ks + row * (DQK * 2);
#pragma unroll
    for (int kk = 0; kk < DQK / 16; ++kk) {
      const int ch = (kk * 2 + c.hl) ^ (row & 7);
      bf16x8 a = lds_read_b128(rbase + ch * 16);
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) s[nq][mt] = mfma32(a, qf[nq][kk], s[nq][mt]);
    }
  }
  // ---- mask (diagonal and tail blocks only; wave-uniform test)
  const int key0 = j * BN;
  const int qmin = c.row0 + c.wave * 32 * NQ;  // smallest local query row of this wave
  const int diag = c.sk - c.sq;                // bottom-right alignment offset
  const bool need_mask = (key0 + BN > c.sk) || (causal && key0 + BN - 1 > qmin + diag);
  if (need_mask) {
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      const int qrow = qmin + nq * 32 + c.l32;
      const int lim = causal ? min(c.sk - 1, qrow + diag) : (c.sk - 1);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + mt * 32 + 8 * (i >> 2) + 4 * c.hl + (i & 3);
          if (key > lim) s[nq][mt][i] = -INFINITY;
        }
    }
  }
  // ---- online softmax (per lane = per query; halves l and l^32 share a query)
  bf16x8 pf[NQ][2][2];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    float mx = s[nq][0][0];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[nq][mt][i]);
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m_run[nq], mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run[nq] - m_use) * scale_log2);
    const float mc = m_use * scale_log2;
    float rs = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(fmaf(s[nq][mt][i], scale_log2, -mc));
        s[nq][mt][i] = pv;
        rs += pv;
      }
    l_run[nq] = l_run[nq] * alpha + rs;
    m_run[nq] = m_new;
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt) o[nq][dt] *= alpha;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[nq][mt][cc][e] = (__bf16)s[nq][mt][cc * 8 + e];
  }
  // ---- O^T += V_blk^T * P^T
  const int g = c.lane >> 4;          // 16-lane group
  const int r = c.lane & 15;          // lane within the group
  const int dv_lane = (g & 1) * 16 + 4 * (r & 3);
#pragma unroll
  for (int dt = 0; dt < DV / 32; ++dt) {
    const int dv = dt * 32 + dv_lane;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int k0 = mt * 32 + cc * 16 + 4 * c.hl + (r >> 2);
        const int k1 = k0 + 8;
        const int ch = dv >> 3;
        const int sub = (dv & 7) * 2;
        const char* p0 = vs + k0 * (DV * 2) + ((ch ^ ((k0 & 3) << 1)) * 16) + sub;
        const char* p1 = vs + k1 * (DV * 2) + ((ch ^ ((k1 & 3) << 1)) * 16) + sub;
        bf16x8 a = join(lds_read_tr16(p0), lds_read_tr16(p1));
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) o[nq][dt] = mfma32(a, pf[nq][mt][cc], o[nq][dt]);
      }
  }
}

}  // namespace

template <int NQ>
__global__ __launch_bounds__(256, (NQ == 1 ? 2 : 1)) void dense_fwd_kernel(DenseParams p) {
  constexpr int BM = 128 * NQ;
  __shared__ __attribute__((aligned(1024))) char lds_k0[K_STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_v0[V_STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_k1[K_STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_v1[V_STAGE_BYTES];

  // ---- XCD-aware work mapping: blocks are dealt round-robin to the 8 XCDs, so give each XCD a
  // contiguous, head-major range of work items (tiles of one head share K/V in that XCD's L2).
  const int x = blockIdx.x;
  const int w = (x & 7) * p.per_xcd + (x >> 3);
  if (w >= p.total_work) return;
  const int split = w % p.num_splits;
  const int t = w / p.num_splits;
  const int item = t % p.n_slots;
  const int h = t / p.n_slots;
  if (item >= *p.num_items) return;
  const int4 it = reinterpret_cast<const int4*>(p.plan)[item];
  const int b = it.x, m = it.y, nb = it.z;

  const int cq0 = p.cu_q[b], sq = p.cu_q[b + 1] - cq0;
  const int ck0 = p.cu_k[b], sk = p.cu_k[b + 1] - ck0;
  const int row0 = m * BM;
  const int rows = min(BM, sq - row0);
  const int blo = (int)(((int64_t)split * nb) / p.num_splits);
  const int bhi = (int)(((int64_t)(split + 1) * nb) / p.num_splits);

  DenseCtx<NQ> c;
  c.lane = threadIdx.x & 63;
  c.wave = threadIdx.x >> 6;
  c.l32 = c.lane & 31;
  c.hl = c.lane >> 5;
  c.kbase = p.k + (int64_t)ck0 * p.k_st + (int64_t)h * p.k_sh;
  c.vbase = p.v + (int64_t)ck0 * p.v_st + (int64_t)h * p.v_sh;
  c.k_st = p.k_st;
  c.v_st = p.v_st;
  c.sk = sk;
  c.sq = sq;
  c.row0 = row0;
#pragma unroll
  for (int i = 0; i < K_CHUNKS_PER_WAVE; ++i) {
    const int pch = (c.wave * K_CHUNKS_PER_WAVE + i) * 64 + c.lane;
    const int row = pch / 24, pc = pch % 24;
    const int lc = pc ^ (row & 7);
    c.krow[i] = row;
    c.koff[i] = row * (int)p.k_st + lc * 8;
  }
#pragma unroll
  for (int i = 0; i < V_CHUNKS_PER_WAVE; ++i) {
    const int pch = (c.wave * V_CHUNKS_PER_WAVE + i) * 64 + c.lane;
    const int row = pch >> 4, pc = pch & 15;
    const int lc = pc ^ ((row & 3) << 1);
    c.vrow[i] = row;
    c.voff[i] = row * (int)p.v_st + lc * 8;
  }

  // ---- Q^T fragments for this wave's query columns (zero beyond the sequence)
  bf16x8 qf[NQ][DQK / 16];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const int r = c.wave * 32 * NQ + nq * 32 + c.l32;
    const bool ok = r < rows;
    const __bf16* qp = p.q + (int64_t)(cq0 + row0 + (ok ? r : 0)) * p.q_st + (int64_t)h * p.q_sh + c.hl * 8;
#pragma unroll
    for (int kk = 0; kk < DQK / 16; ++kk) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + kk * 16);
      qf[nq][kk] = ok ? v : bf16x8{};
    }
  }

  float m_run[NQ], l_run[NQ];
  f32x16 o[NQ][DV / 32];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    m_run[nq] = -INFINITY;
    l_run[nq] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt) o[nq][dt] = f32x16{};
  }

  const bool causal = p.causal != 0;
  const Stage st0{lds_k0, lds_v0}, st1{lds_k1, lds_v1};
  if (blo < bhi) issue_block_load(c, blo, st0);
  wait_vmem();
  __syncthreads();
  // Two blocks per trip so each stage is a distinct LDS object at compile time.
  for (int j = blo; j < bhi; j += 2) {
    if (j + 1 < bhi) issue_block_load(c, j + 1, st1);
    compute_block<NQ>(c, j, lds_k0, lds_v0, qf, m_run, l_run, o, p.scale_log2, causal);
    wait_vmem();
    __syncthreads();
    if (j + 1 >= bhi) break;
    if (j + 2 < bhi) issue_block_load(c, j + 2, st0);
    compute_block<NQ>(c, j + 1, lds_k1, lds_v1, qf, m_run, l_run, o, p.scale_log2, causal);
    wait_vmem();
    __syncthreads();
  }

  // ---- epilogue
  const float sink_v = (p.sink != nullptr && p.o_part == nullptr) ? p.sink[h] : -INFINITY;
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const float l_tot = xhalf_sum(l_run[nq]);
    const int r = c.wave * 32 * NQ + nq * 32 + c.l32;
    float inv, lse_v;
    if (l_tot == 0.f) {
      inv = 0.f;
      lse_v = sink_v;  // -inf without a sink
    } else {
      const float mm = m_run[nq] * p.scale;  // natural-log units
      if (sink_v == -INFINITY) {
        inv = 1.f / l_tot;
        lse_v = mm + __logf(l_tot);
      } else {
        const float mx = fmaxf(mm, sink_v);
        const float a = __expf(mm - mx);
        const float z = l_tot * a + __expf(sink_v - mx);
        inv = a / z;
        lse_v = mx + __logf(z);
      }
    }
    if (r < rows) {
      const int tok = cq0 + row0 + r;
      if (p.o_part != nullptr) {
        float* op = p.o_part + (((int64_t)split * p.total_q + tok) * p.num_heads + h) * DV;
#pragma unroll
        for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int dv = dt * 32 + 8 * g4 + 4 * c.hl;
            f32x4 v = {o[nq][dt][g4 * 4 + 0] * inv, o[nq][dt][g4 * 4 + 1] * inv,
                       o[nq][dt][g4 * 4 + 2] * inv, o[nq][dt][g4 * 4 + 3] * inv};
            *reinterpret_cast<f32x4*>(op + dv) = v;
          }
        if (c.hl == 0) p.lse_part[((int64_t)split * p.total_q + tok) * p.num_heads + h] = lse_v;
      } else {
        __bf16* op = p.out + (int64_t)tok * p.o_st + (int64_t)h * p.o_sh;
#pragma unroll
        for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int dv = dt * 32 + 8 * g4 + 4 * c.hl;
            u32x2 v = {pack_bf16x2(o[nq][dt][g4 * 4 + 0] * inv, o[nq][dt][g4 * 4 + 1] * inv),
                       pack_bf16x2(o[nq][dt][g4 * 4 + 2] * inv, o[nq][dt][g4 * 4 + 3] * inv)};
            *reinterpret_cast<u32x2*>(op + dv) = v;
          }
        if (p.lse != nullptr && c.hl == 0) p.lse[(int64_t)tok * p.l_st + (int64_t)h * p.l_sh] = lse_v;
      }
    }
  }
}

template __global__ void dense_fwd_kernel<1>(DenseParams);
template __global__ void dense_fwd_kernel<2>(DenseParams);

hipError_t launch_dense_fwd(const DenseParams& p, int nq, hipStream_t stream) {
  const int grid = 8 * p.per_xcd;
  if (grid <= 0) return hipSuccess;
  if (nq == 2) {
    hipLaunchKernelGGL(dense_fwd_kernel<2>, dim3(grid), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(dense_fwd_kernel<1>, dim3(grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mla
