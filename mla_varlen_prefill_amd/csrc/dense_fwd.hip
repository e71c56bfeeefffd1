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
// conflicts on the 64-bank LDS while each wave's copy still writes 1 KiB contiguous):
//   K: 64 rows x 24 chunks (384 B/row); chunk c of row r sits at c ^ row_swz(r) (16 rows per
//      operand read hit 16 distinct 16-byte bank groups).
//   V: 64 rows x 16 chunks (256 B/row); chunk c of row r sits at c ^ ((r & 3) << 2) (the four
//      rows of a transposed read hit four distinct 64-byte segments).
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

constexpr float kRescaleLog2 = 8.f;  // rescale O only when a row max grows by more than 2^8

template <int NQ>
struct DenseCtx {
  // per-lane constants
  int lane, wave, l32, hl;
  // problem
  const char* kbase;   // K of this sequence/head at key 0 (bytes)
  const char* vbase;
  int k_st_b, v_st_b;  // token strides in bytes (validated to keep 64-row offsets in 31 bits)
  int sk, sq, row0;
  uint32_t koff[K_CHUNKS_PER_WAVE];  // byte offset of this lane's 16-byte chunk inside a block
  uint32_t voff[V_CHUNKS_PER_WAVE];
  int kdst, vdst;                    // this wave's first 1 KiB slot in a stage (bytes)
  // LDS operand addresses (bytes, relative to a stage)
  int ka[4];                         // K rows: + g*128 + mt*32*384 per 4-step group g
  int va[DV / 32];                   // V rows: + (mt*32 + cc*16 [+8]) * 256 per step
};

// 32-bit value the optimiser must treat as opaque (keeps precomputed offsets 32-bit at their use
// and per-lane arithmetic from being hoisted into long-lived registers).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int NQ>
__device__ __forceinline__ void issue_block_load(const DenseCtx<NQ>& c, int j, char* kst, char* vst) {
  const int key0 = j * BN;
  const char* kb = c.kbase + (int64_t)key0 * c.k_st_b;
  const char* vb = c.vbase + (int64_t)key0 * c.v_st_b;
  if (key0 + BN <= c.sk) {
#pragma unroll
    for (int i = 0; i < K_CHUNKS_PER_WAVE; ++i) g2lds16(kb + opaque(c.koff[i]), kst + c.kdst + i * 1024);
#pragma unroll
    for (int i = 0; i < V_CHUNKS_PER_WAVE; ++i) g2lds16(vb + opaque(c.voff[i]), vst + c.vdst + i * 1024);
  } else {
    // tail block: rows past the sequence re-read its last key (finite values, masked later)
    const int last = c.sk - 1 - key0;
    const int lane = (int)opaque((uint32_t)c.lane);
#pragma unroll
    for (int i = 0; i < K_CHUNKS_PER_WAVE; ++i) {
      const int r = ((c.wave * K_CHUNKS_PER_WAVE + i) * 64 + lane) / 24;
      const int shift = (min(r, last) - r) * c.k_st_b;
      g2lds16(kb + (uint32_t)((int)c.koff[i] + shift), kst + c.kdst + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < V_CHUNKS_PER_WAVE; ++i) {
      const int r = ((c.wave * V_CHUNKS_PER_WAVE + i) * 64 + lane) >> 4;
      const int shift = (min(r, last) - r) * c.v_st_b;
      g2lds16(vb + (uint32_t)((int)c.voff[i] + shift), vst + c.vdst + i * 1024);
    }
  }
}

// NMT: how many of the block's two 32-key tiles this wave computes (2, or 1 when the second tile
// is entirely masked for every row of the wave; a wave with both tiles masked skips the block).
template <int NQ, int NMT, bool MASK>
__device__ __forceinline__ void compute_block(const DenseCtx<NQ>& c, int j, const char* ks,
                                              const char* vs, const bf16x8 (&qf)[NQ][DQK / 16],
                                              float (&m_run)[NQ], float (&l_run)[NQ],
                                              f32x16 (&o)[NQ][DV / 32], float scale_log2,
                                              bool causal) {
  // ---- S^T = K_blk * Q^T: the 32-key tiles are independent accumulator chains, issued
  // alternately, with the K fragments read from LDS PF steps ahead of their MFMA.
  f32x16 s[NQ][2];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) s[nq][0] = s[nq][1] = f32x16{};
  {
    constexpr int NSTEP = NMT * (DQK / 16);  // (kk, mt) steps
    constexpr int PF = 4;
    bf16x8 a[NSTEP];
#pragma unroll
    for (int st = 0; st < PF; ++st) {
      const int kk = st / NMT, mt = st % NMT;
      a[st] = lds_read_b128(ks + c.ka[kk & 3] + (kk >> 2) * 128 + mt * 32 * (DQK * 2));
    }
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      if (st + PF < NSTEP) {
        const int kk2 = (st + PF) / NMT, mt2 = (st + PF) % NMT;
        a[st + PF] = lds_read_b128(ks + c.ka[kk2 & 3] + (kk2 >> 2) * 128 + mt2 * 32 * (DQK * 2));
      }
      const int kk = st / NMT, mt = st % NMT;
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) s[nq][mt] = mfma32(a[st], qf[nq][kk], s[nq][mt]);
      __builtin_amdgcn_sched_barrier(0);  // keep the read PF steps ahead of its MFMA
    }
  }
  if (NMT == 1) {
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[nq][1][i] = -INFINITY;
  }
  // ---- mask (diagonal and tail blocks only; wave-uniform test)
  const int key0 = j * BN;
  const int qmin = c.row0 + c.wave * 32 * NQ;  // smallest local query row of this wave
  const int diag = c.sk - c.sq;                // bottom-right alignment offset
  const bool need_mask = MASK && ((key0 + BN > c.sk) || (causal && key0 + BN - 1 > qmin + diag));
  if (need_mask) {
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      const int qrow = qmin + nq * 32 + c.l32;
      const int lim = (causal ? min(c.sk - 1, qrow + diag) : (c.sk - 1)) - key0 - 4 * c.hl;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kofs = mt * 32 + 8 * (i >> 2) + (i & 3);
          if (kofs > lim) s[nq][mt][i] = -INFINITY;
        }
    }
  }
  // ---- online softmax (per lane = per query; halves l and l^32 share a query), lazy rescale
  bf16x8 pf[NQ][2][2];
  const float tau_raw = kRescaleLog2 / scale_log2;
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    float mx = s[nq][0][0];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = (mt == 0 ? 1 : 0); i < 16; ++i) mx = fmaxf(mx, s[nq][mt][i]);
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m_run[nq], mx);
    if (__ballot(m_new > m_run[nq] + tau_raw) != 0ull) {
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run[nq] - m_use) * scale_log2);
      l_run[nq] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DV / 32; ++dt) o[nq][dt] *= alpha;
      m_run[nq] = m_new;
    }
    const float mc = ((m_run[nq] == -INFINITY) ? 0.f : m_run[nq]) * scale_log2;
    float rs = l_run[nq];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        u32x4 packed;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(s[nq][mt][cc * 8 + 2 * e], scale_log2, -mc));
          const float p1 = fast_exp2(fmaf(s[nq][mt][cc * 8 + 2 * e + 1], scale_log2, -mc));
          packed[e] = pack_bf16x2(p0, p1);
          rs += p0 + p1;
        }
        pf[nq][mt][cc] = __builtin_bit_cast(bf16x8, packed);
      }
    l_run[nq] = rs;
  }
  // ---- O^T += V_blk^T * P^T: the four dv tiles are independent chains; the transposed V reads
  // run PF steps ahead of their MFMA.
  {
    constexpr int NSTEP = 2 * NMT * (DV / 32);   // (mt, cc) x dt
    constexpr int PF = 4;
    bf16x8 a[NSTEP];
#pragma unroll
    for (int st = 0; st < PF; ++st) {
      const int q4 = st / (DV / 32), dt = st % (DV / 32);
      const char* p0 = vs + c.va[dt] + ((q4 >> 1) * 32 + (q4 & 1) * 16) * (DV * 2);
      a[st] = join(lds_read_tr16(p0), lds_read_tr16(p0 + 8 * (DV * 2)));
    }
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      if (st + PF < NSTEP) {
        const int q4 = (st + PF) / (DV / 32), dt = (st + PF) % (DV / 32);
        const char* p0 = vs + c.va[dt] + ((q4 >> 1) * 32 + (q4 & 1) * 16) * (DV * 2);
        a[st + PF] = join(lds_read_tr16(p0), lds_read_tr16(p0 + 8 * (DV * 2)));
      }
      const int q4 = st / (DV / 32), dt = st % (DV / 32);
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) o[nq][dt] = mfma32(a[st], pf[nq][q4 >> 1][q4 & 1], o[nq][dt]);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads PF steps ahead of their MFMA
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
  const int w = p.xcd_remap ? (x & 7) * p.per_xcd + (x >> 3) : x;
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
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.l32 = c.lane & 31;
  c.hl = c.lane >> 5;
  c.kbase = reinterpret_cast<const char*>(p.k + (int64_t)ck0 * p.k_st + (int64_t)h * p.k_sh);
  c.vbase = reinterpret_cast<const char*>(p.v + (int64_t)ck0 * p.v_st + (int64_t)h * p.v_sh);
  c.k_st_b = (int)(p.k_st * 2);
  c.v_st_b = (int)(p.v_st * 2);
  c.sk = sk;
  c.sq = sq;
  c.row0 = row0;
  c.kdst = c.wave * K_CHUNKS_PER_WAVE * 1024;
  c.vdst = c.wave * V_CHUNKS_PER_WAVE * 1024;
#pragma unroll
  for (int i = 0; i < K_CHUNKS_PER_WAVE; ++i) {
    const int pch = (c.wave * K_CHUNKS_PER_WAVE + i) * 64 + c.lane;
    const int row = pch / 24, pc = pch % 24;
    c.koff[i] = (uint32_t)(row * c.k_st_b + ((pc ^ row_swz(row)) * 16));
  }
#pragma unroll
  for (int i = 0; i < V_CHUNKS_PER_WAVE; ++i) {
    const int pch = (c.wave * V_CHUNKS_PER_WAVE + i) * 64 + c.lane;
    const int row = pch >> 4, pc = pch & 15;
    c.voff[i] = (uint32_t)(row * c.v_st_b + ((pc ^ ((row & 3) << 2)) * 16));
  }
  // K operand rows: lane reads row (mt*32 + l32), chunk (kk*2 + hl) stored at chunk ^ row_swz(row)
  // (row_swz(mt*32 + l32) == row_swz(l32)); for kk = 4g + u this is byte
  // row*384 + g*128 + (((2u + hl) ^ row_swz(l32)) * 16).
#pragma unroll
  for (int u = 0; u < 4; ++u) c.ka[u] = c.l32 * (DQK * 2) + (((2 * u + c.hl) ^ row_swz(c.l32)) * 16);
  // V^T operand: 16-lane group g reads rows k0..k0+3 (k0 = 4*hl + (r >> 2) + step offset) at
  // columns dt*32 + (g & 1)*16 + 4*(r & 3); row k0 & 3 == (r >> 2) & 3 fixes the swizzle per lane.
  {
    const int g = c.lane >> 4, r = c.lane & 15;
    const int krel = 4 * c.hl + (r >> 2);
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt) {
      const int dv = dt * 32 + (g & 1) * 16 + 4 * (r & 3);
      c.va[dt] = krel * (DV * 2) + (((dv >> 3) ^ ((krel & 3) << 2)) * 16) + (dv & 7) * 2;
    }
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
  if (blo < bhi) issue_block_load(c, blo, lds_k0, lds_v0);
  wait_vmem();
  __syncthreads();
  // Blocks [blo, jd) need no mask for any row of the tile: they hold no key past the sequence
  // end and, when causal, none past the bottom-right diagonal of the tile's first row.
  const int diag = sk - sq;  // bottom-right alignment offset
  int jd = sk / BN;
  if (causal) {
    const int x = row0 + diag - (BN - 1);
    jd = min(jd, x < 0 ? 0 : x / BN + 1);
  }
  const int jm = max(blo, min(jd, bhi));
  int j = blo;
  // Two unmasked blocks per trip so each stage is a distinct LDS object at compile time.
  for (; j + 1 < jm; j += 2) {
    issue_block_load(c, j + 1, lds_k1, lds_v1);
    compute_block<NQ, 2, false>(c, j, lds_k0, lds_v0, qf, m_run, l_run, o, p.scale_log2, causal);
    wait_vmem();
    __syncthreads();
    if (j + 2 < bhi) issue_block_load(c, j + 2, lds_k0, lds_v0);
    compute_block<NQ, 2, false>(c, j + 1, lds_k1, lds_v1, qf, m_run, l_run, o, p.scale_log2, causal);
    wait_vmem();
    __syncthreads();
  }
  // The rest (at most one unmasked block plus the diagonal and tail blocks), block j in stage 0
  // on entry. Per wave and block, only the leading 32-key tiles that hold a key visible to some
  // row of the wave are computed (0, 1 or 2; wave-uniform).
  const int qmax = row0 + c.wave * 32 * NQ + 32 * NQ - 1;  // largest local query row of the wave
  const int vis_end = min(sk, causal ? qmax + diag + 1 : sk);  // keys [0, vis_end) visible to the wave
  for (int st = 0; j < bhi; ++j, st ^= 1) {
    char* kcur = st ? lds_k1 : lds_k0;
    char* vcur = st ? lds_v1 : lds_v0;
    if (j + 1 < bhi) issue_block_load(c, j + 1, st ? lds_k0 : lds_k1, st ? lds_v0 : lds_v1);
    const int rem = vis_end - j * BN;
    // The one-tile body exists only for one query tile per wave (with two, a second copy of the
    // body does not fit the register file).
    if (rem > 32 || (NQ > 1 && rem > 0))
      compute_block<NQ, 2, true>(c, j, kcur, vcur, qf, m_run, l_run, o, p.scale_log2, causal);
    else if (NQ == 1 && rem > 0)
      compute_block<NQ, 1, true>(c, j, kcur, vcur, qf, m_run, l_run, o, p.scale_log2, causal);
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
