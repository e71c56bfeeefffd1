// Dense varlen MLA prefill forward for gfx950: O = softmax(Q K^T * scale + mask) V, with LSE.
//
// The operation and its conventions (K/V expanded to every head, q/k head 192 = 128 nope + 64
// rope, v head 128, cu_seqlens, causal for new tokens, unmasked context chunks that return the
// LSE) are those of page "FlashAttention backend for MLA prefill" (dispatch,
// run_prefill_new_tokens, run_prefill_context_chunk); the softmax is accumulated online in the
// manner the "Mojo module mla" page names as the Flash attention v2 algorithm.
//
// Work decomposition. A work item is one (query tile, head, key split); its work-group has 4
// waves. The query tile has BM = 128*NQ rows; wave w owns rows [w*32*NQ, (w+1)*32*NQ). Keys
// stream in blocks of BN = 64 through LDS, double-buffered, copied straight from global memory
// into LDS (no register staging). Per block and wave:
//   S^T (keys x queries) = K_blk (A, from LDS) * Q^T (B, registers)       32x32x16 bf16 MFMA
//   each lane owns one query column, so the row max needs one cross-half swap and the row sum
//   stays lane-local until the end;
//   O^T (dv x queries) += V_blk^T (A, LDS transposed reads) * P^T (B, the S^T registers
//   converted to bf16 in place, no data movement).
// The key order inside every 16-key MFMA step is the one the S^T accumulator layout gives each
// lane (keys {4h..4h+3, 8+4h..8+4h+3} for lane half h); the V^T operand is read in the same
// order with two ds_read_b64_tr_b16 of four consecutive keys each.
//
// Scheduling. The grid is persistent: as many work-groups as stay resident (two per CU at
// NQ = 1), each running work item after work item. Work items are dealt to the 8 XCDs by (head,
// split) unit, so every K/V row a unit reads stays in one XCD's L2, and listed inside an XCD
// longest first (the plan's order) within groups of units; an XCD's work-groups take positions
// of that list from a ticket counter, each shortly before starting the item. The item stream is
// pipelined: the last block of an item issues the copy of the next item's first key block and,
// as its own Q^T fragments die (after the S^T products), the loads of the next item's.
// The epilogue turns each wave's output tile around in LDS and writes whole row segments.
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

// A row's probabilities are taken against a reference logit (see compute_block); a block whose
// row sum would pass 2^64 is redone against its exact maximum (P stays far inside bf16 / fp32
// range, and O = sum P V inside fp32 range for any bf16 V).
constexpr float kOverflowSum = 18446744073709551616.f;  // 2^64

// Head dimensions (q/k head DQK, v head DV) and output type of a kernel instance. A work item
// computes DVT = 128 of the DV output columns (DVH = DV / DVT items per row tile and head, all
// computing the same scores): a wave's 32 x 256 fp32 output tile would not fit the registers
// beside its Q fragments.
template <int DQK_, int DV_, bool FP8_, int NW_ = (DQK_ == 256 ? 8 : 4)>
struct Shape {
  static constexpr int DQK = DQK_, DV = DV_;
  static constexpr int DVT = 128, DVH = DV / DVT;
  static constexpr bool FP8 = FP8_;                         // fp8 e4m3 output with a static scale
  // Waves per work-group (32 query rows each). The 256-wide layout needs all of a wave's
  // registers at two waves per SIMD and 96 KB of LDS per work-group, so its work-groups have
  // eight waves (one per CU). The others run two four-wave work-groups per CU, or one of eight
  // waves, whose 256-row tiles halve the key and value copies per query row: faster when items
  // see many keys, slower when they see few (a longer prologue and epilogue per key block).
  static constexpr int NW = NW_;
  // operand reads run PF MFMA steps ahead (fewer where registers are short)
  static constexpr int PF = DQK == 256 ? 3 : 6;
  // The next block's copies are issued one after each of the first S products (256-wide layout;
  // measured 8 % faster there) or all after the first one (the others: spreading them measured 6 %
  // slower on long sequences, where they hold scalar registers through the product loop).
  static constexpr bool SPREAD_COPIES = DQK == 256;
  static constexpr int K_STAGE_BYTES = BN * DQK * 2;
  static constexpr int V_STAGE_BYTES = BN * DVT * 2;
  static constexpr int KCH = BN * (DQK / 8) / (64 * NW);    // wave-wide 1 KiB copies per K block
  static constexpr int VCH = BN * (DVT / 8) / (64 * NW);
  // K operand addressing: the swizzle permutes 16-byte chunks inside groups of KA_GROUP bytes;
  // KA_N per-lane offsets cover one group's MFMA steps.
  static constexpr int KA_GROUP = DQK == 192 ? 128 : 256;
  static constexpr int KA_N = KA_GROUP / 32;
  // The epilogue turns each wave's 32 x DV output tile around in the wave's K copy region, one
  // row segment of EPI_SEG bytes at a time: 128-byte segments when the 4 KiB fit the region, else
  // 64-byte ones.
  static constexpr int EPI_SEG = KCH * 1024 >= 32 * 128 ? 128 : 64;
  static constexpr int EPI_BYTES = 32 * EPI_SEG;
  // The work ticket handed between waves sits past the epilogue area of the wave's K copy region
  // when it fits there, else at the start of the wave's V copy region (which the epilogue never uses).
  static constexpr bool TICKET_IN_K = EPI_BYTES + 4 <= KCH * 1024;
  static_assert((BN * DQK / 8) % (64 * NW) == 0 && (BN * DVT / 8) % (64 * NW) == 0 && DV % DVT == 0, "shape");
};

// K swizzle: chunk c of row r is stored at chunk c ^ kswz(r). 384-byte rows (an odd multiple of
// 128 bytes) use row_swz; rows that are a multiple of 256 bytes start on bank 0, and XOR-ing the
// low four bits with r & 15 gives the 16 rows of every operand read cycle 16 distinct 16-byte bank
// groups.
template <class S>
__device__ __forceinline__ int kswz(int r) {
  return S::DQK == 192 ? row_swz(r) : (r & 15);
}

// Per-lane constants of a work-group (the same for every work item it runs).
template <int NQ, class S>
struct DenseCtx {
  int lane, wave, l32, hl;
  int k_st_b, v_st_b;  // token strides in bytes (validated to keep 64-row offsets in 31 bits)
  uint32_t koff[S::KCH];  // byte offset of this lane's 16-byte chunk inside a block
  uint32_t voff[S::VCH];
  int kdst, vdst;                    // this wave's first 1 KiB slot in a stage (bytes)
  // LDS operand addresses (bytes, relative to a stage)
  int ka[S::KA_N];                   // K rows: + g*KA_GROUP + mt*32*DQK*2 per step group g
  int va[S::DVT / 32];               // V rows: + (mt*32 + cc*16 [+8]) * DVT*2 per step
};

// One work item (wave-uniform): the query tile of sequence b whose local row r is sequence row
// row0 + r (rows [rlo, rows) of the tile exist), head h, key blocks [blo, bhi).
// The item's head, key split and output column tile (columns [dvh * DVT, (dvh + 1) * DVT)) share
// one word: the item stream keeps two items live in scalar registers, where every extra word
// spills.
struct Item {
  const char* kbase;  // K of this sequence/head at key 0 (bytes)
  const char* vbase;
  int cq0, sq, sk, row0, rows, blo, bhi;
  int hsd;  // head (bits 0-15), split (16-22), dvh (23)
  __device__ int h() const { return hsd & 0xFFFF; }
  __device__ int split() const { return (hsd >> 16) & 0x7F; }
  __device__ int dvh() const { return (hsd >> 23) & 1; }
  __device__ int rlo() const { return max(0, -row0); }  // first local row of the sequence
};

// 32-bit value the optimiser must treat as opaque (keeps precomputed offsets 32-bit at their use
// and per-lane arithmetic from being hoisted into long-lived registers).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Copy i (of KCH + VCH wave-wide 1 KiB copies: K first, then V) of key block j of an item into
// a stage. Rows past the end of the sequence re-read its last key (finite values, masked later).
template <int NQ, class S>
__device__ __forceinline__ void issue_copy(const DenseCtx<NQ, S>& c, const Item& it, int j, char* kst, char* vst,
                                           int i) {
  const int key0 = j * BN;
  const bool is_k = i < S::KCH;
  const int ci = is_k ? i : i - S::KCH;
  const int st_b = is_k ? c.k_st_b : c.v_st_b;
  const char* base = (is_k ? it.kbase : it.vbase) + (int64_t)key0 * st_b;
  const uint32_t off = is_k ? c.koff[ci] : c.voff[ci];
  char* dst = is_k ? kst + c.kdst + ci * 1024 : vst + c.vdst + ci * 1024;
  if (key0 + BN <= it.sk) {
    g2lds16(base + opaque(off), dst);
  } else {
    const int lane = (int)opaque((uint32_t)c.lane);
    const int nch = is_k ? S::DQK / 8 : S::DVT / 8;  // 16-byte chunks per row
    const int r = (int)((uint32_t)((c.wave * (is_k ? S::KCH : S::VCH) + ci) * 64 + lane) / (uint32_t)nch);
    const int shift = (min(r, it.sk - 1 - key0) - r) * st_b;
    g2lds16(base + (uint32_t)((int)off + shift), dst);
  }
}

template <int NQ, class S>
__device__ __forceinline__ void issue_block_load(const DenseCtx<NQ, S>& c, const Item& it, int j, char* kst,
                                                 char* vst) {
  const int key0 = j * BN;
  const char* kb = it.kbase + (int64_t)key0 * c.k_st_b;
  const char* vb = it.vbase + (int64_t)key0 * c.v_st_b;
  if (key0 + BN <= it.sk) {
#pragma unroll
    for (int i = 0; i < S::KCH; ++i) g2lds16(kb + opaque(c.koff[i]), kst + c.kdst + i * 1024);
#pragma unroll
    for (int i = 0; i < S::VCH; ++i) g2lds16(vb + opaque(c.voff[i]), vst + c.vdst + i * 1024);
  } else {
    const int last = it.sk - 1 - key0;
    const int lane = (int)opaque((uint32_t)c.lane);
#pragma unroll
    for (int i = 0; i < S::KCH; ++i) {
      const int r = (int)((uint32_t)((c.wave * S::KCH + i) * 64 + lane) / (uint32_t)(S::DQK / 8));
      const int shift = (min(r, last) - r) * c.k_st_b;
      g2lds16(kb + (uint32_t)((int)c.koff[i] + shift), kst + c.kdst + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < S::VCH; ++i) {
      const int r = (int)((uint32_t)((c.wave * S::VCH + i) * 64 + lane) / (uint32_t)(S::DVT / 8));
      const int shift = (min(r, last) - r) * c.v_st_b;
      g2lds16(vb + (uint32_t)((int)c.voff[i] + shift), vst + c.vdst + i * 1024);
    }
  }
}

// NMT: how many of the block's two 32-key tiles this wave computes (2, or 1 when the second tile
// is entirely masked for every row of the wave; a wave with both tiles masked skips the block).
// q_done(kk) runs right after the last product that reads the Q^T fragments qf[.][kk]; copy(st)
// right after S product st.
// The kernel's arguments, re-read from the kernel-argument segment at each use: values needed
// only once per work item are loaded there instead of being held in scalar registers for the
// whole kernel (the optimiser cannot see through the empty asm, so it cannot hoist the loads).
__device__ __forceinline__ const DenseParams& kargs() {
  auto kp = (const __attribute__((address_space(4))) DenseParams*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  return *(const DenseParams*)kp;
}

template <int NQ, int NMT, bool MASK, class S, class QDone, class Copy>
__device__ __forceinline__ void compute_block(const DenseCtx<NQ, S>& c, const Item& it, int j,
                                              const char* ks, const char* vs,
                                              bf16x8 (&qf)[NQ][S::DQK / 16], float (&m_run)[NQ],
                                              float (&l_run)[NQ], f32x16 (&o)[NQ][S::DVT / 32],
                                              float scale_log2, bool causal, QDone&& q_done, Copy&& copy,
                                              bool live) {
  constexpr int DQK = S::DQK, DV = S::DVT, KA_N = S::KA_N, KA_GROUP = S::KA_GROUP;
  if (!live) {
    // The wave sees no key of this block: only the copies and the Q hand-over are issued.
#pragma unroll
    for (int st = 0; st < NMT * (DQK / 16); ++st) {
      copy(st);
      if (st % NMT == NMT - 1) q_done(st / NMT);
    }
    return;
  }
  // ---- S^T = K_blk * Q^T: the 32-key tiles are independent accumulator chains, issued
  // alternately, with the K fragments read from LDS PF steps ahead of their MFMA.
  f32x16 s[NQ][2];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) s[nq][0] = s[nq][1] = f32x16{};
  {
    constexpr int NSTEP = NMT * (DQK / 16);  // (kk, mt) steps
    constexpr int PF = S::PF;
    bf16x8 a[NSTEP];
#pragma unroll
    for (int st = 0; st < PF; ++st) {
      const int kk = st / NMT, mt = st % NMT;
      a[st] = lds_read_b128(ks + c.ka[kk % KA_N] + (kk / KA_N) * KA_GROUP + mt * 32 * (DQK * 2));
    }
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      if (st + PF < NSTEP) {
        const int kk2 = (st + PF) / NMT, mt2 = (st + PF) % NMT;
        a[st + PF] = lds_read_b128(ks + c.ka[kk2 % KA_N] + (kk2 / KA_N) * KA_GROUP + mt2 * 32 * (DQK * 2));
      }
      const int kk = st / NMT, mt = st % NMT;
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) s[nq][mt] = mfma32(a[st], qf[nq][kk], s[nq][mt]);
      copy(st);
      if (mt == NMT - 1) {
        __builtin_amdgcn_sched_barrier(0);  // the old fragments are read before q_done replaces them
        q_done(kk);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the read PF steps ahead of its MFMA
    }
  }
  if (NMT == 1) {
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[nq][1][i] = -INFINITY;
  }
  // ---- mask (diagonal, tail and left-window blocks only; wave-uniform test). Key j is visible
  // to local row i iff j < Sk, j <= i + diag (when right-limited: causal or a right window, whose
  // width is folded into diag) and j >= i + dleft (with a left window).
  const int key0 = j * BN;
  const int qmin = it.row0 + c.wave * 32 * NQ;  // smallest query row of this wave
  const int wl = kargs().win_left;
  const int diag = it.sk - it.sq + kargs().win_right;  // bottom-right alignment offset (+ right window)
  const int dleft = it.sk - it.sq - wl;
  const bool need_mask = MASK && ((key0 + BN > it.sk) || (causal && key0 + BN - 1 > qmin + diag) ||
                                  (wl >= 0 && key0 < qmin + 32 * NQ - 1 + dleft));
  if (need_mask) {
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      const int qrow = qmin + nq * 32 + c.l32;
      const int half = 4 * (int)(opaque(c.lane) >> 5);
      const int lim = (causal ? min(it.sk - 1, qrow + diag) : (it.sk - 1)) - key0 - half;
      const int lo = (wl >= 0 ? qrow + dleft : -(1 << 30)) - key0 - half;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kofs = mt * 32 + 8 * (i >> 2) + (i & 3);
          if (kofs > lim || kofs < lo) s[nq][mt][i] = -INFINITY;
        }
    }
  }
  // ---- softmax against a per-row reference logit (per lane = per query; lanes l and l^32 share
  // a query). A row's reference m_run is the largest logit of the first block in which it sees a
  // key, so the row maximum is only computed while some row of the wave has no reference yet. P =
  // 2^((s - m_run) * scale * log2 e) is summed in fp32 (before its rounding to bf16 for P.V, so
  // the LSE keeps fp32 accuracy on rows with few keys). A block whose running sum would pass 2^64
  // (a logit some 44 nats above the reference) is redone exactly: its maximum becomes the
  // reference and the accumulated O and l are rescaled.
  bf16x8 pf[NQ][2][2];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    auto block_max = [&]() {
      float mx = s[nq][0][0];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = (mt == 0 ? 1 : 0); i < 16; ++i) mx = fmaxf(mx, s[nq][mt][i]);
      return xhalf_max(mx);
    };
    auto exps = [&](float ref, float l0) {
      const float mc = ((ref == -INFINITY) ? 0.f : ref) * scale_log2;
      float rs = l0;
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
      return rs;
    };
    if (__ballot(m_run[nq] == -INFINITY) != 0ull) {
      const float mx = block_max();
      if (m_run[nq] == -INFINITY) m_run[nq] = mx;
    }
    float l_new = exps(m_run[nq], l_run[nq]);
    if (__ballot(!(l_new <= kOverflowSum)) != 0ull) {
      const float m_new = fmaxf(m_run[nq], block_max());
      const float alpha = (m_new == m_run[nq]) ? 1.f : fast_exp2((m_run[nq] - m_new) * scale_log2);
      l_run[nq] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DV / 32; ++dt) o[nq][dt] *= alpha;
      m_run[nq] = m_new;
      l_new = exps(m_run[nq], l_run[nq]);
    }
    l_run[nq] = l_new;
  }
  // ---- O^T += V_blk^T * P^T: the four dv tiles are independent chains; the transposed V reads
  // run PF steps ahead of their MFMA.
  {
    constexpr int NSTEP = 2 * NMT * (DV / 32);   // (mt, cc) x dt
    constexpr int PF = S::PF;
    bf16x8 a[NSTEP];
    // The wave issues these products at raised priority: the other wave on the SIMD, in its
    // softmax or S phase, then takes the issue slots the matrix core leaves (measured +2.5% on
    // long sequences; raising it for the S phase as well gained nothing).
    __builtin_amdgcn_s_setprio(1);
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
    __builtin_amdgcn_s_setprio(0);
  }
}

// One key block: compute block j of item it from the current stage and, optionally, copy block
// ld_j of item ld into the other stage (the copies issued together right after the first S
// product, which then runs while the copies queue: 1 % faster than before it; or spread over
// the S products). The stage pointers are restrict-qualified: the two stages never overlap, and saying so
// lets the compiler order the operand reads of the current stage freely against the copy in
// flight into the other one.
template <int NQ, int NMT, bool MASK, class S, class QDone>
__device__ __forceinline__ void block_step(const DenseCtx<NQ, S>& c, const Item& it, int j, const Item& ld,
                                           int ld_j, bool do_load, char* __restrict__ kn,
                                           char* __restrict__ vn, const char* __restrict__ kc,
                                           const char* __restrict__ vc, bf16x8 (&qf)[NQ][S::DQK / 16],
                                           float (&m_run)[NQ], float (&l_run)[NQ],
                                           f32x16 (&o)[NQ][S::DVT / 32], float scale_log2, bool causal,
                                           QDone&& q_done, bool live = true) {
  static_assert(!S::SPREAD_COPIES || S::KCH + S::VCH <= NMT * (S::DQK / 16), "one copy per S product");
  compute_block<NQ, NMT, MASK>(c, it, j, kc, vc, qf, m_run, l_run, o, scale_log2, causal, q_done, [&](int st) {
    if (S::SPREAD_COPIES && st < S::KCH + S::VCH && do_load) issue_copy(c, ld, ld_j, kn, vn, st);
    if (!S::SPREAD_COPIES && st == 0 && do_load) issue_block_load(c, ld, ld_j, kn, vn);
  }, live);
}

// Read-only metadata (plan, cu_seqlens, sink, item count) is read through the constant address
// space: those loads are scalar, so they never hold a vector-memory counter slot that the
// compiler would make a later block wait for, and their results are wave-uniform registers.
template <class T>
__device__ __forceinline__ T ld_const(const T* ptr, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)ptr)[i];
}

// Positions in the work list of XCD `xcd` (see decode_pos).
template <class S>
__device__ __forceinline__ int list_len(int n_items, int xcd) {
  const DenseParams& p = kargs();
  if (p.xcd_units > 0) return n_items * p.xcd_units;
  const int total = n_items * p.num_heads * p.num_splits * S::DVH;
  return total > xcd ? (total - xcd + 7) / 8 : 0;
}

// Decodes position i of the work list of XCD `xcd` (the positions are handed out by that XCD's
// ticket counter). Work items are (plan item, unit) pairs with units
// u = (h * num_splits + split) * DVH + dvh (the column tiles of a head and split are neighbours).
// When the units divide evenly over the XCDs, XCD k owns the contiguous units
// [k * units/8, (k+1) * units/8) (neighbouring heads, whose rows sit side by side in memory) and
// lists them in groups of group_units, group-major, then plan item (longest first), then unit
// within the group, except that the shortest eighth of the plan items comes last for all units
// together. Otherwise the lists interleave one global order of the same form: XCD k holds
// its positions t = 8*i + k. Returns false past the end of the list.
template <class S>
__device__ __forceinline__ bool decode_pos(int n_items, int xcd, int i, int& item, int& h, int& split, int& dvh) {
  const DenseParams& p = kargs();
  const int units = p.num_heads * p.num_splits * S::DVH;
  const int gu = p.group_units;
  int u;
  if (p.xcd_units > 0) {
    const int xu = p.xcd_units;
    const int n_x = n_items * xu;
    if (i < 0 || i >= n_x) return false;
    // The shortest eighth of the plan items (listed last by the planner) closes the list for all
    // of the XCD's units, item by item, so that the last work to start is short whichever unit
    // it belongs to; the rest goes group by group as above.
    const int n_long = n_items - n_items / 8;
    const int i_tail = n_long * xu;
    if (i >= i_tail) {
      const int r = i - i_tail;
      const int k = r / xu;
      item = n_long + k;
      u = xcd * xu + (r - k * xu);
    } else if (gu == 1) {  // one unit per group: no division by the group size
      const int grp = i / n_long;
      item = i - grp * n_long;
      u = xcd * xu + grp;
    } else {
      const int per_group = n_long * gu;
      const int grp = i / per_group;
      const int r = i - grp * per_group;
      item = r / gu;
      u = xcd * xu + grp * gu + (r - item * gu);
    }
  } else {
    const int total = n_items * units;
    const int n_x = total > xcd ? (total - xcd + 7) / 8 : 0;
    if (i < 0 || i >= n_x) return false;
    const int t = 8 * i + xcd;
    const int per_group = n_items * gu;
    const int grp = t / per_group;
    const int r = t - grp * per_group;
    item = r / gu;
    u = grp * gu + (r - item * gu);
  }
  const int hs = S::DVH == 1 ? u : u / S::DVH;
  dvh = u - hs * S::DVH;
  h = p.num_splits == 1 ? hs : hs / p.num_splits;
  split = hs - h * p.num_splits;
  return true;
}

template <int NQ, class S>
__device__ __forceinline__ Item make_item(int item, int h, int split, int dvh) {
  const DenseParams& p = kargs();
  Item it;
  // two independent loads: the plan entry and the sequence's row ranges the planner stored beside it
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 e = ld_const(reinterpret_cast<const i32x4*>(p.plan), item);
  const i32x4 f = ld_const(reinterpret_cast<const i32x4*>(p.plan_ext), item);
  const int m = e[1], nb = e[2];
  it.cq0 = f[0];
  it.sq = f[1];
  const int ck0 = f[2];
  it.sk = f[3];
  // Query tiles are aligned to the end of the sequence: tile m holds rows [m*BM - pad, (m+1)*BM -
  // pad) with pad = ceil(Sq/BM)*BM - Sq, so the leftover Sq mod BM rows form the first tile, whose
  // rows see the fewest keys under a causal mask.
  constexpr int bm = 32 * S::NW * NQ;
  it.row0 = m * bm - ((it.sq + bm - 1) / bm * bm - it.sq);
  it.rows = min(bm, it.sq - it.row0);
  // with a left window the item's blocks start at the block of the first key its first row sees
  const int blk0 =
      p.win_left >= 0 ? min(max(it.row0 + it.rlo() + it.sk - it.sq - p.win_left, 0), it.sk) / BN : 0;
  if (p.num_splits == 1) {  // (the common case: no 64-bit division)
    it.blo = blk0;
    it.bhi = blk0 + nb;
  } else {
    it.blo = blk0 + (int)(((int64_t)split * nb) / p.num_splits);
    it.bhi = blk0 + (int)(((int64_t)(split + 1) * nb) / p.num_splits);
  }
  it.hsd = h | (split << 16) | (dvh << 23);
  it.kbase = reinterpret_cast<const char*>(p.k + (int64_t)ck0 * p.k_st + (int64_t)h * p.k_sh);
  it.vbase = reinterpret_cast<const char*>(p.v + (int64_t)ck0 * p.v_st + (int64_t)h * p.v_sh + dvh * S::DVT);
  return it;
}

// Q^T fragments of this wave's query columns. Rows outside the sequence re-read its nearest row
// of the tile: their scores stay finite and their outputs are never stored, so no zeroing (and no
// wait) is needed.
template <int NQ, class S>
__device__ __forceinline__ void q_rows(const DenseCtx<NQ, S>& c, const Item& it, const __bf16* (&qp)[NQ]) {
  const DenseParams& p = kargs();
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const int lane = (int)opaque((uint32_t)c.lane);
    const int r = min(max(c.wave * 32 * NQ + nq * 32 + (lane & 31), it.rlo()), it.rows - 1);
    qp[nq] = p.q + (int64_t)(it.cq0 + it.row0 + r) * p.q_st + (int64_t)it.h() * p.q_sh + (lane >> 5) * 8;
  }
}

template <int NQ, class S>
__device__ __forceinline__ void load_q(const DenseCtx<NQ, S>& c, const Item& it, bf16x8 (&qf)[NQ][S::DQK / 16]) {
  const __bf16* qp[NQ];
  q_rows(c, it, qp);
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
    for (int kk = 0; kk < S::DQK / 16; ++kk) qf[nq][kk] = *reinterpret_cast<const bf16x8*>(qp[nq] + kk * 16);
}


// fp32 -> four OCP fp8 e4m3 bytes (round to nearest even), saturated at +-448 first so that no
// value overflows to NaN; byte i of the result encodes x[i].
__device__ __forceinline__ uint32_t pack_fp8x4(float x0, float x1, float x2, float x3) {
  auto sat = [](float x) { return fminf(fmaxf(x, -448.f), 448.f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat(x0), sat(x1), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat(x2), sat(x3), lo, true);
}

template <int NQ, class S>
__device__ __forceinline__ void store_item(const DenseCtx<NQ, S>& c, const Item& it, const float (&m_run)[NQ],
                                           const float (&l_run)[NQ], f32x16 (&o)[NQ][S::DVT / 32],
                                           char* stage) {
  constexpr int DV = S::DVT;  // the columns this item computes: [dvh * DVT, (dvh + 1) * DVT)
  constexpr int ESZ = S::FP8 ? 1 : 2;  // output element bytes
  // The arguments are read once, before any store (a store could otherwise be taken to change them).
  const DenseParams& p = kargs();
  const int h = it.h();
  const float scale = p.scale;
  float* const o_part = p.o_part;
  float* const lse_part = p.lse_part;
  // accumulate 1: merge into the running result held in o_part / lse_part; 2: merge with it and
  // write the final output (sink folded into the merged result) instead
  const bool accumulate = p.accumulate != 0;
  const bool final_merge = p.accumulate == 2;
  const bool to_part = o_part != nullptr && !final_merge;
  const int64_t part_row = (int64_t)it.split() * p.total_q;  // split-mode row base
  const int num_heads = p.num_heads;
  char* const out_h = static_cast<char*>(p.out) + ((int64_t)h * p.o_sh + it.dvh() * DV) * ESZ;
  // every column tile of a row computes the same LSE; the first one stores it (the running
  // merge of accumulate mode is used with a single tile only)
  const bool store_lse = it.dvh() == 0;
  const int64_t o_st_b = p.o_st * ESZ;
  float* const lse = p.lse;
  const int64_t l_st = p.l_st, l_sh = p.l_sh;
  const float sink_v = (p.sink != nullptr && o_part == nullptr) ? ld_const(p.sink, h) : -INFINITY;
  const float sink_f = (p.sink != nullptr && final_merge) ? ld_const(p.sink, h) : -INFINITY;
  // fp8 output: O / out_scale (multiplied by the reciprocal)
  const float q_mul = (S::FP8 && !to_part) ? 1.f / ld_const(p.out_scale, 0) : 1.f;
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const float l_tot = xhalf_sum(l_run[nq]);
    const int r = c.wave * 32 * NQ + nq * 32 + (int)(opaque((uint32_t)c.lane) & 31);
    float inv, lse_v;
    if (l_tot == 0.f) {
      inv = 0.f;
      lse_v = sink_v;  // -inf without a sink
    } else {
      const float mm = m_run[nq] * scale;  // natural-log units
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
    if (r >= it.rlo() && r < it.rows) {
      const int tok = it.cq0 + it.row0 + r;
      if (final_merge) {
        // the running result merged with this one, normalised, then the sink folded in; the
        // merged values replace the accumulators for the output path below
        const float* op = o_part + ((int64_t)tok * num_heads + h) * S::DV + it.dvh() * DV;
        const float l_old = lse_part[(int64_t)tok * num_heads + h];
        f32x4 old[DV / 32][4];
#pragma unroll
        for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) old[dt][g4] = *reinterpret_cast<const f32x4*>(op + dt * 32 + 8 * g4 + 4 * c.hl);
        float w_new = 0.f, w_old = 0.f, lse_m = -INFINITY;
        const float mx = fmaxf(l_old, lse_v);
        if (mx != -INFINITY) {
          const float eo = __expf(l_old - mx), en = __expf(lse_v - mx);
          const float rt = 1.f / (eo + en);
          w_old = eo * rt;
          w_new = inv * en * rt;
          lse_m = mx + __logf(eo + en);
        }
        float fin = 1.f;
        lse_v = lse_m;
        if (sink_f != -INFINITY) {
          const float ms = fmaxf(lse_m, sink_f);
          const float a = __expf(lse_m - ms);
          const float z = a + __expf(sink_f - ms);
          fin = a / z;
          lse_v = ms + __logf(z);
        }
#pragma unroll
        for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              o[nq][dt][g4 * 4 + e] = (o[nq][dt][g4 * 4 + e] * w_new + old[dt][g4][e] * w_old) * fin;
        inv = 1.f;
      }
      if (to_part) {
        float* op = o_part + ((part_row + tok) * num_heads + h) * S::DV + it.dvh() * DV;
        float* lp = lse_part + (part_row + tok) * num_heads + h;
        float w_new = inv, w_old = 0.f;
        f32x4 old[DV / 32][4];
        if (accumulate) {
          // merge with the running result of this row (read in full before any write):
          // LSE = log(e^L_old + e^L_new), O = (e^L_old O_old + e^L_new O_new) / e^LSE
          const float l_old = *lp;
#pragma unroll
          for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) old[dt][g4] = *reinterpret_cast<const f32x4*>(op + dt * 32 + 8 * g4 + 4 * c.hl);
          const float mx = fmaxf(l_old, lse_v);
          if (mx == -INFINITY) {
            w_new = 0.f;
          } else {
            const float eo = __expf(l_old - mx), en = __expf(lse_v - mx);
            const float rt = 1.f / (eo + en);
            w_old = eo * rt;
            w_new = inv * en * rt;
            lse_v = mx + __logf(eo + en);
          }
        }
#pragma unroll
        for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int dv = dt * 32 + 8 * g4 + 4 * c.hl;
            f32x4 v = {o[nq][dt][g4 * 4 + 0] * w_new, o[nq][dt][g4 * 4 + 1] * w_new,
                       o[nq][dt][g4 * 4 + 2] * w_new, o[nq][dt][g4 * 4 + 3] * w_new};
            if (accumulate) v += old[dt][g4] * w_old;
            *reinterpret_cast<f32x4*>(op + dv) = v;
          }
        if (c.hl == 0 && store_lse) *lp = lse_v;
      } else if (lse != nullptr && c.hl == 0 && store_lse) {
        lse[(int64_t)tok * l_st + (int64_t)h * l_sh] = lse_v;
      }
    }
    if (!to_part) {
      // Output through LDS: the lane layout holds pieces of 4 consecutive columns of a row, so the
      // tile is turned around in this wave's own copy region of a free stage, one row segment of
      // SEG bytes at a time (16-byte chunks XOR-swizzled by row), and written as whole segments.
      constexpr int SEG = S::EPI_SEG;
      constexpr int CPR = SEG / 16;      // 16-byte chunks per segment row
      constexpr int RPI = 64 / CPR;      // rows one wave-wide 16-byte access covers
      char* buf = stage + c.kdst;
      const int r0 = c.wave * 32 * NQ + nq * 32;  // first tile row of this 32-row slab
      // lane-derived addresses are computed here, not hoisted into long-lived registers
      const int lane = (int)opaque((uint32_t)c.lane), l32 = lane & 31, hl = lane >> 5;
      const int cc = lane & (CPR - 1);
      constexpr int SEG_DT = SEG / (32 * ESZ);  // 32-column MFMA tiles per segment
      const float w = inv * q_mul;
#pragma unroll
      for (int seg = 0; seg < DV / (32 * SEG_DT); ++seg) {
#pragma unroll
        for (int dd = 0; dd < SEG_DT; ++dd) {
          const int dt = seg * SEG_DT + dd;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            // columns dd*32 + 8*g4 + 4*hl .. +3 of the segment
            if (S::FP8) {
              const uint32_t v = pack_fp8x4(o[nq][dt][g4 * 4 + 0] * w, o[nq][dt][g4 * 4 + 1] * w,
                                            o[nq][dt][g4 * 4 + 2] * w, o[nq][dt][g4 * 4 + 3] * w);
              const int chunk = dd * 2 + (g4 >> 1);
              *reinterpret_cast<uint32_t*>(buf + l32 * SEG + ((chunk ^ (l32 & (CPR - 1))) * 16) + (g4 & 1) * 8 + hl * 4) = v;
            } else {
              const int chunk = dd * 4 + g4;
              u32x2 v = {pack_bf16x2(o[nq][dt][g4 * 4 + 0] * w, o[nq][dt][g4 * 4 + 1] * w),
                         pack_bf16x2(o[nq][dt][g4 * 4 + 2] * w, o[nq][dt][g4 * 4 + 3] * w)};
              *reinterpret_cast<u32x2*>(buf + l32 * SEG + ((chunk ^ (l32 & (CPR - 1))) * 16) + hl * 8) = v;
            }
          }
        }
        u32x4 v[32 / RPI];
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const int rr = i * RPI + lane / CPR;
          v[i] = *reinterpret_cast<const u32x4*>(buf + rr * SEG + ((cc ^ (rr & (CPR - 1))) * 16));
        }
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const int rr = i * RPI + lane / CPR;
          if (r0 + rr >= it.rlo() && r0 + rr < it.rows)
            *reinterpret_cast<u32x4*>(out_h + (int64_t)(it.cq0 + it.row0 + r0 + rr) * o_st_b + seg * SEG + cc * 16) = v[i];
        }
      }
    }
  }
}

}  // namespace

// Two four-wave work-groups per CU when their registers and LDS fit, else one work-group.
template <int NQ, class S>
constexpr int dense_occupancy() {
  return (NQ == 1 && S::NW == 4 && 2 * (S::K_STAGE_BYTES + S::V_STAGE_BYTES) <= 80 * 1024) ? 2 : 1;
}

template <int NQ, class S>
__global__ __launch_bounds__(64 * S::NW, (dense_occupancy<NQ, S>())) void dense_fwd_kernel(DenseParams p) {
  constexpr int DQK = S::DQK, DV = S::DVT, KCH = S::KCH, VCH = S::VCH;
  __shared__ __attribute__((aligned(1024))) char lds_k0[S::K_STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_v0[S::V_STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_k1[S::K_STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_v1[S::V_STAGE_BYTES];

  // Work-groups are dispatched to the XCDs round-robin (work-group x runs on XCD x % 8). The
  // work-groups of one XCD take the positions of its list from a ticket counter, each ticket
  // shortly before the item it names starts (about two key blocks ahead, to hide the atomic's
  // latency). The items in flight on an XCD thus always form a short window of its list, as in
  // the dispatch order of a non-persistent grid, and their K/V rows are shared in that XCD's L2.
  // When an XCD's list is used up, its work-groups go on with the other XCDs' lists in turn
  // (the XCDs do not run at quite the same speed; this evens out their finishing times).
  const int xcd = blockIdx.x & 7;
  const int n_items = min(ld_const(p.num_items, 0), p.n_slots);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto stage_k = [&](int s) { return s ? lds_k1 : lds_k0; };
  auto stage_v = [&](int s) { return s ? lds_v1 : lds_v0; };
  // Thread 0 hands a ticket to every wave through a stage that is free at that moment: one copy
  // in each wave's own copy region, which only that wave's next block copy overwrites (after the
  // wave has read it). In the K region the copy sits past the first EPI_BYTES, which the
  // epilogue of the previous item may still be using in that stage (a wave can still be turning
  // its output around there while thread 0 shares the ticket of the next item); the V region is
  // never used by the epilogue.
  auto ticket_slot = [&](int s, int w) -> char* {
    return S::TICKET_IN_K ? stage_k(s) + w * KCH * 1024 + S::EPI_BYTES : stage_v(s) + w * VCH * 1024;
  };
  auto share_ticket = [&](int sfree, int tk) -> int {
    if (threadIdx.x == 0) {
#pragma unroll
      for (int w = 0; w < S::NW; ++w) *reinterpret_cast<int*>(ticket_slot(sfree, w)) = tk;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*reinterpret_cast<const volatile int*>(ticket_slot(sfree, wave)));
  };
  int fetched = 0;
  int lst = xcd;  // the list tickets are taken from (one 128-byte counter line per list)
  auto fetch = [&] {
    // The zero offset the optimiser cannot see through keeps this a plain per-lane atomic: at a
    // provably uniform address it would be rewritten into a wave-level form that reads its result
    // at once, waiting for the round trip here instead of where the ticket is shared.
    if (threadIdx.x == 0) fetched = atomicAdd(p.counters + lst * 32 + (int)opaque(0u), 1);
  };
  int wi, wh, wsplit, wdvh;
  // Shares the fetched ticket (list in bits 28..30, position below) and decodes it. Past the end
  // of its list, thread 0 reads every list's counter (a hint: reading takes no ticket), takes a
  // ticket from the list with the most positions left and shares that, until one decodes or no
  // list has positions left. The barrier before a re-share lets every wave read the previous
  // ticket first.
  auto take = [&](int sfree) -> bool {
    int tk = share_ticket(sfree, fetched | (lst << 28));
    while (true) {
      lst = tk >> 28;
      if (decode_pos<S>(n_items, lst, tk & 0x0FFFFFFF, wi, wh, wsplit, wdvh)) return true;
      __syncthreads();
      if (threadIdx.x == 0) {
        int best = -1, best_left = 0;
        for (int l = 0; l < 8; ++l) {
          const int taken = __hip_atomic_load(p.counters + l * 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int left = list_len<S>(n_items, l) - taken;
          if (left > best_left) {
            best_left = left;
            best = l;
          }
        }
        fetched = best < 0 ? -1 : ((best << 28) | atomicAdd(p.counters + best * 32, 1));
      }
      tk = share_ticket(sfree, fetched);
      if (tk < 0) return false;
    }
  };
  fetch();
  if (!take(1)) return;

  DenseCtx<NQ, S> c;
  c.lane = threadIdx.x & 63;
  c.wave = wave;
  c.l32 = c.lane & 31;
  c.hl = c.lane >> 5;
  c.k_st_b = (int)(p.k_st * 2);
  c.v_st_b = (int)(p.v_st * 2);
  c.kdst = c.wave * KCH * 1024;
  c.vdst = c.wave * VCH * 1024;
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int pch = (c.wave * KCH + i) * 64 + c.lane;
    const int row = (int)((uint32_t)pch / (DQK / 8)), pc = (int)((uint32_t)pch % (DQK / 8));
    c.koff[i] = (uint32_t)(row * c.k_st_b + ((pc ^ kswz<S>(row)) * 16));
  }
#pragma unroll
  for (int i = 0; i < VCH; ++i) {
    const int pch = (c.wave * VCH + i) * 64 + c.lane;
    const int row = (int)((uint32_t)pch / (DV / 8)), pc = (int)((uint32_t)pch % (DV / 8));
    c.voff[i] = (uint32_t)(row * c.v_st_b + ((pc ^ ((row & 3) << 2)) * 16));
  }
  // K operand rows: lane reads row (mt*32 + l32), chunk (kk*2 + hl) stored at chunk ^ kswz(row)
  // (kswz(mt*32 + l32) == kswz(l32); the swizzle stays inside a KA_GROUP-byte group); for
  // kk = KA_N*g + u this is byte row*DQK*2 + g*KA_GROUP + (((2u + hl) ^ kswz(l32)) * 16).
#pragma unroll
  for (int u = 0; u < S::KA_N; ++u) c.ka[u] = c.l32 * (DQK * 2) + (((2 * u + c.hl) ^ kswz<S>(c.l32)) * 16);
  // V^T operand: 16-lane group gg reads rows k0..k0+3 (k0 = 4*hl + (r >> 2) + step offset) at
  // columns dt*32 + (gg & 1)*16 + 4*(r & 3); row k0 & 3 == (r >> 2) & 3 fixes the swizzle per lane.
  {
    const int gg = c.lane >> 4, r = c.lane & 15;
    const int krel = 4 * c.hl + (r >> 2);
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt) {
      const int dv = dt * 32 + (gg & 1) * 16 + 4 * (r & 3);
      c.va[dt] = krel * (DV * 2) + (((dv >> 3) ^ ((krel & 3) << 2)) * 16) + (dv & 7) * 2;
    }
  }
  const bool causal = p.causal != 0;

  bf16x8 qf[NQ][DQK / 16];
  float m_run[NQ], l_run[NQ];
  f32x16 o[NQ][DV / 32];
  int st = 0;  // stage holding the next block to compute

  auto new_item = [&]() { return make_item<NQ, S>(wi, wh, wsplit, wdvh); };
  Item cur = new_item();
  load_q(c, cur, qf);
  if (cur.blo < cur.bhi) issue_block_load(c, cur, cur.blo, stage_k(st), stage_v(st));
  wait_vmem();
  __syncthreads();

  while (true) {
    bool has_next = false;
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      m_run[nq] = -INFINITY;
      l_run[nq] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DV / 32; ++dt) o[nq][dt] = f32x16{};
    }
    const bool had_blocks = cur.blo < cur.bhi;
    // This wave's query rows [qlo, qlo + 32*NQ); a wave holding no row of the sequence (in the first
    // tile of a sequence whose length is not a multiple of the tile height) only copies.
    const int first = cur.row0 + cur.rlo();  // first sequence row of the tile
    const int qlo = cur.row0 + c.wave * 32 * NQ;
    const bool active = qlo + 32 * NQ > first && qlo < cur.row0 + cur.rows;
    // Hand-over to the next item: its ticket is fetched at the start of block fetch_j, shared at
    // the start of block share_j (where its descriptor is built), and the last block copies its
    // first key block and loads its Q^T fragments. Sharing waits for the ticket, so it comes at
    // least one block after the fetch whenever the item has two blocks or more. (Pulling the next
    // Q tile into L2 ahead of its loads measured slower than loading it cold.)
    const int fetch_j = max(cur.blo, cur.bhi - 4);
    const int share_j = cur.bhi - cur.blo >= 3 ? cur.bhi - 2 : cur.bhi - 1;
    Item nxt = cur;
    if (had_blocks) {
      // Blocks before jd need no mask for any row of the tile: they hold no key past the sequence
      // end and, when causal, none past the bottom-right diagonal of the tile's first row. The
      // last two blocks always run in the later loops, which prepare the hand-over.
      const int diag = cur.sk - cur.sq + p.win_right;
      int jd = cur.sk / BN;
      if (causal) {
        const int x = first + diag - (BN - 1);
        jd = min(jd, x < 0 ? 0 : x / BN + 1);
      }
      const int jm = max(cur.blo, min(jd, cur.bhi - 2));
      // Per wave, only the leading 32-key tiles holding a key visible to some row of the wave
      // are computed (0, 1 or 2; wave-uniform).
      const int qmax = qlo + 32 * NQ - 1;  // largest query row of this wave
      const int vis_end = !active ? 0 : min(cur.sk, causal ? qmax + diag + 1 : cur.sk);

      auto no_q = [](int) {};
      auto prepare = [&](int jj) {  // at the start of block jj, before its copy
        if (jj == fetch_j) fetch();
        if (jj == share_j) {
          has_next = take(st ^ 1);
          if (has_next) nxt = new_item();
        }
      };
      int j = cur.blo;
      // With a left window, the blocks holding a key below the window of the tile's last row need
      // the mask; they come first (at most up to the last block, which runs below).
      if (p.win_left >= 0 && active) {
        const int x = cur.row0 + cur.rows - 1 + cur.sk - cur.sq - p.win_left;  // last row's first key
        const int jl = min(x <= 0 ? 0 : (x + BN - 1) / BN, cur.bhi - 1);
        for (; j < jl; ++j, st ^= 1) {
          prepare(j);
          block_step<NQ, 2, true>(c, cur, j, cur, j + 1, true, stage_k(st ^ 1), stage_v(st ^ 1), stage_k(st),
                                  stage_v(st), qf, m_run, l_run, o, p.scale_log2, causal, no_q);
          wait_vmem();
          __syncthreads();
        }
      }
      // (an inactive wave runs every block but the last in the loop below, where it only copies:
      // the waves' barriers stay in step, as no ticket is shared before block jm)
      for (const int jm_w = active ? jm : j; j < jm_w; ++j, st ^= 1) {
        if (j == fetch_j) fetch();
        block_step<NQ, 2, false>(c, cur, j, cur, j + 1, true, stage_k(st ^ 1), stage_v(st ^ 1), stage_k(st),
                                 stage_v(st), qf, m_run, l_run, o, p.scale_log2, causal, no_q);
        wait_vmem();
        __syncthreads();
      }
      // The one-tile body exists only for one query tile per wave (with two, a second copy of the
      // body does not fit the register file). A wave with no visible key in the block only copies.
      for (; j < cur.bhi - 1; ++j, st ^= 1) {
        prepare(j);  // before jm, at most the fetch, as in the loop above
        const int rem = vis_end - j * BN;
        if (rem > 32 || (NQ > 1 && rem > 0))
          block_step<NQ, 2, true>(c, cur, j, cur, j + 1, true, stage_k(st ^ 1), stage_v(st ^ 1), stage_k(st), stage_v(st),
                                  qf, m_run, l_run, o, p.scale_log2, causal, no_q);
        else if (NQ == 1 && rem > 0)
          block_step<NQ, 1, true>(c, cur, j, cur, j + 1, true, stage_k(st ^ 1), stage_v(st ^ 1), stage_k(st), stage_v(st),
                                  qf, m_run, l_run, o, p.scale_log2, causal, no_q);
        else
          issue_block_load(c, cur, j + 1, stage_k(st ^ 1), stage_v(st ^ 1));
        wait_vmem();
        __syncthreads();
      }
      // Last block: hand over to the next item. Its first key block is copied into the other
      // stage, and each of its Q^T fragments is loaded as soon as the matching fragment of this
      // item has been read for the last time (without a next item, Q is simply re-read). It runs
      // the two-tile body (so that the new fragments have a single definition), or, for a wave
      // that sees no key of the block (the first rows of a causal tile), only the copies and loads.
      {
        prepare(j);
        const __bf16* qp[NQ];
        q_rows(c, nxt, qp);
        block_step<NQ, 2, true>(c, cur, j, nxt, nxt.blo, has_next && nxt.blo < nxt.bhi, stage_k(st ^ 1),
                                stage_v(st ^ 1), stage_k(st), stage_v(st), qf, m_run, l_run, o, p.scale_log2, causal,
                                [&](int kk) {
#pragma unroll
                                  for (int nq = 0; nq < NQ; ++nq)
                                    qf[nq][kk] = *reinterpret_cast<const bf16x8*>(qp[nq] + kk * 16);
                                }, vis_end > j * BN);
        wait_vmem();
        __syncthreads();
        st ^= 1;
      }
    } else {
      fetch();
      has_next = take(st ^ 1);
    }
    // Free stage for the epilogue: the one the last block read (the next item's first block sits
    // in the other), or, for an item without blocks, the one the next item will be copied into.
    store_item(c, cur, m_run, l_run, o, had_blocks ? stage_k(st ^ 1) : stage_k(st));
    if (!has_next) break;
    cur = had_blocks ? nxt : new_item();
    if (!had_blocks) {  // nothing was handed over: start the next item from scratch
      load_q(c, cur, qf);
      if (cur.blo < cur.bhi) issue_block_load(c, cur, cur.blo, stage_k(st), stage_v(st));
      wait_vmem();
      __syncthreads();
    }
  }
}

using Shape192 = Shape<192, 128, false>;
using Shape192F8 = Shape<192, 128, true>;
using Shape192W8 = Shape<192, 128, false, 8>;
using Shape192F8W8 = Shape<192, 128, true, 8>;
using Shape128 = Shape<128, 128, false>;
using Shape128F8 = Shape<128, 128, true>;
using Shape256 = Shape<256, 256, false>;
using Shape256F8 = Shape<256, 256, true>;

template __global__ void dense_fwd_kernel<1, Shape192>(DenseParams);
template __global__ void dense_fwd_kernel<1, Shape192F8>(DenseParams);
template __global__ void dense_fwd_kernel<1, Shape192W8>(DenseParams);
template __global__ void dense_fwd_kernel<1, Shape192F8W8>(DenseParams);
template __global__ void dense_fwd_kernel<1, Shape128>(DenseParams);
template __global__ void dense_fwd_kernel<1, Shape128F8>(DenseParams);
template __global__ void dense_fwd_kernel<1, Shape256>(DenseParams);
template __global__ void dense_fwd_kernel<1, Shape256F8>(DenseParams);

template <int NQ, class S>
static void launch_one(const DenseParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((dense_fwd_kernel<NQ, S>), dim3(grid), dim3(64 * S::NW), 0, stream, p);
}

bool dense_waves_ok(int nw, int dqk, int dv) {
  if (dqk == 192 && dv == 128) return nw == 4 || nw == 8;
  if (dqk == 128 && dv == 128) return nw == Shape128::NW;
  if (dqk == 256 && dv == 256) return nw == Shape256::NW;
  return false;
}

int dense_default_waves(int dqk, int dv) {
  if (dqk == 256 && dv == 256) return Shape256::NW;
  if (dqk == 128 && dv == 128) return Shape128::NW;
  return Shape192::NW;
}

int dense_occupancy_of(int nw, int dqk, int dv) {
  if (dqk == 256 && dv == 256) return dense_occupancy<1, Shape256>();
  if (dqk == 128 && dv == 128) return dense_occupancy<1, Shape128>();
  return nw == 8 ? dense_occupancy<1, Shape192W8>() : dense_occupancy<1, Shape192>();
}

int dense_rows_per_tile(int nw, int dqk, int dv) { return dense_waves_ok(nw, dqk, dv) ? 32 * nw : 0; }

hipError_t launch_dense_fwd(const DenseParams& p, int nw, int dqk, int dv, bool fp8_out, hipStream_t stream) {
  const int grid = 8 * p.wgs_per_xcd;
  if (!dense_waves_ok(nw, dqk, dv)) return hipErrorInvalidValue;
  if (grid <= 0) return hipSuccess;
  if (dqk == 192 && dv == 128) {
    if (nw == 8) {
      if (fp8_out) launch_one<1, Shape192F8W8>(p, grid, stream);
      else launch_one<1, Shape192W8>(p, grid, stream);
    } else {
      if (fp8_out) launch_one<1, Shape192F8>(p, grid, stream);
      else launch_one<1, Shape192>(p, grid, stream);
    }
  } else if (dqk == 128 && dv == 128) {
    if (fp8_out) launch_one<1, Shape128F8>(p, grid, stream);
    else launch_one<1, Shape128>(p, grid, stream);
  } else {
    if (fp8_out) launch_one<1, Shape256F8>(p, grid, stream);
    else launch_one<1, Shape256>(p, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace mla
