// Varlen tile planner: one work-group turns cu_seqlens into the ordered list of query-tile work
// items the dense kernel consumes, on the device (no host synchronisation, capturable).
//
// Prior art: a device-side planner for ragged batches with a counter-clearing helper (page "Mojo
// module mla", mla_prefill_plan_kernel, set_buffer_lengths_to_zero); a metadata call that fills
// an int32 task table before the attention operator (page "SparseFlashMla", Description). The
// format is this library's own: items (b, m, n_blocks, kv_end) for query tiles aligned to the end
// of each sequence (tile m holds rows [m*BM - pad, (m+1)*BM - pad), pad = ceil(Sq/BM)*BM - Sq, so
// the Sq mod BM leftover rows form tile 0, where causal rows see the fewest keys), sequence by
// sequence (sequences with more key blocks first, ties by b) and within a sequence from its last
// query tile to its first (with a left window: n_blocks descending, then slot ascending), unused
// entries -1.
// With a left window n_blocks counts from the block of the first key the tile's first row sees
// (the dense kernel recomputes that block). Long work goes first, and the tiles in flight at
// any time come from few sequences, whose keys and values then stay in L2.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

struct Item {
  int b, m, nb, kv_end;
  int cq0, sq, ck0, sk;
  bool valid;
};

// Item (b, m) of a sequence with rows [cq0, cq0 + sq) and keys [ck0, ck0 + sk).
__device__ __forceinline__ Item plan_item(const PlanParams& p, int b, int m, int cq0, int sq, int ck0, int sk) {
  Item it;
  it.b = b;
  it.m = m;
  it.cq0 = cq0;
  it.ck0 = ck0;
  it.sq = sq;
  it.sk = sk;
  // tile m holds rows [row0, row0 + bm) of the sequence that exist: tiles end at the sequence end
  const int n_tiles = (sq + p.bm - 1) / p.bm;
  const int row0 = it.m * p.bm - (n_tiles * p.bm - sq);
  it.valid = it.m < n_tiles;
  int kv_end = sk;
  if (p.causal) {
    const int i_last = row0 + p.bm - 1;
    kv_end = min(max(i_last + sk - sq + p.win_right + 1, 0), sk);
  }
  const int kv_start = p.win_left >= 0 ? min(max(max(row0, 0) + sk - sq - p.win_left, 0), sk) : 0;
  it.kv_end = kv_end;
  it.nb = kv_end <= kv_start ? 0 : (kv_end + p.bn - 1) / p.bn - kv_start / p.bn;
  return it;
}

__device__ __forceinline__ Item slot_item(const PlanParams& p, int s) {
  const int b = s / p.mt;
  const int cq0 = p.cu_q[b], ck0 = p.cu_k[b];
  return plan_item(p, b, s - b * p.mt, cq0, p.cu_q[b + 1] - cq0, ck0, p.cu_k[b + 1] - ck0);
}

// Entry i of the plan, and (for the dense kernel, when asked for) the sequence's row ranges.
__device__ __forceinline__ void write_item(const PlanParams& p, int i, const Item& it) {
  reinterpret_cast<int4*>(p.plan)[i] = make_int4(it.b, it.m, it.nb, it.kv_end);
  if (p.plan_ext != nullptr) reinterpret_cast<int4*>(p.plan_ext)[i] = make_int4(it.cq0, it.sq, it.ck0, it.sk);
}

}  // namespace

// Plans of up to this many (padded) slots keep every slot's item in LDS between the sort and the
// write-out, so cu_seqlens is read once.
constexpr int kPlanSmall = 1024;

__global__ __launch_bounds__(1024) void plan_kernel(PlanParams p) {
  __shared__ uint32_t keys[kPlanSortCapacity];
  __shared__ int4 slot_e[kPlanSmall], slot_f[kPlanSmall];
  __shared__ int wave_tot[16];
  __shared__ int count_sh;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;  // 1024, or fewer for small plans (sorting path only)
  const int n_slots = p.batch * p.mt;
  if (p.counters != nullptr && tid < 8) p.counters[tid * 32] = 0;

  if (p.win_left < 0 && n_slots <= kPlanSortCapacity && p.batch <= kPlanSmall) {
    // Without a left window the order depends on the sequences alone (more key blocks first, ties
    // by b; each sequence from its last tile to its first): sort the B sequences, then place each
    // sequence's tiles after those of the sequences before it. The same plan as sorting every
    // slot, from log2(B) instead of log2(B * Mt) sort rounds.
    const int B = p.batch;
    int PB = 1;
    while (PB < B) PB <<= 1;
    for (int b = tid; b < PB; b += nthr) {
      uint32_t key = 0xFFFFFFFFu;
      if (b < B) {
        const int cq0 = p.cu_q[b], ck0 = p.cu_k[b];
        const int sq = p.cu_q[b + 1] - cq0, sk = p.cu_k[b + 1] - ck0;
        slot_e[b] = make_int4(cq0, sq, ck0, sk);
        const uint32_t nbs = (uint32_t)min((sk + p.bn - 1) / p.bn, kPlanMaxBlocks);
        key = ((uint32_t)(kPlanMaxBlocks - nbs) << 14) | (uint32_t)b;
      }
      keys[b] = key;
    }
    __syncthreads();
    for (int k = 2; k <= PB; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < PB; i += nthr) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint32_t a = keys[i], c = keys[ixj];
            const bool up = (i & k) == 0;
            if ((a > c) == up) {
              keys[i] = c;
              keys[ixj] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    // inclusive prefix sums of the tile counts in sorted order (one sequence per thread)
    int* pre = reinterpret_cast<int*>(slot_f);
    for (int q = tid; q < PB; q += nthr) {
      int nt = 0;
      if (q < B) nt = min((slot_e[keys[q] & 0x3FFFu].y + p.bm - 1) / p.bm, p.mt);  // slots m < Mt
      pre[q] = nt;
    }
    __syncthreads();
    for (int off = 1; off < PB; off <<= 1) {
      int v[kPlanSmall / 64];
      int n = 0;
      for (int q = tid; q < PB; q += nthr) v[n++] = q >= off ? pre[q - off] : 0;
      __syncthreads();
      n = 0;
      for (int q = tid; q < PB; q += nthr) pre[q] += v[n++];
      __syncthreads();
    }
    const int count = pre[B - 1];
    for (int i = tid; i < p.capacity; i += nthr) {
      if (i < count) {
        int lo = 0, hi = B - 1;  // the first sorted sequence whose tiles reach past i
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (pre[mid] > i) hi = mid; else lo = mid + 1;
        }
        const int b = (int)(keys[lo] & 0x3FFFu);
        const int4 e = slot_e[b];
        const int nt = min((e.y + p.bm - 1) / p.bm, p.mt);
        const int t = i - (lo > 0 ? pre[lo - 1] : 0);
        write_item(p, i, plan_item(p, b, nt - 1 - t, e.x, e.y, e.z, e.w));
      } else {
        reinterpret_cast<int4*>(p.plan)[i] = make_int4(-1, -1, -1, -1);
      }
    }
    if (tid == 0) *p.num_items = count;
  } else if (n_slots <= kPlanSortCapacity) {
    int P = 1;
    while (P < n_slots) P <<= 1;
    const bool small = P <= kPlanSmall;
    for (int s = tid; s < P; s += nthr) {
      uint32_t key = 0xFFFFFFFFu;
      if (s < n_slots) {
        const Item it = slot_item(p, s);
        if (small) {
          slot_e[s] = make_int4(it.b, it.m, it.nb, it.kv_end);
          slot_f[s] = make_int4(it.cq0, it.sq, it.ck0, it.sk);
        }
        if (it.valid) {
          if (p.win_left < 0) {
            // sequences with more key blocks first (ties by b), each from its last tile to its first
            const uint32_t nbs = (uint32_t)min((it.sk + p.bn - 1) / p.bn, kPlanMaxBlocks);
            key = ((uint32_t)(kPlanMaxBlocks - nbs) << 14) | (uint32_t)(it.b * p.mt + (p.mt - 1 - it.m));
          } else {
            // with a left window: longest item first, ties by slot
            const uint32_t nb = (uint32_t)min(it.nb, kPlanMaxBlocks);
            key = ((uint32_t)(kPlanMaxBlocks - nb) << 14) | (uint32_t)s;
          }
        }
      }
      keys[s] = key;
    }
    if (tid == 0) count_sh = 0;
    __syncthreads();
    // bitonic sort, ascending: longest first, ties by slot; invalid (all ones) last
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P; i += nthr) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint32_t a = keys[i], c = keys[ixj];
            const bool up = (i & k) == 0;
            if ((a > c) == up) {
              keys[i] = c;
              keys[ixj] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < P; i += nthr) {
      const bool v = keys[i] != 0xFFFFFFFFu;
      const bool next_v = (i + 1 < P) && keys[i + 1] != 0xFFFFFFFFu;
      if (v && !next_v) count_sh = i + 1;  // the single last valid entry
    }
    __syncthreads();
    const int count = count_sh;
    for (int i = tid; i < p.capacity; i += nthr) {
      if (i < count) {
        const int low = (int)(keys[i] & 0x3FFFu);  // b * Mt + (Mt - 1 - m), or the slot with a left window
        const int kb = low / p.mt;
        const int slot = p.win_left < 0 ? kb * p.mt + (p.mt - 1 - (low - kb * p.mt)) : low;
        if (small) {
          reinterpret_cast<int4*>(p.plan)[i] = slot_e[slot];
          if (p.plan_ext != nullptr) reinterpret_cast<int4*>(p.plan_ext)[i] = slot_f[slot];
        } else {
          write_item(p, i, slot_item(p, slot));
        }
      } else {
        reinterpret_cast<int4*>(p.plan)[i] = make_int4(-1, -1, -1, -1);
      }
    }
    if (tid == 0) *p.num_items = count;
  } else {
    // Too many slots to sort in LDS: compact the items in slot order.
    const int lane = tid & 63, wave = tid >> 6;
    int base = 0;
    for (int s0 = 0; s0 < n_slots; s0 += 1024) {
      const int s = s0 + tid;
      Item it;
      it.valid = false;
      if (s < n_slots) it = slot_item(p, s);
      const uint64_t mask = __ballot(it.valid);
      const int pre = __popcll(mask & ((1ull << lane) - 1ull));
      if (lane == 0) wave_tot[wave] = __popcll(mask);
      __syncthreads();
      int off = base, tot = 0;
      for (int wv = 0; wv < 16; ++wv) {
        if (wv < wave) off += wave_tot[wv];
        tot += wave_tot[wv];
      }
      if (it.valid) write_item(p, off + pre, it);
      base += tot;
      __syncthreads();
    }
    for (int i = base + tid; i < p.capacity; i += 1024)
      reinterpret_cast<int4*>(p.plan)[i] = make_int4(-1, -1, -1, -1);
    if (tid == 0) *p.num_items = base;
  }
}

hipError_t launch_plan(const PlanParams& p, hipStream_t stream) {
  // A plan of up to 1024 slots is sorted by as many threads as its padded size (at least one
  // wave, and at least the 8 that clear the ticket counters): fewer waves to synchronise.
  const int64_t n_slots = (int64_t)p.batch * p.mt;
  int threads = 1024;
  if (n_slots <= 1024) {
    threads = 64;
    while (threads < n_slots) threads <<= 1;
  }
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
