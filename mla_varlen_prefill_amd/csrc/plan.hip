// Varlen tile planner: one work-group turns cu_seqlens into the ordered list of query-tile work
// items the dense kernel consumes, on the device (no host synchronisation, capturable).
//
// Prior art: a GPU kernel that plans varying-length sequences through a fixed-size buffer and a
// helper that zeroes its counters (page "Mojo module mla", mla_prefill_plan_kernel,
// set_buffer_lengths_to_zero); a metadata call producing a fixed-size int32 task split before
// the attention call (page "SparseFlashMla", Description). The format is this library's own:
// items (b, m, n_blocks, kv_end), sequence by sequence (sequences with more key blocks first,
// ties by b) and within a sequence from its last query tile to its first (with a left window:
// n_blocks descending, then slot ascending), unused entries -1.
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

__device__ __forceinline__ Item slot_item(const PlanParams& p, int s) {
  Item it;
  it.b = s / p.mt;
  it.m = s - it.b * p.mt;
  it.cq0 = p.cu_q[it.b];
  it.ck0 = p.cu_k[it.b];
  const int sq = p.cu_q[it.b + 1] - it.cq0;
  const int sk = p.cu_k[it.b + 1] - it.ck0;
  it.sq = sq;
  it.sk = sk;
  it.valid = it.m * p.bm < sq;
  int kv_end = sk;
  if (p.causal) {
    const int i_last = min((it.m + 1) * p.bm, sq) - 1;
    kv_end = min(max(i_last + sk - sq + p.win_right + 1, 0), sk);
  }
  const int kv_start = p.win_left >= 0 ? min(max(it.m * p.bm + sk - sq - p.win_left, 0), sk) : 0;
  it.kv_end = kv_end;
  it.nb = kv_end <= kv_start ? 0 : (kv_end + p.bn - 1) / p.bn - kv_start / p.bn;
  return it;
}

// Entry i of the plan, and (for the dense kernel, when asked for) the sequence's row ranges.
__device__ __forceinline__ void write_item(const PlanParams& p, int i, const Item& it) {
  reinterpret_cast<int4*>(p.plan)[i] = make_int4(it.b, it.m, it.nb, it.kv_end);
  if (p.plan_ext != nullptr) reinterpret_cast<int4*>(p.plan_ext)[i] = make_int4(it.cq0, it.sq, it.ck0, it.sk);
}

}  // namespace

__global__ __launch_bounds__(1024) void plan_kernel(PlanParams p) {
  __shared__ uint32_t keys[kPlanSortCapacity];
  __shared__ int wave_tot[16];
  __shared__ int count_sh;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;  // 1024, or fewer for small plans (sorting path only)
  const int n_slots = p.batch * p.mt;
  if (p.counters != nullptr && tid < 8) p.counters[tid * 32] = 0;

  if (n_slots <= kPlanSortCapacity) {
    int P = 1;
    while (P < n_slots) P <<= 1;
    for (int s = tid; s < P; s += nthr) {
      uint32_t key = 0xFFFFFFFFu;
      if (s < n_slots) {
        const Item it = slot_item(p, s);
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
        write_item(p, i, slot_item(p, p.win_left < 0 ? kb * p.mt + (p.mt - 1 - (low - kb * p.mt)) : low));
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
