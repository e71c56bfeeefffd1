// C-ABI host layer of libmla_prefill.so: argument validation, workspace layout, the split-KV
// heuristic and kernel launches on the caller's stream. No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/mla_prefill.h"
#include "kernels.h"

namespace {

constexpr int kAbiVersion = 2;
constexpr int kDenseBN = 64;
constexpr int kDenseDqk = 192;
constexpr int kDenseDv = 128;
constexpr int kSparseDqk = 576;
constexpr int kSparseDv = 512;
constexpr int kMaxSplits = 64;
constexpr int kMaxDevices = 64;

struct DeviceInfo {
  int cus = 0;
  bool gfx950 = false;
  bool ok = false;
};

DeviceInfo g_dev[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

const DeviceInfo* device_info() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_dev_once[dev], [dev]() {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
    g_dev[dev].cus = prop.multiProcessorCount;
    g_dev[dev].gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev[dev].ok = true;
  });
  return g_dev[dev].ok ? &g_dev[dev] : nullptr;
}

// ---- scratch of the allocation-free dense entry point ---------------------------------------
// The plan, the ticket counters and the split partials of one mla_prefill_varlen_noalloc call
// live in this array instead of a caller workspace. Every GPU the library runs on holds its own
// copy from module load until the process ends; host code never uses the array's name as an
// address (it is a host-side stand-in), only the device address resolved below.
constexpr size_t kNoAllocScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

void* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of the current device's copy of `scratch`, resolved once per device with that
// device current; null if the device cannot be queried or the lookup failed.
void* scratch_device_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = p;
  });
  return g_scratch_ptr[dev];
}

// ---- launch timing (measurement aid) ------------------------------------------------------
constexpr int kNumKernels = 5;
constexpr size_t kMaxPending = 65536;

struct Profiler {
  std::mutex mu;
  std::atomic<bool> enabled{false};
  std::atomic<uint32_t> kinds{0xFFFFFFFFu};  // bit k: time kernel kind k
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Rec> pending;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  double total_ms[kNumKernels] = {};
  int64_t count[kNumKernels] = {};
};
Profiler g_prof;

// Launch `fn` (which enqueues one kernel on `stream`), bracketed by timing events when enabled.
template <typename F>
hipError_t timed_launch(int kind, hipStream_t stream, F&& fn) {
  if (!g_prof.enabled.load(std::memory_order_relaxed) || ((g_prof.kinds.load(std::memory_order_relaxed) >> kind) & 1u) == 0)
    return fn();
  std::pair<hipEvent_t, hipEvent_t> ev{nullptr, nullptr};
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.pending.size() >= kMaxPending) return fn();
    if (!g_prof.pool.empty()) {
      ev = g_prof.pool.back();
      g_prof.pool.pop_back();
    }
  }
  if (ev.first == nullptr) {
    if (hipEventCreate(&ev.first) != hipSuccess || hipEventCreate(&ev.second) != hipSuccess) return fn();
  }
  if (hipEventRecord(ev.first, stream) != hipSuccess) return fn();
  const hipError_t e = fn();
  if (e != hipSuccess) return e;
  if (hipEventRecord(ev.second, stream) != hipSuccess) return hipErrorUnknown;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.pending.push_back({kind, ev.first, ev.second});
  return hipSuccess;
}

// Query rows per dense work-group of the default (four-wave) instances.
int dense_bm() { return 128; }

// Head dimensions the dense kernels are built for: (q/k head, v head) = (192, 128), the default
// MLA layout 128 nope + 64 rope with v 128, and the other layouts (64 + 64, v 128) = (128, 128),
// (192 + 64, v 256) and (256 + 0, v 256) = (256, 256).
bool dense_dims_ok(int dqk, int dv) {
  return (dqk == 192 && dv == 128) || (dqk == 128 && dv == 128) || (dqk == 256 && dv == 256);
}

// Instance of a dense call: waves per work-group, resident work-groups per CU and tile height.
// The (192, 128) layout takes eight waves (256-row tiles) when a tile's rows see many keys: with
// at least 256 query rows in some sequence and at least 2048 keys (8192 under the causal mask,
// where a taller tile also computes a larger triangle of masked scores). Measured against four
// waves: 2-3% faster without the mask at 2048-4096 keys, 1.6% faster at 16384 causal, even at
// 4096-8192 causal, 1.5% slower on causal batches of 2048-token sequences. MLA_DENSE_WAVES (4 or
// 8) overrides the choice.
struct DenseShape {
  int dqk, dv, nw, occ, bm;
  bool fp8;
};
DenseShape with_waves(DenseShape d, int nw) {
  d.nw = nw;
  d.occ = mla::dense_occupancy_of(nw, d.dqk, d.dv);
  d.bm = mla::dense_rows_per_tile(nw, d.dqk, d.dv);
  return d;
}
DenseShape dense_shape(int dqk, int dv, bool fp8, int32_t max_q, int32_t max_k, bool causal) {
  DenseShape d{dqk, dv, mla::dense_default_waves(dqk, dv), 1, 128, fp8};
  if (dqk == 192 && dv == 128) {
    static const int forced = []() {
      const char* e = std::getenv("MLA_DENSE_WAVES");
      return e != nullptr ? std::atoi(e) : 0;
    }();
    const bool tall = max_q >= 256 && max_k >= (causal ? 8192 : 2048);
    d.nw = (forced == 4 || forced == 8) ? forced : (tall ? 8 : 4);
  }
  return with_waves(d, d.nw);
}

// Dense scheduling groups: each XCD works through `n` (head, split) units at a time (longest
// item first within a group). MLA_DENSE_GROUP overrides the default.
int dense_group_per_xcd() {
  static int n = []() {
    const char* e = std::getenv("MLA_DENSE_GROUP");
    const int v = e != nullptr ? std::atoi(e) : 0;
    return v > 0 ? v : 1;
  }();
  return n;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// MLA_VALIDATE (nonzero): check cu_seqlens contents on the host before launching (synchronises).
bool validate_inputs() {
  const char* e = std::getenv("MLA_VALIDATE");
  return e != nullptr && std::atoi(e) != 0;
}

// cu [batch + 1] starts at 0 and is non-decreasing with lengths <= max_len; its last entry equals
// `last` (exact) or is at most `last` (!exact); last < 0: not checked.
mla_status_t check_cu(const int32_t* cu, int32_t batch, int64_t last, bool exact, int32_t max_len,
                      hipStream_t stream) {
  std::vector<int32_t> h((size_t)batch + 1);
  if (hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MLA_ERR_HIP;
  if (h[0] != 0) return MLA_ERR_INVALID_ARG;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t len = (int64_t)h[b + 1] - h[b];
    if (len < 0 || len > max_len) return MLA_ERR_INVALID_ARG;
  }
  if (last >= 0 && (exact ? h[batch] != last : h[batch] > last)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}
inline bool stride_ok(int64_t s) { return s >= 0 && (s & 7) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct VarlenLayout {
  int32_t bm, mt, n_slots, splits;
  int32_t wgs_per_xcd;  // persistent dense grid: 8 * wgs_per_xcd work-groups
  size_t off_count, off_tickets, off_plan, off_plan_ext, off_opart, off_lpart, total;
};

int32_t resolve_splits(int32_t batch, int32_t max_q, int32_t max_k, int32_t heads,
                       int32_t num_splits, const DenseShape& ds) {
  if (num_splits >= 1) return num_splits;
  // Heuristic (our own; the pages name a num_splits_heuristic over M-blocks and SM count): split
  // the keys only when the (tile, head) work items cannot fill every CU with its resident
  // work-groups, and keep at least four key blocks per split.
  const DeviceInfo* di = device_info();
  const int cus = (di != nullptr && di->cus > 0) ? di->cus : 256;
  const int64_t conc = (int64_t)cus * ds.occ;
  const int64_t items = (int64_t)batch * cdiv(max_q, ds.bm) * heads;
  if (items <= 0 || items >= conc) return 1;
  const int64_t max_blocks = cdiv(max_k, kDenseBN);
  int64_t s = cdiv(conc, items);
  s = std::min<int64_t>(s, std::max<int64_t>(1, max_blocks / 4));
  s = std::min<int64_t>(s, kMaxSplits);
  return (int32_t)std::max<int64_t>(1, s);
}

VarlenLayout varlen_layout(int32_t batch, int32_t total_q, int32_t max_q, int32_t max_k,
                           int32_t heads, int32_t num_splits, const DenseShape& ds) {
  VarlenLayout L{};
  L.bm = ds.bm;
  L.mt = (int32_t)cdiv(std::max(max_q, 0), L.bm);
  L.n_slots = batch * L.mt;
  L.splits = resolve_splits(batch, max_q, max_k, heads, num_splits, ds);
  {
    // Persistent dense grid: every resident work-group slot, but no more work-groups than work
    // items.
    const DeviceInfo* di = device_info();
    const int cus = (di != nullptr && di->cus > 0) ? di->cus : 256;
    const int occ = ds.occ;
    const int64_t max_work = (int64_t)L.n_slots * heads * L.splits * (ds.dv / 128);
    const int64_t per_xcd = std::max<int64_t>(1, (int64_t)(cus / 8) * occ);
    int64_t want = per_xcd;
    if (const char* e = std::getenv("MLA_DENSE_WGS_PER_XCD")) want = std::max(1, std::atoi(e));
    L.wgs_per_xcd = (int32_t)std::max<int64_t>(1, std::min<int64_t>(want, cdiv(max_work, 8)));
  }
  L.off_count = 0;
  L.off_tickets = 256;  // 8 per-XCD ticket counters, one 128-byte line each, zeroed by the plan kernel
  L.off_plan = L.off_tickets + 8 * 128;
  L.off_plan_ext = align256(L.off_plan + (size_t)L.n_slots * 16);
  size_t off = align256(L.off_plan_ext + (size_t)L.n_slots * 16);
  L.off_opart = off;
  L.off_lpart = off;
  if (L.splits > 1) {
    L.off_opart = off;
    off = align256(off + (size_t)L.splits * total_q * heads * ds.dv * sizeof(float));
    L.off_lpart = off;
    off = align256(off + (size_t)L.splits * total_q * heads * sizeof(float));
  }
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_ALIGNMENT: return "MLA_ERR_ALIGNMENT";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
  }
}

int32_t mla_abi_version(void) { return kAbiVersion; }

void mla_dense_tile_shape(int32_t* block_m, int32_t* block_n) {
  if (block_m != nullptr) *block_m = dense_bm();
  if (block_n != nullptr) *block_n = kDenseBN;
}

mla_status_t mla_prefill_plan(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t batch, int32_t max_seqlen_q, int32_t block_m,
                              int32_t block_n, int32_t causal, int32_t window_left,
                              int32_t window_right, int32_t* plan, int32_t plan_capacity,
                              int32_t* num_items, void* hip_stream) {
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr || plan == nullptr || num_items == nullptr)
    return MLA_ERR_INVALID_ARG;
  auto pow2 = [](int32_t x) { return x >= 16 && x <= 1024 && (x & (x - 1)) == 0; };
  if (batch < 0 || max_seqlen_q < 0 || !pow2(block_m) || !pow2(block_n) || plan_capacity < 0 ||
      window_left < -1 || window_right < -1)
    return MLA_ERR_INVALID_ARG;
  const int32_t right = causal ? 0 : window_right;
  const int64_t mt = cdiv(max_seqlen_q, block_m);
  if ((int64_t)batch * mt > plan_capacity) return MLA_ERR_INVALID_ARG;
  if (!aligned16(plan)) return MLA_ERR_ALIGNMENT;
  if (device_info() == nullptr) return MLA_ERR_HIP;
  mla::PlanParams pp{cu_seqlens_q, cu_seqlens_k, batch, (int32_t)mt, block_m, block_n,
                     right >= 0 ? 1 : 0, right >= 0 ? right : 0, window_left,
                     plan, plan_capacity, num_items};
  return timed_launch(MLA_KERNEL_PLAN, (hipStream_t)hip_stream,
                      [&] { return mla::launch_plan(pp, (hipStream_t)hip_stream); }) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

int32_t mla_prefill_varlen_num_splits(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
                                      int32_t causal, int32_t num_splits) {
  if (num_splits < 0 || num_splits > kMaxSplits || !dense_dims_ok(head_dim_qk, head_dim_v)) return -1;
  // the instance the bf16-output call runs (FP8 output selects the same tile height and residency)
  return resolve_splits(batch, max_seqlen_q, max_seqlen_k, num_heads, num_splits,
                        dense_shape(head_dim_qk, head_dim_v, false, max_seqlen_q, max_seqlen_k, causal != 0));
}

size_t mla_prefill_varlen_workspace_size(int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                         int32_t max_seqlen_k, int32_t num_heads,
                                         int32_t head_dim_v, int32_t causal, int32_t num_splits) {
  if (batch < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_heads <= 0 ||
      num_splits < 0 || num_splits > kMaxSplits || (head_dim_v != 128 && head_dim_v != 256))
    return 0;
  // enough for every instance with this v head (tile height and output type vary the layout)
  size_t need = 0;
  const int dqks[2] = {head_dim_v == 128 ? 192 : 256, 128};
  for (int dqk : dqks) {
    if (!dense_dims_ok(dqk, head_dim_v)) continue;
    for (bool fp8 : {false, true})
      need = std::max(need, varlen_layout(batch, total_q, max_seqlen_q, max_seqlen_k, num_heads, num_splits,
                                          dense_shape(dqk, head_dim_v, fp8, max_seqlen_q, max_seqlen_k,
                                                      causal != 0)).total);
  }
  return need;
}

static mla_status_t varlen_call(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, int32_t causal, int32_t window_left, int32_t window_right,
    int32_t num_splits, const float* sink, const float* out_scale,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream,
    float* part_o = nullptr, float* part_lse = nullptr, int accumulate = 0, bool check = true,
    bool noalloc = false) {
  // out_scale: null for bf16 output, else fp8 e4m3 output of O / *out_scale.
  // part_o / part_lse (internal use): write the normalised fp32 result [total_q, H, Dv] and its
  // LSE [total_q, H] there instead of `out` / `lse`, unsplit and without the sink; with
  // accumulate = 1, merge it into the running result already held there; with 2, merge it with
  // that result and write the final `out` / `lse` (sink folded in) instead. check = false skips
  // the MLA_VALIDATE checks (cu_seqlens built by the library itself). noalloc: the workspace is
  // this device's copy of `scratch` (the caller passes none).
  if (part_o != nullptr) num_splits = 1;
  if (q == nullptr || k == nullptr || v == nullptr || cu_seqlens_q == nullptr ||
      cu_seqlens_k == nullptr || out == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (batch < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_heads <= 0 ||
      num_splits < 0 || num_splits > kMaxSplits || !std::isfinite(softmax_scale) || !(softmax_scale > 0.f) ||
      window_left < -1 || window_right < -1)
    return MLA_ERR_INVALID_ARG;
  const int32_t right = causal ? 0 : window_right;  // causal is the right window 0
  if (!dense_dims_ok(head_dim_qk, head_dim_v) || num_heads > 65535 ||
      max_seqlen_k > (1 << 24) || k_stride_tok >= (1 << 23) || v_stride_tok >= (1 << 23))
    return MLA_ERR_UNSUPPORTED;  // key-block byte offsets are kept in 31 bits
  const bool fp8 = out_scale != nullptr && (part_o == nullptr || accumulate == 2);
  const DenseShape ds = dense_shape(head_dim_qk, head_dim_v, fp8, max_seqlen_q, max_seqlen_k, causal != 0);
  // fp8 rows are written in 16-byte pieces: strides in whole 16-element units
  const bool ostride_ok = fp8 ? ((o_stride_tok & 15) == 0 && (o_stride_head & 15) == 0)
                              : (stride_ok(o_stride_tok) && stride_ok(o_stride_head));
  const int64_t H = num_heads;
  auto rows_ok = [H](int64_t st, int64_t sh, int64_t width) {
    return sh >= 0 && st >= 0 && (H == 1 || sh >= width) && st >= (H - 1) * sh + width;
  };
  if (!rows_ok(q_stride_tok, q_stride_head, head_dim_qk) || !rows_ok(k_stride_tok, k_stride_head, head_dim_qk) ||
      !rows_ok(v_stride_tok, v_stride_head, head_dim_v) || !rows_ok(o_stride_tok, o_stride_head, head_dim_v))
    return MLA_ERR_INVALID_ARG;
  if (lse != nullptr && (lse_stride_tok < 0 || lse_stride_head < 0)) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !stride_ok(q_stride_tok) || !stride_ok(q_stride_head) || !stride_ok(k_stride_tok) ||
      !stride_ok(k_stride_head) || !stride_ok(v_stride_tok) || !stride_ok(v_stride_head) || !ostride_ok ||
      (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) ||
      (out_scale != nullptr && (reinterpret_cast<uintptr_t>(out_scale) & 3u) != 0))
    return MLA_ERR_ALIGNMENT;
  if (batch == 0 || total_q == 0) return MLA_OK;
  const VarlenLayout L = varlen_layout(batch, total_q, max_seqlen_q, max_seqlen_k, num_heads, num_splits, ds);
  const int dv_tiles = head_dim_v / 128;  // work items per (row tile, head, split): 128 columns each
  if ((int64_t)L.n_slots * num_heads * L.splits * dv_tiles > INT32_MAX - 8) return MLA_ERR_UNSUPPORTED;
  if (noalloc) {
    if (L.total > kNoAllocScratchBytes) return MLA_ERR_WORKSPACE;
    workspace = scratch_device_ptr();
    workspace_bytes = kNoAllocScratchBytes;
    if (workspace == nullptr) return MLA_ERR_HIP;
  }
  if (workspace == nullptr || workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGNMENT;
  const DeviceInfo* di = device_info();
  if (di == nullptr) return MLA_ERR_HIP;
  if (!di->gfx950) return MLA_ERR_UNSUPPORTED;

  hipStream_t stream = (hipStream_t)hip_stream;
  if (check && validate_inputs()) {
    mla_status_t st = check_cu(cu_seqlens_q, batch, total_q, true, max_seqlen_q, stream);
    if (st == MLA_OK) st = check_cu(cu_seqlens_k, batch, -1, true, max_seqlen_k, stream);
    if (st != MLA_OK) return st;
  }
  char* ws = static_cast<char*>(workspace);
  int32_t* num_items = reinterpret_cast<int32_t*>(ws + L.off_count);
  int32_t* plan = reinterpret_cast<int32_t*>(ws + L.off_plan);

  int32_t* tickets = reinterpret_cast<int32_t*>(ws + L.off_tickets);
  int32_t* plan_ext = reinterpret_cast<int32_t*>(ws + L.off_plan_ext);
  mla::PlanParams pp{cu_seqlens_q, cu_seqlens_k, batch, L.mt, L.bm, kDenseBN, right >= 0 ? 1 : 0,
                     right >= 0 ? right : 0, window_left, plan, L.n_slots, num_items, tickets, plan_ext};
  if (timed_launch(MLA_KERNEL_PLAN, stream, [&] { return mla::launch_plan(pp, stream); }) != hipSuccess)
    return MLA_ERR_HIP;

  mla::DenseParams dp{};
  dp.q = static_cast<const __bf16*>(q); dp.q_st = q_stride_tok; dp.q_sh = q_stride_head;
  dp.k = static_cast<const __bf16*>(k); dp.k_st = k_stride_tok; dp.k_sh = k_stride_head;
  dp.v = static_cast<const __bf16*>(v); dp.v_st = v_stride_tok; dp.v_sh = v_stride_head;
  dp.cu_q = cu_seqlens_q;
  dp.cu_k = cu_seqlens_k;
  dp.plan = plan;
  dp.plan_ext = plan_ext;
  dp.num_items = num_items;
  dp.n_slots = L.n_slots;
  dp.num_heads = num_heads;
  dp.num_splits = L.splits;
  dp.causal = right >= 0 ? 1 : 0;
  dp.win_right = right >= 0 ? right : 0;
  dp.win_left = window_left;
  dp.scale = softmax_scale;
  dp.scale_log2 = softmax_scale * 1.4426950408889634f;
  dp.sink = sink;
  dp.out = out; dp.o_st = o_stride_tok; dp.o_sh = o_stride_head;
  dp.out_scale = fp8 ? out_scale : nullptr;
  dp.lse = lse; dp.l_st = lse_stride_tok; dp.l_sh = lse_stride_head;
  dp.total_q = total_q;
  if (L.splits > 1) {
    dp.o_part = reinterpret_cast<float*>(ws + L.off_opart);
    dp.lse_part = reinterpret_cast<float*>(ws + L.off_lpart);
  } else if (part_o != nullptr) {
    dp.o_part = part_o;
    dp.lse_part = part_lse;
    dp.accumulate = accumulate;
  }
  {
    dp.wgs_per_xcd = L.wgs_per_xcd;
    const int units = num_heads * L.splits * dv_tiles;
    const char* map = std::getenv("MLA_DENSE_XCD_MAP");
    const bool contiguous = units % 8 == 0 && !(map != nullptr && std::string(map) == "interleave");
    if (contiguous) {
      dp.xcd_units = units / 8;
      const int gu = dense_group_per_xcd();
      dp.group_units = (dp.xcd_units % gu == 0) ? gu : dp.xcd_units;
    } else {
      dp.xcd_units = 0;
      const int gu = 8 * dense_group_per_xcd();
      dp.group_units = (units % gu == 0) ? gu : units;
    }
    dp.counters = tickets;
  }
  if (timed_launch(MLA_KERNEL_DENSE, stream, [&] { return mla::launch_dense_fwd(dp, ds.nw, ds.dqk, ds.dv, ds.fp8, stream); }) !=
      hipSuccess)
    return MLA_ERR_HIP;

  if (L.splits > 1) {
    mla::CombineParams cp{};
    cp.o_part = dp.o_part;
    cp.lse_part = dp.lse_part;
    cp.num_splits = L.splits;
    cp.rows = total_q * num_heads;
    cp.num_heads = num_heads;
    cp.dv = head_dim_v;
    cp.sink = sink;
    cp.out = dp.out; cp.o_st = o_stride_tok; cp.o_sh = o_stride_head;
    cp.out_scale = dp.out_scale;
    cp.lse = lse; cp.l_st = lse_stride_tok; cp.l_sh = lse_stride_head;
    if (timed_launch(MLA_KERNEL_COMBINE, stream, [&] { return mla::launch_combine(cp, stream); }) != hipSuccess)
      return MLA_ERR_HIP;
  }
  return MLA_OK;
}

mla_status_t mla_prefill_varlen(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, int32_t causal, int32_t num_splits, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream) {
  return varlen_call(q, q_stride_tok, q_stride_head, k, k_stride_tok, k_stride_head, v, v_stride_tok,
                     v_stride_head, cu_seqlens_q, cu_seqlens_k, batch, total_q, max_seqlen_q,
                     max_seqlen_k, num_heads, head_dim_qk, head_dim_v, softmax_scale, causal, -1, -1,
                     num_splits, sink, nullptr, out, o_stride_tok, o_stride_head, lse, lse_stride_tok,
                     lse_stride_head, workspace, workspace_bytes, hip_stream);
}

mla_status_t mla_prefill_varlen_noalloc(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, int32_t causal, int32_t num_splits, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head, void* hip_stream) {
  // Same launches as mla_prefill_varlen; MLA_VALIDATE is not honoured here (its host copy
  // allocates and synchronises).
  return varlen_call(q, q_stride_tok, q_stride_head, k, k_stride_tok, k_stride_head, v, v_stride_tok,
                     v_stride_head, cu_seqlens_q, cu_seqlens_k, batch, total_q, max_seqlen_q,
                     max_seqlen_k, num_heads, head_dim_qk, head_dim_v, softmax_scale, causal, -1, -1,
                     num_splits, sink, nullptr, out, o_stride_tok, o_stride_head, lse, lse_stride_tok,
                     lse_stride_head, nullptr, 0, hip_stream, nullptr, nullptr, 0, false, true);
}

mla_status_t mla_prefill_varlen_window(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, int32_t causal, int32_t window_left, int32_t window_right,
    int32_t num_splits, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream) {
  return varlen_call(q, q_stride_tok, q_stride_head, k, k_stride_tok, k_stride_head, v, v_stride_tok,
                     v_stride_head, cu_seqlens_q, cu_seqlens_k, batch, total_q, max_seqlen_q,
                     max_seqlen_k, num_heads, head_dim_qk, head_dim_v, softmax_scale, causal,
                     window_left, window_right, num_splits, sink, nullptr, out, o_stride_tok, o_stride_head,
                     lse, lse_stride_tok, lse_stride_head, workspace, workspace_bytes, hip_stream);
}

mla_status_t mla_prefill_varlen_fp8(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, int32_t causal, int32_t window_left, int32_t window_right,
    int32_t num_splits, const float* sink, const float* out_scale,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (out_scale == nullptr) return MLA_ERR_INVALID_ARG;
  return varlen_call(q, q_stride_tok, q_stride_head, k, k_stride_tok, k_stride_head, v, v_stride_tok,
                     v_stride_head, cu_seqlens_q, cu_seqlens_k, batch, total_q, max_seqlen_q,
                     max_seqlen_k, num_heads, head_dim_qk, head_dim_v, softmax_scale, causal,
                     window_left, window_right, num_splits, sink, out_scale, out, o_stride_tok, o_stride_head,
                     lse, lse_stride_tok, lse_stride_head, workspace, workspace_bytes, hip_stream);
}

namespace {

// Workspace of mla_prefill_chunked_context: the dense workspace, then the chunk's row offsets,
// the bounded K/V buffer and the fp32 accumulators.
struct ChunkedLayout {
  size_t dense, off_cu, off_k, off_v, off_acc, off_la, total;
};

ChunkedLayout chunked_layout(int32_t batch, int32_t total_q, int32_t max_q, int32_t heads, int32_t chunk) {
  ChunkedLayout C{};
  // enough for the dense calls of a chunked call with either tile height
  const int32_t max_k = std::max(max_q, chunk);
  size_t dense = 0;
  for (int nw : {4, 8})
    dense = std::max(dense, varlen_layout(batch, total_q, max_q, max_k, heads, 1,
                                          with_waves(dense_shape(kDenseDqk, kDenseDv, false, max_q, max_k, false),
                                                     nw)).total);
  C.dense = align256(dense);
  const size_t rows = (size_t)batch * chunk;
  const size_t th = (size_t)total_q * heads;
  C.off_cu = C.dense;
  C.off_k = align256(C.off_cu + (size_t)(batch + 1) * 4);
  C.off_v = align256(C.off_k + rows * heads * kDenseDqk * 2);
  C.off_acc = align256(C.off_v + rows * heads * kDenseDv * 2);
  C.off_la = align256(C.off_acc + th * kDenseDv * 4);
  C.total = align256(C.off_la + th * 4);
  return C;
}

}  // namespace

size_t mla_prefill_chunked_context_workspace_size(int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                                  int32_t num_heads, int32_t chunk_tokens) {
  if (batch < 0 || total_q < 0 || max_seqlen_q < 0 || num_heads <= 0 || chunk_tokens <= 0) return 0;
  return chunked_layout(batch, total_q, max_seqlen_q, num_heads, chunk_tokens).total;
}

mla_status_t mla_latent_upproject(const void* latent, int64_t latent_stride_row,
                                  const int32_t* cu_seqlens_ctx, int32_t batch, int32_t ctx_start,
                                  int32_t chunk_tokens, const void* w_kv, int64_t w_stride_row,
                                  int32_t num_heads, int32_t* cu_chunk, void* k_out, void* v_out,
                                  void* hip_stream) {
  if (latent == nullptr || cu_seqlens_ctx == nullptr || w_kv == nullptr || cu_chunk == nullptr ||
      k_out == nullptr || v_out == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (batch < 0 || ctx_start < 0 || chunk_tokens <= 0 || num_heads <= 0 || latent_stride_row < kSparseDqk ||
      w_stride_row < 512)
    return MLA_ERR_INVALID_ARG;
  if (batch > 65535 || num_heads > 32767 || chunk_tokens > (1 << 24) || w_stride_row >= (1 << 23))
    return MLA_ERR_UNSUPPORTED;  // a head's W_KV rows are addressed with 32-bit byte offsets
  if (!aligned16(latent) || !aligned16(w_kv) || !aligned16(k_out) || !aligned16(v_out) ||
      !stride_ok(latent_stride_row) || !stride_ok(w_stride_row) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_ctx) & 3u) != 0 || (reinterpret_cast<uintptr_t>(cu_chunk) & 3u) != 0)
    return MLA_ERR_ALIGNMENT;
  if (batch == 0) return MLA_OK;
  const DeviceInfo* di = device_info();
  if (di == nullptr) return MLA_ERR_HIP;
  if (!di->gfx950) return MLA_ERR_UNSUPPORTED;
  hipStream_t stream = (hipStream_t)hip_stream;
  if (mla::launch_chunk_cu(cu_seqlens_ctx, batch, ctx_start, chunk_tokens, cu_chunk, stream) != hipSuccess)
    return MLA_ERR_HIP;
  mla::UpprojParams up{};
  up.latent = static_cast<const __bf16*>(latent); up.lat_st = latent_stride_row;
  up.cu_ctx = cu_seqlens_ctx; up.cu_chunk = cu_chunk;
  up.batch = batch; up.c0 = ctx_start; up.w = chunk_tokens;
  up.w_kv = static_cast<const __bf16*>(w_kv); up.w_st = w_stride_row;
  up.num_heads = num_heads;
  up.kbuf = static_cast<__bf16*>(k_out); up.k_st = (int64_t)num_heads * kDenseDqk; up.k_sh = kDenseDqk;
  up.vbuf = static_cast<__bf16*>(v_out); up.v_st = (int64_t)num_heads * kDenseDv; up.v_sh = kDenseDv;
  return timed_launch(MLA_KERNEL_UPPROJ, stream, [&] { return mla::launch_upproj(up, stream); }) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

mla_status_t mla_prefill_chunked_context(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
    const int32_t* cu_seqlens_q, const void* latent, int64_t latent_stride_row,
    const int32_t* cu_seqlens_ctx, const void* w_kv, int64_t w_stride_row,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_ctx,
    int32_t num_heads, int32_t chunk_tokens, float softmax_scale, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (latent == nullptr || cu_seqlens_ctx == nullptr || w_kv == nullptr || q == nullptr || out == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (batch < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_ctx < 0 || num_heads <= 0 ||
      chunk_tokens <= 0 || latent_stride_row < kSparseDqk || w_stride_row < 512 || !std::isfinite(softmax_scale) ||
      !(softmax_scale > 0.f))
    return MLA_ERR_INVALID_ARG;
  if (batch > 65535 || num_heads > 32767 || chunk_tokens > (1 << 24) ||
      (int64_t)batch * chunk_tokens > INT32_MAX || (int64_t)num_heads * kDenseDqk >= (1 << 23) ||
      w_stride_row >= (1 << 23))
    return MLA_ERR_UNSUPPORTED;
  if (!aligned16(latent) || !aligned16(w_kv) || !stride_ok(latent_stride_row) || !stride_ok(w_stride_row) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_ctx) & 3u) != 0)
    return MLA_ERR_ALIGNMENT;
  if (batch == 0 || total_q == 0) return MLA_OK;
  const ChunkedLayout C = chunked_layout(batch, total_q, max_seqlen_q, num_heads, chunk_tokens);
  if (workspace == nullptr || workspace_bytes < C.total) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGNMENT;
  hipStream_t stream = (hipStream_t)hip_stream;
  if (validate_inputs()) {
    mla_status_t vs = check_cu(cu_seqlens_q, batch, total_q, true, max_seqlen_q, stream);
    if (vs == MLA_OK) vs = check_cu(cu_seqlens_ctx, batch, -1, true, max_seqlen_ctx, stream);
    if (vs != MLA_OK) return vs;
  }
  char* ws = static_cast<char*>(workspace);
  float* acc = reinterpret_cast<float*>(ws + C.off_acc);
  float* la = reinterpret_cast<float*>(ws + C.off_la);
  int32_t* cu_chunk = reinterpret_cast<int32_t*>(ws + C.off_cu);
  void* kbuf = ws + C.off_k;
  void* vbuf = ws + C.off_v;
  // Without context the result is the causal prefill of the new tokens.
  if (max_seqlen_ctx == 0)
    return varlen_call(q, q_stride_tok, q_stride_head, k, k_stride_tok, k_stride_head, v, v_stride_tok,
                       v_stride_head, cu_seqlens_q, cu_seqlens_q, batch, total_q, max_seqlen_q, max_seqlen_q,
                       num_heads, kDenseDqk, kDenseDv, softmax_scale, 1, -1, -1, 1, sink, nullptr, out,
                       o_stride_tok, o_stride_head, lse, lse_stride_tok, lse_stride_head, ws, C.dense, hip_stream,
                       nullptr, nullptr, 0, false);
  // 1. the new tokens against themselves, causally: the first accumulated part
  mla_status_t st = varlen_call(q, q_stride_tok, q_stride_head, k, k_stride_tok, k_stride_head, v, v_stride_tok,
                                v_stride_head, cu_seqlens_q, cu_seqlens_q, batch, total_q, max_seqlen_q,
                                max_seqlen_q, num_heads, kDenseDqk, kDenseDv, softmax_scale, 1, -1, -1, 1,
                                nullptr, nullptr, out, o_stride_tok, o_stride_head, nullptr, 0, 0, ws, C.dense,
                                hip_stream, acc, la, 0, false);
  if (st != MLA_OK) return st;
  // 2. each context chunk: up-project into the bounded buffer, attend without a mask and merge the
  //    chunk's result into the running one in the attention kernel's epilogue; the last chunk's
  //    epilogue writes the final output, with the sink folded in once
  const int64_t kst = (int64_t)num_heads * kDenseDqk, vst = (int64_t)num_heads * kDenseDv;
  for (int64_t c0 = 0; c0 < max_seqlen_ctx; c0 += chunk_tokens) {
    st = mla_latent_upproject(latent, latent_stride_row, cu_seqlens_ctx, batch, (int32_t)c0, chunk_tokens, w_kv,
                              w_stride_row, num_heads, cu_chunk, kbuf, vbuf, hip_stream);
    if (st != MLA_OK) return st;
    const bool last = c0 + chunk_tokens >= max_seqlen_ctx;
    st = varlen_call(q, q_stride_tok, q_stride_head, kbuf, kst, kDenseDqk, vbuf, vst, kDenseDv, cu_seqlens_q,
                     cu_chunk, batch, total_q, max_seqlen_q, chunk_tokens, num_heads, kDenseDqk, kDenseDv,
                     softmax_scale, 0, -1, -1, 1, last ? sink : nullptr, nullptr, out, o_stride_tok, o_stride_head,
                     last ? lse : nullptr, lse_stride_tok, lse_stride_head, ws, C.dense, hip_stream, acc, la,
                     last ? 2 : 1, false);
    if (st != MLA_OK) return st;
  }
  return MLA_OK;
}

size_t mla_prefill_sparse_workspace_size(int32_t num_tokens, int32_t num_heads, int32_t topk,
                                         int32_t head_dim_v) {
  (void)num_tokens;
  (void)num_heads;
  (void)topk;
  (void)head_dim_v;
  return 0;
}

}  // extern "C"

namespace {

// Checks shared by the physical-row and the paged sparse entry points, then the launch.
mla_status_t sparse_call(mla::SparseParams& sp, const void* q, int64_t q_stride_tok,
                         int64_t q_stride_head, const void* kv, int64_t kv_stride_row, int64_t n_kv,
                         const int32_t* indices, int64_t idx_stride_tok, int32_t topk,
                         const int32_t* topk_length, int32_t num_tokens, int32_t num_heads,
                         int32_t head_dim_qk, int32_t head_dim_v, float softmax_scale,
                         const float* sink, void* out, int64_t o_stride_tok, int64_t o_stride_head,
                         float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
                         void* hip_stream) {
  if (q == nullptr || kv == nullptr || indices == nullptr || out == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (num_tokens < 0 || num_heads <= 0 || n_kv < 0 || topk <= 0 || !std::isfinite(softmax_scale) ||
      !(softmax_scale > 0.f))
    return MLA_ERR_INVALID_ARG;
  if (head_dim_qk != kSparseDqk || head_dim_v != kSparseDv || num_heads > 128 || topk > 8192 ||
      n_kv > INT32_MAX || kv_stride_row > INT32_MAX)
    return MLA_ERR_UNSUPPORTED;
  const int64_t H = num_heads;
  if (idx_stride_tok < topk || kv_stride_row < kSparseDqk || q_stride_head < 0 || o_stride_head < 0 ||
      (H > 1 && (q_stride_head < kSparseDqk || o_stride_head < kSparseDv)) ||
      q_stride_tok < (H - 1) * q_stride_head + kSparseDqk ||
      o_stride_tok < (H - 1) * o_stride_head + kSparseDv ||
      (lse != nullptr && (lse_stride_tok < 0 || lse_stride_head < 0)))
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || !stride_ok(q_stride_tok) ||
      !stride_ok(q_stride_head) || !stride_ok(kv_stride_row) || !stride_ok(o_stride_tok) ||
      !stride_ok(o_stride_head) || (reinterpret_cast<uintptr_t>(indices) & 3u) != 0 ||
      (topk_length != nullptr && (reinterpret_cast<uintptr_t>(topk_length) & 3u) != 0) ||
      (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0))
    return MLA_ERR_ALIGNMENT;
  if (num_tokens == 0) return MLA_OK;
  const DeviceInfo* di = device_info();
  if (di == nullptr) return MLA_ERR_HIP;
  if (!di->gfx950) return MLA_ERR_UNSUPPORTED;

  sp.q = static_cast<const __bf16*>(q); sp.q_st = q_stride_tok; sp.q_sh = q_stride_head;
  sp.kv = static_cast<const __bf16*>(kv); sp.kv_st = kv_stride_row; sp.n_kv = n_kv;
  sp.idx = indices; sp.idx_st = idx_stride_tok; sp.topk = topk;
  sp.topk_length = topk_length;
  sp.num_tokens = num_tokens;
  sp.max_wgs = di->cus > 0 ? di->cus : 256;
  sp.num_heads = num_heads;
  sp.scale = softmax_scale;
  sp.scale_log2 = softmax_scale * 1.4426950408889634f;
  sp.sink = sink;
  sp.out = static_cast<__bf16*>(out); sp.o_st = o_stride_tok; sp.o_sh = o_stride_head;
  sp.lse = lse; sp.l_st = lse_stride_tok; sp.l_sh = lse_stride_head;
  return timed_launch(MLA_KERNEL_SPARSE, (hipStream_t)hip_stream,
                      [&] { return mla::launch_sparse_fwd(sp, (hipStream_t)hip_stream); }) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

mla_status_t mla_prefill_sparse(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* kv, int64_t kv_stride_row, int64_t n_kv,
    const int32_t* indices, int64_t idx_stride_tok, int32_t topk,
    const int32_t* topk_length,
    int32_t num_tokens, int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream) {
  (void)workspace;
  (void)workspace_bytes;
  mla::SparseParams sp{};
  return sparse_call(sp, q, q_stride_tok, q_stride_head, kv, kv_stride_row, n_kv, indices,
                     idx_stride_tok, topk, topk_length, num_tokens, num_heads, head_dim_qk,
                     head_dim_v, softmax_scale, sink, out, o_stride_tok, o_stride_head, lse,
                     lse_stride_tok, lse_stride_head, hip_stream);
}

mla_status_t mla_prefill_sparse_paged(
    const void* q, int64_t q_stride_tok, int64_t q_stride_head,
    const void* kv_cache, int64_t kv_stride_row, int32_t num_blocks, int32_t block_size,
    const int32_t* block_table, int64_t bt_stride_seq, int32_t max_blocks_per_seq,
    const int32_t* cu_seqlens_q, int32_t batch, const int32_t* seqused_kv,
    const int32_t* seqused_q,
    const int32_t* indices, int64_t idx_stride_tok, int32_t topk,
    const int32_t* topk_length,
    int32_t num_tokens, int32_t num_heads, int32_t head_dim_qk, int32_t head_dim_v,
    float softmax_scale, const float* sink,
    void* out, int64_t o_stride_tok, int64_t o_stride_head,
    float* lse, int64_t lse_stride_tok, int64_t lse_stride_head,
    void* workspace, size_t workspace_bytes, void* hip_stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (block_table == nullptr || cu_seqlens_q == nullptr) return MLA_ERR_INVALID_ARG;
  if (batch <= 0 || num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 ||
      bt_stride_seq < max_blocks_per_seq)
    return MLA_ERR_INVALID_ARG;
  if (block_size > 1024 || (int64_t)num_blocks * block_size > INT32_MAX ||
      (int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return MLA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) != 0 ||
      (seqused_kv != nullptr && (reinterpret_cast<uintptr_t>(seqused_kv) & 3u) != 0) ||
      (seqused_q != nullptr && (reinterpret_cast<uintptr_t>(seqused_q) & 3u) != 0))
    return MLA_ERR_ALIGNMENT;
  if (validate_inputs() && num_tokens > 0) {
    const mla_status_t vs = check_cu(cu_seqlens_q, batch, num_tokens, false, INT32_MAX, (hipStream_t)hip_stream);
    if (vs != MLA_OK) return vs;
  }
  mla::SparseParams sp{};
  sp.block_table = block_table; sp.bt_st = bt_stride_seq;
  sp.max_blocks = max_blocks_per_seq; sp.block_size = block_size; sp.num_blocks = num_blocks;
  sp.cu_q = cu_seqlens_q; sp.batch = batch; sp.seqused = seqused_kv; sp.seqused_q = seqused_q;
  return sparse_call(sp, q, q_stride_tok, q_stride_head, kv_cache, kv_stride_row,
                     (int64_t)num_blocks * block_size, indices, idx_stride_tok, topk, topk_length,
                     num_tokens, num_heads, head_dim_qk, head_dim_v, softmax_scale, sink, out,
                     o_stride_tok, o_stride_head, lse, lse_stride_tok, lse_stride_head, hip_stream);
}

mla_status_t mla_combine(const float* o_part, const float* lse_part, int32_t num_splits,
                         int32_t num_tokens, int32_t num_heads, int32_t head_dim_v,
                         const float* sink, void* out, int64_t o_stride_tok,
                         int64_t o_stride_head, float* lse, int64_t lse_stride_tok,
                         int64_t lse_stride_head, void* hip_stream) {
  if (o_part == nullptr || lse_part == nullptr || out == nullptr) return MLA_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > 256 || num_tokens < 0 || num_heads <= 0 || head_dim_v <= 0 ||
      (head_dim_v & 7) != 0 || head_dim_v > 1024)
    return MLA_ERR_INVALID_ARG;
  const int64_t H = num_heads;
  if (o_stride_head < 0 || (H > 1 && o_stride_head < head_dim_v) ||
      o_stride_tok < (H - 1) * o_stride_head + head_dim_v ||
      (lse != nullptr && (lse_stride_tok < 0 || lse_stride_head < 0)))
    return MLA_ERR_INVALID_ARG;
  if ((int64_t)num_tokens * num_heads > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if (!aligned16(o_part) || !aligned16(out) || !stride_ok(o_stride_tok) || !stride_ok(o_stride_head) ||
      (reinterpret_cast<uintptr_t>(lse_part) & 3u) != 0 ||
      (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0))
    return MLA_ERR_ALIGNMENT;
  if (num_tokens == 0) return MLA_OK;
  if (device_info() == nullptr) return MLA_ERR_HIP;
  mla::CombineParams cp{};
  cp.o_part = o_part;
  cp.lse_part = lse_part;
  cp.num_splits = num_splits;
  cp.rows = num_tokens * num_heads;
  cp.num_heads = num_heads;
  cp.dv = head_dim_v;
  cp.sink = sink;
  cp.out = out; cp.o_st = o_stride_tok; cp.o_sh = o_stride_head;
  cp.lse = lse; cp.l_st = lse_stride_tok; cp.l_sh = lse_stride_head;
  return timed_launch(MLA_KERNEL_COMBINE, (hipStream_t)hip_stream,
                      [&] { return mla::launch_combine(cp, (hipStream_t)hip_stream); }) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

mla_status_t mla_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (int i = 0; i < kNumKernels; ++i) {
    g_prof.total_ms[i] = 0.0;
    g_prof.count[i] = 0;
  }
  g_prof.enabled.store(enable != 0);
  return MLA_OK;
}

mla_status_t mla_profile_select(uint32_t kinds) {
  g_prof.kinds.store(kinds);
  return MLA_OK;
}

mla_status_t mla_profile_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= kNumKernels || total_ms == nullptr || launches == nullptr)
    return MLA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  bool ok = true;
  for (auto& r : g_prof.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      ok = false;
    } else {
      g_prof.total_ms[r.kind] += ms;
      g_prof.count[r.kind] += 1;
    }
    g_prof.pool.push_back({r.a, r.b});
  }
  g_prof.pending.clear();
  *total_ms = g_prof.total_ms[kernel];
  *launches = g_prof.count[kernel];
  return ok ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
