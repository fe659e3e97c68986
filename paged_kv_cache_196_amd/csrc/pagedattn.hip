// pagedattn.hip — the C ABI declared in include/pagedattn.h: descriptor
// checks, dispatch to the kernel variants (compiled in their own
// translation units, see dispatch.h) and the host block manager.
//
// One decode call is one kernel launch on the caller's stream: the decode
// kernel (matrix-core or vector-ALU engine) with a grid of one resident
// wave of workgroups.  Each workgroup rebuilds the block-count prefix in
// LDS, walks its equal share of the flattened (sequence, KV head, logical
// block) units and writes `out` for every (sequence, KV head) it holds
// whole; the pieces of a (sequence, KV head) split across workgroups meet
// in the workspace, where the last one to finish folds them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string.h>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pagedattn.h"
#include "block_manager.h"
#include "dispatch.h"
#include "kernel_args.h"
#include "pa_device.h"

namespace pa {

inline bool use_mfma(const pa_desc* d) {
  if (d->kernel == PA_KERNEL_MFMA) return true;
  if (d->kernel == PA_KERNEL_VALU) return false;
  return d->dtype != PA_F32;
}

Variant decode_variant(const pa_desc* d, int G) {
  const int B = d->block_size;
  const bool mf = use_mfma(d);
  switch (d->dtype) {
    case PA_F32: return mf ? Variant{} : decode_variant_f32_valu(B, G);
    case PA_F16: return mf ? decode_variant_f16_mfma(B, G) : decode_variant_f16_valu(B, G);
    case PA_BF16: return mf ? decode_variant_bf16_mfma(B, G) : decode_variant_bf16_valu(B, G);
    default: return Variant{};
  }
}

// How a descriptor's query group runs: the kernel for group size G and
// `split` = (query heads per KV head) / G virtual KV heads per pool head.
// G is the largest built size that divides the query group, so a group
// the kernels hold directly runs as one (split = 1); a larger one (MQA's
// 32 or 64 heads on one KV head, 8 on the vector ALU) runs as several
// virtual groups that each read the K/V tiles of their pool head.
struct Plan {
  Variant v;
  int G = 0, split = 1, shift = 0;
  int hkv = 0;  // virtual KV heads: num_kv_heads * split
};

template <class Get>
Plan make_plan(const pa_desc* d, Get get, int max_g) {
  Plan p;
  const int group = d->num_q_heads / d->num_kv_heads;
  for (int g = max_g; g >= 1; g /= 2) {
    if (group % g != 0) continue;
    const Variant v = get(g);
    if (!v.launch) continue;
    p.v = v;
    p.G = g;
    p.split = group / g;
    p.shift = (p.split & (p.split - 1)) == 0 ? __builtin_ctz((unsigned)p.split) : -1;
    p.hkv = d->num_kv_heads * p.split;
    return p;
  }
  return p;
}

// max_g caps the kernel group (a power of two), e.g. to bound the
// workspace a group's partials take.
Plan plan_decode(const pa_desc* d, int max_g = 64) {
  return make_plan(d, [d](int g) { return decode_variant(d, g); }, max_g);
}

// Per-device facts queried once.
struct DeviceInfo {
  bool ok = false;
  int cus = 0;
};

DeviceInfo device_info() {
  static std::mutex mu;
  static DeviceInfo cache[64];
  static bool known[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DeviceInfo{};
  std::lock_guard<std::mutex> lk(mu);
  if (!known[dev]) {
    hipDeviceProp_t p;
    DeviceInfo info;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess && strncmp(p.gcnArchName, "gfx950", 6) == 0) {
      info.ok = true;
      info.cus = p.multiProcessorCount;
    }
    cache[dev] = info;
    known[dev] = true;
  }
  return cache[dev];
}

// Dynamic LDS of a decode workgroup: the block-count prefix (S + 1 ints)
// and a copy of the lengths (S ints).
size_t prefix_lds(int S) { return (size_t)(2 * S + 1) * sizeof(int); }

// ------------------------------------------- allocation-free decode scratch
//
// paged_attn_decode_noalloc keeps its workspace (split counters and
// partials) in this file-scope device array instead of a caller buffer:
// one copy per GPU, alive until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the device address hipGetSymbolAddress returns, looked
// up once per device with that device current.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's scratch, nullptr if the lookup failed.
void* scratch_ptr() {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

__global__ void clear_ints_kernel(int* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// Workspace layout for `slots` partial slots (two per workgroup) and
// `counters` split counters: counters first (padded to 256 bytes), then
// the weighted-V partials [slots][G][kD] and the (max, sum) pairs
// [slots][G][2], all fp32.
size_t ws_layout_bytes(int counters, int slots, int G) {
  const size_t cnt = ((size_t)counters * sizeof(int) + 255) & ~(size_t)255;
  return cnt + sizeof(float) * (size_t)slots * G * (kD + 2);
}

void bind_workspace(Args* a, void* ws, int counters, int slots, int G) {
  const size_t cnt = ((size_t)counters * sizeof(int) + 255) & ~(size_t)255;
  a->counters = static_cast<int*>(ws);
  a->ws_o = reinterpret_cast<float*>(static_cast<char*>(ws) + cnt);
  a->ws_ml = a->ws_o + (size_t)slots * G * kD;
}

// Workspace of a shared-prefix call: the ordinary decode workspace first
// (split counters and narrow partials, same layout), then the member
// pairs' counters [S*Hkv], their whole-contribution slots pair_o
// [S*Hkv][2][G][kD] / pair_ml [S*Hkv][2][G][2], and the wide slots of item
// fragments wide_o [2*kMaxSharedGrid][kWideCols][kD] / wide_ml [..][2].
constexpr int kMaxSharedGrid = 512;

struct SharedWs {
  size_t pcnt, pair_o, pair_ml, wide_o, wide_ml, total;
};

SharedWs shared_ws_layout(const pa_desc* d) {
  const size_t G = (size_t)(d->num_q_heads / d->num_kv_heads);
  const size_t pairs = (size_t)d->num_seqs * d->num_kv_heads;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  SharedWs w;
  // the leading part also serves the plain decode these calls fall back to
  const int g_plain = plan_decode(d).G;
  size_t off = al(ws_layout_bytes(kMaxGrid, 2 * kMaxGrid, std::max((int)G, g_plain)));
  if (d->num_seqs > kMaxSeqs) {  // runs as the ordinary decode: the leading part alone
    w.pcnt = w.pair_o = w.pair_ml = w.wide_o = w.wide_ml = w.total = off;
    return w;
  }
  w.pcnt = off;
  off = al(off + sizeof(int) * pairs);
  w.pair_o = off;
  off = al(off + sizeof(float) * pairs * 2 * G * kD);
  w.pair_ml = off;
  off = al(off + sizeof(float) * pairs * 2 * G * 2);
  w.wide_o = off;
  off = al(off + sizeof(float) * 2 * kMaxSharedGrid * kWideCols * kD);
  w.wide_ml = off;
  off = al(off + sizeof(float) * 2 * kMaxSharedGrid * kWideCols * 2);
  w.total = off;
  return w;
}

void bind_shared_workspace(Args* a, void* ws, const SharedWs& w) {
  char* base = static_cast<char*>(ws);
  a->pcnt = reinterpret_cast<int*>(base + w.pcnt);
  a->pair_o = reinterpret_cast<float*>(base + w.pair_o);
  a->pair_ml = reinterpret_cast<float*>(base + w.pair_ml);
  a->wide_o = reinterpret_cast<float*>(base + w.wide_o);
  a->wide_ml = reinterpret_cast<float*>(base + w.wide_ml);
}

// The shared-prefix kernel of a descriptor: matrix cores (fp16 / bf16, kernel
// AUTO or MFMA), for query groups it holds directly (1, 2, 4 or 8 heads per
// KV head, no virtual split); an empty Variant otherwise.
Variant pick_shared(const pa_desc* d) {
  if (!use_mfma(d)) return Variant{};
  const int G = d->num_q_heads / d->num_kv_heads;
  if (d->dtype == PA_BF16) return decode_shared_variant_bf16(d->block_size, G);
  if (d->dtype == PA_F16) return decode_shared_variant_f16(d->block_size, G);
  return Variant{};
}

size_t shared_lds(int S, int ngroups) { return (size_t)shared_lds_ints(S, ngroups) * sizeof(int); }

// Member partials a shared-prefix workgroup can keep in LDS until its next
// count-in: the most (up to the count-in list length) whose dynamic LDS
// still lets the kernel run, found by bisection on the occupancy query and
// cached per (kernel, LDS of the schedule).
int stage_capacity(const Variant& v, size_t base, size_t entry) {
  static std::mutex mu;
  static std::unordered_map<uint64_t, int> cache;
  const uint64_t key = (uint64_t)(uintptr_t)v.launch * 1000003u ^ (uint64_t)base * 131u ^ entry;
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int lo = 0, hi = kDefer;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (v.occ(base + (size_t)mid * entry) > 0) lo = mid; else hi = mid - 1;
  }
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = lo;
  return lo;
}

// Prefill plan of a descriptor: matrix cores only (fp16 / bf16), query
// groups as in the decode plan.
struct PrefillPlan {
  PrefillFn fn = nullptr;
  int G = 0, split = 1, shift = 0;
};

PrefillPlan plan_prefill(const pa_desc* d) {
  PrefillPlan p;
  if (d->kernel == PA_KERNEL_VALU || d->dtype == PA_F32) return p;
  const int group = d->num_q_heads / d->num_kv_heads;
  for (int g = 16; g >= 1; g /= 2) {
    if (group % g != 0) continue;
    const PrefillFn fn = d->dtype == PA_BF16 ? prefill_variant_bf16(d->block_size, g)
                                             : prefill_variant_f16(d->block_size, g);
    if (!fn) continue;
    p.fn = fn;
    p.G = g;
    p.split = group / g;
    p.shift = (p.split & (p.split - 1)) == 0 ? __builtin_ctz((unsigned)p.split) : -1;
    return p;
  }
  return p;
}

}  // namespace pa

using namespace pa;

// A decode launch keeps its batch's length prefix in LDS, so it takes at
// most kMaxSeqs sequences: a larger batch runs as consecutive launches of
// at most kMaxSeqs sequences on the caller's stream.  Sequences are
// independent, and every launch leaves the workspace's counters at zero
// for the next.  call(slice descriptor, first sequence) launches one.
template <class F>
static int32_t decode_in_slices(const void* q, const int32_t* bt, const int32_t* lens, void* out,
                                const pa_desc* d, F call) {
  if (!q || !bt || !lens || !out) return PA_ERR_NULL;
  pa_desc ds = *d;
  for (int32_t s0 = 0; s0 < d->num_seqs; s0 += kMaxSeqs) {
    ds.num_seqs = std::min(kMaxSeqs, d->num_seqs - s0);
    const int32_t st = call(&ds, s0);
    if (st != PA_OK) return st;
  }
  return PA_OK;
}

// Byte offset of sequence s0's rows in q (input type) or out (output type).
static int64_t rows_bytes(const pa_desc* d, int64_t s0, int32_t dtype) {
  return s0 * d->num_q_heads * d->head_dim * (int64_t)pa_dtype_size(dtype);
}

extern "C" {

const char* pa_status_str(int32_t s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: invalid size or num_q_heads % num_kv_heads != 0";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unknown dtype or unsupported out_dtype";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: configuration not built (head_dim, block_size, group, kernel)";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: q, pools and out must be 16-byte aligned";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: kernel launch failed";
    case PA_ERR_TABLE: return "PA_ERR_TABLE: block table entry or sequence length out of range";
    case PA_ERR_DEVICE: return "PA_ERR_DEVICE: no gfx950 device current";
    case PA_ERR_NOMEM: return "PA_ERR_NOMEM: not enough free physical blocks";
    case PA_ERR_SCRATCH:
      return "PA_ERR_SCRATCH: the call needs more than the 8 MiB static scratch of "
             "paged_attn_decode_noalloc";
    default: return "unknown pa_status";
  }
}

size_t pa_dtype_size(int32_t dt) {
  switch (dt) {
    case PA_F32: return 4;
    case PA_F16:
    case PA_BF16: return 2;
    default: return 0;
  }
}

int64_t pa_blocks_for_len(int64_t len, int32_t block_size) {
  if (len <= 0 || block_size <= 0) return 0;
  return (len + block_size - 1) / block_size;
}

int32_t pa_check_desc(const pa_desc* d) {
  if (!d) return PA_ERR_NULL;
  if (d->num_seqs < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 ||
      d->block_size <= 0 || d->num_blocks <= 0 || d->max_blocks_per_seq <= 0 ||
      d->cached_prefix_blocks < 0)
    return PA_ERR_SHAPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_SHAPE;
  if (pa_dtype_size(d->dtype) == 0) return PA_ERR_DTYPE;
  if (d->out_dtype != PA_F32 && d->out_dtype != d->dtype) return PA_ERR_DTYPE;
  if (d->head_dim != kD) return PA_ERR_UNSUPPORTED;
  if (d->block_size != 16 && d->block_size != 32) return PA_ERR_UNSUPPORTED;
  if (d->kernel < PA_KERNEL_AUTO || d->kernel > PA_KERNEL_MFMA) return PA_ERR_UNSUPPORTED;
  if (d->kernel == PA_KERNEL_MFMA && d->dtype == PA_F32) return PA_ERR_UNSUPPORTED;
  const Plan p = plan_decode(d);
  if (!p.v.launch) return PA_ERR_UNSUPPORTED;
  // flat unit indices of one decode launch (at most kMaxSeqs sequences) are int32
  if ((int64_t)std::min(d->num_seqs, kMaxSeqs) * d->max_blocks_per_seq * p.hkv >= ((int64_t)1 << 31))
    return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

size_t pa_pool_bytes(const pa_desc* d) {
  if (pa_check_desc(d) != PA_OK) return 0;
  return (size_t)d->num_blocks * d->num_kv_heads * d->block_size * d->head_dim *
         pa_dtype_size(d->dtype);
}

int64_t pa_k_elem_offset(const pa_desc* d, int32_t block, int32_t kv_head, int32_t slot, int32_t dim) {
  if (pa_check_desc(d) != PA_OK) return -1;
  if (block < 0 || block >= d->num_blocks || kv_head < 0 || kv_head >= d->num_kv_heads || slot < 0 ||
      slot >= d->block_size || dim < 0 || dim >= d->head_dim)
    return -1;
  return (((int64_t)block * d->num_kv_heads + kv_head) * d->block_size + slot) * d->head_dim + dim;
}

int64_t pa_v_elem_offset(const pa_desc* d, int32_t block, int32_t kv_head, int32_t slot, int32_t dim) {
  if (pa_check_desc(d) != PA_OK) return -1;
  if (block < 0 || block >= d->num_blocks || kv_head < 0 || kv_head >= d->num_kv_heads || slot < 0 ||
      slot >= d->block_size || dim < 0 || dim >= d->head_dim)
    return -1;
  const int64_t tile = ((int64_t)block * d->num_kv_heads + kv_head) * d->block_size * d->head_dim;
  return tile + ((int64_t)(slot / kSub) * d->head_dim + dim) * kSub + slot % kSub;
}

size_t pa_workspace_bytes(const pa_desc* d) {
  if (pa_check_desc(d) != PA_OK) return 0;
  return ws_layout_bytes(kMaxGrid, 2 * kMaxGrid, plan_decode(d).G);
}

int32_t pa_validate_host(const pa_desc* d, const int32_t* bt, const int32_t* lens) {
  const int32_t st = pa_check_desc(d);
  if (st != PA_OK) return st;
  if (d->num_seqs > 0 && (!bt || !lens)) return PA_ERR_NULL;
  const int64_t cap = (int64_t)d->max_blocks_per_seq * d->block_size;
  for (int32_t b = 0; b < d->num_seqs; ++b) {
    if (lens[b] < 0 || lens[b] > cap) return PA_ERR_TABLE;
    const int64_t n = pa_blocks_for_len(lens[b], d->block_size);
    for (int64_t j = 0; j < n; ++j) {
      const int32_t id = bt[(int64_t)b * d->max_blocks_per_seq + j];
      if (id < 0 || id >= d->num_blocks) return PA_ERR_TABLE;
    }
  }
  return PA_OK;
}

// Workgroups of a decode launch with plan p: every CU filled to the
// kernel's occupancy, at most kMaxGrid; -1 if no workgroup fits a CU.
static int plan_grid(const Plan& p, int S) {
  const DeviceInfo info = device_info();
  if (!info.ok) return -1;
  const int per_cu = p.v.occ(prefix_lds(S));
  if (per_cu <= 0) return -1;  // the workgroup's LDS does not fit a CU
  return std::min(info.cus * per_cu, kMaxGrid);
}

int32_t pa_decode_grid(const pa_desc* d) {
  if (pa_check_desc(d) != PA_OK) return -1;
  return plan_grid(plan_decode(d), std::min(d->num_seqs, kMaxSeqs));
}

// Checks the call (a caller workspace too when check_ws) and fills every
// field of the kernel arguments except the workspace pointers
// (bind_workspace).  Argument errors come before any device query.
// *grid = 0: nothing to launch.
static int32_t prepare(const void* q, const void* k_pool, const void* v_pool, const int32_t* bt,
                       const int32_t* lens, float scale, void* out, const pa_desc* d,
                       const Plan& p, bool check_ws, const void* ws, size_t ws_bytes, Args* a,
                       int* grid) {
  const int32_t st = pa_check_desc(d);
  if (st != PA_OK) return st;
  *grid = 0;
  if (d->num_seqs == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !bt || !lens || !out) return PA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)out) & 15u) return PA_ERR_ALIGN;
  if (check_ws && (!ws || ws_bytes < pa_workspace_bytes(d) || ((uintptr_t)ws & 15u)))
    return PA_ERR_WORKSPACE;
  if (!device_info().ok) return PA_ERR_DEVICE;
  const int g = plan_grid(p, d->num_seqs);
  if (g <= 0) return PA_ERR_UNSUPPORTED;  // LDS of this batch size and group does not fit
  a->q = q;
  a->kp = k_pool;
  a->vp = v_pool;
  a->bt = bt;
  a->lens = lens;
  a->out = out;
  a->scale_log2 = scale * kLog2e;
  a->S = d->num_seqs;
  a->Hq = d->num_q_heads;
  a->Hkv = p.hkv;
  a->Hp = d->num_kv_heads;
  a->kv_split = p.split;
  a->kv_shift = p.shift;
  a->mbs = d->max_blocks_per_seq;
  a->nwg = g;
  a->out_f32 = d->out_dtype == PA_F32 ? 1 : 0;
  a->cached_blocks = d->cached_prefix_blocks;
  a->grp_start = nullptr;
  a->grp_shared = nullptr;
  a->ngroups = 0;
  a->pcnt = nullptr;
  a->pair_o = a->pair_ml = a->wide_o = a->wide_ml = nullptr;
  a->stage_cap = 0;
  *grid = g;
  return PA_OK;
}

int32_t paged_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* bt, const int32_t* lens, float scale, void* out,
                          const pa_desc* d, void* ws, size_t ws_bytes, void* stream) {
  Args a;
  int grid = 0;
  const int32_t st0 = pa_check_desc(d);
  if (st0 != PA_OK) return st0;
  if (d->num_seqs > kMaxSeqs)
    return decode_in_slices(q, bt, lens, out, d, [&](const pa_desc* ds, int64_t s0) {
      return paged_attn_decode(static_cast<const char*>(q) + rows_bytes(d, s0, d->dtype), k_pool,
                               v_pool, bt + s0 * d->max_blocks_per_seq, lens + s0, scale,
                               static_cast<char*>(out) + rows_bytes(d, s0, d->out_dtype), ds, ws,
                               ws_bytes, stream);
    });
  const Plan p = plan_decode(d);
  const int32_t st = prepare(q, k_pool, v_pool, bt, lens, scale, out, d, p, true, ws, ws_bytes,
                             &a, &grid);
  if (st != PA_OK || grid == 0) return st;
  bind_workspace(&a, ws, kMaxGrid, 2 * kMaxGrid, p.G);
  if (p.v.launch(a, grid, prefix_lds(a.S), static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

int32_t paged_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* bt, const int32_t* lens, float scale, void* out,
                                  const pa_desc* d, void* stream) {
  Args a;
  int grid = 0;
  const int32_t st0 = pa_check_desc(d);
  if (st0 != PA_OK) return st0;
  if (d->num_seqs > kMaxSeqs)
    return decode_in_slices(q, bt, lens, out, d, [&](const pa_desc* ds, int64_t s0) {
      return paged_attn_decode_noalloc(static_cast<const char*>(q) + rows_bytes(d, s0, d->dtype),
                                       k_pool, v_pool, bt + s0 * d->max_blocks_per_seq, lens + s0,
                                       scale, static_cast<char*>(out) + rows_bytes(d, s0, d->out_dtype),
                                       ds, stream);
    });
  // A column-split group whose partials would overflow the static scratch
  // runs as virtual groups of 16 heads instead.
  Plan p = plan_decode(d);
  if (p.G > 16) {
    const int g = plan_grid(p, d->num_seqs);
    if (g > 0 && ws_layout_bytes(g, 2 * g, p.G) > kScratchBytes) p = plan_decode(d, 16);
  }
  const int32_t st = prepare(q, k_pool, v_pool, bt, lens, scale, out, d, p, false, nullptr, 0,
                             &a, &grid);
  if (st != PA_OK || grid == 0) return st;
  const int G = p.G;
  if (ws_layout_bytes(grid, 2 * grid, G) > kScratchBytes) return PA_ERR_SCRATCH;
  void* ws = scratch_ptr();
  if (!ws) return PA_ERR_DEVICE;
  bind_workspace(&a, ws, grid, 2 * grid, G);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the split counters must start at zero: a fill kernel (no memset node,
  // so the pair of launches can also be captured into a graph)
  hipLaunchKernelGGL(clear_ints_kernel, dim3(1), dim3(256), 0, s, a.counters, grid);
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  if (p.v.launch(a, grid, prefix_lds(a.S), s) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

size_t pa_shared_workspace_bytes(const pa_desc* d) {
  if (pa_check_desc(d) != PA_OK) return 0;
  return shared_ws_layout(d).total;
}

int32_t pa_validate_shared_host(const pa_desc* d, const int32_t* bt, const int32_t* lens,
                                const int32_t* group_start, const int32_t* group_shared,
                                int32_t num_groups) {
  const int32_t st = pa_validate_host(d, bt, lens);
  if (st != PA_OK) return st;
  if (num_groups < 0) return PA_ERR_SHAPE;
  if (num_groups == 0) return PA_OK;
  if (!group_start || !group_shared) return PA_ERR_NULL;
  if (group_start[0] < 0 || group_start[num_groups] > d->num_seqs) return PA_ERR_SHAPE;
  const int64_t B = d->block_size, mbs = d->max_blocks_per_seq;
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t f = group_start[g], e = group_start[g + 1];
    if (e < f || group_shared[g] < 0) return PA_ERR_SHAPE;
    if (e - f < 2 || group_shared[g] == 0) continue;
    // the member covering the most shared blocks holds the reference row
    int32_t ref = f;
    int64_t most = -1;
    for (int32_t b = f; b < e; ++b) {
      const int64_t nb = std::min<int64_t>(pa_blocks_for_len(lens[b], d->block_size), group_shared[g]);
      if (nb > most) {
        most = nb;
        ref = b;
      }
    }
    for (int32_t b = f; b < e; ++b) {
      const int64_t nb = std::min<int64_t>(pa_blocks_for_len(lens[b], d->block_size), group_shared[g]);
      for (int64_t j = 0; j < nb; ++j)
        if (bt[b * mbs + j] != bt[ref * mbs + j]) return PA_ERR_TABLE;
    }
  }
  (void)B;
  return PA_OK;
}

int32_t pa_decode_shared_grid(const pa_desc* d, int32_t num_groups) {
  if (pa_check_desc(d) != PA_OK || num_groups < 0) return -1;
  if (d->num_seqs > kMaxSeqs) return pa_decode_grid(d);  // runs as the ordinary decode
  const DeviceInfo info = device_info();
  if (!info.ok) return -1;
  const Variant v = pick_shared(d);
  if (!v.launch) return -1;
  const int per_cu = v.occ(shared_lds(d->num_seqs, num_groups));
  if (per_cu <= 0) return -1;
  int grid = info.cus * per_cu;
  if (grid > kMaxSharedGrid) grid = kMaxSharedGrid;
  return grid;
}

int32_t paged_attn_decode_shared(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* bt, const int32_t* lens,
                                 const int32_t* group_start, const int32_t* group_shared,
                                 int32_t num_groups, float scale, void* out, const pa_desc* d,
                                 void* ws, size_t ws_bytes, void* stream) {
  const int32_t st0 = pa_check_desc(d);
  if (st0 != PA_OK) return st0;
  if (num_groups < 0) return PA_ERR_SHAPE;
  if (num_groups > 0 && (!group_start || !group_shared)) return PA_ERR_NULL;
  if (d->num_seqs > 0 && (!ws || ws_bytes < shared_ws_layout(d).total || ((uintptr_t)ws & 15u)))
    return PA_ERR_WORKSPACE;
  const Variant v = pick_shared(d);
  // no group to share, not the matrix-core kernel, or a batch whose
  // schedule does not fit the workgroup's LDS (more than kMaxSeqs
  // sequences: the ordinary decode, in slices)
  if (num_groups == 0 || !v.launch || d->num_seqs > kMaxSeqs)
    return paged_attn_decode(q, k_pool, v_pool, bt, lens, scale, out, d, ws, ws_bytes, stream);
  Args a;
  int grid = 0;
  // the shared kernel's groups are held directly (split 1), as in the plain plan
  const int32_t st = prepare(q, k_pool, v_pool, bt, lens, scale, out, d, plan_decode(d), true, ws,
                             ws_bytes, &a, &grid);
  if (st != PA_OK || grid == 0) return st;
  grid = pa_decode_shared_grid(d, num_groups);
  if (grid <= 0) return PA_ERR_UNSUPPORTED;  // LDS of this batch and its groups does not fit
  a.nwg = grid;
  const int G = d->num_q_heads / d->num_kv_heads;
  bind_workspace(&a, ws, kMaxGrid, 2 * kMaxGrid, G);
  bind_shared_workspace(&a, ws, shared_ws_layout(d));
  a.grp_start = group_start;
  a.grp_shared = group_shared;
  a.ngroups = num_groups;
  const size_t base = shared_lds(a.S, num_groups);
  const size_t entry = sizeof(float) * (size_t)(G * kD + 2 * G);
  a.stage_cap = stage_capacity(v, base, entry);
  if (v.launch(a, grid, base + (size_t)a.stage_cap * entry, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

int32_t pa_validate_append_host(const pa_desc* d, const int32_t* bt, const int32_t* pos) {
  const int32_t st = pa_check_desc(d);
  if (st != PA_OK) return st;
  if (d->num_seqs > 0 && (!bt || !pos)) return PA_ERR_NULL;
  const int64_t cap = (int64_t)d->max_blocks_per_seq * d->block_size;
  std::unordered_set<int64_t> seen;
  for (int32_t b = 0; b < d->num_seqs; ++b) {
    const int32_t t = pos[b];
    if (t < 0) continue;
    if (t >= cap) return PA_ERR_TABLE;
    const int32_t id = bt[(int64_t)b * d->max_blocks_per_seq + t / d->block_size];
    if (id < 0 || id >= d->num_blocks) return PA_ERR_TABLE;
    if (!seen.insert((int64_t)id * d->block_size + t % d->block_size).second) return PA_ERR_TABLE;
  }
  return PA_OK;
}

int32_t paged_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                        const int32_t* bt, const int32_t* pos, const pa_desc* d, void* stream) {
  const int32_t st = pa_check_desc(d);
  if (st != PA_OK) return st;
  if (d->num_seqs == 0) return PA_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !bt || !pos) return PA_ERR_NULL;
  if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_pool | (uintptr_t)v_pool) & 15u)
    return PA_ERR_ALIGN;
  if (!device_info().ok) return PA_ERR_DEVICE;
  AppendArgs a;
  a.kn = k_new;
  a.vn = v_new;
  a.kp = k_pool;
  a.vp = v_pool;
  a.bt = bt;
  a.pos = pos;
  a.S = d->num_seqs;
  a.Hkv = d->num_kv_heads;
  a.B = d->block_size;
  a.mbs = d->max_blocks_per_seq;
  const int grid = (int)(((int64_t)a.S * a.Hkv + kAuxWaves - 1) / kAuxWaves);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return launch_append(a, (int)pa_dtype_size(d->dtype), grid, s) == hipSuccess ? PA_OK
                                                                              : PA_ERR_LAUNCH;
}

int32_t pa_validate_copy_host(const pa_desc* d, const int32_t* src, const int32_t* dst,
                              int32_t n) {
  const int32_t st = pa_check_desc(d);
  if (st != PA_OK) return st;
  if (n < 0) return PA_ERR_SHAPE;
  if (n > 0 && (!src || !dst)) return PA_ERR_NULL;
  std::unordered_set<int32_t> dsts, srcs;
  for (int32_t i = 0; i < n; ++i) {
    if (src[i] < 0 || src[i] >= d->num_blocks || dst[i] < 0 || dst[i] >= d->num_blocks)
      return PA_ERR_TABLE;
    if (!dsts.insert(dst[i]).second) return PA_ERR_TABLE;
    srcs.insert(src[i]);
  }
  for (int32_t x : dsts)
    if (srcs.count(x)) return PA_ERR_TABLE;
  return PA_OK;
}

int32_t paged_kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst,
                             int32_t n, const pa_desc* d, void* stream) {
  const int32_t st = pa_check_desc(d);
  if (st != PA_OK) return st;
  if (n < 0) return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!k_pool || !v_pool || !src || !dst) return PA_ERR_NULL;
  if (((uintptr_t)k_pool | (uintptr_t)v_pool) & 15u) return PA_ERR_ALIGN;
  const DeviceInfo info = device_info();
  if (!info.ok) return PA_ERR_DEVICE;
  CopyArgs a;
  a.kp = static_cast<char*>(k_pool);
  a.vp = static_cast<char*>(v_pool);
  a.src = src;
  a.dst = dst;
  a.block_bytes = (int64_t)d->num_kv_heads * d->block_size * d->head_dim * pa_dtype_size(d->dtype);
  a.chunks = (int32_t)(a.block_bytes / kChunkBytes);  // head_dim 128, B in {16, 32}: exact
  const int64_t total = (int64_t)n * 2 * a.chunks;
  if (total >= ((int64_t)1 << 31)) return PA_ERR_UNSUPPORTED;
  a.total = (int32_t)total;
  int64_t grid = (total + kCopyUnroll - 1) / kCopyUnroll;
  const int64_t cap = (int64_t)info.cus * 8;
  if (grid > cap) grid = cap;
  return launch_copy_blocks(a, (int)grid, static_cast<hipStream_t>(stream)) == hipSuccess
             ? PA_OK
             : PA_ERR_LAUNCH;
}

int32_t paged_kv_block_scores(const void* k_pool, const void* v_pool, const int32_t* bt,
                              const int32_t* lens, float* scores, int32_t* evict,
                              const pa_desc* d, void* stream) {
  const int32_t st = pa_check_desc(d);
  if (st != PA_OK) return st;
  if (d->num_seqs == 0) return PA_OK;
  if (!k_pool || !v_pool || !bt || !lens || !scores || !evict) return PA_ERR_NULL;
  if (((uintptr_t)k_pool | (uintptr_t)v_pool) & 15u) return PA_ERR_ALIGN;
  if (((uintptr_t)scores | (uintptr_t)evict) & 3u) return PA_ERR_ALIGN;
  if (!device_info().ok) return PA_ERR_DEVICE;
  ScoreArgs a;
  a.kp = k_pool;
  a.vp = v_pool;
  a.bt = bt;
  a.lens = lens;
  a.scores = scores;
  a.evict = evict;
  a.S = d->num_seqs;
  a.Hkv = d->num_kv_heads;
  a.mbs = d->max_blocks_per_seq;
  return launch_block_scores(a, d->dtype, d->block_size, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? PA_OK
             : PA_ERR_LAUNCH;
}

struct pa_block_manager {
  pa::BlockManager m;
};

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  try {
    return new pa_block_manager{pa::BlockManager(num_blocks, block_size)};
  } catch (...) {
    return nullptr;
  }
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_num_free(const pa_block_manager* bm) { return bm ? bm->m.num_free() : -1; }

int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block) {
  return bm ? bm->m.refcount(block) : -1;
}

int32_t pa_bm_alloc(pa_block_manager* bm, int32_t n, int32_t* ids) {
  if (!bm || (n > 0 && !ids)) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (!bm->m.reserve(n)) return PA_ERR_NOMEM;
  bm->m.take_reserved_n(n, ids);
  return PA_OK;
}

int32_t pa_bm_release(pa_block_manager* bm, const int32_t* ids, int32_t n) {
  if (!bm || (n > 0 && !ids)) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  return bm->m.drop_n(ids, n) == n ? PA_OK : PA_ERR_TABLE;
}

int32_t pa_bm_share(pa_block_manager* bm, const int32_t* ids, int32_t n) {
  if (!bm || (n > 0 && !ids)) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i)
    if (!bm->m.share(ids[i])) return PA_ERR_TABLE;
  return PA_OK;
}

int32_t pa_bm_prepare_append(pa_block_manager* bm, int32_t* bt, int32_t mbs, const int32_t* lens,
                             int32_t num_seqs, int32_t* pos, int32_t* cow_src, int32_t* cow_dst,
                             int32_t* num_cow) {
  if (!bm || !num_cow) return PA_ERR_NULL;
  *num_cow = 0;
  if (num_seqs < 0 || mbs <= 0) return PA_ERR_SHAPE;
  if (num_seqs > 0 && (!bt || !lens || !pos || !cow_src || !cow_dst)) return PA_ERR_NULL;
  const int32_t B = bm->m.block_size();
  // Pass 1: validate every sequence and decide what it needs (a copy of a
  // block shared only within this batch is needed once: after the first
  // writer copies it, the next one owns it alone); count the fresh blocks.
  enum : uint8_t { kKeep = 0, kFresh = 1, kCopy = 2 };
  std::vector<uint8_t> act(num_seqs > 0 ? num_seqs : 0, kKeep);
  std::unordered_map<int32_t, int32_t> drops;
  int32_t need = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t L = lens[b];
    if (L < 0) continue;
    if (L / B >= mbs) return PA_ERR_TABLE;
    if (L % B == 0) {
      act[b] = kFresh;
      ++need;
      continue;
    }
    const int32_t e = bt[(int64_t)b * mbs + L / B];
    const int32_t rc = bm->m.refcount(e) - (drops.count(e) ? drops[e] : 0);
    if (rc <= 0) return PA_ERR_TABLE;
    if (rc > 1) {
      act[b] = kCopy;
      ++need;
      ++drops[e];
    }
  }
  // All or nothing: the fresh blocks are reserved before any is taken, and
  // taken in one go (in the order single takes would give them: the drops
  // below never free a block, since each drops one of several references).
  if (!bm->m.reserve(need)) return PA_ERR_NOMEM;
  std::vector<int32_t> fresh(need > 0 ? need : 1);
  bm->m.take_reserved_n(need, fresh.data());
  int32_t next = 0;
  // Pass 2: apply the decisions (cannot fail).
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t L = lens[b];
    if (L < 0) {
      pos[b] = -1;
      continue;
    }
    int32_t* entry = bt + (int64_t)b * mbs + L / B;
    if (act[b] == kFresh) {
      *entry = fresh[next++];
    } else if (act[b] == kCopy) {
      const int32_t id = fresh[next++];
      cow_src[*num_cow] = *entry;
      cow_dst[*num_cow] = id;
      ++*num_cow;
      bm->m.drop(*entry);
      *entry = id;
    }
    pos[b] = L;
  }
  return PA_OK;
}

int32_t pa_validate_prefill_host(const pa_desc* d, const int32_t* bt, const int32_t* lens,
                                 const int32_t* q_start, int32_t max_q_len) {
  const int32_t st = pa_validate_host(d, bt, lens);
  if (st != PA_OK) return st;
  if (!q_start) return PA_ERR_NULL;
  if (max_q_len < 0) return PA_ERR_SHAPE;
  if (q_start[0] != 0) return PA_ERR_TABLE;
  for (int32_t b = 0; b < d->num_seqs; ++b) {
    const int64_t n = (int64_t)q_start[b + 1] - q_start[b];
    if (n < 0 || n > max_q_len || n > lens[b]) return PA_ERR_TABLE;
  }
  return PA_OK;
}

int32_t paged_attn_prefill(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* bt, const int32_t* lens, const int32_t* q_start,
                           int32_t max_q_len, float scale, void* out, const pa_desc* d,
                           void* stream) {
  const int32_t st = pa_check_desc(d);
  if (st != PA_OK) return st;
  if (max_q_len < 0) return PA_ERR_SHAPE;
  const PrefillPlan pp = plan_prefill(d);
  if (!pp.fn) return PA_ERR_UNSUPPORTED;
  if (d->num_seqs == 0 || max_q_len == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !bt || !lens || !q_start || !out) return PA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)out) & 15u) return PA_ERR_ALIGN;
  if (!device_info().ok) return PA_ERR_DEVICE;
  // row blocks of one workgroup: kPrefillWaves waves of kPrefillTiles column tiles
  const int rows_per_block = kPrefillWaves * kPrefillTiles * (kSub / pp.G);
  const int64_t tiles = (max_q_len + rows_per_block - 1) / rows_per_block;
  const int64_t hkv = (int64_t)d->num_kv_heads * pp.split;  // virtual KV heads
  const int64_t pairs = hkv * d->num_seqs;
  const int64_t blocks = 8 * ((pairs + 7) / 8) * tiles;  // XCD-major order (prefill_kernel)
  if (blocks >= ((int64_t)1 << 31)) return PA_ERR_UNSUPPORTED;
  PrefillArgs a;
  a.q = q;
  a.kp = k_pool;
  a.vp = v_pool;
  a.bt = bt;
  a.lens = lens;
  a.qs = q_start;
  a.out = out;
  a.scale_log2 = scale * kLog2e;
  a.S = d->num_seqs;
  a.Hq = d->num_q_heads;
  a.Hkv = (int32_t)hkv;
  a.Hp = d->num_kv_heads;
  a.kv_split = pp.split;
  a.kv_shift = pp.shift;
  a.mbs = d->max_blocks_per_seq;
  a.tiles = (int32_t)tiles;
  a.out_f32 = d->out_dtype == PA_F32 ? 1 : 0;
  pp.fn(a, dim3((unsigned)blocks), static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"
