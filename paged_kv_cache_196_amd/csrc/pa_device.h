// pa_device.h — device-side building blocks shared by the gfx950 decode and
// merge kernels: element types, wave64 cross-lane helpers, the work schedule
// (which workgroup handles which logical blocks of which (sequence, KV head))
// and the cross-wave / cross-partition combination of softmax partials.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kD = 128;          // head_dim the kernels are built for
constexpr int kWaves = 8;        // waves per decode workgroup (one workgroup per CU)
constexpr int kThreads = 64 * kWaves;
constexpr int kAuxWaves = 4;     // waves per workgroup of the cache-write and scan kernels
constexpr int kAuxThreads = 64 * kAuxWaves;
constexpr int kSub = 16;         // tokens per sub-tile (unit of the streaming loop)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxGrid = 2048;   // upper bound on decode workgroups (sizes the workspace)
constexpr int kWideCols = 32;    // MFMA columns of a prefix item: members x query heads
constexpr int kMaxSeqs = 8192;   // sequences per decode launch (LDS prefix array); larger batches run in slices

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Element-type tags.
struct F32 { static constexpr int kEsize = 4; static constexpr int kCode = 0; };
struct F16 { static constexpr int kEsize = 2; static constexpr int kCode = 1; };
struct BF16 { static constexpr int kEsize = 2; static constexpr int kCode = 2; };

// Kernel arguments (one struct, passed by value).
struct Args {
  const void* q;
  const void* kp;
  const void* vp;
  const int32_t* bt;
  const int32_t* lens;
  void* out;
  float* ws_o;    // [kMaxGrid*2][G][kD] partial weighted-V sums
  float* ws_ml;   // [kMaxGrid*2][G][2]  partial (max, sum of exp), log2 domain
  int* counters;  // [kMaxGrid] pieces finished per split (sequence, KV head)
  float scale_log2;  // scale * log2(e): scores are kept in base-2 exponent units
  int32_t S, Hq, Hkv, mbs, nwg, out_f32;
  // Virtual KV heads: a query group of split * G heads runs as `split`
  // groups of G, one per virtual KV head; Hkv counts virtual heads, Hp the
  // pool's heads, and virtual head v reads pool head v / split (shift =
  // log2(split) when a power of two, else -1).
  int32_t Hp, kv_split, kv_shift;
  int32_t cached_blocks;  // leading logical blocks read with the cache-retaining policy
  // Prefix groups (shared-prefix calls only; ngroups = 0 otherwise).
  const int32_t* grp_start;   // [ngroups + 1] group i = sequences grp_start[i] .. grp_start[i+1]-1
  const int32_t* grp_shared;  // [ngroups] leading table entries every member shares
  int32_t ngroups;
  int* pcnt;       // [S*Hkv] arrival counters of member pairs
  float* pair_o;   // [S*Hkv][2][G][kD] whole contributions: [0] item, [1] private part
  float* pair_ml;  // [S*Hkv][2][G][2]
  float* wide_o;   // [2*kMaxGrid][kWideCols][kD] item fragments cut by chunk boundaries
  float* wide_ml;  // [2*kMaxGrid][kWideCols][2]
  int32_t stage_cap;  // member partials the workgroup's LDS can hold until its next count-in
};

// Pool KV head of virtual KV head kvh (the K/V tiles it reads).
template <class A>
__device__ __forceinline__ int pool_head(const A& a, int kvh) {
  return a.kv_shift >= 0 ? kvh >> a.kv_shift : kvh / a.kv_split;
}

// ------------------------------------------------------------ conversions

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
}

// Two consecutive 16-bit elements packed in one dword -> floats.
template <class T>
__device__ __forceinline__ void unpack2(uint32_t u, float& a, float& b) {
  if constexpr (T::kCode == BF16::kCode) {
    a = bf16_lo(u);
    b = bf16_hi(u);
  } else {
    a = f16_lo(u);
    b = f16_hi(u);
  }
}

// One 16-byte chunk -> E floats (E = 16 / esize).
template <class T>
__device__ __forceinline__ void chunk_to_float(const uint4& c, float* f) {
  if constexpr (T::kCode == F32::kCode) {
    f[0] = __uint_as_float(c.x);
    f[1] = __uint_as_float(c.y);
    f[2] = __uint_as_float(c.z);
    f[3] = __uint_as_float(c.w);
  } else {
    unpack2<T>(c.x, f[0], f[1]);
    unpack2<T>(c.y, f[2], f[3]);
    unpack2<T>(c.z, f[4], f[5]);
    unpack2<T>(c.w, f[6], f[7]);
  }
}

// float -> output element, round to nearest even.
template <class T>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, int out_f32) {
  if (out_f32) {
    static_cast<float*>(out)[idx] = v;
  } else if constexpr (T::kCode == BF16::kCode) {
    static_cast<__bf16*>(out)[idx] = (__bf16)v;
  } else if constexpr (T::kCode == F16::kCode) {
    static_cast<_Float16*>(out)[idx] = (_Float16)v;
  } else {
    static_cast<float*>(out)[idx] = v;
  }
}

// ----------------------------------------------------- cross-lane helpers
// DPP moves within a row of 16 lanes (quad_perm / half-mirror / mirror).
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum / max over the 16 lanes of a row; every lane of the row gets the result.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  return x;
}

// Lane exchange across rows of 16: lane i receives lane i ^ m (m = 16, 32).
__device__ __forceinline__ float xor_lanes(float x, int m) { return __shfl_xor(x, m); }

// Butterfly steps across the four 16-lane rows without the LDS crossbar.
// v_permlane32_swap(x, x) leaves rows (0,1,0,1) in one result and (2,3,2,3)
// in the other; v_permlane16_swap(x, x) leaves (0,0,2,2) and (1,1,3,3).
// Combining the two results is the i ^ 32 (resp. i ^ 16) butterfly.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------ K/V tile access
//
// Each (physical block, KV head) tile is read through a raw buffer resource
// whose base is the tile itself: the per-tile address arithmetic stays on
// the scalar unit (the tile base is wave-uniform), every lane's offset
// inside the tile is a constant, and the hardware range check of the
// resource (num_records = tile bytes) keeps every access inside the tile.
// Loads carry the streaming (non-temporal) cache policy: each K/V byte is
// used once per call, and on gfx950 this policy let random 4 KiB tile
// gathers reach ~6.4-6.6 TB/s versus ~5.9 TB/s with the default policy.
// Blocks that several sequences of the batch share (a common prefix) are
// read with the default, cache-retaining policy instead, so that every
// sequence after the first finds them in L2 or the Infinity Cache.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStreamPolicy = 2;                // nt
constexpr int kCachedPolicy = 0;                // default
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* pool, int64_t byte_off,
                                                            int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(pool)) + byte_off, (short)0, bytes, kRsrcWord3);
}
template <int kPolicy>
__device__ __forceinline__ uint4 tile_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kPolicy);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int kPolicy>
__device__ __forceinline__ uint2 tile_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kPolicy);
  return make_uint2(v.x, v.y);
}

// True in every lane when any lane of the wave has `pred` set.
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Read-only int32 data seen through the constant address space: the kernels
// never write the block tables, so a wave-uniform index becomes a scalar
// load (s_load), which waits on lgkmcnt and leaves the vector-memory queue
// of in-flight K/V loads alone.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ const_i32_ptr as_constant(const int32_t* p) {
  return (const_i32_ptr)(p);
}

// ------------------------------------------------------------ schedule
//
// Work unit = one logical block of one (sequence, KV head).  Units are
// flattened sequence-major: unit (b, kvh, j) has index
//     cum[b] * Hkv + kvh * n_b + j,      n_b = ceil(L_b / B),
// and cum[] is the exclusive prefix sum of n_b.  The W = cum[S] * Hkv units
// are cut into nwg equal contiguous chunks; chunk k (one workgroup) handles
// [k*c, min((k+1)*c, W)) with c = ceil(W / nwg).  Within a chunk the work
// falls into pieces, one per (sequence, KV head) it meets; at most the first
// and the last piece are partial (the pair continues in a neighbouring
// chunk).  Whole pairs are written straight to `out`.  A partial piece's
// (max, sum of exp, weighted V) belongs in workspace slot
// 2*k + (piece is first in chunk ? 0 : 1); each split is folded exactly
// once, by the workgroup that completes it: the one whose count-in is the
// last, or a chunk's final piece that finds every other piece already
// counted in and folds without publishing its own (finish_late).

__device__ __forceinline__ int blocks_of(int len, int B) { return len > 0 ? (len + B - 1) / B : 0; }

// cum[0..S] (exclusive prefix of block counts) and a copy of the lengths in
// LDS.  All threads call.
__device__ inline void build_prefix(const int32_t* __restrict__ lens, int S, int B, int* cum,
                                    int* lens_s, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < S; base += kThreads) {
    const int b = base + tid;
    const int len = b < S ? lens[b] : 0;
    if (b < S) lens_s[b] = len;
    int x = blocks_of(len, B);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = carry, total = carry;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) before += wsum[w];
      total += wsum[w];
    }
    if (b < S) cum[b + 1] = before + x;
    carry = total;
    __syncthreads();
  }
  if (tid == 0) cum[0] = 0;
  __syncthreads();
}

// Sequence whose units contain flat index f (0 <= f < W): the last b with
// cum[b]*Hkv <= f.  Skips empty sequences by construction.
__device__ __forceinline__ int find_seq(const int* cum, int S, int Hkv, int f) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cum[mid] * Hkv <= f) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Chunk handled by workgroup `wg`.  Consecutive chunks go to workgroups on
// the same XCD (workgroups are dispatched round-robin over the 8 XCDs), so
// sequences that share prefix blocks tend to hit the same L2.
__device__ __forceinline__ int chunk_of_wg(int wg, int nwg) {
  if (nwg % 8 != 0) return wg;
  return (wg % 8) * (nwg / 8) + wg / 8;
}

// One piece of work: the tokens [tok_begin, tok_end) of (sequence b, KV
// head kvh), nsub 16-token sub-tiles.  When the pair is split over several
// chunks, its pieces occupy workspace slots first_slot (chunk kfirst) and
// 2*k (chunks kfirst+1 .. kfirst+npieces-1); this piece is `slot`.
//
// Kinds.  A whole piece covers its pair and writes `out` itself.  A partial
// piece that opens its chunk and has more work after it is "early": it is
// published and counted in as soon as it is merged, mid-chunk.  Any other
// partial piece ends its chunk ("late"); by then its partners have usually
// been counted in, so it folds the split without publishing its own part.
//
// A piece of a member pair (a sequence whose leading blocks are attended by
// its prefix group's item, shared_prefix.h) is of kind kMember whatever its
// extent: the pair always has at least two contributions (the item's and
// its private blocks'), published and counted in on the pair's own counter.
enum : int { kWhole = 0, kEarly = 1, kLate = 2, kMember = 3 };

struct Piece {
  int b, kvh, L;
  int tok_begin, tok_end, nsub;
  int kind;
  int slot, kfirst, npieces, first_slot;
};

__device__ __forceinline__ Piece uniform_piece(const Piece& p) {
  Piece u;
  u.b = uniform(p.b);
  u.kvh = uniform(p.kvh);
  u.L = uniform(p.L);
  u.tok_begin = uniform(p.tok_begin);
  u.tok_end = uniform(p.tok_end);
  u.nsub = uniform(p.nsub);
  u.kind = uniform(p.kind);
  u.slot = uniform(p.slot);
  u.kfirst = uniform(p.kfirst);
  u.npieces = uniform(p.npieces);
  u.first_slot = uniform(p.first_slot);
  return u;
}

// ------------------------------------------------ partial combination
//
// Merge of softmax partials ("39 · PagedAttention", §3 "On the GPU", merge
// equation): m = max(m1, m2); l = l1 e^(m1-m) + l2 e^(m2-m); the weighted-V
// sums rescale the same way, and out = o / l.  Scores here are in base-2
// units (scaled by log2 e), so e^(m1-m) becomes 2^(m1-m).  An empty partial
// (m = -inf, l = 0, o = 0) is the identity.
//
// Two levels use it: the kWaves waves of a workgroup (through LDS, at the
// end of every piece) and the pieces of a (sequence, KV head) that chunk
// boundaries cut (through the workspace, by the workgroup that counts the
// last of those pieces in).

constexpr int kQueryLdsBytes = 32768;
constexpr int kFoldLoads = 64;  // workspace loads per thread in flight when folding a split

// Query groups wider than one MFMA column tile (MQA: 32 or 64 heads on one
// KV head): every wave scores each K/V sub-tile it loads against two
// column tiles of 16 heads (32 heads), and the waves form G / 32 column
// groups of kColWaves waves; a group takes its 32 heads and deals the
// sub-tiles among its own waves.  Two groups (64 heads) read the same
// sub-tiles, kept within a few passes of each other by barriers in the
// stream (stream_batch), so each is fetched from HBM once.
// Merging goes through the 16-column wave arrays one column tile (round)
// at a time.
template <int G>
constexpr int kTilesPerWave = G > 16 ? 2 : 1;
template <int G>
constexpr int kColGroups = G > 16 ? G / 32 : 1;
template <int G>
constexpr int kColWaves = kWaves / kColGroups<G>;
static_assert(kColGroups<64> <= kWaves, "one wave at least per column group");

// Pieces listed per batch: their query groups are staged in LDS together.
template <class T, int G>
constexpr int piece_batch() {
  constexpr int per = G * kD * T::kEsize;
  constexpr int n = kQueryLdsBytes / per;
  return n > 32 ? 32 : n;
}

// A softmax partial (log2-domain max m, sum of exponentials l, weighted-V
// sum o) for the outputs this thread owns: flat index idx = threadIdx.x +
// r * kThreads of the G x kD outputs, (g, d) = (idx / kD, idx % kD).
template <int G>
struct Partial {
  static constexpr int kOut = (G * kD + kThreads - 1) / kThreads;
  // pieces per fold round (half the loads in flight for column-split
  // groups, whose many outputs per thread would not fit the registers)
  static constexpr int kLoads = G > 16 ? kFoldLoads / 2 : kFoldLoads;
  static constexpr int kPer = kLoads / kOut < 32 ? kLoads / kOut : 32;
  float m[kOut], l[kOut], o[kOut];
};

// Schedule of a shared-prefix call, in dynamic LDS (built by the prologue
// of shared_prefix.h).  Sequence b attends its first shb[b] blocks through
// its sub-group's item and the rest as private blocks; cum is the prefix
// of private units (private blocks plus V virtual units per sequence with
// any), icum of item block counts; cI / cP the chunk sizes of the item and
// private unit spaces.  The scalars live in the workgroup's LDS struct;
// the array addresses are recomputed from the dynamic LDS symbol wherever
// they are used (shared_info), so that every access compiles to an LDS
// access (a pointer kept in memory would come back as a generic pointer,
// whose loads also wait for the wave's outstanding global stores).
struct SharedScalars {
  int nsg, cI, cP, V, B;
};

struct SharedInfo {
  const int* lens;      // [S]
  const int* shb;       // [S]
  const int* seq_sg;    // [S] sub-group of b, -1 when b has no item
  const int* cum;       // [S + 1]
  const int* sg_first;  // [nsg] first member
  const int* sg_count;  // [nsg] members
  const int* sg_ref;    // [nsg] member whose table row covers the whole item
  const int* sg_len;    // [nsg] tokens the item covers (longest member's shared part)
  const int* icum;      // [nsg + 1]
  int nsg, cI, cP, B;
  int V;                // virtual units charged per (sequence, KV head) with private blocks
};

// Dynamic LDS layout of a shared-prefix call (ints): lens, shb, seq_sg (S
// each), cum (S + 1), the group bounds and shared counts as loaded
// (ngroups + 1 each), gbase (ngroups + 1), four sub-group arrays (S each)
// and icum (S + 1).
struct SharedLayout {
  int *lens, *shb, *seq_sg, *cum, *gstart, *gshared, *gbase, *sg_first, *sg_count, *sg_ref,
      *sg_len, *icum;
  float* stage;  // [stage_cap][G * kD + 2 * G] member partials awaiting their count-in
};
__host__ __device__ constexpr int64_t shared_lds_ints(int64_t S, int64_t ngroups) {
  return 9 * S + 3 * (ngroups + 1) + 2;
}
__device__ __forceinline__ SharedLayout shared_layout(int S, int ng) {
  extern __shared__ int pa_shared_dyn[];
  SharedLayout l;
  l.lens = pa_shared_dyn;
  l.shb = l.lens + S;
  l.seq_sg = l.shb + S;
  l.cum = l.seq_sg + S;
  l.gstart = l.cum + S + 1;
  l.gshared = l.gstart + ng + 1;
  l.gbase = l.gshared + ng + 1;
  l.sg_first = l.gbase + ng + 1;
  l.sg_count = l.sg_first + S;
  l.sg_ref = l.sg_count + S;
  l.sg_len = l.sg_ref + S;
  l.icum = l.sg_len + S;
  l.stage = reinterpret_cast<float*>(l.icum + S + 1);
  return l;
}

// Where the contributions of member pair `pair` (= b * Hkv + kvh) live:
// first its item's (one whole-item partial in the pair slot, or one per
// fragment in the wide chunk slots first_i, 2 * (kf_i + 1), ...), then its
// private pieces' (one in the pair slot, or one per piece in the narrow
// chunk slots).  mi is the member's place among its item's columns.
struct MemberLayout {
  int pair, mi;
  int nfr, kf_i, first_i;  // item contributions
  int npp, kf_p, first_p;  // private contributions (npp = 0: none)
  int stage, own;          // LDS stage entry of contribution `own` (-1: none)
};

constexpr int kDefer = 128;  // member contributions waiting for their count-in

template <class T, int G, bool kWide = false>
struct MergeSmem {
  static constexpr int kBatch = piece_batch<T, G>();
  static constexpr int kFoldMl = Partial<G>::kPer * G;
  // the wide (prefix item) phase: every wave holds 16 columns of `o` and
  // the (max, sum) of its columns among all kWideCols in m / l
  // a column-split group: every wave holds the 16 columns of its tile
  static constexpr int kOCols = (kWide && G < 16) || G > 16 ? 16 : G;
  static constexpr int kMCols = kWide && G < kWideCols ? kWideCols : (G > 16 ? 16 : G);
  static constexpr int kDefers = kWide ? kDefer : 1;
  float o[kWaves][kOCols][kD + 4];
  float m[kWaves][kMCols];
  float l[kWaves][kMCols];
  // (max, sum) of the pieces of one folding round
  float pm[kFoldMl];
  float pl[kFoldMl];
  int flag;
  int seen;        // arrival count read for the piece being finished (-1: not read)
  int early_seen;  // count returned to this chunk's early piece (-1: none)
  // the chunk's current batch of pieces and their query groups
  Piece plist[kBatch];
  int npl, next_f;
  uint4 q[kBatch][G * kD * T::kEsize / 16];
  // this chunk's early and late pieces (folded at the end of the chunk
  // when this workgroup completes their split)
  Piece early, late;
  int fold_late;
  // member contributions published and not yet counted in (pair indices)
  int dpair[kDefers];
  int dlast[kDefers];
  int dstage[kDefers];  // LDS stage entry of a listed private part (-1: published)
  int dpiece[kDefers];  // its piece index among the pair's private pieces (-1: item part)
  MemberLayout dlay[kDefers];
  int dn, nstage;
  SharedScalars ssc;
  // The workgroup's own partial of a late piece (all G heads), kept in the
  // wave-partial arrays (free by then) with its heads laid out flat.
  __device__ float& own_o(int g, int d) { return (&o[0][0][0])[g * (kD + 4) + d]; }
  __device__ float& own_m(int g) { return (&m[0][0])[g]; }
  __device__ float& own_l(int g) { return (&l[0][0])[g]; }
  static_assert(kWaves * kOCols >= G && kWaves * kMCols >= G, "own partial fits the wave arrays");
};

// The shared-prefix schedule of this call (see SharedInfo).
template <class Smem>
__device__ __forceinline__ SharedInfo shared_info(const Args& a, const Smem& sm) {
  const SharedLayout l = shared_layout(a.S, a.ngroups);
  SharedInfo si;
  si.lens = l.lens;
  si.shb = l.shb;
  si.seq_sg = l.seq_sg;
  si.cum = l.cum;
  si.sg_first = l.sg_first;
  si.sg_count = l.sg_count;
  si.sg_ref = l.sg_ref;
  si.sg_len = l.sg_len;
  si.icum = l.icum;
  si.nsg = sm.ssc.nsg;
  si.cI = sm.ssc.cI;
  si.cP = sm.ssc.cP;
  si.V = sm.ssc.V;
  si.B = sm.ssc.B;
  return si;
}

__device__ __forceinline__ float rescale(float mi, float m) {
  return mi == -INFINITY ? 0.f : fast_exp2(mi - m);
}

// Workspace partials are exchanged between workgroups that may sit on
// different XCDs (separate L2s).  Every partial value is written and read
// with an agent-scope atomic (relaxed), so each one is coherent across the
// XCDs by itself; the arrival counters order them:
//   publish: every wave completes its partial stores (compiler barrier and
//     a wait for its vector memory counter), the workgroup synchronises,
//     and one thread counts in with an agent-scope read-modify-write;
//   fold: the thread that saw every other piece counted in (from its
//     count-in, or from a load of the counter) issues an agent-scope
//     acquire fence, and the workgroup reads the partials after a barrier.
// The count-in is not a release operation: on gfx950 an agent-scope release
// writes back the whole L2 of the XCD (buffer_wbl2), which measured 6 % of
// a GQA batch-64 call (one per workgroup) for nothing it has to order here,
// since the published values are atomic stores that have completed before
// the count-in is issued.  The acquire fence measured free.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int count_in(int* c) {
  return __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int counted(const int* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Pairs with the release count-ins whose total the calling thread saw.
__device__ __forceinline__ void acquire_counted() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void reset_count(int* c) {
  __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt immediate with vmcnt = 0 and the other counters at their
// maximum (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt
// high bits [15:14]): waits for vector memory operations only.
constexpr int kVmcntZero = 0x0F70;
// Waits until this wave's stores (and loads) have completed; no memory
// access is moved across it by the compiler either.
__device__ __forceinline__ void drain_vmem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Merge the kWaves wave partials the waves left in `sm` into this thread's
// outputs.  Callers synchronise before (waves wrote sm) and after.
// Merge of output (g, d) over waves w0 .. w0 + W - 1, whose partials of
// the head sit at column gl of the wave arrays.
template <int W, class Smem>
__device__ __forceinline__ void merge_output(const Smem& sm, int w0, int gl, int d, float& M,
                                             float& l, float& o) {
  M = sm.m[w0][gl];
#pragma unroll
  for (int w = 1; w < W; ++w) M = fmaxf(M, sm.m[w0 + w][gl]);
  o = 0.f;
  l = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const float f = rescale(sm.m[w0 + w][gl], M);
    o += f * sm.o[w0 + w][gl][d];
    l += f * sm.l[w0 + w][gl];
  }
}

template <class T, int G, class Smem>
__device__ inline void merge_waves(const Smem& sm, Partial<G>& pt) {
#pragma unroll
  for (int r = 0; r < Partial<G>::kOut; ++r) {
    const int idx = threadIdx.x + r * kThreads;
    pt.m[r] = -INFINITY;
    pt.l[r] = 0.f;
    pt.o[r] = 0.f;
    if (idx >= G * kD) continue;
    merge_output<kWaves>(sm, 0, idx / kD, idx % kD, pt.m[r], pt.l[r], pt.o[r]);
  }
}

template <class T, int G>
__device__ inline void store_result(const Args& a, const Piece& pc, const Partial<G>& pt) {
#pragma unroll
  for (int r = 0; r < Partial<G>::kOut; ++r) {
    const int idx = threadIdx.x + r * kThreads;
    if (idx >= G * kD) continue;
    const int g = idx / kD, d = idx % kD;
    store_out<T>(a.out, ((int64_t)pc.b * a.Hq + pc.kvh * G + g) * kD + d, pt.o[r] / pt.l[r],
                 a.out_f32);
  }
}

// A partial's rows: weighted-V sums o_base[g][kD], (max, sum) ml_base[g][2].
template <int G>
__device__ inline void store_rows(float* o_base, float* ml_base, const Partial<G>& pt) {
#pragma unroll
  for (int r = 0; r < Partial<G>::kOut; ++r) {
    const int idx = threadIdx.x + r * kThreads;
    if (idx >= G * kD) continue;
    const int g = idx / kD, d = idx % kD;
    st_agent(o_base + (int64_t)g * kD + d, pt.o[r]);
    if (d == 0) {
      st_agent(ml_base + (int64_t)g * 2 + 0, pt.m[r]);
      st_agent(ml_base + (int64_t)g * 2 + 1, pt.l[r]);
    }
  }
}

template <int G>
__device__ inline void store_partial(const Args& a, int slot, const Partial<G>& pt) {
  store_rows<G>(a.ws_o + (int64_t)slot * G * kD, a.ws_ml + (int64_t)slot * G * 2, pt);
}

// Folds the npieces partials of a split (sequence, KV head) and writes
// out = o / l.  The pieces are combined in piece order whoever folds, so
// the result does not depend on which workgroup arrived last.  The
// partial in workspace slot `own_slot` is the caller's own and is taken
// from `own` (its outputs) and sm.m[0] / sm.l[0] (its per-head max and
// sum) instead of memory; own_slot = -1 reads every piece.  Each round
// issues the weighted-V loads of up to kPer pieces together with their
// (max, sum) loads, so a split of up to kPer pieces costs one round trip.
// All threads call; the caller has seen every piece counted in.
template <class T, int G, class Smem>
__device__ inline void fold_split(const Args& a, Smem& sm, const Piece& pc,
                                  const Partial<G>& own, int own_slot) {
  constexpr int kOut = Partial<G>::kOut;
  constexpr int kPer = Partial<G>::kPer;
  auto slot_of = [&](int p) { return p == 0 ? pc.first_slot : 2 * (pc.kfirst + p); };
  Partial<G> acc;
#pragma unroll
  for (int r = 0; r < kOut; ++r) {
    acc.m[r] = -INFINITY;
    acc.l[r] = 0.f;
    acc.o[r] = 0.f;
  }
  for (int p0 = 0; p0 < pc.npieces; p0 += kPer) {
    const int np = min(kPer, pc.npieces - p0);
    float v[kOut][kPer];
#pragma unroll
    for (int r = 0; r < kOut; ++r) {
      const int idx = min(threadIdx.x + r * kThreads, G * kD - 1);
      const int g = idx / kD, d = idx % kD;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int slot = slot_of(p0 + q);
        v[r][q] = q >= np ? 0.f
                  : slot == own_slot ? own.o[r]
                  : ld_agent(a.ws_o + ((int64_t)slot * G + g) * kD + d);
      }
    }
    for (int e = threadIdx.x; e < np * G; e += kThreads) {
      const int slot = slot_of(p0 + e / G), g = e % G;
      const float* ml = a.ws_ml + ((int64_t)slot * G + g) * 2;
      const bool mine = slot == own_slot;
      sm.pm[e] = mine ? sm.own_m(g) : ld_agent(ml);
      sm.pl[e] = mine ? sm.own_l(g) : ld_agent(ml + 1);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kOut; ++r) {
      const int g = min(threadIdx.x + r * kThreads, G * kD - 1) / kD;
      float M = acc.m[r];
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        if (q < np) M = fmaxf(M, sm.pm[q * G + g]);
      const float f0 = rescale(acc.m[r], M);
      float l = acc.l[r] * f0, o = acc.o[r] * f0;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        if (q < np) {
          const float f = rescale(sm.pm[q * G + g], M);
          l += f * sm.pl[q * G + g];
          o += f * v[r][q];
        }
      }
      acc.m[r] = M;
      acc.l[r] = l;
      acc.o[r] = o;
    }
    __syncthreads();
  }
  store_result<T, G>(a, pc, acc);
}

// ------------------------------------------------ member pairs (prefix groups)
//
// A member pair's result is the fold of its contributions (MemberLayout),
// each published to the workspace by the workgroup that computed it and
// then counted in on the pair's counter a.pcnt[pair]; the workgroup whose
// count-in completes the pair folds it.  Count-ins are batched: a
// workgroup lists the contributions it published (sm.dpair) and counts
// them in together (flush_members) when the list is full, at the end of
// its chunk and after its prefix items, so no wave waits for a count-in in
// the middle of the stream.  Publication and reading follow the counter
// protocol above (count_in: acquire-release at agent scope after every
// wave's stores completed and a barrier; partials read after a barrier
// that follows the count-ins).

__device__ inline MemberLayout member_layout(const Args& a, const SharedInfo& si, int pair) {
  MemberLayout m;
  const int b = pair / a.Hkv, kvh = pair % a.Hkv;
  const int s = si.seq_sg[b];
  m.pair = pair;
  m.mi = b - si.sg_first[s];
  const int nI = blocks_of(si.sg_len[s], si.B);
  const int uI = si.icum[s] * a.Hkv + kvh * nI;
  m.kf_i = uI / si.cI;
  m.nfr = (uI + nI - 1) / si.cI - m.kf_i + 1;
  m.first_i = 2 * m.kf_i + (uI != m.kf_i * si.cI ? 1 : 0);
  const int np = blocks_of(si.lens[b], si.B) - si.shb[b];
  m.npp = m.kf_p = m.first_p = 0;
  m.stage = -1;
  m.own = -1;
  if (np > 0) {
    const int uP = si.cum[b] * a.Hkv + kvh * (np + si.V);
    m.kf_p = uP / si.cP;
    m.npp = (uP + np - 1) / si.cP - m.kf_p + 1;
    m.first_p = 2 * m.kf_p + (uP != m.kf_p * si.cP ? 1 : 0);
  }
  return m;
}

// Bases of contribution i (0 <= i < nfr + npp) of a member pair: weighted-V
// rows [G][kD] and (max, sum) pairs [G][2].
template <int G>
__device__ inline void member_contrib(const Args& a, const MemberLayout& m, int i, const float*& o,
                                      const float*& ml) {
  if (i < m.nfr) {
    if (m.nfr == 1) {
      o = a.pair_o + (int64_t)(2 * m.pair) * G * kD;
      ml = a.pair_ml + (int64_t)(2 * m.pair) * G * 2;
    } else {
      const int slot = i == 0 ? m.first_i : 2 * (m.kf_i + i);
      const int64_t col = (int64_t)slot * kWideCols + m.mi * G;
      o = a.wide_o + col * kD;
      ml = a.wide_ml + col * 2;
    }
    return;
  }
  i -= m.nfr;
  if (m.npp == 1) {
    o = a.pair_o + (int64_t)(2 * m.pair + 1) * G * kD;
    ml = a.pair_ml + (int64_t)(2 * m.pair + 1) * G * 2;
  } else {
    const int slot = i == 0 ? m.first_p : 2 * (m.kf_p + i);
    o = a.ws_o + (int64_t)slot * G * kD;
    ml = a.ws_ml + (int64_t)slot * G * 2;
  }
}

constexpr int kMemberFoldU = 8;  // outputs per thread folded together at a chunk end

// LDS stage entry e: a member partial's weighted-V sums [G][kD], then its
// maxima [G] and sums [G].
template <int G>
__device__ __forceinline__ float* stage_entry(const Args& a, int e) {
  return shared_layout(a.S, a.ngroups).stage + (int64_t)e * (G * kD + 2 * G);
}

// Folds the nf member pairs listed in sm.dpair / sm.dlay and writes out.
// Each thread takes U outputs at a time and issues the loads of their
// contributions two at a time, so that a round of folds costs one memory
// round trip per two contributions.  Contributions are combined in their
// fixed order whichever workgroup folds.  All threads call.
template <class T, int G, int U, class Smem>
__device__ inline void fold_members(const Args& a, Smem& sm, int nf) {
  constexpr int kPer = G * kD;
  const int total = nf * kPer;
  for (int x0 = 0; x0 < total; x0 += kThreads * U) {
    float M[U], L[U], O[U];
    int pi[U], g[U], d[U], E[U];
    int emax = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int x = x0 + threadIdx.x + u * kThreads;
      const int xc = x < total ? x : total - 1;
      pi[u] = xc / kPer;
      g[u] = (xc % kPer) / kD;
      d[u] = xc % kD;
      E[u] = x < total ? sm.dlay[pi[u]].nfr + sm.dlay[pi[u]].npp : 0;
      emax = max(emax, E[u]);
      M[u] = -INFINITY;
      L[u] = 0.f;
      O[u] = 0.f;
    }
    for (int i0 = 0; i0 < emax; i0 += 2) {
      float vo[U][2], vm[U][2], vl[U][2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          vo[u][j] = 0.f;
          vm[u][j] = -INFINITY;
          vl[u][j] = 0.f;
          if (i0 + j < E[u]) {
            const MemberLayout& m = sm.dlay[pi[u]];
            if (m.stage >= 0 && i0 + j == m.own) {
              const float* e = stage_entry<G>(a, m.stage);
              vo[u][j] = e[g[u] * kD + d[u]];
              vm[u][j] = e[G * kD + g[u]];
              vl[u][j] = e[G * kD + G + g[u]];
            } else {
              const float* o;
              const float* ml;
              member_contrib<G>(a, m, i0 + j, o, ml);
              vo[u][j] = ld_agent(o + g[u] * kD + d[u]);
              vm[u][j] = ld_agent(ml + g[u] * 2);
              vl[u][j] = ld_agent(ml + g[u] * 2 + 1);
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float Mn = fmaxf(M[u], fmaxf(vm[u][0], vm[u][1]));
        const float f0 = rescale(M[u], Mn), f1 = rescale(vm[u][0], Mn), f2 = rescale(vm[u][1], Mn);
        L[u] = L[u] * f0 + f1 * vl[u][0] + f2 * vl[u][1];
        O[u] = O[u] * f0 + f1 * vo[u][0] + f2 * vo[u][1];
        M[u] = Mn;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (x0 + threadIdx.x + u * kThreads >= total) continue;
      const int pair = sm.dlay[pi[u]].pair;
      const int b = pair / a.Hkv, kvh = pair % a.Hkv;
      store_out<T>(a.out, ((int64_t)b * a.Hq + kvh * G + g[u]) * kD + d[u], O[u] / L[u], a.out_f32);
    }
  }
}

// Counts in the contributions listed in sm.dpair and folds the pairs this
// workgroup completes.  A private part still in the LDS stage first checks
// whether every other contribution of its pair is already counted in: then
// the workgroup folds the pair from the stage without publishing or counting
// in (nobody else can fold it, and the counter is put back to zero);
// otherwise it is published from the stage and counted in like the rest.
// All threads call; the list and the stage are empty afterwards.
template <class T, int G, int U, class Smem>
__device__ inline void flush_members(const Args& a, Smem& sm) {
  constexpr int kEntry = G * kD + 2 * G;
  const int n = uniform(sm.dn);  // callers come here after a barrier
  if (n == 0) return;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int pair = sm.dpair[i];
    MemberLayout m = member_layout(a, shared_info(a, sm), pair);
    const int st = sm.dstage[i];
    int fast = 0;
    if (st >= 0) {
      m.stage = st;
      m.own = m.nfr + sm.dpiece[i];
      fast = counted(a.pcnt + pair) == m.nfr + m.npp - 1 ? 2 : 0;
    }
    sm.dlast[i] = fast;
    sm.dlay[i] = m;
  }
  __syncthreads();
  // publish the staged parts that do not complete their pair
  for (int i = 0; i < n; ++i) {
    const MemberLayout& m = sm.dlay[i];
    if (m.stage < 0 || sm.dlast[i] != 0) continue;
    const float* e = stage_entry<G>(a, m.stage);
    const float* o;
    const float* ml;
    member_contrib<G>(a, m, m.own, o, ml);
    for (int x = threadIdx.x; x < kEntry; x += kThreads) {
      if (x < G * kD) {
        st_agent(const_cast<float*>(o) + x, e[x]);
      } else {
        const int g = (x - G * kD) % G, which = (x - G * kD) / G;  // 0: max, 1: sum
        st_agent(const_cast<float*>(ml) + 2 * g + which, e[x]);
      }
    }
  }
  drain_vmem();     // this wave's partial stores have completed ...
  __syncthreads();  // ... and every other wave's
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const MemberLayout& m = sm.dlay[i];
    int* cnt = a.pcnt + m.pair;
    bool fold = sm.dlast[i] == 2;
    if (!fold) fold = count_in(cnt) == m.nfr + m.npp - 1;
    if (fold) {
      reset_count(cnt);
      acquire_counted();
    }
    sm.dlast[i] = fold;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // keep the pairs to fold, in list order (in place: a lane writes at or
    // below the entry it read, and every lane reads before any writes)
    const int lane = threadIdx.x;
    const uint64_t below = (uint64_t(1) << lane) - 1;
    int nf = 0;
    for (int base = 0; base < n; base += 64) {
      const int i = base + lane;
      const bool keep = i < n && sm.dlast[i];
      const MemberLayout m = sm.dlay[i < n ? i : 0];
      const uint64_t km = __builtin_amdgcn_ballot_w64(keep);
      if (keep) sm.dlay[nf + __builtin_popcountll(km & below)] = m;
      nf += __builtin_popcountll(km);
    }
    if (lane == 0) sm.dn = nf;
  }
  __syncthreads();
  const int nf = sm.dn;
  if (nf > 0) fold_members<T, G, U>(a, sm, nf);
  __syncthreads();
  if (threadIdx.x == 0) {
    sm.dn = 0;
    sm.nstage = 0;
  }
  __syncthreads();
}

// A piece of a member pair, merged across the waves (pt): publish it in its
// slot and list it for the next count-in.  The list has room: it is
// flushed between batches of pieces whenever a whole batch might not fit
// (run_decode_shared), so no count-in or fold runs inside the stream.  All
// threads call.
template <class T, int G, class Smem>
__device__ inline void publish_member(const Args& a, Smem& sm, const Piece& pc, const Partial<G>& pt) {
  if constexpr (Smem::kDefers > 1) {
    const int pair = pc.b * a.Hkv + pc.kvh;
    const int ns = uniform(sm.nstage);
    const bool stage = ns < a.stage_cap;
    if (stage) {
      float* e = stage_entry<G>(a, ns);
#pragma unroll
      for (int r = 0; r < Partial<G>::kOut; ++r) {
        const int idx = threadIdx.x + r * kThreads;
        if (idx >= G * kD) continue;
        const int g = idx / kD, d = idx % kD;
        e[idx] = pt.o[r];
        if (d == 0) {
          e[G * kD + g] = pt.m[r];
          e[G * kD + G + g] = pt.l[r];
        }
      }
    } else if (pc.npieces == 1) {
      store_rows<G>(a.pair_o + (int64_t)(2 * pair + 1) * G * kD,
                    a.pair_ml + (int64_t)(2 * pair + 1) * G * 2, pt);
    } else {
      store_partial<G>(a, pc.slot, pt);
    }
    if (threadIdx.x == 0) {
      const int i = sm.dn;
      sm.dpair[i] = pair;
      sm.dstage[i] = stage ? ns : -1;
      sm.dpiece[i] = pc.npieces == 1 ? 0 : pc.slot / 2 - pc.kfirst;
      sm.dn = i + 1;
    }
    // sm.nstage moves on after the barrier that ends finish_piece (every
    // wave reads it above)
  }
}

// The last piece of a chunk when it is partial ("late").  sm.seen is the
// split's arrival count read while the waves were merging (-1 if not
// read).  When every other piece has already counted in, this workgroup
// folds the split from its own partial: no store of its own part and no
// atomic.  Otherwise it publishes its partial, counts itself in, and folds
// if it turned out to be the last.  The fold itself runs at the end of the
// chunk (finish_chunk), outside the streaming loop, from the own partial
// left in LDS.
template <class T, int G, class Smem>
__device__ inline void finish_late(const Args& a, Smem& sm, const Piece& pc,
                                   const Partial<G>& pt) {
  int* cnt = a.counters + pc.kfirst;
  bool fold = uniform(sm.seen) == pc.npieces - 1;
  if (fold) {
    if (threadIdx.x == 0) reset_count(cnt);
    // merge_waves of every wave reads the wave arrays, overwritten below
    __syncthreads();
  } else {
    store_partial<G>(a, pc.slot, pt);
    drain_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int last = count_in(cnt) == pc.npieces - 1;
      if (last) reset_count(cnt);
      sm.flag = last;
    }
    __syncthreads();
    fold = uniform(sm.flag);
  }
  if (!fold) return;
  // every thread has finished reading the wave partials (barrier above)
#pragma unroll
  for (int r = 0; r < Partial<G>::kOut; ++r) {
    const int idx = threadIdx.x + r * kThreads;
    if (idx >= G * kD) continue;
    const int g = idx / kD, d = idx % kD;
    sm.own_o(g, d) = pt.o[r];
    if (d == 0) {
      sm.own_m(g) = pt.m[r];
      sm.own_l(g) = pt.l[r];
    }
  }
  if (threadIdx.x == 0) {
    sm.late = pc;
    sm.fold_late = 1;
  }
}

// finish_piece for a column-split group (two column tiles per wave): the
// wave partials go through the 16-column wave arrays one column tile per
// round (Engine::to_lds of that round), and each output of the round is
// merged and emitted on its own (out for a whole piece, the piece's
// workspace slot otherwise), so only a few are live in registers while
// the next sub-tiles are in flight.  A late piece always publishes its
// partial; when this workgroup completes its split, the fold at the end of
// the chunk reads every piece, its own included, from the workspace.  All
// threads call; thread 0 has set sm.seen.
template <class T, int G, class Engine, class Smem, class State>
__device__ inline void finish_piece_rounds(const Args& a, Smem& sm, const Piece& pc,
                                           const State& st, int wave) {
  constexpr int W = kColWaves<G>;
  constexpr int kPerRound = kColGroups<G> * 16 * kD;  // outputs of one round
  static_assert(kPerRound % kThreads == 0, "every thread owns the same number of outputs");
  const bool whole = pc.kind == kWhole;
  float* const o_base = a.ws_o + (int64_t)pc.slot * G * kD;
  float* const ml_base = a.ws_ml + (int64_t)pc.slot * G * 2;
#pragma unroll
  for (int round = 0; round < kTilesPerWave<G>; ++round) {
    __syncthreads();  // the wave arrays are free (the previous round's merges are done)
    Engine::to_lds(sm, st, wave, round);
    __syncthreads();
#pragma unroll 2
    for (int r = 0; r < kPerRound / kThreads; ++r) {
      const int idx = threadIdx.x + r * kThreads;
      const int cg = idx / (16 * kD), c = idx / kD % 16, d = idx % kD;
      const int g = cg * 32 + round * 16 + c;
      float M, l, o;
      merge_output<W>(sm, cg * W, c, d, M, l, o);
      if (whole) {
        store_out<T>(a.out, ((int64_t)pc.b * a.Hq + pc.kvh * G + g) * kD + d, o / l, a.out_f32);
      } else {
        st_agent(o_base + (int64_t)g * kD + d, o);
        if (d == 0) {
          st_agent(ml_base + (int64_t)g * 2 + 0, M);
          st_agent(ml_base + (int64_t)g * 2 + 1, l);
        }
      }
    }
  }
  if (!whole) {
    drain_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
      int* cnt = a.counters + pc.kfirst;
      if (pc.kind == kEarly) {
        sm.early_seen = count_in(cnt);
        sm.early = pc;
      } else {
        // the last arrival folds: either every other piece was already
        // counted in when the stream began this one, or this count-in is
        // the last
        const bool last = sm.seen == pc.npieces - 1 || count_in(cnt) == pc.npieces - 1;
        if (last) {
          reset_count(cnt);
          sm.late = pc;
          sm.fold_late = 1;
        }
      }
    }
  }
  __syncthreads();
}

// Emit a piece after its waves wrote their partials to LDS (to_lds) and
// thread 0 set sm.seen.  All threads call.  A whole piece writes `out`.
// An early piece publishes its partial and counts itself in at once
// (sm.early_seen keeps the returned count; the rare case that it was the
// last is folded at the end of the chunk).  A late piece finishes its
// split (finish_late).  Values returned by memory are moved to LDS where
// they arrive, so no load is left in flight into a register that the
// streaming loop reuses.
template <class T, int G, class Smem>
__device__ inline void finish_piece(const Args& a, Smem& sm, const Piece& pc) {
  __syncthreads();
  Partial<G> pt;
  merge_waves<T, G>(sm, pt);
  if (pc.kind == kWhole) {
    store_result<T, G>(a, pc, pt);
  } else if (pc.kind == kMember) {
    publish_member<T, G>(a, sm, pc, pt);
  } else if (pc.kind == kEarly) {
    store_partial<G>(a, pc.slot, pt);
    drain_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
      sm.early_seen = count_in(a.counters + pc.kfirst);
      sm.early = pc;
    }
  } else {
    finish_late<T, G>(a, sm, pc, pt);
  }
  __syncthreads();
  if constexpr (Smem::kDefers > 1) {
    // the stage entry publish_member filled (if any) is taken now that
    // every wave has read the stage count; the next reader comes after the
    // next barrier
    if (pc.kind == kMember && threadIdx.x == 0 && sm.nstage < a.stage_cap) ++sm.nstage;
  }
}

// End of the chunk: fold the late piece's split if finish_late chose to
// (own partial in LDS), and the early piece's split if its count-in was
// the last one.  All threads call.
template <class T, int G, class Smem>
__device__ inline void finish_chunk(const Args& a, Smem& sm) {
  if (threadIdx.x == 0) {
    sm.flag = sm.early_seen >= 0 && sm.early_seen == sm.early.npieces - 1;
    // thread 0 read the counts of both splits: acquire before their folds
    if (sm.flag || sm.fold_late) acquire_counted();
  }
  __syncthreads();
  if (uniform(sm.fold_late)) {
    const Piece pc = uniform_piece(sm.late);
    Partial<G> own;
    if constexpr (kTilesPerWave<G> > 1) {
      // column-split groups published their own partial too: read every piece
#pragma unroll
      for (int r = 0; r < Partial<G>::kOut; ++r) own.m[r] = own.l[r] = own.o[r] = 0.f;
      fold_split<T, G>(a, sm, pc, own, -1);
    } else {
#pragma unroll
      for (int r = 0; r < Partial<G>::kOut; ++r) {
        const int idx = min(threadIdx.x + r * kThreads, G * kD - 1);
        const int g = idx / kD, d = idx % kD;
        own.m[r] = sm.own_m(g);
        own.l[r] = sm.own_l(g);
        own.o[r] = sm.own_o(g, d);
      }
      fold_split<T, G>(a, sm, pc, own, pc.slot);
    }
  }
  if (uniform(sm.flag)) {
    const Piece pc = uniform_piece(sm.early);
    if (threadIdx.x == 0) reset_count(a.counters + pc.kfirst);
    Partial<G> none;
#pragma unroll
    for (int r = 0; r < Partial<G>::kOut; ++r) none.m[r] = none.l[r] = none.o[r] = 0.f;
    fold_split<T, G>(a, sm, pc, none, -1);
  }
  if constexpr (Smem::kDefers > 1) flush_members<T, G, kMemberFoldU>(a, sm);
}

// out = 0 for sequences of length 0 (every query head).  Sequences are
// shared among workgroups round-robin.
template <class T>
__device__ inline void zero_empty_sequences(const Args& a, int chunk, const int* lens_s) {
  for (int b = chunk; b < a.S; b += a.nwg) {
    if (lens_s[b] > 0) continue;
    for (int i = threadIdx.x; i < a.Hq * kD; i += kThreads)
      store_out<T>(a.out, (int64_t)b * a.Hq * kD + i, 0.f, a.out_f32);
  }
}

// ------------------------------------------------------------ driver
//
// Per workgroup: the chunk's pieces are listed in LDS a batch at a time and
// their query groups staged in LDS.  The batch's sub-tiles are numbered
// through its pieces in order and dealt round-robin to the waves (wave w
// takes sub-tiles w, w + kWaves, ...), so every wave streams one
// continuous sequence of sub-tiles whatever the piece boundaries: each
// wave's count differs from the others' by at most one per batch.  A wave
// keeps two sub-tiles in flight (registers t0, t1) and computes one while
// the next loads; its table lookups run one sub-tile ahead on the scalar
// unit.  When the next sub-tile belongs to a later piece, the wave first
// finishes the pieces in between (finish_piece; every wave finishes every
// piece, in order, so their barriers pair up), and the loads already in
// flight keep streaming meanwhile.  Past the end of its share a wave
// issues the same loads at its last sub-tile through an empty resource (no
// memory access, never computed), so every load is issued unconditionally
// and the compiler waits for exactly the one it consumes.

// Arrival count of a late two-piece split, read by thread 0 as its waves
// finish streaming (the load overlaps the wave merge); -1 otherwise.  Splits
// over more pieces have partners that end at the same time, so the read
// would rarely find them all counted in.
__device__ __forceinline__ int split_seen(const Args& a, const Piece& pc) {
  if (pc.kind != kLate || pc.npieces != 2 || threadIdx.x != 0) return -1;
  return counted(a.counters + pc.kfirst);
}

// Stage the batch's query groups in LDS (all threads; the caller
// synchronises before they are read).
template <class T, int G, class Smem>
__device__ inline void stage_queries(const Args& a, Smem& sm, int npl) {
  constexpr int kQChunks = G * kD * T::kEsize / 16;  // 16-byte chunks per query group
  for (int x = threadIdx.x; x < npl * kQChunks; x += kThreads) {
    const int p = x / kQChunks, k = x % kQChunks;
    const Piece& pc = sm.plist[p];
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
        ((int64_t)pc.b * a.Hq + (int64_t)pc.kvh * G) * kD * T::kEsize);
    sm.q[p][k] = src[k];
  }
}

template <class T, int B, int G, class Engine>
__device__ inline void stream_batch(const Args& a, typename Engine::Smem& sm) {
  using Tile = typename Engine::Tile;
  using State = typename Engine::State;
  using Query = typename Engine::Query;
  const int wave = uniform(threadIdx.x >> 6);
  const int npl = uniform(sm.npl);

  // Stream position: sub-tile j of piece p (p == npl: past the end), with
  // the fields of piece p that addressing and masking need.
  struct Cur {
    int p, j, n, b, kvh, tb, te;
  };
  auto settle = [&](Cur& c) {  // move an overflowing j on to the piece holding it
    while (c.p < npl) {
      c.n = uniform(sm.plist[c.p].nsub);
      if (c.j < c.n) break;
      c.j -= c.n;
      ++c.p;
    }
    if (c.p < npl) {
      c.b = uniform(sm.plist[c.p].b);
      c.kvh = uniform(sm.plist[c.p].kvh);
      c.tb = uniform(sm.plist[c.p].tok_begin);
      c.te = uniform(sm.plist[c.p].tok_end);
    }
  };
  // The waves of a column group deal the sub-tiles among themselves (all
  // kWaves waves when the group is one column tile).
  constexpr int kStride = kColWaves<G>;
  auto advance = [&](Cur& c) {
    c.j += kStride;
    if (c.j >= c.n) settle(c);
  };
  Cur c{0, wave % kStride, 0, 0, 0, 0, 0};
  settle(c);

  int cur = 0;  // piece whose state the wave holds
  State st;
  Engine::reset(st);
  Query q;
  // Column groups (64 heads) read the same sub-tiles, each group dealing
  // them over its own waves.  Left to drift, the second read of a sub-tile
  // mostly missed L2 (FETCH_SIZE 1.9 x the K/V bytes; 1.02 x with these
  // barriers), so the groups meet at a workgroup barrier at every
  // kSyncSub-th position of the stream (positions number the batch's
  // sub-tiles through its pieces, as dealt; a barrier every 1, 2, 4, 8
  // passes measured 344, 333, 328 and 335 us on the 64-head batch).
  // A wave takes the barrier at position X before computing its first
  // sub-tile at or past X, and the finish of piece p (its own barriers) at
  // the position where piece p + 1 starts, ties going to the finish: every
  // wave meets the same barriers in the same order, only at different
  // sub-tiles of its own.
  constexpr bool kSync = kColGroups<G> > 1;
  constexpr int kSyncSub = 8 * kColWaves<G>;  // four passes of the group
  int cur_end = 0;                            // stream position where piece cur + 1 starts
  int next_sync = kSyncSub;                   // position of the next barrier
  int total = 0;                              // the batch's stream length
  if constexpr (kSync) {
    cur_end = uniform(sm.plist[0].nsub);
    for (int p = 0; p < npl; ++p) total += uniform(sm.plist[p].nsub);
  }
  // Finish pieces cur .. p-1 and start piece p (p <= npl), taking the
  // barriers up to position pos on the way (column groups).  The late
  // piece is the last of the chunk, so it is only ever finished after the
  // streaming loop (enter(npl, total - 1, true)); only there is its arrival
  // count read, which keeps that load and its wait out of the loop.
  auto enter = [&](int p, int pos, bool last) {
    const int cur0 = cur;
    while (true) {
      const bool fin = cur < p;
      if constexpr (kSync) {
        if (next_sync <= pos && (!fin || next_sync < cur_end)) {
          __syncthreads();
          next_sync += kSyncSub;
          continue;
        }
      }
      if (!fin) break;
      const Piece pc = uniform_piece(sm.plist[cur]);
      const int seen = last ? split_seen(a, pc) : -1;
      if constexpr (kTilesPerWave<G> > 1) {
        if (threadIdx.x == 0) sm.seen = seen;
        finish_piece_rounds<T, G, Engine>(a, sm, pc, st, wave);
      } else {
        Engine::to_lds(sm, st, wave);
        if (threadIdx.x == 0) sm.seen = seen;
        finish_piece<T, G>(a, sm, pc);
      }
      Engine::reset(st);
      ++cur;
      if constexpr (kSync) {
        if (cur < npl) cur_end += uniform(sm.plist[cur].nsub);
      }
    }
    if (cur != cur0 && p < npl) Engine::load_query(sm, p, q);
  };

  if (c.p < npl) {
    Cur last = c;  // last position inside the batch (address of the empty loads past the end)
    auto row_phys = [&](const Cur& u) {
      return as_constant(a.bt + (int64_t)u.b * a.mbs)[(u.tb + kSub * u.j) / B];
    };
    // The tile's address is wave-uniform; say so, so that the buffer
    // resource stays in scalar registers whatever the compiler concludes
    // about the cursor's control flow.
    // A load past the end of the wave's share (live = false) keeps the
    // instruction stream unconditional but goes through a resource of zero
    // bytes: the range check drops every lane's access, so it returns zeros
    // without touching memory.
    auto load = [&](const Cur& u, int phys, bool live, Tile& t) {
      const int tok = uniform(u.tb + kSub * u.j), kvh = uniform(u.kvh);
      phys = uniform(phys);
      const int bytes = uniform(live ? B * kD * T::kEsize : 0);
      // column groups re-read each other's sub-tiles: keep them cached
      if (kColGroups<G> > 1 || tok / B < a.cached_blocks)
        Engine::template load_tile<kCachedPolicy>(a, kvh, tok % B, phys, bytes, t);
      else
        Engine::template load_tile<kStreamPolicy>(a, kvh, tok % B, phys, bytes, t);
    };
    // Each tile register carries (piece, valid tokens) of its sub-tile.
    // The first two positions and their table entries are resolved before
    // any tile load, so both loads leave back to back, and the query
    // groups are staged after them: the batch starts with two memory round
    // trips instead of three.
    const Cur c0 = c;
    int p0 = c.p, v0 = c.te - (c.tb + kSub * c.j);
    int s0 = wave % kStride, s1 = s0 + kStride;  // stream positions of t0, t1
    int snext = s1 + kStride;                    // of the next refill
    advance(c);
    if (c.p < npl) last = c;
    const Cur c1 = last;
    const bool live1 = c.p < npl;
    int p1 = c.p, v1 = c.te - (c.tb + kSub * c.j);
    advance(c);
    if (c.p < npl) last = c;
    const int ph0 = row_phys(c0), ph1 = row_phys(c1);
    int ph = row_phys(last);
    Tile t0, t1;
    load(c0, ph0, true, t0);
    load(c1, ph1, live1, t1);
    stage_queries<T, G>(a, sm, npl);
    __syncthreads();  // query groups staged
    Engine::load_query(sm, 0, q);
    // Load the stream's next sub-tile into t and return its (piece, valid
    // tokens).
    auto refill = [&](Tile& t, int& pn, int& vn, int& sn) {
      pn = c.p;
      vn = c.te - (c.tb + kSub * c.j);
      sn = snext;
      snext += kStride;
      load(last, ph, c.p < npl, t);
      advance(c);
      if (c.p < npl) last = c;
      ph = row_phys(last);
    };
    // Every pass through the body refills t0 and then t1 (an empty load
    // when past the end), so the loads in flight at the top of the loop are
    // always t0's followed by t1's and the compiler's wait before each
    // compute covers exactly that tile.  The loop leaves only at the
    // bottom.
    enter(p0, s0, false);
    while (true) {
      int n0, w0, n1, w1, m0, m1;
      Engine::compute(a, sm, q, st, t0, v0);
      refill(t0, n0, w0, m0);
      const bool more = p1 < npl;
      if (more) {
        enter(p1, s1, false);
        Engine::compute(a, sm, q, st, t1, v1);
      }
      refill(t1, n1, w1, m1);
      p0 = n0;
      v0 = w0;
      s0 = m0;
      p1 = n1;
      v1 = w1;
      s1 = m1;
      if (!more || p0 >= npl) break;
      enter(p0, s0, false);
    }
  } else {
    stage_queries<T, G>(a, sm, npl);
    __syncthreads();  // query groups staged
  }
  // the rest of the batch's pieces and barriers (those before its end)
  enter(npl, total - 1, true);
}

// Lists the chunk's next batch of pieces (flat range [sm.next_f, e)) in
// sm.plist with the 64 lanes of wave 0: lane t looks at the t-th
// (sequence, KV head) pair after the one holding the batch's first block,
// a ballot drops pairs of empty sequences and gives every piece its place,
// and further rounds of 64 continue until the batch is full or the chunk
// ends.  Pieces are contiguous in flat order, so the next batch starts
// where the last listed piece ends.
// With prefix groups (kShared) cum counts private blocks only: sequence b's
// units start after its shb[b] leading blocks (attended by its item), and
// every piece of a sequence with an item is a member piece.
//
// V > 0: every (sequence, KV head) with blocks is charged V virtual units
// after its real ones (cum counts n_b + V for such sequences), so that the
// equal chunks balance time rather than blocks: a piece costs a merge and
// its output on top of its blocks.  A chunk boundary inside those virtual
// units leaves no piece there; pieces, kinds and split counts follow the
// real blocks only.
template <int B, bool kShared, class Smem>
__device__ inline void list_batch(const Args& a, Smem& sm, const int* cum, const int* lens_s,
                                  const int* shb, int s, int e, int chunk, int c, int V) {
  const int lane = threadIdx.x & 63;
  const int f0 = uniform(sm.next_f);
  if (lane == 0) {
    sm.npl = 0;
    sm.next_f = e;
  }
  if (f0 >= e) return;
  const int b0 = uniform(find_seq(cum, a.S, a.Hkv, f0));
  const int nb0 = cum[b0 + 1] - cum[b0];
  const int kvh0 = uniform((f0 - cum[b0] * a.Hkv) / nb0);
  const uint64_t below = (uint64_t(1) << lane) - 1;
  int n = 0;
  for (int lin = kvh0; n < Smem::kBatch; lin += 64) {
    const int L = lin + lane;
    const int b = b0 + L / a.Hkv, kvh = L % a.Hkv;
    int nb = 0, real = 0, ustart = 0;
    if (b < a.S) {
      nb = cum[b + 1] - cum[b];  // units of each KV head of b (real + V)
      real = nb > 0 ? nb - V : 0;
      ustart = cum[b] * a.Hkv + kvh * nb;
    }
    const int f = L == kvh0 ? f0 : ustart;
    const bool past = b >= a.S || (nb > 0 && ustart >= e);
    const bool ok = !past && real > 0 && f - ustart < real;
    const uint64_t okm = __builtin_amdgcn_ballot_w64(ok);
    const int idx = n + __builtin_popcountll(okm & below);
    if (ok && idx < Smem::kBatch) {
      const int pe = min(e, ustart + real);
      const int j0 = f - ustart, j1 = pe - ustart;
      Piece pc;
      pc.b = b;
      pc.kvh = kvh;
      pc.L = lens_s[b];
      const int off = kShared ? shb[b] * B : 0;
      pc.tok_begin = off + j0 * B;
      pc.tok_end = min(off + j1 * B, pc.L);
      pc.nsub = (pc.tok_end - pc.tok_begin + kSub - 1) / kSub;
      pc.kind = (kShared && off > 0) ? kMember
                : (j0 == 0 && j1 == real) ? kWhole : (f == s && pe < e) ? kEarly : kLate;
      pc.slot = 2 * chunk + (f == s ? 0 : 1);
      pc.kfirst = ustart / c;
      pc.npieces = (ustart + real - 1) / c - pc.kfirst + 1;
      pc.first_slot = 2 * pc.kfirst + (ustart != pc.kfirst * c ? 1 : 0);
      sm.plist[idx] = pc;
      if (idx == Smem::kBatch - 1) sm.next_f = pe;
    }
    n += __builtin_popcountll(okm);
    if (__builtin_amdgcn_ballot_w64(past) != 0) break;
  }
  if (lane == 0) sm.npl = min(n, Smem::kBatch);
}

template <class T, int B, int G, class Engine>
__device__ inline void run_decode(const Args& a) {
  using Smem = typename Engine::Smem;
  extern __shared__ int dyn[];
  int* cum = dyn;               // S + 1
  int* lens_s = dyn + a.S + 1;  // S
  __shared__ int wsum[kWaves];
  __shared__ Smem sm;
  build_prefix(a.lens, a.S, B, cum, lens_s, wsum);
  const int chunk = chunk_of_wg(blockIdx.x, a.nwg);
  zero_empty_sequences<T>(a, chunk, lens_s);
  const int W = cum[a.S] * a.Hkv;
  if (W == 0) return;
  const int c = (W + a.nwg - 1) / a.nwg;
  const int s = chunk * c;
  const int e = min(W, s + c);
  if (threadIdx.x == 0) {
    sm.next_f = s;
    sm.fold_late = 0;
    sm.early_seen = -1;
  }
  __syncthreads();
  while (true) {
    if (threadIdx.x < 64) list_batch<B, false>(a, sm, cum, lens_s, nullptr, s, e, chunk, c, 0);
    __syncthreads();
    const int npl = sm.npl;
    if (npl == 0) break;
    stream_batch<T, B, G, Engine>(a, sm);
    __syncthreads();
  }
  finish_chunk<T, G>(a, sm);
}

}  // namespace pa
