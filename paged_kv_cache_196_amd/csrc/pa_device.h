// pa_device.h — device-side building blocks shared by the gfx950 decode and
// merge kernels: element types, wave64 cross-lane helpers, the work schedule
// (which workgroup handles which logical blocks of which (sequence, KV head))
// and the cross-wave / cross-partition combination of softmax partials.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kD = 128;          // head_dim the kernels are built for
constexpr int kWaves = 4;        // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kSub = 16;         // tokens per sub-tile (unit of the streaming loop)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxGrid = 2048;   // upper bound on decode workgroups (sizes the workspace)
constexpr int kMaxSeqs = 8192;   // sequences per call (LDS prefix array)

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
};

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
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kKvPolicy = 2;                    // nt
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* pool, int64_t byte_off,
                                                            int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(pool)) + byte_off, (short)0, bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 tile_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kKvPolicy);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 tile_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kKvPolicy);
  return make_uint2(v.x, v.y);
}

// Streaming loop of one wave over its sub-tiles first, first + kWaves, ...,
// last, with kDepth sub-tiles in flight.  Every step issues its prefetch
// unconditionally (past `last` the index is clamped to it, a harmless
// re-read), so the compiler waits for exactly the oldest tile instead of
// draining every outstanding load; the table entry of the load after next
// is fetched (scalar load) one step early.
template <int kDepth, class Tile, class PhysFn, class LoadFn, class ComputeFn, class ProgressFn>
__device__ __forceinline__ void stream_subtiles(int first, int last, PhysFn phys_of, LoadFn load,
                                                ComputeFn compute, ProgressFn progress) {
  static_assert(kDepth >= 1 && kDepth <= 4, "prefetch depth");
  Tile t[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    const int j = min(first + d * kWaves, last);
    load(j, phys_of(j), t[d]);
  }
  int pn = phys_of(min(first + kDepth * kWaves, last));
  int i = first;
  auto step = [&](Tile& tile) -> bool {
    progress(i);
    compute(tile, i);
    load(min(i + kDepth * kWaves, last), pn, tile);
    pn = phys_of(min(i + (kDepth + 1) * kWaves, last));
    i += kWaves;
    return i > last;
  };
  while (true) {
    if (step(t[0])) break;
    if constexpr (kDepth > 1) { if (step(t[1])) break; }
    if constexpr (kDepth > 2) { if (step(t[2])) break; }
    if constexpr (kDepth > 3) { if (step(t[3])) break; }
  }
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
// [k*c, min((k+1)*c, W)) with c = ceil(W / nwg).  A chunk meets at most two
// (sequence, KV head) pairs only partly (its first and its last piece);
// every pair in between is processed whole and written straight to `out`.
// Partial pieces store (max, sum of exp, weighted V) in the workspace slot
// 2*k + (piece is first in chunk ? 0 : 1); the merge kernel folds them.

__device__ __forceinline__ int blocks_of(int len, int B) { return len > 0 ? (len + B - 1) / B : 0; }

// cum[0..S] in LDS (exclusive prefix of block counts).  All threads call.
__device__ inline void build_prefix(const int32_t* __restrict__ lens, int S, int B, int* cum,
                                    int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < S; base += kThreads) {
    const int b = base + tid;
    int x = b < S ? blocks_of(lens[b], B) : 0;
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
// boundaries cut (through the workspace, done by the workgroup that
// finishes the last of those pieces).

constexpr int kMergeBatch = 128;  // pieces staged in LDS at a time when folding a split

template <int G>
struct MergeSmem {
  float o[kWaves][G][kD + 4];
  float m[kWaves][G];
  float l[kWaves][G];
  // folding the pieces of a split (sequence, KV head)
  float pm[kMergeBatch * G];
  float pl[kMergeBatch * G];
  float M[G], L[G], scale[G];
  int last;
};

__device__ __forceinline__ float rescale(float mi, float m) {
  return mi == -INFINITY ? 0.f : fast_exp2(mi - m);
}

// Workspace partials are exchanged between workgroups that may sit on
// different XCDs (separate L2s).  They are written and read with relaxed
// agent-scope atomics (coherent at device scope without whole-L2
// write-back / invalidate), and a writer waits for its stores to complete
// before it counts itself in.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One piece of work: logical blocks [j0, j1) of (sequence b, KV head kvh).
// When the (sequence, KV head) is split over several chunks, its pieces
// occupy workspace slots first_slot (chunk kfirst) and 2*k (chunks
// kfirst+1 .. kfirst+npieces-1); this piece is `slot`.
struct Piece {
  int b, kvh, j0, j1, L;
  bool complete;
  int slot, kfirst, npieces, first_slot;
  int done_before;  // units of the chunk finished before this piece
  int chunk_len;    // units in the chunk
};

// Issue priority from a workgroup's progress through its chunk.  Two or more
// workgroups share a CU, and the older one's waves win arbitration; left
// alone, the first workgroup on every CU finished its (equal) chunk in ~60 %
// of the time of the second, which then streamed with half the CU's loads
// in flight.  Waves that are further behind get the higher priority, so the
// co-resident workgroups progress together.
__device__ __forceinline__ void set_priority_for_progress(int done, int total) {
  const int q = (4 * done) / max(total, 1);
  if (q <= 0) __builtin_amdgcn_s_setprio(3);
  else if (q == 1) __builtin_amdgcn_s_setprio(2);
  else if (q == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Folds the npieces partials of a split (sequence, KV head) from the
// workspace and writes out = o / l.  All threads of the workgroup call.
template <class T, int G>
__device__ inline void fold_split(const Args& a, MergeSmem<G>& sm, const Piece& pc) {
  auto slot_of = [&](int p) { return p == 0 ? pc.first_slot : 2 * (pc.kfirst + p); };
  constexpr int kOut = (G * kD + kThreads - 1) / kThreads;  // outputs per thread
  float o[kOut];
#pragma unroll
  for (int r = 0; r < kOut; ++r) o[r] = 0.f;
  if (threadIdx.x < G) {
    sm.M[threadIdx.x] = -INFINITY;
    sm.L[threadIdx.x] = 0.f;
  }
  for (int p0 = 0; p0 < pc.npieces; p0 += kMergeBatch) {
    const int np = min(kMergeBatch, pc.npieces - p0);
    for (int e = threadIdx.x; e < np * G; e += kThreads) {
      const float* ml = a.ws_ml + ((int64_t)slot_of(p0 + e / G) * G + e % G) * 2;
      sm.pm[e] = ld_agent(ml);
      sm.pl[e] = ld_agent(ml + 1);
    }
    __syncthreads();
    if (threadIdx.x < G) {
      const int g = threadIdx.x;
      float Mb = sm.M[g];
      for (int p = 0; p < np; ++p) Mb = fmaxf(Mb, sm.pm[p * G + g]);
      const float sc = rescale(sm.M[g], Mb);
      float L = sm.L[g] * sc;
      for (int p = 0; p < np; ++p) L += rescale(sm.pm[p * G + g], Mb) * sm.pl[p * G + g];
      sm.scale[g] = sc;
      sm.M[g] = Mb;
      sm.L[g] = L;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < np * G; e += kThreads) sm.pm[e] = rescale(sm.pm[e], sm.M[e % G]);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kOut; ++r) {
      const int idx = threadIdx.x + r * kThreads;
      if (idx < G * kD) o[r] *= sm.scale[idx / kD];
    }
    // kChunk pieces x kOut outputs of loads in flight before any is used.
    constexpr int kChunk = kOut >= 8 ? 2 : 16 / kOut;
    for (int p = 0; p < np; p += kChunk) {
      float v[kOut][kChunk];
#pragma unroll
      for (int r = 0; r < kOut; ++r) {
        const int idx = min(threadIdx.x + r * kThreads, G * kD - 1);
        const int g = idx / kD, d = idx % kD;
#pragma unroll
        for (int q = 0; q < kChunk; ++q)
          v[r][q] = p + q < np ? ld_agent(a.ws_o + ((int64_t)slot_of(p0 + p + q) * G + g) * kD + d) : 0.f;
      }
#pragma unroll
      for (int r = 0; r < kOut; ++r) {
        const int g = min(threadIdx.x + r * kThreads, G * kD - 1) / kD;
#pragma unroll
        for (int q = 0; q < kChunk; ++q)
          if (p + q < np) o[r] += sm.pm[(p + q) * G + g] * v[r][q];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < kOut; ++r) {
    const int idx = threadIdx.x + r * kThreads;
    if (idx < G * kD) {
      const int g = idx / kD, d = idx % kD;
      store_out<T>(a.out, ((int64_t)pc.b * a.Hq + pc.kvh * G + g) * kD + d, o[r] / sm.L[g], a.out_f32);
    }
  }
}

// Combine the kWaves wave partials held in `sm` and emit the piece's result:
// the final output (complete piece), or a workspace partial followed, when
// this is the last piece of its split to finish, by the fold of the split.
// All threads call; the caller has synchronised after the waves wrote `sm`.
template <class T, int G>
__device__ inline void emit_piece(const Args& a, MergeSmem<G>& sm, const Piece& pc) {
  for (int idx = threadIdx.x; idx < G * kD; idx += kThreads) {
    const int g = idx / kD, d = idx % kD;
    float M = sm.m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.m[w][g]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = rescale(sm.m[w][g], M);
      o += f * sm.o[w][g][d];
      l += f * sm.l[w][g];
    }
    if (pc.complete) {
      const int64_t oi = ((int64_t)pc.b * a.Hq + pc.kvh * G + g) * kD + d;
      store_out<T>(a.out, oi, o / l, a.out_f32);
    } else {
      st_agent(a.ws_o + ((int64_t)pc.slot * G + g) * kD + d, o);
      if (d == 0) {
        st_agent(a.ws_ml + ((int64_t)pc.slot * G + g) * 2 + 0, M);
        st_agent(a.ws_ml + ((int64_t)pc.slot * G + g) * 2 + 1, l);
      }
    }
  }
  if (pc.complete) return;
  // Count this piece in once every thread's partial stores have completed;
  // the workgroup that brings the count to npieces folds the split and
  // returns the counter to zero for the next call.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(a.counters + pc.kfirst, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == pc.npieces - 1;
    if (last) __hip_atomic_store(a.counters + pc.kfirst, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = last;
  }
  __syncthreads();
  if (sm.last) fold_split<T, G>(a, sm, pc);
}

// out = 0 for sequences of length 0 (every query head).  Sequences are
// shared among workgroups round-robin.
template <class T>
__device__ inline void zero_empty_sequences(const Args& a, int chunk) {
  for (int b = chunk; b < a.S; b += a.nwg) {
    if (a.lens[b] > 0) continue;
    for (int i = threadIdx.x; i < a.Hq * kD; i += kThreads)
      store_out<T>(a.out, (int64_t)b * a.Hq * kD + i, 0.f, a.out_f32);
  }
}

// Drives one decode workgroup: builds the prefix, walks its chunk piece by
// piece and hands each piece to Engine::piece.
template <class T, int B, int G, class Engine>
__device__ inline void run_decode(const Args& a) {
  extern __shared__ int cum[];                      // S + 1 ints
  __shared__ int wsum[kWaves];
  __shared__ typename Engine::Smem sm;
  build_prefix(a.lens, a.S, B, cum, wsum);
  const int chunk = chunk_of_wg(blockIdx.x, a.nwg);
  zero_empty_sequences<T>(a, chunk);
  const int W = cum[a.S] * a.Hkv;
  if (W == 0) return;
  const int c = (W + a.nwg - 1) / a.nwg;
  const int s = chunk * c;
  const int e = min(W, s + c);
  int f = s;
  while (f < e) {
    Piece pc;
    pc.b = find_seq(cum, a.S, a.Hkv, f);
    const int nb = cum[pc.b + 1] - cum[pc.b];
    const int base = cum[pc.b] * a.Hkv;
    pc.kvh = (f - base) / nb;
    pc.j0 = (f - base) - pc.kvh * nb;
    const int ustart = base + pc.kvh * nb;
    const int pe = min(e, ustart + nb);
    pc.j1 = pc.j0 + (pe - f);
    pc.L = a.lens[pc.b];
    pc.complete = (pc.j0 == 0) && (pc.j1 == nb);
    pc.slot = 2 * chunk + (f == s ? 0 : 1);
    pc.kfirst = ustart / c;
    pc.npieces = (ustart + nb - 1) / c - pc.kfirst + 1;
    pc.first_slot = 2 * pc.kfirst + (ustart != pc.kfirst * c ? 1 : 0);
    pc.done_before = f - s;
    pc.chunk_len = e - s;
    Engine::piece(a, sm, pc);
    f = pe;
  }
}

}  // namespace pa
