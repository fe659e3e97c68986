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
// chunk).  Whole pairs are written straight to `out`; a partial piece
// leaves (max, sum of exp, weighted V) in workspace slot
// 2*k + (piece is first in chunk ? 0 : 1), and the split is folded by the
// workgroup that counts its last piece in.

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
struct Piece {
  int b, kvh, L;
  int tok_begin, tok_end, nsub;
  int complete;
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
  u.complete = uniform(p.complete);
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

constexpr int kMergeBatch = 128;  // pieces staged in LDS at a time when folding a split
constexpr int kQueryLdsBytes = 32768;

// Pieces listed per batch: their query groups are staged in LDS together.
template <class T, int G>
constexpr int piece_batch() {
  constexpr int per = G * kD * T::kEsize;
  constexpr int n = kQueryLdsBytes / per;
  return n > 32 ? 32 : n;
}

template <class T, int G>
struct MergeSmem {
  static constexpr int kBatch = piece_batch<T, G>();
  float o[kWaves][G][kD + 4];
  float m[kWaves][G];
  float l[kWaves][G];
  // folding the pieces of a split (sequence, KV head)
  float pm[kMergeBatch * G];
  float pl[kMergeBatch * G];
  float M[G], L[G], scale[G];
  int last[2];
  // the chunk's current batch of pieces and their query groups
  Piece plist[kBatch];
  int npl, next_f;
  uint4 q[kBatch][G * kD * T::kEsize / 16];
  // partial pieces of this chunk awaiting their count (first, last)
  Piece commit[2];
  int ncommit;
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

// Folds the npieces partials of a split (sequence, KV head) from the
// workspace and writes out = o / l.  All threads of the workgroup call.
template <class T, int G>
__device__ inline void fold_split(const Args& a, MergeSmem<T, G>& sm, const Piece& pc) {
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
  __syncthreads();
}

// Combine the kWaves wave partials held in `sm` and emit the piece's result:
// the final output (whole piece) or its workspace partial, which is counted
// in later (commit_splits).  All threads call; the caller has synchronised
// after the waves wrote `sm`.
template <class T, int G>
__device__ inline void emit_piece(const Args& a, MergeSmem<T, G>& sm, const Piece& pc) {
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
  if (!pc.complete && threadIdx.x == 0) sm.commit[sm.ncommit++] = pc;
}

// At the end of the chunk: wait until this workgroup's partial stores have
// completed, count each partial piece in on its split's counter, and fold
// the splits this workgroup completed (returning their counters to zero).
template <class T, int G>
__device__ inline void commit_splits(const Args& a, MergeSmem<T, G>& sm) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int n = sm.ncommit;
  if (threadIdx.x == 0) {
    for (int k = 0; k < n; ++k) {
      const Piece& pc = sm.commit[k];
      const int old = __hip_atomic_fetch_add(a.counters + pc.kfirst, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == pc.npieces - 1;
      if (last)
        __hip_atomic_store(a.counters + pc.kfirst, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.last[k] = last;
    }
  }
  __syncthreads();
  for (int k = 0; k < n; ++k)
    if (sm.last[k]) fold_split<T, G>(a, sm, sm.commit[k]);
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
// their query groups staged in LDS.  Each wave then streams its sub-tiles
// (wave w takes sub-tiles w, w + kWaves, ... of every piece) with one pair
// of sub-tiles in flight while it computes the previous pair.  The prefetch
// runs across piece boundaries, so the next piece's first tiles are already
// in flight while the workgroup merges and emits a finished piece.  A
// wave's sub-tile count in each piece is padded to even with a dummy (a
// re-read, not computed) so the two tile registers keep a fixed role; past
// the batch the prefetch re-reads the last pair.  Every prefetch is issued
// unconditionally so the compiler waits for exactly the pair it consumes.

template <class T, int B, int G, class Engine>
__device__ inline void stream_batch(const Args& a, typename Engine::Smem& sm, int chunk) {
  using Tile = typename Engine::Tile;
  using State = typename Engine::State;
  using Query = typename Engine::Query;
  const int wave = uniform(threadIdx.x >> 6);
  const int npl = uniform(sm.npl);

  auto count = [&](int p) {  // this wave's sub-tiles in piece p
    const int n = uniform(sm.plist[p].nsub);
    return n > wave ? (n - 1 - wave) / kWaves + 1 : 0;
  };
  auto first_piece_from = [&](int p) {
    while (p < npl && count(p) == 0) ++p;
    return p;
  };
  // Pair cursor: piece p, local pair start k (even).  Advances to the next
  // piece in which this wave has sub-tiles.
  struct Cur {
    int p, k;
  };
  auto advance = [&](Cur c) {
    c.k += 2;
    if (c.k >= count(c.p)) {
      c.p = first_piece_from(c.p + 1);
      c.k = 0;
    }
    return c;
  };
  auto row_of = [&](const Piece& pc) { return as_constant(a.bt + (int64_t)pc.b * a.mbs); };
  // physical blocks of the pair at cursor c (second = first for a dummy)
  auto pair_phys = [&](Cur c, int& ph0, int& ph1) {
    const Piece pc = uniform_piece(sm.plist[c.p]);
    const int n = count(c.p);
    const int i0 = wave + kWaves * c.k;
    const int i1 = wave + kWaves * min(c.k + 1, n - 1);
    const auto row = row_of(pc);
    ph0 = row[(pc.tok_begin + kSub * i0) / B];
    ph1 = row[(pc.tok_begin + kSub * i1) / B];
  };
  auto pair_load = [&](Cur c, int ph0, int ph1, Tile& t0, Tile& t1) {
    const Piece pc = uniform_piece(sm.plist[c.p]);
    const int n = count(c.p);
    Engine::load_tile(a, pc, wave + kWaves * c.k, ph0, t0);
    Engine::load_tile(a, pc, wave + kWaves * min(c.k + 1, n - 1), ph1, t1);
  };

  Cur cc{first_piece_from(0), 0};
  if (cc.p < npl) {
    // prologue: the first pair, then the scalar table reads of the next
    Cur pf = cc, lastv = cc;
    Tile t0, t1;
    int ph0, ph1;
    pair_phys(pf, ph0, ph1);
    pair_load(pf, ph0, ph1, t0, t1);
    pf = advance(pf);
    if (pf.p >= npl) pf = lastv; else lastv = pf;
    pair_phys(pf, ph0, ph1);
    __syncthreads();  // query groups staged (see run_decode)

    for (int p = 0; p < npl; ++p) {
      State st;
      Engine::reset(st);
      const Piece pc = uniform_piece(sm.plist[p]);
      if (cc.p == p) {
        Query q;
        Engine::load_query(sm, p, q);
        const int n = count(p);
        while (true) {
          Engine::compute(a, sm, pc, q, st, t0, wave + kWaves * cc.k);
          // prefetch the next pair (possibly in a later piece) into t0, t1
          const Piece pn = uniform_piece(sm.plist[pf.p]);
          const int nn = count(pf.p);
          Engine::load_tile(a, pn, wave + kWaves * pf.k, ph0, t0);
          if (cc.k + 1 < n) Engine::compute(a, sm, pc, q, st, t1, wave + kWaves * (cc.k + 1));
          Engine::load_tile(a, pn, wave + kWaves * min(pf.k + 1, nn - 1), ph1, t1);
          cc = advance(cc);
          pf = advance(pf);
          if (pf.p >= npl) pf = lastv; else lastv = pf;
          pair_phys(pf, ph0, ph1);
          if (cc.p != p) break;
        }
      }
      Engine::to_lds(sm, st, wave);
      __syncthreads();
      emit_piece<T, G>(a, sm, pc);
      __syncthreads();
    }
  } else {
    __syncthreads();  // query groups staged
    for (int p = 0; p < npl; ++p) {
      State st;
      Engine::reset(st);
      Engine::to_lds(sm, st, wave);
      __syncthreads();
      emit_piece<T, G>(a, sm, uniform_piece(sm.plist[p]));
      __syncthreads();
    }
  }
  (void)chunk;
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
    sm.ncommit = 0;
  }
  __syncthreads();
  constexpr int kQChunks = G * kD * T::kEsize / 16;  // 16-byte chunks per query group
  while (true) {
    if (threadIdx.x == 0) {
      int f = sm.next_f, n = 0;
      while (f < e && n < Smem::kBatch) {
        Piece pc;
        pc.b = find_seq(cum, a.S, a.Hkv, f);
        const int nb = cum[pc.b + 1] - cum[pc.b];
        const int base = cum[pc.b] * a.Hkv;
        pc.kvh = (f - base) / nb;
        const int j0 = (f - base) - pc.kvh * nb;
        const int ustart = base + pc.kvh * nb;
        const int pe = min(e, ustart + nb);
        const int j1 = j0 + (pe - f);
        pc.L = lens_s[pc.b];
        pc.tok_begin = j0 * B;
        pc.tok_end = min(j1 * B, pc.L);
        pc.nsub = (pc.tok_end - pc.tok_begin + kSub - 1) / kSub;
        pc.complete = (j0 == 0) && (j1 == nb);
        pc.slot = 2 * chunk + (f == s ? 0 : 1);
        pc.kfirst = ustart / c;
        pc.npieces = (ustart + nb - 1) / c - pc.kfirst + 1;
        pc.first_slot = 2 * pc.kfirst + (ustart != pc.kfirst * c ? 1 : 0);
        sm.plist[n++] = pc;
        f = pe;
      }
      sm.npl = n;
      sm.next_f = f;
    }
    __syncthreads();
    const int npl = sm.npl;
    if (npl == 0) break;
    // Stage the batch's query groups in LDS (issued before any tile load).
    for (int x = threadIdx.x; x < npl * kQChunks; x += kThreads) {
      const int p = x / kQChunks, k = x % kQChunks;
      const Piece& pc = sm.plist[p];
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
          ((int64_t)pc.b * a.Hq + (int64_t)pc.kvh * G) * kD * T::kEsize);
      sm.q[p][k] = src[k];
    }
    stream_batch<T, B, G, Engine>(a, sm, chunk);
    __syncthreads();
  }
  commit_splits<T, G>(a, sm);
}

}  // namespace pa
