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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

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

template <int G>
struct MergeSmem {
  float o[kWaves][G][kD + 4];
  float m[kWaves][G];
  float l[kWaves][G];
};

__device__ __forceinline__ float rescale(float mi, float m) {
  return mi == -INFINITY ? 0.f : fast_exp2(mi - m);
}

// Combine the kWaves wave partials held in `sm` and emit the piece's result:
// the final output (complete piece) or a workspace partial.  All threads call;
// the caller has synchronised after the waves wrote `sm`.
template <class T, int G>
__device__ inline void emit_piece(const Args& a, MergeSmem<G>& sm, int b, int kvh,
                                  bool complete, int slot) {
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
    if (complete) {
      const int64_t oi = ((int64_t)b * a.Hq + kvh * G + g) * kD + d;
      store_out<T>(a.out, oi, o / l, a.out_f32);
    } else {
      a.ws_o[((int64_t)slot * G + g) * kD + d] = o;
      if (d == 0) {
        a.ws_ml[((int64_t)slot * G + g) * 2 + 0] = M;
        a.ws_ml[((int64_t)slot * G + g) * 2 + 1] = l;
      }
    }
  }
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
    const int b = find_seq(cum, a.S, a.Hkv, f);
    const int nb = cum[b + 1] - cum[b];
    const int base = cum[b] * a.Hkv;
    const int kvh = (f - base) / nb;
    const int j0 = (f - base) - kvh * nb;
    const int pe = min(e, base + (kvh + 1) * nb);
    const int j1 = j0 + (pe - f);
    const bool complete = (j0 == 0) && (j1 == nb);
    const int slot = 2 * chunk + (f == s ? 0 : 1);
    Engine::piece(a, sm, b, kvh, j0, j1, a.lens[b], complete, slot);
    f = pe;
  }
}

}  // namespace pa
