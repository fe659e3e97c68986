// kernel_args.h — argument structs of the cache-write, eviction-scan and
// prefill kernels (passed by value), shared by the kernels and the C ABI.
#pragma once

#include <stdint.h>

namespace pa {

struct AppendArgs {
  const void* kn;  // [S][Hkv][kD] new keys
  const void* vn;  // [S][Hkv][kD] new values
  void* kp;
  void* vp;
  const int32_t* bt;
  const int32_t* pos;  // [S] logical slot of the new token (< 0: none)
  int32_t S, Hkv, B, mbs;
};

struct CopyArgs {
  char* kp;
  char* vp;
  const int32_t* src;
  const int32_t* dst;
  int64_t block_bytes;  // one block of one pool
  int32_t chunks;       // 4 KiB chunks per block of one pool
  int32_t total;        // num_pairs * 2 pools * chunks
};

constexpr int kChunkBytes = 4096;
constexpr int kCopyUnroll = 4;  // chunks per workgroup pass

struct ScoreArgs {
  const void* kp;
  const void* vp;
  const int32_t* bt;
  const int32_t* lens;
  float* scores;   // [S][mbs]
  int32_t* evict;  // [S]
  int32_t S, Hkv, mbs;
};

struct PrefillArgs {
  const void* q;       // [total_q][Hq][kD]
  const void* kp;
  const void* vp;
  const int32_t* bt;   // [S][mbs]
  const int32_t* lens; // [S]
  const int32_t* qs;   // [S + 1] row offsets
  void* out;           // [total_q][Hq][kD]
  float scale_log2;
  int32_t S, Hq, Hkv, mbs, tiles, out_f32;  // tiles: column tiles per (sequence, KV head)
  int32_t Hp, kv_split, kv_shift;           // virtual KV heads, as in the decode arguments
};

constexpr int kPrefillTiles = 2;  // 16-column tiles per wave: they share every K/V sub-tile read
// Four waves per prefill workgroup and two workgroups per CU: the waves
// sharing a SIMD belong to different workgroups, whose per-step barriers
// are independent, so one's softmax overlaps the other's matrix products.
constexpr int kPrefillWaves = 4;
constexpr int kPrefillThreads = 64 * kPrefillWaves;

}  // namespace pa
