// decode_inst.h — the decode kernel template and its per-variant launcher
// and occupancy query.  Each decode translation unit includes this header
// and instantiates one element type and engine for every block size and
// group size it builds.
#pragma once

#include "dispatch.h"
#include "decode_mfma.h"
#include "decode_valu.h"

namespace pa {

template <class T, int B, int G, bool kMfma>
__global__ __launch_bounds__(kThreads) void decode_kernel(Args a) {
  if constexpr (kMfma)
    run_decode<T, B, G, MfmaEngine<T, B, G>>(a);
  else
    run_decode<T, B, G, ValuEngine<T, B, G>>(a);
}

template <class T, int B, int G, bool M>
hipError_t launch_decode(const Args& a, int grid, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<T, B, G, M>), dim3(grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <class T, int B, int G, bool M>
int decode_occupancy(size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<T, B, G, M>, kThreads, lds) !=
      hipSuccess)
    return 0;
  return n;
}

template <class T, int B, int G, bool M>
Variant make_variant() {
  Variant v;
  v.launch = &launch_decode<T, B, G, M>;
  v.occ = &decode_occupancy<T, B, G, M>;
  return v;
}

// Group sizes built: 1, 2, 4, 8, 16 on the matrix cores, and 32, 64 as
// column-split groups (MQA); on the vector
// ALU those whose registers hold without spilling (1, 2, 4 for 16-bit
// types, 1 for fp32).  Other query groups run as virtual groups of one of
// these (the host's plan).
template <class T, int B, bool M>
Variant pick_group(int G) {
  constexpr int kMaxG = M ? 16 : T::kEsize == 4 ? 1 : 4;
  switch (G) {
    case 1: return make_variant<T, B, 1, M>();
    case 2:
      if constexpr (kMaxG >= 2) return make_variant<T, B, 2, M>();
      return Variant{};
    case 4:
      if constexpr (kMaxG >= 4) return make_variant<T, B, 4, M>();
      return Variant{};
    case 8:
      if constexpr (kMaxG >= 8) return make_variant<T, B, 8, M>();
      return Variant{};
    case 16:
      if constexpr (kMaxG >= 16) return make_variant<T, B, 16, M>();
      return Variant{};
    case 32:
      if constexpr (M) return make_variant<T, B, 32, M>();
      return Variant{};
    case 64:
      if constexpr (M) return make_variant<T, B, 64, M>();
      return Variant{};
    default: return Variant{};
  }
}

template <class T, bool M>
Variant pick_block(int B, int G) {
  if (B == 16) return pick_group<T, 16, M>(G);
  if (B == 32) return pick_group<T, 32, M>(G);
  return Variant{};
}

}  // namespace pa
