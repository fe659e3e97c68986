// decode_shared_inst.h — the shared-prefix decode kernel template and its
// launcher / occupancy query, instantiated per element type.
#pragma once

#include "dispatch.h"
#include "shared_prefix.h"

namespace pa {

template <class T, int B, int G>
__global__ __launch_bounds__(kThreads) void decode_shared_kernel(Args a) {
  run_decode_shared<T, B, G>(a);
}

template <class T, int B, int G>
hipError_t launch_decode_shared(const Args& a, int grid, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((decode_shared_kernel<T, B, G>), dim3(grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <class T, int B, int G>
int decode_shared_occupancy(size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_shared_kernel<T, B, G>, kThreads,
                                                   lds) != hipSuccess)
    return 0;
  return n;
}

// Group sizes 1 .. 8 (items of 32 .. 4 members).  At G = 16 an item would
// pair two members only; those calls run the ordinary decode.
template <class T, int B>
Variant shared_pick_group(int G) {
  Variant v;
  switch (G) {
#define PA_SHARED_CASE(g)                             \
  case g:                                             \
    v.launch = &launch_decode_shared<T, B, g>;        \
    v.occ = &decode_shared_occupancy<T, B, g>;        \
    break;
    PA_SHARED_CASE(1)
    PA_SHARED_CASE(2)
    PA_SHARED_CASE(4)
    PA_SHARED_CASE(8)
#undef PA_SHARED_CASE
    default: break;
  }
  return v;
}

template <class T>
Variant shared_pick(int B, int G) {
  if (B == 16) return shared_pick_group<T, 16>(G);
  if (B == 32) return shared_pick_group<T, 32>(G);
  return Variant{};
}

}  // namespace pa
