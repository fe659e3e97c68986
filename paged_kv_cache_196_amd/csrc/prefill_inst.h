// prefill_inst.h — prefill launchers for one element type: every block
// size and group size built.
#pragma once

#include "dispatch.h"
#include "prefill_mfma.h"

namespace pa {

template <class T, int B, int G>
void launch_prefill(const PrefillArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<T, B, G>), grid, dim3(kPrefillThreads), 0, s, a);
}

template <class T, int B>
PrefillFn prefill_for_group(int G) {
  switch (G) {
    case 1: return launch_prefill<T, B, 1>;
    case 2: return launch_prefill<T, B, 2>;
    case 4: return launch_prefill<T, B, 4>;
    case 8: return launch_prefill<T, B, 8>;
    case 16: return launch_prefill<T, B, 16>;
    default: return nullptr;
  }
}

template <class T>
PrefillFn prefill_pick(int B, int G) {
  if (B == 16) return prefill_for_group<T, 16>(G);
  if (B == 32) return prefill_for_group<T, 32>(G);
  return nullptr;
}

}  // namespace pa
