// cache_kernels.hip — launchers of the kernels that write the cache
// (append, copy-on-write block copy) and of the block-wise eviction scan.
#include "dispatch.h"
#include "evict_scan.h"
#include "kv_write.h"

namespace pa {

hipError_t launch_append(const AppendArgs& a, int esize, int grid, hipStream_t s) {
  if (esize == 4)
    hipLaunchKernelGGL(append_kernel<4>, dim3(grid), dim3(kAuxThreads), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<2>, dim3(grid), dim3(kAuxThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kAuxThreads), 0, s, a);
  return hipGetLastError();
}

template <class T>
hipError_t launch_scores(const ScoreArgs& a, int B, hipStream_t s) {
  const dim3 grid((unsigned)((a.mbs + kAuxWaves - 1) / kAuxWaves), (unsigned)a.S);
  if (B == 16)
    hipLaunchKernelGGL((block_score_kernel<T, 16>), grid, dim3(kAuxThreads), 0, s, a);
  else
    hipLaunchKernelGGL((block_score_kernel<T, 32>), grid, dim3(kAuxThreads), 0, s, a);
  return hipGetLastError();
}

// Scores, then the per-sequence choice, on one stream.
hipError_t launch_block_scores(const ScoreArgs& a, int dtype_code, int B, hipStream_t s) {
  hipError_t e;
  switch (dtype_code) {
    case F32::kCode: e = launch_scores<F32>(a, B, s); break;
    case F16::kCode: e = launch_scores<F16>(a, B, s); break;
    default: e = launch_scores<BF16>(a, B, s); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(evict_choice_kernel, dim3((unsigned)((a.S + kAuxWaves - 1) / kAuxWaves)),
                     dim3(kAuxThreads), 0, s, a, B);
  return hipGetLastError();
}

}  // namespace pa
