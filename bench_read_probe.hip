// bench_read_probe.hip — streaming-read reference used by bench.py.
//
// Reads every byte of a device buffer once with 16-byte vector loads and
// keeps nothing but a running XOR per lane, so its time is the time to
// stream the buffer out of HBM.  The benchmark reports the decode
// kernel's KV bandwidth as a fraction of the best rate this probe reaches
// on the same device, beside the fraction of the published HBM peak.
// Measurement only: it is not part of the decode library.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup w reads the contiguous 16-byte words [w*per, (w+1)*per); each
// pass keeps U loads per lane in flight.  The one store is taken only if
// the XOR of the workgroup's first lane equals a fixed constant, which
// keeps the loads live without writing anything in practice.
template <int U, bool kNontemporal>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         float* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per;
  const size_t end = beg + per < n16 ? beg + per : n16;
  uint32_t acc = 0;
  size_t i = beg + threadIdx.x;
  for (; i + (size_t)(U - 1) * 256 < end; i += (size_t)U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = kNontemporal ? __builtin_nontemporal_load(src + i + (size_t)u * 256) : src[i + (size_t)u * 256];
    __builtin_amdgcn_sched_barrier(0);  // every load of the pass issued before the first use
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += 256) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (threadIdx.x == 0 && acc == 0x9E3779B9u) sink[blockIdx.x] = 1.f;
}

}  // namespace

// Launches the probe over `bytes` bytes at `src` (a multiple of 16) with
// `grid` workgroups of 256 threads on `stream`.  `sink` holds at least
// `grid` floats.  variant 0: plain loads, 1: nontemporal loads.  Returns
// 0, or a nonzero HIP error / -1 for arguments out of range.
extern "C" int pa_bench_read_probe(const void* src, size_t bytes, float* sink, int grid,
                                   int variant, void* stream) {
  if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 || grid <= 0 ||
      grid > (1 << 20) || (variant != 0 && variant != 1))
    return -1;
  const size_t n16 = bytes / 16;
  const auto s = static_cast<hipStream_t>(stream);
  const auto* p = static_cast<const u32x4*>(src);
  if (variant == 1)
    hipLaunchKernelGGL((read_probe_kernel<8, true>), dim3(grid), dim3(256), 0, s, p, n16, sink);
  else
    hipLaunchKernelGGL((read_probe_kernel<8, false>), dim3(grid), dim3(256), 0, s, p, n16, sink);
  return static_cast<int>(hipGetLastError());
}
