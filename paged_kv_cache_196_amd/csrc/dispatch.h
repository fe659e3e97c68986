// dispatch.h — host-side launchers of the gfx950 kernels, one getter per
// translation unit, so that the kernel instantiations compile in parallel
// (decode per element type and engine, prefill per element type, and the
// cache-write / eviction-scan kernels) and the C ABI (pagedattn.hip) picks
// among them at run time.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_device.h"

namespace pa {

struct PrefillArgs;
struct AppendArgs;
struct CopyArgs;
struct ScoreArgs;

// One decode kernel instantiation: its launcher and its occupancy query
// (resident workgroups per CU for a given dynamic LDS size).
using LaunchFn = hipError_t (*)(const Args&, int grid, size_t lds, hipStream_t);
using OccFn = int (*)(size_t lds);
struct Variant {
  LaunchFn launch = nullptr;
  OccFn occ = nullptr;
};

// Decode variants for block size B and group size G; an empty Variant when
// that pair is not built.
Variant decode_variant_bf16_mfma(int B, int G);
Variant decode_variant_f16_mfma(int B, int G);
Variant decode_variant_bf16_valu(int B, int G);
Variant decode_variant_f16_valu(int B, int G);
Variant decode_variant_f32_valu(int B, int G);

// Shared-prefix decode variants (matrix cores, fp16 / bf16; shared_prefix.h).
Variant decode_shared_variant_bf16(int B, int G);
Variant decode_shared_variant_f16(int B, int G);

// Prefill launchers (matrix cores: fp16 / bf16), nullptr when not built.
using PrefillFn = void (*)(const PrefillArgs&, dim3, hipStream_t);
PrefillFn prefill_variant_bf16(int B, int G);
PrefillFn prefill_variant_f16(int B, int G);

// Cache writes and eviction scoring; each returns hipGetLastError().
hipError_t launch_append(const AppendArgs& a, int esize, int grid, hipStream_t s);
hipError_t launch_copy_blocks(const CopyArgs& a, int grid, hipStream_t s);
hipError_t launch_block_scores(const ScoreArgs& a, int dtype_code, int B, hipStream_t s);

}  // namespace pa
