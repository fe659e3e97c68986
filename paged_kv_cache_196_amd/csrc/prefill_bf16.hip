// prefill_bf16.hip — causal paged prefill kernels for bf16 inputs.
#include "dispatch.h"
#include "prefill_inst.h"

namespace pa {

PrefillFn prefill_variant_bf16(int B, int G) { return prefill_pick<BF16>(B, G); }

}  // namespace pa
