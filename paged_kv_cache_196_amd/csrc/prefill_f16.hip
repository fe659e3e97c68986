// prefill_f16.hip — causal paged prefill kernels for fp16 inputs.
#include "dispatch.h"
#include "prefill_inst.h"

namespace pa {

PrefillFn prefill_variant_f16(int B, int G) { return prefill_pick<F16>(B, G); }

}  // namespace pa
