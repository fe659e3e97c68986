// decode_bf16_shared.hip — shared-prefix decode kernels for BF16 inputs
// (prefix groups read once per group; matrix cores), every block size and
// group size built.
#include "decode_shared_inst.h"

namespace pa {

Variant decode_shared_variant_bf16(int B, int G) { return shared_pick<BF16>(B, G); }

}  // namespace pa
