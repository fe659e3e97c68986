// decode_f16_mfma.hip — matrix-core decode kernels for F16 inputs, every block
// size and group size built (one translation unit per element type and
// engine so that the instantiations compile in parallel).
#include "decode_inst.h"

namespace pa {

Variant decode_variant_f16_mfma(int B, int G) { return pick_block<F16, true>(B, G); }

}  // namespace pa
