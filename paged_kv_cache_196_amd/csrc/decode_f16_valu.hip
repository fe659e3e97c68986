// decode_f16_valu.hip — vector-ALU decode kernels for F16 inputs, every block
// size and group size built (one translation unit per element type and
// engine so that the instantiations compile in parallel).
#include "decode_inst.h"

namespace pa {

Variant decode_variant_f16_valu(int B, int G) { return pick_block<F16, false>(B, G); }

}  // namespace pa
