// Decode-kernel instantiations, f16 activations.
#define FP4_ACT 1
#define FP4_DECODE_FN launch_decode_f16
#include "decode_inst.inc"
