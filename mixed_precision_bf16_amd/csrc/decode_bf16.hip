// Decode-kernel instantiations, bf16 activations.
#define FP4_ACT 0
#define FP4_DECODE_FN launch_decode_bf16
#include "decode_inst.inc"
