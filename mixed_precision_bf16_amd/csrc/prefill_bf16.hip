// Prefill-kernel instantiations, bf16 activations.
#define FP4_ACT 0
#define FP4_PREFILL_FN launch_prefill_bf16
#include "prefill_inst.inc"
