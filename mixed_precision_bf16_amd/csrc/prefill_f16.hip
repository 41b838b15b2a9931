// Prefill-kernel instantiations, f16 activations.
#define FP4_ACT 1
#define FP4_PREFILL_FN launch_prefill_f16
#include "prefill_inst.inc"
