// Instantiations of the prefill attention kernel for head_dim 64: f16 or
// bf16 inputs, f32 or input-type output, causal or full, with or without
// phase-A issue priority.
#include "fa_internal.h"
#include "fa_prefill_kernel.h"

namespace fa {

const void* prefill_kernel_hd64(bool in_bf16, bool out_f32, bool causal, bool prio) {
    return pick_kernel<64>(in_bf16, out_f32, causal, prio);
}

}  // namespace fa
