// Decode-step kernels for a state whose launch holds only LORES_FP8 (E4M3)
// heads (see lores_step_impl.h).
#include "lores_step_impl.h"

namespace lores {

hipError_t launch_step_fp8(int dk, bool per_channel, bool delta, bool in_bf16,
                         const StepPtrs &p, const StepMeta &m, hipStream_t s) {
    return launch_classes<LORES_FP8, -1>(dk, per_channel, delta, in_bf16, p, m, s);
}

}  // namespace lores
