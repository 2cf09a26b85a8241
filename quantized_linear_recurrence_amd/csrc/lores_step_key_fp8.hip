// Decode-step kernels for LORES_FP8 heads with key-column scales (see
// lores_step_impl.h).
#include "lores_step_impl.h"

namespace lores {

hipError_t launch_step_key_fp8(int dk, bool per_channel, bool delta, bool in_bf16,
                              const StepPtrs &p, const StepMeta &m, hipStream_t s) {
    return launch_classes_key<LORES_FP8>(dk, per_channel, delta, in_bf16, p, m, s);
}

}  // namespace lores
