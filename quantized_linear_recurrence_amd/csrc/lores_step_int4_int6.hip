// Fused decode-step kernels for a launch holding LORES_INT4 and LORES_INT6
// heads (the mix that promotes the slowest-decaying heads from 4 to 6 bits):
// tasks of both classes alternate inside each wavefront (see
// lores_step_impl.h).
#include "lores_step_impl.h"

namespace lores {

hipError_t launch_step_int4_int6(int dk, bool per_channel, bool delta, bool in_bf16,
                               const StepPtrs &p, const StepMeta &m, hipStream_t s) {
    return launch_classes<LORES_INT4, LORES_INT6>(dk, per_channel, delta, in_bf16, p, m, s);
}

}  // namespace lores
