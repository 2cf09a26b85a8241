// Fused decode-step kernels for a launch holding LORES_BF16 and LORES_INT8 heads:
// work-groups of both classes share the device, so the VALU-heavier and the
// HBM-heavier class overlap (see lores_step_impl.h).
#include "lores_step_impl.h"

namespace lores {

hipError_t launch_step_bf16_int8(int dk, bool per_channel, bool delta, bool in_bf16,
                               const StepPtrs &p, const StepMeta &m, hipStream_t s) {
    return launch_classes<LORES_BF16, LORES_INT8>(dk, per_channel, delta, in_bf16, p, m, s);
}

}  // namespace lores
