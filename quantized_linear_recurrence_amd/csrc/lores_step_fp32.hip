// Decode-step kernels for LORES_FP32 heads (see lores_step_impl.h).
#include "lores_step_impl.h"

namespace lores {

hipError_t launch_step_fp32(int dk, bool per_channel, bool delta, bool in_bf16,
                          const StepPtrs &p, const ClassMeta &m, hipStream_t s) {
    return launch_prec<LORES_FP32>(dk, per_channel, delta, in_bf16, p, m, s);
}

}  // namespace lores
