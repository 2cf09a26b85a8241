// Windowed requantization for int4 states: instantiation unit of
// lores_window_impl.h (one per precision, so they compile in parallel).
#include "lores_window_impl.h"

namespace lores {

hipError_t launch_window_step_int4(int dk, bool delta, bool in_bf16, bool key, bool pc,
                                 const StepPtrs &p, const StepMeta &m, hipStream_t s) {
    return window_prec<LORES_INT4>(dk, delta, in_bf16, key, pc, p, m, s);
}

hipError_t launch_window_dequant_int4(int dk, bool key, const uint8_t *codes, const float *scales,
                                    const float *win, float *out, const StepMeta &m,
                                    hipStream_t s) {
    return window_dequant_prec<LORES_INT4>(dk, key, codes, scales, win, out, m, s);
}

}  // namespace lores
