// Windowed requantization: dispatch of a window step or dequantization to
// the instantiation unit of the class's precision (lores_window_<prec>.hip;
// the kernels are in lores_window_impl.h).
#include "lores_internal.h"

namespace lores {

hipError_t launch_window_step(int prec, int dk, bool delta, bool in_bf16, bool key, bool pc,
                              const StepPtrs &p, const StepMeta &m, hipStream_t s) {
    if (m.wpos < 1 || m.wpos > m.window || m.window < 2) return hipErrorInvalidValue;
    switch (prec) {
        case LORES_INT8: return launch_window_step_int8(dk, delta, in_bf16, key, pc, p, m, s);
        case LORES_INT4: return launch_window_step_int4(dk, delta, in_bf16, key, pc, p, m, s);
        case LORES_INT6: return launch_window_step_int6(dk, delta, in_bf16, key, pc, p, m, s);
        case LORES_FP8: return launch_window_step_fp8(dk, delta, in_bf16, key, pc, p, m, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_window_dequant(int prec, int dk, bool key, const uint8_t *codes,
                                 const float *scales, const float *win, float *out,
                                 const StepMeta &m, hipStream_t s) {
    switch (prec) {
        case LORES_INT8: return launch_window_dequant_int8(dk, key, codes, scales, win, out, m, s);
        case LORES_INT4: return launch_window_dequant_int4(dk, key, codes, scales, win, out, m, s);
        case LORES_INT6: return launch_window_dequant_int6(dk, key, codes, scales, win, out, m, s);
        case LORES_FP8: return launch_window_dequant_fp8(dk, key, codes, scales, win, out, m, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lores
