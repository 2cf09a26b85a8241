// Host-only stand-ins for the kernel launchers of liblores, so that the host
// code (csrc/lores_api.cpp) can be built with AddressSanitizer and
// UndefinedBehaviorSanitizer and driven without a GPU.  Each stand-in records
// the launch it was asked for and touches no memory.
#include "../../quantized_linear_recurrence_amd/csrc/lores_internal.h"

#include "launch_log.h"

LaunchLog g_launches;

extern "C" const char *hipGetErrorString(hipError_t) { return "stub"; }

// The thread's sticky last error, as HIP keeps it: hipGetLastError returns
// and clears it.  Tests plant one (an earlier caller's failure) or make the
// next stand-in launch fail.
hipError_t g_sticky_error = hipSuccess;
bool g_fail_next_launch = false;
extern "C" hipError_t hipGetLastError(void) {
    const hipError_t e = g_sticky_error;
    g_sticky_error = hipSuccess;
    return e;
}

namespace lores {

// Like the real launchers: enqueue, then return the thread's last error.
static hipError_t rec(const char *kind, int p0, int p1, const StepMeta &m) {
    const int Hc[2] = {m.cls[0].Hc, m.cls[1].Hc};
    const int groups[2] = {m.cls[0].groups, m.cls[1].groups};
    g_launches.add(kind, p0, p1, m.wpos, m.window, m.n_cls, m.n_rb, Hc, groups, m.win_pc);
    if (g_fail_next_launch) {
        g_fail_next_launch = false;
        g_sticky_error = hipErrorLaunchFailure;
    }
    return hipGetLastError();
}

#define LORES_STUB(name, p0, p1)                                                               \
    hipError_t name(int, bool, bool, bool, const StepPtrs &, const StepMeta &m, hipStream_t) {  \
        return rec(#name, p0, p1, m);                                                          \
    }
LORES_STUB(launch_step_fp32, LORES_FP32, -1)
LORES_STUB(launch_step_bf16, LORES_BF16, -1)
LORES_STUB(launch_step_int8, LORES_INT8, -1)
LORES_STUB(launch_step_int4, LORES_INT4, -1)
LORES_STUB(launch_step_int6, LORES_INT6, -1)
LORES_STUB(launch_step_fp8, LORES_FP8, -1)
LORES_STUB(launch_step_int8_int4, LORES_INT8, LORES_INT4)
LORES_STUB(launch_step_int4_int6, LORES_INT4, LORES_INT6)
LORES_STUB(launch_step_bf16_int8, LORES_BF16, LORES_INT8)
LORES_STUB(launch_step_bf16_int4, LORES_BF16, LORES_INT4)
LORES_STUB(launch_step_key_int8, LORES_INT8, -2)
LORES_STUB(launch_step_key_int4, LORES_INT4, -2)
LORES_STUB(launch_step_key_int6, LORES_INT6, -2)
LORES_STUB(launch_step_key_fp8, LORES_FP8, -2)
#undef LORES_STUB

hipError_t launch_window_step(int prec, int, bool, bool, bool key, bool pc, const StepPtrs &,
                              const StepMeta &m, hipStream_t) {
    return rec(key ? (pc ? "window_key_pc" : "window_key") : (pc ? "window_pc" : "window"), prec,
               -1, m);
}
hipError_t launch_dequant(int prec, int, const uint8_t *, const float *, float *,
                          const StepMeta &m, hipStream_t, bool) {
    return rec("dequant", prec, -1, m);
}
hipError_t launch_window_dequant(int prec, int, bool, const uint8_t *, const float *,
                                 const float *, float *, const StepMeta &m, hipStream_t) {
    return rec("window_dequant", prec, -1, m);
}
hipError_t launch_quant(int prec, int, const float *, uint8_t *, float *, const StepMeta &m,
                        hipStream_t, bool) {
    return rec("quant", prec, -1, m);
}
hipError_t launch_fill_zero(void *, uint64_t, hipStream_t) {
    StepMeta m{};
    return rec("fill_zero", -1, -1, m);
}

}  // namespace lores
