// Internal declarations shared by the host API (lores_api.cpp) and the HIP
// kernels (lores_step_*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lores.h"

namespace lores {

// Per-launch description of one precision class of a state.  Passed by value
// as a kernel argument (about 2.1 KiB), so the head table needs no device
// allocation.  Launch grid: x = groups of kWavesPerGroup (head slot, row
// block) tasks, y = sequence b.
struct ClassMeta {
    int32_t B, H, Hc, dv, dv_pad, n_rb;
    int64_t unit_bytes;        // code bytes per (sequence, head) unit
    uint64_t seed, t;
    int64_t seq_base, head_base;
    uint32_t heads[LORES_MAX_HEADS];   // slot -> head index of this class (dwords: scalar loads)
};

// Pointers of one decode-step launch.
struct StepPtrs {
    const void *q, *k, *v;
    const float *alpha, *beta;
    float *o;
    uint8_t *codes;   // class code segment
    float *scales;    // class scale segment (int classes), else nullptr
};

// Launchers, one translation unit per precision class.  Each returns the
// launch status; `dk` is one of 32, 64, 96, 128.
hipError_t launch_step_fp32(int dk, bool per_channel, bool delta, bool in_bf16,
                            const StepPtrs &p, const ClassMeta &m, hipStream_t s);
hipError_t launch_step_bf16(int dk, bool per_channel, bool delta, bool in_bf16,
                            const StepPtrs &p, const ClassMeta &m, hipStream_t s);
hipError_t launch_step_int8(int dk, bool per_channel, bool delta, bool in_bf16,
                            const StepPtrs &p, const ClassMeta &m, hipStream_t s);
hipError_t launch_step_int4(int dk, bool per_channel, bool delta, bool in_bf16,
                            const StepPtrs &p, const ClassMeta &m, hipStream_t s);

hipError_t launch_dequant(int prec, int dk, const uint8_t *codes, const float *scales,
                          float *out, const ClassMeta &m, hipStream_t s);
hipError_t launch_fill_zero(void *buf, uint64_t bytes, hipStream_t s);

// Tasks (one wavefront each) per 256-thread work-group.
constexpr int kWavesPerGroup = 4;

}  // namespace lores
