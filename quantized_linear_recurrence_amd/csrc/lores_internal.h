// Internal declarations shared by the host API (lores_api.cpp) and the HIP
// kernels (lores_step_*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lores.h"

namespace lores {

// One precision class inside a decode-step launch.
struct ClassDesc {
    int32_t prec;          // LORES_* code
    int32_t Hc;            // heads of the class
    int32_t groups;        // work-groups along grid x: ceil(tasks / wavefronts per group)
    int32_t head_off;      // first entry of the class's head list in StepMeta::heads
    int64_t unit_bytes;    // code bytes per (sequence, head) unit
};

// Description of one launch, passed by value as a kernel argument (about
// 2.2 KiB), so no device allocation is needed.  Grid: x runs over the
// work-groups of class 0 then class 1 (kWavesPerGroup (head slot, row block)
// tasks each; a fused int pair first pairs the two classes' tasks, in groups
// of kPairWavesPerGroup); y strides over sequences blockIdx.y,
// blockIdx.y + gridDim.y, ...
struct StepMeta {
    int32_t B, H, dv, dv_pad, n_rb, n_cls;
    int32_t rounding;                  // LORES_ROUND_*
    int32_t wpos;                      // windowed states: position p of step t (1 .. window),
                                       // or, for the dequantization, the buffered tokens
    int32_t window;                    // W (1: requantize every step)
    int32_t win_pc;                    // windowed states: the window's tokens carry one
                                       // decay per key channel (else a scalar per unit)
    uint64_t seed, t;
    int64_t seq_base, head_base;
    ClassDesc cls[2];
    uint32_t heads[LORES_MAX_HEADS];   // head indices, class by class (dwords: scalar loads)
};

// Pointers of one decode-step launch (codes / scales per class of the launch).
struct StepPtrs {
    const void *q, *k, *v;
    const float *alpha, *beta;
    float *o;
    uint8_t *codes[2];
    float *scales[2];        // int classes, else nullptr
    float *win[2];           // window buffers of a windowed state, else nullptr
};

// Floats of one unit's window block: W - 1 slots of g (d_v_pad), then W - 1
// of k (d_k), then W - 1 of alpha (d_k: one decay per key channel, or a
// scalar decay in element 0), padded to 16 bytes.
__host__ __device__ inline int64_t window_unit_floats(int window, int dv_pad, int dk) {
    return ((int64_t)(window - 1) * (dv_pad + 2 * dk) + 3) / 4 * 4;
}

// One launch covers one class or one of the fused pairs (int8, int4),
// (int4, int6), (bf16, int8), (bf16, int4); `p1` is -1 for a single class.  Returns the
// launch status; `dk` is one of 32, 64, 96, 128.
hipError_t launch_step(int dk, bool per_channel, bool delta, bool in_bf16, int p0, int p1,
                       const StepPtrs &p, const StepMeta &m, hipStream_t s, bool key = false);
bool fusable_pair(int p0, int p1);

// Per-translation-unit launchers behind launch_step.
hipError_t launch_step_fp32(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_bf16(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_int8(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_int4(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_int6(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_fp8(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_int8_int4(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_int4_int6(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_bf16_int8(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_bf16_int4(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
// key-column scales (one class per launch, d_k = 64 or 128)
hipError_t launch_step_key_int8(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_key_int4(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_key_int6(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);
hipError_t launch_step_key_fp8(int, bool, bool, bool, const StepPtrs &, const StepMeta &, hipStream_t);

// Windowed states (scalar decay, d_k 64 or 128; `key`: key-column scales):
// the step at window position m.wpos < m.window (read the stored state,
// buffer the token) or = m.window (rebuild, step and requantize).  One class
// per launch.
hipError_t launch_window_step(int prec, int dk, bool delta, bool in_bf16, bool key, bool pc,
                              const StepPtrs &p, const StepMeta &m, hipStream_t s);

// The per-precision window launchers behind the two above
// (lores_window_<prec>.hip).
#define LORES_WINDOW_PREC(N)                                                                   \
    hipError_t launch_window_step_##N(int dk, bool delta, bool in_bf16, bool key, bool pc,     \
                                      const StepPtrs &p, const StepMeta &m, hipStream_t s);    \
    hipError_t launch_window_dequant_##N(int dk, bool key, const uint8_t *codes,              \
                                         const float *scales, const float *win, float *out,    \
                                         const StepMeta &m, hipStream_t s);
LORES_WINDOW_PREC(int8)
LORES_WINDOW_PREC(int4)
LORES_WINDOW_PREC(int6)
LORES_WINDOW_PREC(fp8)
#undef LORES_WINDOW_PREC

// Dequant uses the same StepMeta with one class; `key`: key-column scales.
hipError_t launch_dequant(int prec, int dk, const uint8_t *codes, const float *scales,
                          float *out, const StepMeta &m, hipStream_t s, bool key);
// The current state of a windowed class: the stored state followed by the
// first m.wpos (>= 1) buffered tokens.
hipError_t launch_window_dequant(int prec, int dk, bool key, const uint8_t *codes,
                                 const float *scales, const float *win, float *out,
                                 const StepMeta &m, hipStream_t s);
hipError_t launch_quant(int prec, int dk, const float *X, uint8_t *codes, float *scales,
                        const StepMeta &m, hipStream_t s, bool key);
hipError_t launch_fill_zero(void *buf, uint64_t bytes, hipStream_t s);

// Tasks (one wavefront each) per 256-thread work-group.
constexpr int kWavesPerGroup = 4;
// Wavefronts per work-group of a fused int-pair launch (512 threads: one
// group per CU at two wavefronts per SIMD, sharing a work queue).
constexpr int kPairWavesPerGroup = 8;

// Wavefronts per work-group of the launches whose wavefronts exchange
// key-column maxima (key-column steps and quantization): a unit's n_rb row
// blocks must share one work-group, so units of three row blocks run in
// three-wavefront groups, units of more than four (32-row tasks at d_k =
// 256) in groups of their own size, and all others in kWavesPerGroup.
__host__ __device__ constexpr int key_group_waves(int n_rb) {
    return n_rb == 3 ? 3 : n_rb <= kWavesPerGroup ? kWavesPerGroup : n_rb;
}
// wavefronts of the largest key-column work-group: a unit of 32-row tasks
// (d_k = 256) has up to 8 row blocks
constexpr int kMaxKeyGroupWaves = 8;

}  // namespace lores
