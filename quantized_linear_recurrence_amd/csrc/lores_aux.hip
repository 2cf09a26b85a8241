// Auxiliary kernels: packed state -> fp32 (lores_dequant_state), fp32 ->
// packed state (lores_quant_state) and the zero fill that sets S_0 = 0 (a
// plain kernel rather than a memset node, so a caller may capture it in a
// graph).
#include "lores_step_impl.h"

namespace lores {

// value = scale * code for int heads (fl of the product), the stored value
// for bf16 / fp32 heads.  Same row mapping as the step: a wavefront per 64
// rows, or per 32 rows split across lane pairs at d_k = 256 (lane L + 32
// takes the second half of the columns).
// KEY: the scale of element j is the unit's key-column scale s_j.
template <int DK, int PREC, bool KEY = false>
__global__ void __launch_bounds__(64 * kWavesPerGroup)
lores_dequant_kernel(const uint8_t *__restrict__ codes, const float *__restrict__ scales,
                     float *__restrict__ out, const StepMeta meta) {
    constexpr bool SPLIT = DK > 128;
    constexpr int CPL = SPLIT ? DK / 2 : DK, RPW = SPLIT ? 32 : 64;
    constexpr int E = Prec<PREC>::E;
    constexpr int NCH = row_chunks<CPL, PREC>();     // chunks of the lane's columns
    const int lane = threadIdx.x & 63;
    const int half = SPLIT ? lane >> 5 : 0;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const ClassDesc &cd = meta.cls[0];
    const int task = blockIdx.x * kWavesPerGroup + wv;
    if (task >= cd.Hc * meta.n_rb) return;
    const int slot = task / meta.n_rb;
    const int rb = task - slot * meta.n_rb;
    const int b = blockIdx.y;
    const long unit = (long)b * cd.Hc + slot;
    const int h = (int)meta.heads[cd.head_off + slot];
    const long bh = (long)b * meta.H + h;
    const int row = rb * RPW + (lane & (RPW - 1));
    if (row >= meta.dv) return;
    const long dv_pad = meta.dv_pad;
    const u32x4 *cp = reinterpret_cast<const u32x4 *>(codes + unit * cd.unit_bytes) + row +
                      half * NCH * dv_pad;
    float s = 0.0f;
    if constexpr (has_scale<PREC>() && !KEY) s = scales[unit * dv_pad + row];
    // the scale of element j (wave-uniform loads for key columns)
    auto sc = [&](int j) {
        if constexpr (KEY) return scales[unit * DK + half * CPL + j];
        else return s;
    };
    float *orow = out + (bh * meta.dv + row) * DK + half * CPL;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    if constexpr (PREC == LORES_INT6) {
        u32x4 cw[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) cw[c] = cp[c * dv_pad];
#pragma unroll
        for (int j = 0; j < CPL; j += 4) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // an odd column holds its code negated
                const float f = (float)int6_field(cw, j + e);
                x[e] = sc(j + e) * ((e & 1) ? 32.0f - f : f - 32.0f);
            }
            *reinterpret_cast<f32x4 *>(orow + j) = f32x4{x[0], x[1], x[2], x[3]};
        }
    } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const u32x4 v = cp[c * dv_pad];
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
            float x[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (c * E + e >= CPL) {              // the padding of a half chunk
                    x[e] = 0.0f;
                    continue;
                }
                if constexpr (PREC == LORES_FP8) {
                    x[e] = sc(c * E + e) * fp8_value(wd[e >> 2], e & 3);
                } else if constexpr (PREC == LORES_INT8) {
                    // an odd column holds its code negated
                    const float f = (float)((wd[e >> 2] >> (8 * (e & 3))) & 0xFFu);
                    x[e] = sc(c * E + e) * ((e & 1) ? 128.0f - f : f - 128.0f);
                } else if constexpr (PREC == LORES_INT4) {
                    const uint32_t w = wd[e >> 3];
                    const float f = (float)((w >> (4 * (e & 7))) & 0xFu);
                    x[e] = sc(c * E + e) * ((e & 1) ? 8.0f - f : f - 8.0f);
                } else if constexpr (PREC == LORES_BF16) {
                    const uint32_t w = wd[e >> 1];
                    x[e] = __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
                } else {
                    x[e] = __uint_as_float(wd[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                if (c * E + e < CPL)
                    *reinterpret_cast<f32x4 *>(orow + c * E + e) = f32x4{x[e], x[e + 1], x[e + 2], x[e + 3]};
            }
        }
    }
}

// fp32 rows -> packed rows of one class with the step's own requantization
// (requantize_row), keyed at meta.t.  Same row mapping as the step (split
// rows at d_k = 256: the row maximum combined across the lane pair).
// KEY: key-column scales from the column maxima of the unit's rows (the
// unit's row blocks are consecutive wavefronts of one work-group).
template <int DK, int PREC, bool KEY = false>
__global__ void __launch_bounds__(64 * (KEY && DK > 128 ? kMaxKeyGroupWaves : kWavesPerGroup))
lores_quant_kernel(const float *__restrict__ X, uint8_t *__restrict__ codes,
                   float *__restrict__ scales, const StepMeta meta) {
    constexpr bool SPLIT = DK > 128;
    constexpr int CPL = SPLIT ? DK / 2 : DK, RPW = SPLIT ? 32 : 64;
    const int lane = threadIdx.x & 63;
    const int half = SPLIT ? lane >> 5 : 0;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const ClassDesc &cd = meta.cls[0];
    const int task = blockIdx.x * (KEY ? key_group_waves(meta.n_rb) : kWavesPerGroup) + wv;
    if (task >= cd.Hc * meta.n_rb) {
        if constexpr (KEY) {
            if (meta.n_rb > 1) lds_barrier();      // the work-group's one barrier
        }
        return;
    }
    const int slot = task / meta.n_rb;
    const int rb = task - slot * meta.n_rb;
    const int b = blockIdx.y;
    const long unit = (long)b * cd.Hc + slot;
    const int h = (int)meta.heads[cd.head_off + slot];
    const long bh = (long)b * meta.H + h;
    const int row = rb * RPW + (lane & (RPW - 1));
    const bool active = row < meta.dv;
    const long dv_pad = meta.dv_pad;
    // padding lanes read the last real row and store nothing
    const float *xrow = X + (bh * meta.dv + (active ? row : meta.dv - 1)) * DK + half * CPL;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    float U[CPL];
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; c += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(xrow + c);
        U[c] = v.x;
        U[c + 1] = v.y;
        U[c + 2] = v.z;
        U[c + 3] = v.w;
    }
    const CodeRows io(codes + unit * cd.unit_bytes, cd.unit_bytes, row, dv_pad,
                      half * row_chunks<CPL, PREC>());
    if constexpr (KEY) {
        constexpr int SLOT = key_slot<DK>(), LW = key_lds_waves<DK>();
        constexpr int NCM = SPLIT ? 4 : key_groups<DK>();
        __shared__ float cmax[2 * LW * SLOT];               // maxima, staging
        float cm[NCM], snew[NCM], inv[CPL / 16];
        if constexpr (SPLIT) col_absmax_split(U, cm);
        else col_absmax<DK>(U, cm);
        auto col_of = [](int j, int L) {
            if constexpr (SPLIT) return key_col_split<CPL>(j, L);
            else return key_col(j, L);
        };
        key_scales(cm, cmax, cmax + LW * SLOT, wv, rb, meta.n_rb, Prec<PREC>::R, snew, inv,
                   col_of, half * CPL);
        if (rb == 0) {
#pragma unroll
            for (int t = 0; t < NCM; ++t) {
                const int col = col_of(t, lane);
                if (col < DK) scales[unit * DK + col] = snew[t];
            }
        }
        requantize_row<CPL, PREC, true>(U, 0.0f, meta, b, h, row, active, io, nullptr, inv,
                                        half * CPL);
    } else {
#pragma unroll
        for (int j = 0; j < CPL; ++j) m = fmaxf(m, fabsf(U[j]));
        if constexpr (SPLIT) m = pair_max(m);
        requantize_row<CPL, PREC>(U, m, meta, b, h, row, active, io,
                                  has_scale<PREC>() ? scales + unit * dv_pad + row : nullptr,
                                  nullptr, half * CPL);
    }
}

template <int PREC>
static hipError_t quant_prec(int dk, const float *X, uint8_t *codes, float *scales,
                             const StepMeta &m, hipStream_t s, bool key) {
    const dim3 grid((m.cls[0].Hc * m.n_rb + kWavesPerGroup - 1) / kWavesPerGroup, m.B);
    const dim3 block(64 * kWavesPerGroup);
    if constexpr (has_scale<PREC>()) {
        if (key) {
            const int gw = key_group_waves(m.n_rb);
            const dim3 kgrid((m.cls[0].Hc * m.n_rb + gw - 1) / gw, m.B), kblock(64 * gw);
            switch (dk) {
                case 32: hipLaunchKernelGGL((lores_quant_kernel<32, PREC, true>), kgrid, kblock, 0, s, X, codes, scales, m); break;
                case 64: hipLaunchKernelGGL((lores_quant_kernel<64, PREC, true>), kgrid, kblock, 0, s, X, codes, scales, m); break;
                case 96: hipLaunchKernelGGL((lores_quant_kernel<96, PREC, true>), kgrid, kblock, 0, s, X, codes, scales, m); break;
                case 128: hipLaunchKernelGGL((lores_quant_kernel<128, PREC, true>), kgrid, kblock, 0, s, X, codes, scales, m); break;
                case 160: hipLaunchKernelGGL((lores_quant_kernel<160, PREC, true>), kgrid, kblock, 0, s, X, codes, scales, m); break;
                case 192: hipLaunchKernelGGL((lores_quant_kernel<192, PREC, true>), kgrid, kblock, 0, s, X, codes, scales, m); break;
                case 224: hipLaunchKernelGGL((lores_quant_kernel<224, PREC, true>), kgrid, kblock, 0, s, X, codes, scales, m); break;
                case 256: hipLaunchKernelGGL((lores_quant_kernel<256, PREC, true>), kgrid, kblock, 0, s, X, codes, scales, m); break;
                default: return hipErrorInvalidValue;
            }
            return hipGetLastError();
        }
    }
    switch (dk) {
        case 32: hipLaunchKernelGGL((lores_quant_kernel<32, PREC>), grid, block, 0, s, X, codes, scales, m); break;
        case 64: hipLaunchKernelGGL((lores_quant_kernel<64, PREC>), grid, block, 0, s, X, codes, scales, m); break;
        case 96: hipLaunchKernelGGL((lores_quant_kernel<96, PREC>), grid, block, 0, s, X, codes, scales, m); break;
        case 128: hipLaunchKernelGGL((lores_quant_kernel<128, PREC>), grid, block, 0, s, X, codes, scales, m); break;
        case 160: hipLaunchKernelGGL((lores_quant_kernel<160, PREC>), grid, block, 0, s, X, codes, scales, m); break;
        case 192: hipLaunchKernelGGL((lores_quant_kernel<192, PREC>), grid, block, 0, s, X, codes, scales, m); break;
        case 224: hipLaunchKernelGGL((lores_quant_kernel<224, PREC>), grid, block, 0, s, X, codes, scales, m); break;
        case 256: hipLaunchKernelGGL((lores_quant_kernel<256, PREC>), grid, block, 0, s, X, codes, scales, m); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quant(int prec, int dk, const float *X, uint8_t *codes, float *scales,
                        const StepMeta &m, hipStream_t s, bool key) {
    switch (prec) {
        case LORES_FP32: return quant_prec<LORES_FP32>(dk, X, codes, scales, m, s, key);
        case LORES_BF16: return quant_prec<LORES_BF16>(dk, X, codes, scales, m, s, key);
        case LORES_INT8: return quant_prec<LORES_INT8>(dk, X, codes, scales, m, s, key);
        case LORES_INT4: return quant_prec<LORES_INT4>(dk, X, codes, scales, m, s, key);
        case LORES_INT6: return quant_prec<LORES_INT6>(dk, X, codes, scales, m, s, key);
        case LORES_FP8: return quant_prec<LORES_FP8>(dk, X, codes, scales, m, s, key);
        default: return hipErrorInvalidValue;
    }
}

template <int PREC>
static hipError_t dequant_prec(int dk, const uint8_t *codes, const float *scales, float *out,
                               const StepMeta &m, hipStream_t s, bool key) {
    const dim3 grid((m.cls[0].Hc * m.n_rb + kWavesPerGroup - 1) / kWavesPerGroup, m.B);
    const dim3 block(64 * kWavesPerGroup);
    if constexpr (has_scale<PREC>()) {
        if (key) {
            switch (dk) {
                case 32: hipLaunchKernelGGL((lores_dequant_kernel<32, PREC, true>), grid, block, 0, s, codes, scales, out, m); break;
                case 64: hipLaunchKernelGGL((lores_dequant_kernel<64, PREC, true>), grid, block, 0, s, codes, scales, out, m); break;
                case 96: hipLaunchKernelGGL((lores_dequant_kernel<96, PREC, true>), grid, block, 0, s, codes, scales, out, m); break;
                case 128: hipLaunchKernelGGL((lores_dequant_kernel<128, PREC, true>), grid, block, 0, s, codes, scales, out, m); break;
                case 160: hipLaunchKernelGGL((lores_dequant_kernel<160, PREC, true>), grid, block, 0, s, codes, scales, out, m); break;
                case 192: hipLaunchKernelGGL((lores_dequant_kernel<192, PREC, true>), grid, block, 0, s, codes, scales, out, m); break;
                case 224: hipLaunchKernelGGL((lores_dequant_kernel<224, PREC, true>), grid, block, 0, s, codes, scales, out, m); break;
                case 256: hipLaunchKernelGGL((lores_dequant_kernel<256, PREC, true>), grid, block, 0, s, codes, scales, out, m); break;
                default: return hipErrorInvalidValue;
            }
            return hipGetLastError();
        }
    }
    switch (dk) {
        case 32: hipLaunchKernelGGL((lores_dequant_kernel<32, PREC>), grid, block, 0, s, codes, scales, out, m); break;
        case 64: hipLaunchKernelGGL((lores_dequant_kernel<64, PREC>), grid, block, 0, s, codes, scales, out, m); break;
        case 96: hipLaunchKernelGGL((lores_dequant_kernel<96, PREC>), grid, block, 0, s, codes, scales, out, m); break;
        case 128: hipLaunchKernelGGL((lores_dequant_kernel<128, PREC>), grid, block, 0, s, codes, scales, out, m); break;
        case 160: hipLaunchKernelGGL((lores_dequant_kernel<160, PREC>), grid, block, 0, s, codes, scales, out, m); break;
        case 192: hipLaunchKernelGGL((lores_dequant_kernel<192, PREC>), grid, block, 0, s, codes, scales, out, m); break;
        case 224: hipLaunchKernelGGL((lores_dequant_kernel<224, PREC>), grid, block, 0, s, codes, scales, out, m); break;
        case 256: hipLaunchKernelGGL((lores_dequant_kernel<256, PREC>), grid, block, 0, s, codes, scales, out, m); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_dequant(int prec, int dk, const uint8_t *codes, const float *scales,
                          float *out, const StepMeta &m, hipStream_t s, bool key) {
    switch (prec) {
        case LORES_FP32: return dequant_prec<LORES_FP32>(dk, codes, scales, out, m, s, key);
        case LORES_BF16: return dequant_prec<LORES_BF16>(dk, codes, scales, out, m, s, key);
        case LORES_INT8: return dequant_prec<LORES_INT8>(dk, codes, scales, out, m, s, key);
        case LORES_INT4: return dequant_prec<LORES_INT4>(dk, codes, scales, out, m, s, key);
        case LORES_INT6: return dequant_prec<LORES_INT6>(dk, codes, scales, out, m, s, key);
        case LORES_FP8: return dequant_prec<LORES_FP8>(dk, codes, scales, out, m, s, key);
        default: return hipErrorInvalidValue;
    }
}

// bytes is a multiple of 16 (segments are 256-byte aligned and padded).
__global__ void __launch_bounds__(256) lores_fill_zero_kernel(u32x4 *__restrict__ p, uint64_t n) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_fill_zero(void *buf, uint64_t bytes, hipStream_t s) {
    const uint64_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    uint64_t groups = (n + 255) / 256;
    if (groups > 65536) groups = 65536;
    hipLaunchKernelGGL(lores_fill_zero_kernel, dim3((unsigned)groups), dim3(256), 0, s,
                       reinterpret_cast<u32x4 *>(buf), n);
    return hipGetLastError();
}

}  // namespace lores
