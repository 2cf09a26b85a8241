// Windowed requantization: a state rounded once per window of W decode steps,
// the window's tokens buffered at fp32 (the reading of the PACE and
// LeapQuant abstracts: rounding once every few tokens with the tokens in
// between kept in a buffer; recurrence and quantizer as in
// lores_step_impl.h).
//
// Windows are the steps t = kW + 1 .. (k + 1) W, position p = (t - 1) mod W
// + 1.  The stored codes and scales hold X_0, the state at the window start;
// a unit's window block holds slots tau = 1 .. W - 1 of (g_tau, k_tau,
// alpha_tau), what the recurrence needs to rebuild S from X_0 in fp32:
//   S'_1 = fl(c fl(s alpha_1)),  S'_tau = fl(U_{tau-1} alpha_tau),
//   U_tau = fma(g_tau, k_tau, S'_tau).
// With a scalar decay the same state is, in closed form,
//   S_{p-1} = c_{p-1} X_0 + sum_{tau < p} d_tau g_tau k_tau^T,
//   c_{p-1} = prod_{sigma < p} alpha_sigma,  d_tau = prod_{tau < sigma < p} alpha_sigma,
// so a step inside the window needs only X_0 . k, X_0 . q (two dot products
// per stored row, read-only) and the buffered tokens' dot products with k and
// q (per unit):
//   r_i = alpha_p (c s_i sum_j c_ij k_j + sum_tau d_tau g_tau,i (k_tau . k)),
//   o_i = alpha_p (c s_i sum_j c_ij q_j + sum_tau d_tau g_tau,i (k_tau . q)) + g_i (k . q).
// The last step of a window replays the buffer in the exact order above, so
// its requantized state is the fp32 recurrence's, and steps as usual.
#include "lores_step_impl.h"

namespace lores {

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// x . y for two row vectors (register i holds element 16 i + lane % 16): the
// registers' products, then a sum over the 16 lanes of a row (lane ^ 1,
// lane ^ 2, lane ^ 7 within 8, lane ^ 8), which every row holds alike.
template <int NV>
__device__ __forceinline__ float rowdot(const float *x, const float *y) {
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) p = __builtin_fmaf(x[i], y[i], p);
    p += dpp_f<0xB1>(p);      // quad_perm [1, 0, 3, 2]
    p += dpp_f<0x4E>(p);      // quad_perm [2, 3, 0, 1]
    p += dpp_f<0x141>(p);     // row_half_mirror
    p += dpp_f<0x128>(p);     // row_ror:8
    return p;
}

// Element j of a stored row held in chunk registers cw: the offset-binary
// integer (code + off) of an int row, the E4M3 value of an fp8 row.  j is a
// constant once the callers' loops are unrolled.
template <int PREC>
__device__ __forceinline__ float stored(const u32x4 *cw, int j) {
    if constexpr (PREC == LORES_INT6) {
        return (float)int6_field(cw, j);
    } else if constexpr (PREC == LORES_FP8) {
        return fp8_value(cw[j >> 4][(j >> 2) & 3], j & 3);
    } else if constexpr (PREC == LORES_INT8) {
        return (float)((cw[j >> 4][(j >> 2) & 3] >> (8 * (j & 3))) & 0xFFu);
    } else {
        const uint32_t w = cw[j >> 5][(j >> 3) & 3];
        const uint32_t nib = (j & 1) ? and_opaque(w >> 4, 0x0F0F0F0Fu) : and_opaque(w, 0x0F0F0F0Fu);
        return (float)((nib >> (8 * ((j & 7) >> 1))) & 0xFFu);
    }
}

// fl(code * a): int rows as fma(code + off, a, -off a), exact since off * a is
// a power-of-two multiple of a
template <int PREC>
__device__ __forceinline__ float scaled_code(const u32x4 *cw, int j, float a, float na) {
    if constexpr (PREC == LORES_FP8) return stored<PREC>(cw, j) * a;
    else return __builtin_fmaf(stored<PREC>(cw, j), a, na);
}

struct WindowTask {
    int slot, rb, h, row, lrow;
    long unit, bh;
    bool active;
};

__device__ __forceinline__ bool window_task(const StepMeta &meta, WindowTask &w) {
    const ClassDesc &cd = meta.cls[0];
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int task = blockIdx.x * kWavesPerGroup + wv;
    if (task >= cd.Hc * meta.n_rb) return false;
    w.slot = task / meta.n_rb;
    w.rb = task - w.slot * meta.n_rb;
    const int b = blockIdx.y;
    w.unit = (long)b * cd.Hc + w.slot;
    w.h = (int)meta.heads[cd.head_off + w.slot];
    w.bh = (long)b * meta.H + w.h;
    w.row = w.rb * 64 + (threadIdx.x & 63);
    w.active = w.row < meta.dv;
    w.lrow = w.active ? w.row : meta.dv - 1;
    return true;
}

// ---------------------------------------------------------------------------
// a step inside a window (p < W): read X_0, buffer the token
// ---------------------------------------------------------------------------
// KEY: key-column scales: X_0 . k = sum_j c_ij (s_j k_j), so the dot products
// take s o k and s o q and there is no row scale.
template <int DK, int PREC, bool DELTA, bool BF16IN, bool KEY>
__global__ void __launch_bounds__(64 * kWavesPerGroup)
lores_window_read_kernel(const void *__restrict__ qp, const void *__restrict__ kp,
                         const void *__restrict__ vp, const float *__restrict__ alphap,
                         const float *__restrict__ betap, float *__restrict__ op,
                         const uint8_t *__restrict__ codes, const float *__restrict__ scales,
                         float *__restrict__ win, const StepMeta meta) {
    constexpr int NCH = row_chunks<DK, PREC>(), NV = DK / 16;
    WindowTask w;
    if (!window_task(meta, w)) return;
    const int lane = threadIdx.x & 63;
    const long dv_pad = meta.dv_pad;
    const u32x4 *cp = reinterpret_cast<const u32x4 *>(codes + w.unit * meta.cls[0].unit_bytes) + w.lrow;
    u32x4 cw[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) cw[c] = __builtin_nontemporal_load(cp + c * dv_pad);
    const float s = KEY ? 1.0f : scales[w.unit * dv_pad + w.lrow];
    const float v = in_scalar<BF16IN>(vp, w.bh * meta.dv + w.lrow);
    const float beta = betap[w.bh], alpha = alphap[w.bh];
    float kv[NV], qv[NV], ks[NV], qs[NV];
    const long kb = w.bh * DK + (lane & 15);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        kv[i] = in_scalar<BF16IN>(kp, kb + 16 * i);
        qv[i] = in_scalar<BF16IN>(qp, kb + 16 * i);
        if constexpr (KEY) {
            const float sc = scales[w.unit * DK + 16 * i + (lane & 15)];
            ks[i] = sc * kv[i];
            qs[i] = sc * qv[i];
        } else {
            ks[i] = kv[i];
            qs[i] = qv[i];
        }
    }
    const int p = meta.wpos, nslot = meta.window - 1;
    float *ub = win + w.unit * window_unit_floats(meta.window, meta.dv_pad, DK);
    float *gslot = ub, *kslot = ub + (long)nslot * dv_pad, *aslot = kslot + (long)nslot * DK;

    // sum_j c_ij k_j and sum_j c_ij q_j over the stored row (codes unscaled):
    // int rows take the stored offset-binary integers c + off and subtract
    // off * sum_j k_j once (a different rounding of the same sum)
    float A = 0.0f, Bq = 0.0f;
#pragma unroll
    for (int gi = 0; gi < NV; ++gi) {
        float x[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = stored<PREC>(cw, 16 * gi + e);
        if constexpr (DELTA) dot16(A, x, ks[gi]);
        dot16(Bq, x, qs[gi]);
    }
    if constexpr (PREC != LORES_FP8) {
        float ones[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) ones[i] = 1.0f;
        if constexpr (DELTA) A = __builtin_fmaf(-Prec<PREC>::OFF, rowdot<NV>(ks, ones), A);
        Bq = __builtin_fmaf(-Prec<PREC>::OFF, rowdot<NV>(qs, ones), Bq);
    }

    // the buffered tokens, latest first: d_tau = product of the later decays
    float rs = 0.0f, os = 0.0f, d = 1.0f;
    for (int tau = p - 1; tau >= 1; --tau) {
        const float gt = gslot[(long)(tau - 1) * dv_pad + w.lrow];
        float kt[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) kt[i] = kslot[(long)(tau - 1) * DK + 16 * i + (lane & 15)];
        const float dg = d * gt;
        if constexpr (DELTA) rs = __builtin_fmaf(dg, rowdot<NV>(kt, kv), rs);
        os = __builtin_fmaf(dg, rowdot<NV>(kt, qv), os);
        d = d * aslot[tau - 1];
    }
    // d is now c_{p-1}, the product of the window's earlier decays
    const float cs = d * s;
    float g;
    if constexpr (DELTA) {
        const float r = alpha * __builtin_fmaf(cs, A, rs);
        g = beta * (v - r);
    } else {
        g = beta * v;
    }
    const float o = __builtin_fmaf(g, rowdot<NV>(kv, qv), alpha * __builtin_fmaf(cs, Bq, os));
    if (w.active) {
        op[w.bh * meta.dv + w.row] = o;
        gslot[(long)(p - 1) * dv_pad + w.row] = g;
    }
    if (w.rb == 0) {
        if (lane < 16) {
#pragma unroll
            for (int i = 0; i < NV; ++i) kslot[(long)(p - 1) * DK + 16 * i + lane] = kv[i];
        }
        if (lane == 0) aslot[p - 1] = alpha;
    }
}

// ---------------------------------------------------------------------------
// the current state of a windowed unit: the stored state followed by the
// first meta.wpos buffered tokens (lores_dequant_state)
// ---------------------------------------------------------------------------
template <int DK, int PREC, bool KEY>
__global__ void __launch_bounds__(64 * kWavesPerGroup)
lores_window_dequant_kernel(const uint8_t *__restrict__ codes, const float *__restrict__ scales,
                            const float *__restrict__ win, float *__restrict__ out,
                            const StepMeta meta) {
    constexpr int NCH = row_chunks<DK, PREC>(), NV = DK / 16;
    WindowTask w;
    if (!window_task(meta, w)) return;
    const int lane = threadIdx.x & 63;
    const long dv_pad = meta.dv_pad;
    const u32x4 *lp = reinterpret_cast<const u32x4 *>(codes + w.unit * meta.cls[0].unit_bytes) + w.lrow;
    u32x4 cw[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) cw[c] = lp[c * dv_pad];
    const int nslot = meta.window - 1, n = meta.wpos;
    const float *ub = win + w.unit * window_unit_floats(meta.window, meta.dv_pad, DK);
    const float *gslot = ub, *kslot = ub + (long)nslot * dv_pad, *aslot = kslot + (long)nslot * DK;
    float U[DK];
    // token 1: fl(c fl(s alpha_1)), with the row's or column j's scale s
    const float s = KEY ? 0.0f : scales[w.unit * dv_pad + w.lrow];
#pragma unroll
    for (int j = 0; j < DK; ++j) {
        const float a1 = (KEY ? scales[w.unit * DK + j] : s) * aslot[0];
        float na1 = 0.0f;
        if constexpr (PREC != LORES_FP8) na1 = a1 * -Prec<PREC>::OFF;
        U[j] = scaled_code<PREC>(cw, j, a1, na1);
    }
    for (int tau = 1; tau <= n; ++tau) {
        const float gt = gslot[(long)(tau - 1) * dv_pad + w.lrow];
        float kt[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) kt[i] = kslot[(long)(tau - 1) * DK + 16 * i + (lane & 15)];
#pragma unroll
        for (int gi = 0; gi < NV; ++gi) axpy16(&U[16 * gi], gt, kt[gi]);
        if (tau < n) {
            const float an = aslot[tau];
#pragma unroll
            for (int j = 0; j < DK; ++j) U[j] = U[j] * an;
        }
    }
    if (!w.active) return;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    float *orow = out + (w.bh * meta.dv + w.row) * DK;
#pragma unroll
    for (int j = 0; j < DK; j += 4) *reinterpret_cast<f32x4 *>(orow + j) = f32x4{U[j], U[j + 1], U[j + 2], U[j + 3]};
}

// Inside a window: one task per wavefront (a read-only pass, many waves per
// SIMD).  The window's last step: the step kernel's task stream
// with the buffer replayed between pass 1 and the token's own update.
template <int DK, int PREC, bool KEY>
static hipError_t window_dk(bool delta, bool bf16, const StepPtrs &p, const StepMeta &m,
                            hipStream_t s) {
    if (m.wpos == m.window) {
        if (delta) return bf16 ? launch_one<DK, false, true, true, PREC, -1, KEY, true>(p, m, s)
                               : launch_one<DK, false, true, false, PREC, -1, KEY, true>(p, m, s);
        return bf16 ? launch_one<DK, false, false, true, PREC, -1, KEY, true>(p, m, s)
                    : launch_one<DK, false, false, false, PREC, -1, KEY, true>(p, m, s);
    }
    const dim3 grid((m.cls[0].Hc * m.n_rb + kWavesPerGroup - 1) / kWavesPerGroup, m.B);
    const dim3 block(64 * kWavesPerGroup);
#define LORES_WIN_LAUNCH(D, BF)                                                                 \
    hipLaunchKernelGGL((lores_window_read_kernel<DK, PREC, D, BF, KEY>), grid, block, 0, s, p.q,   \
                       p.k, p.v, p.alpha, p.beta, p.o, p.codes[0], p.scales[0], p.win[0], m);
    if (delta) {
        if (bf16) { LORES_WIN_LAUNCH(true, true) } else { LORES_WIN_LAUNCH(true, false) }
    } else {
        if (bf16) { LORES_WIN_LAUNCH(false, true) } else { LORES_WIN_LAUNCH(false, false) }
    }
#undef LORES_WIN_LAUNCH
    return hipGetLastError();
}

template <int PREC>
static hipError_t window_prec(int dk, bool delta, bool bf16, bool key, const StepPtrs &p,
                              const StepMeta &m, hipStream_t s) {
    switch (dk) {
        case 64: return key ? window_dk<64, PREC, true>(delta, bf16, p, m, s)
                            : window_dk<64, PREC, false>(delta, bf16, p, m, s);
        case 128: return key ? window_dk<128, PREC, true>(delta, bf16, p, m, s)
                             : window_dk<128, PREC, false>(delta, bf16, p, m, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_window_step(int prec, int dk, bool delta, bool in_bf16, bool key,
                              const StepPtrs &p, const StepMeta &m, hipStream_t s) {
    if (m.wpos < 1 || m.wpos > m.window || m.window < 2) return hipErrorInvalidValue;
    switch (prec) {
        case LORES_INT8: return window_prec<LORES_INT8>(dk, delta, in_bf16, key, p, m, s);
        case LORES_INT4: return window_prec<LORES_INT4>(dk, delta, in_bf16, key, p, m, s);
        case LORES_INT6: return window_prec<LORES_INT6>(dk, delta, in_bf16, key, p, m, s);
        case LORES_FP8: return window_prec<LORES_FP8>(dk, delta, in_bf16, key, p, m, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_window_dequant(int prec, int dk, bool key, const uint8_t *codes,
                                 const float *scales, const float *win, float *out,
                                 const StepMeta &m, hipStream_t s) {
    const dim3 grid((m.cls[0].Hc * m.n_rb + kWavesPerGroup - 1) / kWavesPerGroup, m.B);
    const dim3 block(64 * kWavesPerGroup);
#define LORES_WD(DK, P)                                                                         \
    do {                                                                                        \
        if (key)                                                                                \
            hipLaunchKernelGGL((lores_window_dequant_kernel<DK, P, true>), grid, block, 0, s,   \
                               codes, scales, win, out, m);                                     \
        else                                                                                    \
            hipLaunchKernelGGL((lores_window_dequant_kernel<DK, P, false>), grid, block, 0, s,  \
                               codes, scales, win, out, m);                                     \
    } while (0)
    if (dk == 64) {
        switch (prec) {
            case LORES_INT8: LORES_WD(64, LORES_INT8); break;
            case LORES_INT4: LORES_WD(64, LORES_INT4); break;
            case LORES_INT6: LORES_WD(64, LORES_INT6); break;
            case LORES_FP8: LORES_WD(64, LORES_FP8); break;
            default: return hipErrorInvalidValue;
        }
    } else if (dk == 128) {
        switch (prec) {
            case LORES_INT8: LORES_WD(128, LORES_INT8); break;
            case LORES_INT4: LORES_WD(128, LORES_INT4); break;
            case LORES_INT6: LORES_WD(128, LORES_INT6); break;
            case LORES_FP8: LORES_WD(128, LORES_FP8); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        return hipErrorInvalidValue;
    }
#undef LORES_WD
    return hipGetLastError();
}

}  // namespace lores
