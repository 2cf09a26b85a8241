// Windowed requantization (kernels and launch templates; one translation
// unit per state precision instantiates them): a state rounded once per
// window of W decode steps,
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
// With one decay per key channel the products are per column: with
// C_j = prod_{sigma < p} alpha_sigma,j and D_tau,j = prod_{tau < sigma < p}
// alpha_sigma,j the decayed state S'_p = S_{p-1} diag(alpha_p) reads
//   r_i = s_i sum_j c_ij (C alpha_p k)_j + sum_tau g_tau,i ((D_tau alpha_p k_tau) . k),
//   o_i = s_i sum_j c_ij (C alpha_p q)_j + sum_tau g_tau,i ((D_tau alpha_p k_tau) . q)
//         + g_i (k . q),
// the same dot products with per-column weights (row vectors).
// The last step of a window replays the buffer in the exact order above, so
// its requantized state is the fp32 recurrence's, and steps as usual.
#pragma once

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
// integer of an int row (code + off, or off - code in an odd column, which
// holds its code negated), the E4M3 value of an fp8 row.  j is a constant
// once the callers' loops are unrolled.
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

// A stored row of d_k > 128 columns is two halves, the second starting on a
// chunk: its chunks, and element j of it.
template <int DK, int PREC>
constexpr int stored_chunks() {
    return DK > 128 ? 2 * row_chunks<DK / 2, PREC>() : row_chunks<DK, PREC>();
}
template <int DK, int PREC>
__device__ __forceinline__ float stored_at(const u32x4 *cw, int j) {
    if constexpr (DK > 128) {
        constexpr int H = DK / 2, NH = row_chunks<H, PREC>();
        return j < H ? stored<PREC>(cw, j) : stored<PREC>(cw + NH, j - H);
    } else {
        return stored<PREC>(cw, j);
    }
}

// fl(code * a): int rows as fma(code + off, a, -off a), exact since off * a is
// a power-of-two multiple of a (an odd column: fma(off - code, -a, off a))
template <int DK, int PREC>
__device__ __forceinline__ float scaled_code(const u32x4 *cw, int j, float a, float na) {
    if constexpr (PREC == LORES_FP8) return stored_at<DK, PREC>(cw, j) * a;
    else if (j & 1) return __builtin_fmaf(stored_at<DK, PREC>(cw, j), -a, -na);
    else return __builtin_fmaf(stored_at<DK, PREC>(cw, j), a, na);
}

struct WindowTask {
    int slot, rb, h, row, lrow;
    long unit, bh;
    bool active;
};

__device__ __forceinline__ bool window_task(const StepMeta &meta, WindowTask &w) {
    const ClassDesc &cd = meta.cls[0];
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // tasks of 64 rows (the split rows of the step at d_k = 256 do not apply
    // here: these kernels hold no fp32 row beside the codes)
    const int nrb = (int)(meta.dv_pad / 64);
    const int task = blockIdx.x * kWavesPerGroup + wv;
    if (task >= cd.Hc * nrb) return false;
    w.slot = task / nrb;
    w.rb = task - w.slot * nrb;
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
// take s o k and s o q and there is no row scale.  PC: one decay per key
// channel (alpha [B][H][d_k]; every token of the window has one).
template <int DK, int PREC, bool DELTA, bool BF16IN, bool KEY, bool PC>
__global__ void __launch_bounds__(64 * kWavesPerGroup)
lores_window_read_kernel(const void *__restrict__ qp, const void *__restrict__ kp,
                         const void *__restrict__ vp, const float *__restrict__ alphap,
                         const float *__restrict__ betap, float *__restrict__ op,
                         const uint8_t *__restrict__ codes, const float *__restrict__ scales,
                         float *__restrict__ win, const StepMeta meta) {
    constexpr int NCH = stored_chunks<DK, PREC>(), NV = DK / 16;
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
    const float beta = betap[w.bh], alpha = PC ? 1.0f : alphap[w.bh];
    float kv[NV], qv[NV], sc[NV], av[NV];
    const long kb = w.bh * DK + (lane & 15);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        kv[i] = in_scalar<BF16IN>(kp, kb + 16 * i);
        qv[i] = in_scalar<BF16IN>(qp, kb + 16 * i);
        sc[i] = KEY ? scales[w.unit * DK + 16 * i + (lane & 15)] : 1.0f;
        av[i] = PC ? alphap[kb + 16 * i] : 1.0f;
    }
    const int p = meta.wpos, nslot = meta.window - 1;
    float *ub = win + w.unit * window_unit_floats(meta.window, meta.dv_pad, DK);
    float *gslot = ub, *kslot = ub + (long)nslot * dv_pad, *aslot = kslot + (long)nslot * DK;

    // the buffered tokens, latest first.  Scalar decay: d = the product of
    // the later decays, then (after the loop) c_{p-1}.  Per channel: E = the
    // later decays times alpha_p, column by column, then C alpha_p.
    float rs = 0.0f, os = 0.0f, d = 1.0f, E[PC ? NV : 1];
    if constexpr (PC) {
#pragma unroll
        for (int i = 0; i < NV; ++i) E[i] = av[i];
    }
    for (int tau = p - 1; tau >= 1; --tau) {
        const float gt = gslot[(long)(tau - 1) * dv_pad + w.lrow];
        float kt[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) kt[i] = kslot[(long)(tau - 1) * DK + 16 * i + (lane & 15)];
        if constexpr (PC) {
            float ek[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) ek[i] = E[i] * kt[i];
            if constexpr (DELTA) rs = __builtin_fmaf(gt, rowdot<NV>(ek, kv), rs);
            os = __builtin_fmaf(gt, rowdot<NV>(ek, qv), os);
#pragma unroll
            for (int i = 0; i < NV; ++i) E[i] = E[i] * aslot[(long)(tau - 1) * DK + 16 * i + (lane & 15)];
        } else {
            const float dg = d * gt;
            if constexpr (DELTA) rs = __builtin_fmaf(dg, rowdot<NV>(kt, kv), rs);
            os = __builtin_fmaf(dg, rowdot<NV>(kt, qv), os);
            d = d * aslot[(long)(tau - 1) * DK];
        }
    }

    // sum_j c_ij w_j over the stored row (codes unscaled) with the weights
    // w = s o k and s o q (scalar decay; s = 1 for value rows) or s o C alpha_p
    // o k and ... o q (per channel): int rows take the stored offset-binary
    // integers and subtract off * sum_j w_j once (a different rounding of the
    // same sum).  An odd column holds off - c, so its weight enters negated
    // (the odd lanes of a row vector hold the odd columns).
    const float wsign = (PREC != LORES_FP8 && (lane & 1)) ? -1.0f : 1.0f;
    float wk[NV], wq[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        float f = sc[i] * wsign;
        if constexpr (PC) f = f * E[i];
        wk[i] = f * kv[i];
        wq[i] = f * qv[i];
    }
    float A = 0.0f, Bq = 0.0f;
#pragma unroll
    for (int gi = 0; gi < NV; ++gi) {
        float x[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = stored_at<DK, PREC>(cw, 16 * gi + e);
        if constexpr (DELTA) dot16(A, x, wk[gi]);
        dot16(Bq, x, wq[gi]);
    }
    if constexpr (PREC != LORES_FP8) {
        float ones[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) ones[i] = 1.0f;
        if constexpr (DELTA) A = __builtin_fmaf(-Prec<PREC>::OFF, rowdot<NV>(wk, ones), A);
        Bq = __builtin_fmaf(-Prec<PREC>::OFF, rowdot<NV>(wq, ones), Bq);
    }

    // scalar decay: d is now c_{p-1}, the product of the window's earlier decays
    const float cs = PC ? s : d * s;
    const float da = PC ? 1.0f : alpha;
    float g;
    if constexpr (DELTA) {
        const float r = da * __builtin_fmaf(cs, A, rs);
        g = beta * (v - r);
    } else {
        g = beta * v;
    }
    const float o = __builtin_fmaf(g, rowdot<NV>(kv, qv), da * __builtin_fmaf(cs, Bq, os));
    if (w.active) {
        op[w.bh * meta.dv + w.row] = o;
        gslot[(long)(p - 1) * dv_pad + w.row] = g;
    }
    if (w.rb == 0) {
        if (lane < 16) {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                kslot[(long)(p - 1) * DK + 16 * i + lane] = kv[i];
                if constexpr (PC) aslot[(long)(p - 1) * DK + 16 * i + lane] = av[i];
            }
        }
        if constexpr (!PC) {
            if (lane == 0) aslot[(long)(p - 1) * DK] = alpha;
        }
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
    constexpr int NCH = stored_chunks<DK, PREC>();
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
    // columns are independent in the replay: blocks of at most 128 of them,
    // which tile the row exactly (two halves above d_k = 128)
    constexpr int CB = DK > 128 ? DK / 2 : DK, NVB = CB / 16;
    static_assert(DK % CB == 0 && CB <= 128, "column blocks tile the row");
    const bool pc = meta.win_pc != 0;
    const float s = KEY ? 0.0f : scales[w.unit * dv_pad + w.lrow];
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    float *orow = out + (w.bh * meta.dv + w.row) * DK;
#pragma unroll
    for (int j0 = 0; j0 < DK; j0 += CB) {
        float U[CB];
        // token 1: fl(c fl(s alpha_1,j)), with the row's or column j's scale s
        // and the token's decay of column j (a scalar decay: every column alike)
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            const float a1 = (KEY ? scales[w.unit * DK + j0 + j] : s) * aslot[pc ? j0 + j : 0];
            float na1 = 0.0f;
            if constexpr (PREC != LORES_FP8) na1 = a1 * -Prec<PREC>::OFF;
            U[j] = scaled_code<DK, PREC>(cw, j0 + j, a1, na1);
        }
        for (int tau = 1; tau <= n; ++tau) {
            const float gt = gslot[(long)(tau - 1) * dv_pad + w.lrow];
            float kt[NVB];
#pragma unroll
            for (int i = 0; i < NVB; ++i)
                kt[i] = kslot[(long)(tau - 1) * DK + j0 + 16 * i + (lane & 15)];
#pragma unroll
            for (int gi = 0; gi < NVB; ++gi) axpy16(&U[16 * gi], gt, kt[gi]);
            if (tau < n) {
                const float *an = aslot + (long)tau * DK;
#pragma unroll
                for (int j = 0; j < CB; ++j) U[j] = U[j] * an[pc ? j0 + j : 0];
            }
        }
        if (w.active) {
#pragma unroll
            for (int j = 0; j < CB; j += 4)
                *reinterpret_cast<f32x4 *>(orow + j0 + j) = f32x4{U[j], U[j + 1], U[j + 2], U[j + 3]};
        }
    }
}

// Inside a window: one task per wavefront (a read-only pass, many waves per
// SIMD).  The window's last step: the step kernel's task stream
// with the buffer replayed between pass 1 and the token's own update.
template <int DK, int PREC, bool KEY, bool PC>
static hipError_t window_dk(bool delta, bool bf16, const StepPtrs &p, const StepMeta &m,
                            hipStream_t s) {
    if (m.wpos == m.window) {
        if (delta) return bf16 ? launch_one<DK, PC, true, true, PREC, -1, KEY, true>(p, m, s)
                               : launch_one<DK, PC, true, false, PREC, -1, KEY, true>(p, m, s);
        return bf16 ? launch_one<DK, PC, false, true, PREC, -1, KEY, true>(p, m, s)
                    : launch_one<DK, PC, false, false, PREC, -1, KEY, true>(p, m, s);
    }
    const dim3 grid((m.cls[0].Hc * (m.dv_pad / 64) + kWavesPerGroup - 1) / kWavesPerGroup, m.B);
    const dim3 block(64 * kWavesPerGroup);
#define LORES_WIN_LAUNCH(D, BF)                                                                 \
    hipLaunchKernelGGL((lores_window_read_kernel<DK, PREC, D, BF, KEY, PC>), grid, block, 0, s,    \
                       p.q, p.k, p.v, p.alpha, p.beta, p.o, p.codes[0], p.scales[0], p.win[0], m);
    if (delta) {
        if (bf16) { LORES_WIN_LAUNCH(true, true) } else { LORES_WIN_LAUNCH(true, false) }
    } else {
        if (bf16) { LORES_WIN_LAUNCH(false, true) } else { LORES_WIN_LAUNCH(false, false) }
    }
#undef LORES_WIN_LAUNCH
    return hipGetLastError();
}

template <int PREC>
static hipError_t window_prec(int dk, bool delta, bool bf16, bool key, bool pc,
                              const StepPtrs &p, const StepMeta &m, hipStream_t s) {
#define LORES_WIN_KEY_PC(DK)                                                                    \
    (key ? (pc ? window_dk<DK, PREC, true, true>(delta, bf16, p, m, s)                          \
               : window_dk<DK, PREC, true, false>(delta, bf16, p, m, s))                        \
         : (pc ? window_dk<DK, PREC, false, true>(delta, bf16, p, m, s)                         \
               : window_dk<DK, PREC, false, false>(delta, bf16, p, m, s)))
    switch (dk) {
        case 32: return LORES_WIN_KEY_PC(32);
        case 64: return LORES_WIN_KEY_PC(64);
        case 96: return LORES_WIN_KEY_PC(96);
        case 128: return LORES_WIN_KEY_PC(128);
        case 160: return LORES_WIN_KEY_PC(160);
        case 192: return LORES_WIN_KEY_PC(192);
        case 224: return LORES_WIN_KEY_PC(224);
        case 256: return LORES_WIN_KEY_PC(256);
        default: return hipErrorInvalidValue;
    }
#undef LORES_WIN_KEY_PC
}

// The current state of one windowed class (lores_dequant_state): the stored
// state followed by the buffered tokens.
template <int PREC>
static hipError_t window_dequant_prec(int dk, bool key, const uint8_t *codes, const float *scales,
                                      const float *win, float *out, const StepMeta &m,
                                      hipStream_t s) {
    const dim3 grid((m.cls[0].Hc * (m.dv_pad / 64) + kWavesPerGroup - 1) / kWavesPerGroup, m.B);
    const dim3 block(64 * kWavesPerGroup);
#define LORES_WD(DK, KEY)                                                                       \
    hipLaunchKernelGGL((lores_window_dequant_kernel<DK, PREC, KEY>), grid, block, 0, s, codes,   \
                       scales, win, out, m)
    switch (dk) {
        case 32: if (key) LORES_WD(32, true); else LORES_WD(32, false); break;
        case 64: if (key) LORES_WD(64, true); else LORES_WD(64, false); break;
        case 96: if (key) LORES_WD(96, true); else LORES_WD(96, false); break;
        case 128: if (key) LORES_WD(128, true); else LORES_WD(128, false); break;
        case 160: if (key) LORES_WD(160, true); else LORES_WD(160, false); break;
        case 192: if (key) LORES_WD(192, true); else LORES_WD(192, false); break;
        case 224: if (key) LORES_WD(224, true); else LORES_WD(224, false); break;
        case 256: if (key) LORES_WD(256, true); else LORES_WD(256, false); break;
        default: return hipErrorInvalidValue;
    }
#undef LORES_WD
    return hipGetLastError();
}

}  // namespace lores
