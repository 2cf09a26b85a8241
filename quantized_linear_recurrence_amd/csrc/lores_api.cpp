// Host side of the LoReS C ABI: layout planning, argument validation,
// decay-based precision assignment and kernel dispatch.  Every exported
// function validates first and launches nothing on error; no exception
// leaves this file.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <numeric>
#include <string>
#include <vector>

#include "lores_internal.h"

struct lores_state {
    int32_t B, H, dk, dv, dv_pad, n_rb;
    uint8_t prec[LORES_MAX_HEADS];
    int32_t slot[LORES_MAX_HEADS];
    int32_t n_class[LORES_NUM_PREC];
    uint16_t heads[LORES_NUM_PREC][LORES_MAX_HEADS];
    int64_t codes_off[LORES_NUM_PREC], scales_off[LORES_NUM_PREC], unit_bytes[LORES_NUM_PREC];
    uint64_t total;
    uint8_t *base;
    int32_t rounding;        // LORES_ROUND_*
    int32_t axis;            // LORES_SCALE_*
    int32_t window;          // W: steps per requantization of the scaled classes
    int32_t n_buf;           // tokens of the current window held in the buffer
    int32_t win_pc;          // those tokens carry one decay per key channel
    int64_t win_off[LORES_NUM_PREC], unit_win[LORES_NUM_PREC];   // bytes
};

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return LORES_OK;
}

bool is_int_prec(int p) { return p == LORES_INT8 || p == LORES_INT4 || p == LORES_INT6; }

// classes stored with one fp32 scale per value row
bool has_scales(int p) { return is_int_prec(p) || p == LORES_FP8; }

// Bytes per stored row: d_k elements of 32, 16, 8, 4 or 6 bits in whole
// 16-byte chunks (only int6 rows can end in a partly used chunk).
// 16-byte chunks of a stored row; a row of d_k > 128 is two halves of d_k / 2
// columns, each padded to whole chunks (the step splits it across two lanes)
int64_t row_bytes(int prec, int dk) {
    static const int bits[LORES_NUM_PREC] = {32, 16, 8, 4, 6, 8};
    if (dk > 128) return 2 * row_bytes(prec, dk / 2);
    return (int64_t)((dk * bits[prec] + 127) / 128) * 16;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~(uint64_t)255; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_dims(int32_t B, int32_t H, int32_t dk, int32_t dv) {
    if (B < 1 || B > 65535) return fail(LORES_EINVAL, "B must be in [1, 65535] (got %d)", B);
    if (H < 1 || H > LORES_MAX_HEADS)
        return fail(LORES_EINVAL, "H must be in [1, %d] (got %d)", LORES_MAX_HEADS, H);
    if (dk < 32 || dk % 32 != 0)
        return fail(LORES_EINVAL, "d_k must be a positive multiple of 32 (got %d)", dk);
    if (dk > 256) return fail(LORES_EINVAL, "d_k must be at most 256 (got %d)", dk);
    if (dv < 1 || dv > LORES_MAX_DV)
        return fail(LORES_EINVAL, "d_v must be in [1, %d] (got %d)", LORES_MAX_DV, dv);
    return LORES_OK;
}

// fp32 scales per (sequence, head) unit of a scaled class
int64_t unit_scales(const lores_state *st) {
    return st->axis == LORES_SCALE_KEY ? st->dk : st->dv_pad;
}

// Fill st's layout from its dimensions, head_prec and axis; returns status.
int plan(lores_state *st, const uint8_t *head_prec) {
    std::memset(st->n_class, 0, sizeof st->n_class);
    for (int h = 0; h < st->H; ++h) {
        const int p = head_prec[h];
        if (p < 0 || p >= LORES_NUM_PREC)
            return fail(LORES_EINVAL, "head_prec[%d] = %d is not a precision code", h, p);
        st->prec[h] = (uint8_t)p;
        st->slot[h] = st->n_class[p];
        st->heads[p][st->n_class[p]++] = (uint16_t)h;
    }
    st->dv_pad = (st->dv + LORES_ROW_BLOCK - 1) / LORES_ROW_BLOCK * LORES_ROW_BLOCK;
    // tasks of 64 rows, or of 32 rows split across lane pairs at d_k > 128
    st->n_rb = st->dk > 128 ? (st->dv + 31) / 32 : st->dv_pad / LORES_ROW_BLOCK;
    uint64_t off = 0;
    for (int c = 0; c < LORES_NUM_PREC; ++c) {
        st->codes_off[c] = st->scales_off[c] = st->win_off[c] = -1;
        st->unit_win[c] = 0;
        st->unit_bytes[c] = row_bytes(c, st->dk) * st->dv_pad;
        if (!st->n_class[c]) continue;
        const double units = (double)st->B * st->n_class[c];
        if (units * st->unit_bytes[c] > 9.0e18) return fail(LORES_EINVAL, "state too large");
        off = align256(off);
        st->codes_off[c] = (int64_t)off;
        off += (uint64_t)st->B * st->n_class[c] * st->unit_bytes[c];
        if (has_scales(c)) {
            off = align256(off);
            st->scales_off[c] = (int64_t)off;
            off += (uint64_t)st->B * st->n_class[c] * unit_scales(st) * sizeof(float);
        }
        st->win_off[c] = -1;
        st->unit_win[c] = 0;
        if (has_scales(c) && st->window > 1) {
            st->unit_win[c] = lores::window_unit_floats(st->window, st->dv_pad, st->dk) * 4;
            off = align256(off);
            st->win_off[c] = (int64_t)off;
            off += (uint64_t)st->B * st->n_class[c] * st->unit_win[c];
        }
        // launch grid: y = sequence (at most 65535), x = groups of row-block tasks
    }
    st->total = align256(off);
    return LORES_OK;
}

// Launch description for the classes in `cls` (one, or a fused pair).
lores::StepMeta make_meta(const lores_state *st, const int *cls, int n_cls) {
    lores::StepMeta m;
    std::memset(&m, 0, sizeof m);
    m.B = st->B;
    m.H = st->H;
    m.dv = st->dv;
    m.dv_pad = st->dv_pad;
    m.n_rb = st->n_rb;
    m.n_cls = n_cls;
    m.rounding = st->rounding;
    int off = 0;
    for (int i = 0; i < n_cls; ++i) {
        const int c = cls[i];
        lores::ClassDesc &d = m.cls[i];
        d.prec = c;
        d.Hc = st->n_class[c];
        const int gw = st->axis == LORES_SCALE_KEY && has_scales(c)
                           ? lores::key_group_waves(st->n_rb) : lores::kWavesPerGroup;
        d.groups = (d.Hc * st->n_rb + gw - 1) / gw;
        d.head_off = off;
        d.unit_bytes = st->unit_bytes[c];
        for (int k = 0; k < d.Hc; ++k) m.heads[off + k] = st->heads[c][k];
        off += d.Hc;
    }
    // a launch of the two int classes pairs task p of one with task p of the
    // other in one wavefront; `groups` then counts only the unpaired rest, in
    // the kPairWavesPerGroup-wavefront groups of such launches
    if (n_cls == 2 && is_int_prec(cls[0]) && is_int_prec(cls[1])) {
        const int n0 = m.cls[0].Hc * st->n_rb, n1 = m.cls[1].Hc * st->n_rb;
        const int paired = n0 < n1 ? n0 : n1;
        for (int i = 0; i < 2; ++i) {
            const int rest = (i ? n1 : n0) - paired;
            m.cls[i].groups = (rest + lores::kPairWavesPerGroup - 1) / lores::kPairWavesPerGroup;
        }
    }
    return m;
}

}  // namespace

namespace lores {

bool fusable_pair(int p0, int p1) {
    return (p0 == LORES_INT8 && p1 == LORES_INT4) || (p0 == LORES_INT4 && p1 == LORES_INT6) ||
           (p0 == LORES_BF16 && p1 == LORES_INT8) || (p0 == LORES_BF16 && p1 == LORES_INT4);
}

hipError_t launch_step(int dk, bool pc, bool delta, bool bf16, int p0, int p1, const StepPtrs &p,
                       const StepMeta &m, hipStream_t s, bool key) {
    if (key) {
        if (p1 >= 0) return hipErrorInvalidValue;
        switch (p0) {
            case LORES_INT8: return launch_step_key_int8(dk, pc, delta, bf16, p, m, s);
            case LORES_INT4: return launch_step_key_int4(dk, pc, delta, bf16, p, m, s);
            case LORES_INT6: return launch_step_key_int6(dk, pc, delta, bf16, p, m, s);
            case LORES_FP8: return launch_step_key_fp8(dk, pc, delta, bf16, p, m, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (p1 < 0) {
        switch (p0) {
            case LORES_FP32: return launch_step_fp32(dk, pc, delta, bf16, p, m, s);
            case LORES_BF16: return launch_step_bf16(dk, pc, delta, bf16, p, m, s);
            case LORES_INT8: return launch_step_int8(dk, pc, delta, bf16, p, m, s);
            case LORES_INT4: return launch_step_int4(dk, pc, delta, bf16, p, m, s);
            case LORES_INT6: return launch_step_int6(dk, pc, delta, bf16, p, m, s);
            case LORES_FP8: return launch_step_fp8(dk, pc, delta, bf16, p, m, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (p0 == LORES_INT8 && p1 == LORES_INT4) return launch_step_int8_int4(dk, pc, delta, bf16, p, m, s);
    if (p0 == LORES_INT4 && p1 == LORES_INT6) return launch_step_int4_int6(dk, pc, delta, bf16, p, m, s);
    if (p0 == LORES_BF16 && p1 == LORES_INT8) return launch_step_bf16_int8(dk, pc, delta, bf16, p, m, s);
    if (p0 == LORES_BF16 && p1 == LORES_INT4) return launch_step_bf16_int4(dk, pc, delta, bf16, p, m, s);
    return hipErrorInvalidValue;
}

}  // namespace lores

// Every launcher enqueues its kernels and returns the thread's last HIP
// error.  That error is sticky: one left by earlier work on this thread (the
// caller's, or a failed query) would be reported as the launch's own.  So it
// is consumed right before each launcher call, and a returned error is then
// the launch's.
static void consume_stale_hip_error() { (void)hipGetLastError(); }

extern "C" {

const char *lores_last_error(void) { return g_err.c_str(); }

int lores_spec_version(void) { return LORES_SPEC_VERSION; }

static int alloc_impl(int32_t B, int32_t H, int32_t d_k, int32_t d_v, const uint8_t *head_prec,
                      int32_t scale_axis, int32_t window, void *d_buf, size_t *bytes,
                      void *stream, lores_state **out) {
    try {
        int rc = check_dims(B, H, d_k, d_v);
        if (rc) return rc;
        if (!head_prec) return fail(LORES_EINVAL, "head_prec is NULL");
        if (!bytes) return fail(LORES_EINVAL, "bytes is NULL");
        if (scale_axis != LORES_SCALE_VALUE && scale_axis != LORES_SCALE_KEY)
            return fail(LORES_EINVAL, "scale_axis must be LORES_SCALE_VALUE (0) or "
                                      "LORES_SCALE_KEY (1), got %d", scale_axis);
        lores_state tmp;
        tmp.B = B;
        tmp.H = H;
        tmp.dk = d_k;
        tmp.dv = d_v;
        tmp.base = nullptr;
        tmp.rounding = LORES_ROUND_STOCHASTIC;
        tmp.axis = scale_axis;
        tmp.window = window;
        tmp.n_buf = 0;
        tmp.win_pc = 0;
        rc = plan(&tmp, head_prec);
        if (rc) return rc;
        if (!d_buf) {
            *bytes = (size_t)tmp.total;
            return ok();
        }
        if (!out) return fail(LORES_EINVAL, "out is NULL");
        if (!aligned(d_buf, 256)) return fail(LORES_EINVAL, "d_buf must be 256-byte aligned");
        if (*bytes < tmp.total)
            return fail(LORES_ESIZE, "buffer holds %zu bytes, the layout needs %llu", *bytes,
                        (unsigned long long)tmp.total);
        lores_state *st = new (std::nothrow) lores_state(tmp);
        if (!st) return fail(LORES_ENOMEM, "host allocation of the state handle failed");
        st->base = (uint8_t *)d_buf;
        consume_stale_hip_error();
        hipError_t e = lores::launch_fill_zero(d_buf, tmp.total, (hipStream_t)stream);
        if (e != hipSuccess) {
            delete st;
            return fail(LORES_EHIP, "zero fill launch failed: %s", hipGetErrorString(e));
        }
        *out = st;
        return ok();
    } catch (...) {
        return fail(LORES_EINVAL, "internal error in lores_state_alloc");
    }
}

int lores_state_alloc_axis(int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                           const uint8_t *head_prec, int32_t scale_axis, void *d_buf,
                           size_t *bytes, void *stream, lores_state **out) {
    return alloc_impl(B, H, d_k, d_v, head_prec, scale_axis, 1, d_buf, bytes, stream, out);
}

int lores_state_alloc(int32_t B, int32_t H, int32_t d_k, int32_t d_v, const uint8_t *head_prec,
                      void *d_buf, size_t *bytes, void *stream, lores_state **out) {
    return alloc_impl(B, H, d_k, d_v, head_prec, LORES_SCALE_VALUE, 1, d_buf, bytes, stream, out);
}

int lores_state_alloc_window(int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                             const uint8_t *head_prec, int32_t scale_axis, int32_t window,
                             void *d_buf, size_t *bytes, void *stream, lores_state **out) {
    if (window < 1 || window > LORES_MAX_WINDOW)
        return fail(LORES_EINVAL, "window must be in [1, %d] (got %d)", LORES_MAX_WINDOW, window);
    return alloc_impl(B, H, d_k, d_v, head_prec, scale_axis, window, d_buf, bytes, stream, out);
}

void lores_state_free(lores_state *st) { delete st; }

int lores_state_layout(const lores_state *st, lores_layout *out) {
    if (!st || !out) return fail(LORES_EINVAL, "NULL argument");
    out->B = st->B;
    out->H = st->H;
    out->d_k = st->dk;
    out->d_v = st->dv;
    out->d_v_pad = st->dv_pad;
    for (int c = 0; c < LORES_NUM_PREC; ++c) {
        out->n_class[c] = st->n_class[c];
        out->codes_offset[c] = st->codes_off[c];
        out->scales_offset[c] = st->scales_off[c];
        out->unit_code_bytes[c] = st->unit_bytes[c];
    }
    out->total_bytes = st->total;
    out->scale_axis = st->axis;
    out->unit_scales = (int32_t)unit_scales(st);
    out->window = st->window;
    out->window_fill = st->n_buf;
    for (int c = 0; c < LORES_NUM_PREC; ++c) {
        out->window_offset[c] = st->win_off[c];
        out->unit_window_bytes[c] = st->unit_win[c];
    }
    return ok();
}

int lores_state_set_rounding(lores_state *st, int32_t mode) {
    if (!st) return fail(LORES_EINVAL, "state handle is NULL");
    if (mode != LORES_ROUND_STOCHASTIC && mode != LORES_ROUND_NEAREST)
        return fail(LORES_EINVAL, "rounding mode must be LORES_ROUND_STOCHASTIC (0) or "
                                  "LORES_ROUND_NEAREST (1), got %d", mode);
    st->rounding = mode;
    return ok();
}

int lores_state_head_map(const lores_state *st, uint8_t *prec_out, int32_t *slot_out) {
    if (!st || !prec_out || !slot_out) return fail(LORES_EINVAL, "NULL argument");
    for (int h = 0; h < st->H; ++h) {
        prec_out[h] = st->prec[h];
        slot_out[h] = st->slot[h];
    }
    return ok();
}

int lores_decay_stat(const float *alpha, int64_t n, int32_t H, int32_t width, double *stat) {
    try {
        if (!alpha || !stat) return fail(LORES_EINVAL, "NULL argument");
        if (n < 1 || H < 1 || width < 1) return fail(LORES_EINVAL, "n, H and width must be >= 1");
        std::vector<double> acc(H, 0.0);
        for (int64_t i = 0; i < n; ++i) {
            const float *row = alpha + i * (int64_t)H * width;
            for (int h = 0; h < H; ++h) {
                double s = 0.0;
                for (int w = 0; w < width; ++w) {
                    const float a = row[(int64_t)h * width + w];
                    if (!(a > 0.0f)) return fail(LORES_EINVAL, "alpha must be > 0 (row %lld, head %d)", (long long)i, h);
                    s += std::log((double)a);
                }
                acc[h] += s;
            }
        }
        const double cnt = (double)n * width;
        for (int h = 0; h < H; ++h) stat[h] = acc[h] / cnt;
        return ok();
    } catch (...) {
        return fail(LORES_EINVAL, "internal error in lores_decay_stat");
    }
}

int lores_assign_precision(const double *stat, int32_t H, const double *tier_frac,
                           const uint8_t *tier_prec, int32_t n_tiers, uint8_t *head_prec) {
    try {
        if (!stat || !tier_frac || !tier_prec || !head_prec) return fail(LORES_EINVAL, "NULL argument");
        if (H < 1 || H > LORES_MAX_HEADS) return fail(LORES_EINVAL, "H must be in [1, %d]", LORES_MAX_HEADS);
        if (n_tiers < 1) return fail(LORES_EINVAL, "n_tiers must be >= 1");
        for (int k = 0; k < n_tiers; ++k) {
            if (tier_prec[k] >= LORES_NUM_PREC)
                return fail(LORES_EINVAL, "tier_prec[%d] is not a precision code", k);
            if (!(tier_frac[k] >= 0.0) || !std::isfinite(tier_frac[k]))
                return fail(LORES_EINVAL, "tier_frac[%d] must be finite and >= 0", k);
        }
        for (int h = 0; h < H; ++h)
            if (std::isnan(stat[h])) return fail(LORES_EINVAL, "stat[%d] is NaN", h);
        std::vector<int> order(H);
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(),
                         [&](int a, int b) { return stat[a] > stat[b]; });   // slowest first
        int pos = 0;
        for (int k = 0; k < n_tiers; ++k) {
            int count;
            if (k == n_tiers - 1) {
                count = H - pos;
            } else {
                const double want = std::floor(tier_frac[k] * H + 0.5);
                count = (int)std::min<double>(want, (double)(H - pos));
            }
            for (int i = 0; i < count; ++i) head_prec[order[pos + i]] = tier_prec[k];
            pos += count;
        }
        return ok();
    } catch (...) {
        return fail(LORES_EINVAL, "internal error in lores_assign_precision");
    }
}

// Launches of one decode step: the classes present, where a fusable pair
// shares one launch and anything else gets one launch per class.
static int plan_launches(const lores_state *st, int groups[LORES_NUM_PREC][2],
                         int width[LORES_NUM_PREC]) {
    int present[LORES_NUM_PREC], n = 0;
    for (int c = 0; c < LORES_NUM_PREC; ++c)
        if (st->n_class[c]) present[n++] = c;
    if (n == 2 && st->axis == LORES_SCALE_VALUE && st->window == 1 &&
        lores::fusable_pair(present[0], present[1])) {
        groups[0][0] = present[0];
        groups[0][1] = present[1];
        width[0] = 2;
        return 1;
    }
    for (int i = 0; i < n; ++i) {
        groups[i][0] = present[i];
        width[i] = 1;
    }
    return n;
}

int lores_step_launches(const lores_state *st, int32_t *n) {
    if (!st || !n) return fail(LORES_EINVAL, "NULL argument");
    int groups[LORES_NUM_PREC][2], width[LORES_NUM_PREC];
    *n = plan_launches(st, groups, width);
    return ok();
}

int lores_decode_step(lores_state *st, const void *q, const void *k, const void *v,
                      int32_t in_bf16, const float *alpha, int32_t alpha_per_channel,
                      const float *beta, int32_t delta, uint64_t seed, uint64_t t,
                      int64_t seq_base, int64_t head_base, float *o, void *stream) {
    try {
        if (!st) return fail(LORES_EINVAL, "state handle is NULL");
        if (!q || !k || !v || !alpha || !beta || !o)
            return fail(LORES_EINVAL, "q, k, v, alpha, beta and o must be non-NULL device pointers");
        // q, k, alpha, beta are read as dwords (bf16 q and k as pairs), v one
        // element per lane, o one fp32 per lane
        if (!aligned(q, 4) || !aligned(k, 4) || !aligned(alpha, 4) || !aligned(beta, 4) ||
            !aligned(o, 4) || !aligned(v, in_bf16 ? 2 : 4))
            return fail(LORES_EINVAL, "q, k, alpha, beta and o must be 4-byte aligned, v aligned "
                                      "to its element size");
        if (in_bf16 != 0 && in_bf16 != 1) return fail(LORES_EINVAL, "in_bf16 must be 0 or 1");
        if (alpha_per_channel != 0 && alpha_per_channel != 1)
            return fail(LORES_EINVAL, "alpha_per_channel must be 0 or 1");
        if (delta != 0 && delta != 1) return fail(LORES_EINVAL, "delta must be 0 or 1 (got %d)", delta);
        if (t < 1) return fail(LORES_EINVAL, "t must be >= 1 (t = 0 is the initial state)");
        if (seq_base < 0 || (uint64_t)seq_base + (uint64_t)st->B > (1ull << 32))
            return fail(LORES_EINVAL, "seq_base + B must lie in [0, 2^32]");
        if (head_base < 0 || (uint64_t)head_base + (uint64_t)st->H > (1ull << 32))
            return fail(LORES_EINVAL, "head_base + H must lie in [0, 2^32]");
        const hipStream_t s = (hipStream_t)stream;
        // windowed states: the step's position in its window must follow the
        // tokens the buffer holds
        const bool windowed = st->window > 1;
        int wpos = 1;
        if (windowed) {
            wpos = (int)((t - 1) % (uint64_t)st->window) + 1;
            if (wpos != st->n_buf + 1)
                return fail(LORES_EINVAL, "windowed state: the buffer holds %d tokens of the current "
                                          "window, so the next step is at window position %d, but "
                                          "t = %llu is at position %d (steps must come in order)",
                            st->n_buf, st->n_buf + 1, (unsigned long long)t, wpos);
            // the buffered tokens and this one share one kind of decay
            if (wpos > 1 && alpha_per_channel != st->win_pc)
                return fail(LORES_EINVAL, "windowed state: the window's buffered tokens carry %s "
                                          "decay, this step %s (alpha_per_channel may change only "
                                          "at a window's first step)",
                            st->win_pc ? "a per-channel" : "a scalar",
                            alpha_per_channel ? "a per-channel one" : "a scalar one");
        }
        int groups[LORES_NUM_PREC][2], width[LORES_NUM_PREC];
        const int n_launch = plan_launches(st, groups, width);
        for (int l = 0; l < n_launch; ++l) {
            lores::StepMeta m = make_meta(st, groups[l], width[l]);
            m.seed = seed;
            m.t = t;
            m.seq_base = seq_base;
            m.head_base = head_base;
            m.wpos = wpos;
            m.window = st->window;
            lores::StepPtrs p;
            std::memset(&p, 0, sizeof p);
            p.q = q;
            p.k = k;
            p.v = v;
            p.alpha = alpha;
            p.beta = beta;
            p.o = o;
            for (int i = 0; i < width[l]; ++i) {
                const int c = groups[l][i];
                p.codes[i] = st->base + st->codes_off[c];
                p.scales[i] = has_scales(c) ? (float *)(st->base + st->scales_off[c]) : nullptr;
            }
            const int p1 = width[l] == 2 ? groups[l][1] : -1;
            const bool key = st->axis == LORES_SCALE_KEY && has_scales(groups[l][0]);
            hipError_t e;
            consume_stale_hip_error();
            if (windowed && has_scales(groups[l][0])) {
                p.win[0] = (float *)(st->base + st->win_off[groups[l][0]]);
                m.win_pc = alpha_per_channel;
                e = lores::launch_window_step(groups[l][0], st->dk, delta, in_bf16, key,
                                              alpha_per_channel != 0, p, m, s);
            } else {
                e = lores::launch_step(st->dk, alpha_per_channel, delta, in_bf16, groups[l][0], p1, p,
                                       m, s, key);
            }
            if (e != hipSuccess)
                return fail(LORES_EHIP, "decode-step launch failed: %s", hipGetErrorString(e));
        }
        if (windowed) {
            st->n_buf = wpos == st->window ? 0 : wpos;
            st->win_pc = alpha_per_channel;
        }
        return ok();
    } catch (...) {
        return fail(LORES_EINVAL, "internal error in lores_decode_step");
    }
}

int lores_quant_state(lores_state *st, const float *X, uint64_t seed, int64_t seq_base,
                      int64_t head_base, void *stream) {
    try {
        if (!st || !X) return fail(LORES_EINVAL, "NULL argument");
        if (!aligned(X, 16)) return fail(LORES_EINVAL, "X must be 16-byte aligned");
        if (seq_base < 0 || (uint64_t)seq_base + (uint64_t)st->B > (1ull << 32))
            return fail(LORES_EINVAL, "seq_base + B must lie in [0, 2^32]");
        if (head_base < 0 || (uint64_t)head_base + (uint64_t)st->H > (1ull << 32))
            return fail(LORES_EINVAL, "head_base + H must lie in [0, 2^32]");
        for (int c = 0; c < LORES_NUM_PREC; ++c) {
            if (!st->n_class[c]) continue;
            lores::StepMeta m = make_meta(st, &c, 1);
            m.seed = seed;
            m.t = 0;
            m.seq_base = seq_base;
            m.head_base = head_base;
            float *sc = has_scales(c) ? (float *)(st->base + st->scales_off[c]) : nullptr;
            consume_stale_hip_error();
            hipError_t e = lores::launch_quant(c, st->dk, X, st->base + st->codes_off[c], sc, m,
                                               (hipStream_t)stream,
                                               st->axis == LORES_SCALE_KEY && has_scales(c));
            if (e != hipSuccess)
                return fail(LORES_EHIP, "quantize launch failed: %s", hipGetErrorString(e));
        }
        st->n_buf = 0;
        return ok();
    } catch (...) {
        return fail(LORES_EINVAL, "internal error in lores_quant_state");
    }
}

int lores_dequant_state(const lores_state *st, float *out, void *stream) {
    try {
        if (!st || !out) return fail(LORES_EINVAL, "NULL argument");
        if (!aligned(out, 16)) return fail(LORES_EINVAL, "out must be 16-byte aligned");
        for (int c = 0; c < LORES_NUM_PREC; ++c) {
            if (!st->n_class[c]) continue;
            lores::StepMeta m = make_meta(st, &c, 1);
            const float *sc = has_scales(c) ? (const float *)(st->base + st->scales_off[c]) : nullptr;
            hipError_t e;
            consume_stale_hip_error();
            if (st->window > 1 && st->n_buf > 0 && has_scales(c)) {
                m.wpos = st->n_buf;
                m.win_pc = st->win_pc;
                m.window = st->window;
                e = lores::launch_window_dequant(c, st->dk, st->axis == LORES_SCALE_KEY,
                                                 st->base + st->codes_off[c], sc,
                                                 (const float *)(st->base + st->win_off[c]), out, m,
                                                 (hipStream_t)stream);
            } else {
                e = lores::launch_dequant(c, st->dk, st->base + st->codes_off[c], sc, out, m,
                                          (hipStream_t)stream,
                                          st->axis == LORES_SCALE_KEY && has_scales(c));
            }
            if (e != hipSuccess) return fail(LORES_EHIP, "dequant launch failed: %s", hipGetErrorString(e));
        }
        return ok();
    } catch (...) {
        return fail(LORES_EINVAL, "internal error in lores_dequant_state");
    }
}

}  // extern "C"
