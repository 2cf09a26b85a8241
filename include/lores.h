/*
 * lores.h - C ABI of the LoReS quantized recurrent-state decode step for
 * AMD Instinct MI355X (gfx950).
 *
 * The method: "Quantizing Recurrent Language Models Is Easier Than You Think"
 * (structured summary page).  Each (sequence, head) unit keeps a recurrent
 * state S in R^{d_v x d_k} that every decode step updates in place:
 *
 *   S_t = S_{t-1} diag(alpha_t) (I - delta beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *   o_t = S_t q_t
 *
 * (section "Introduction and Theoretical Foundation", general recurrence form)
 * while the state is stored quantized, dequantized, updated and requantized
 * every step (section "Intra-State Quantization Approach", property 3), with
 * one scale per value row (section "Intra-State Quantization (Section 4)",
 * scale grouping and Proposition 1), stochastic rounding (same section,
 * Rounding and Proposition 3) and a per-head precision chosen from the decay
 * rate (same section, decay-based mixed precision).
 *
 * Conventions for every entry point:
 *   - Return value: LORES_OK (0) or a negative LORES_E* code.  On error,
 *     lores_last_error() (thread-local) describes it.  No C++ exception
 *     crosses this boundary.  Validation happens before any GPU work, so a
 *     call that fails validation launches nothing.
 *   - "device" pointers point to HIP device memory owned by the caller; the
 *     library never allocates or frees device memory.  "host" pointers point
 *     to ordinary host memory, read or written synchronously.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued asynchronously on it; inputs must stay alive
 *     and unmodified until that work has run.
 *   - Calls on one lores_state handle are not re-entrant across streams.
 *   - LORES_EHIP reports that a launch of this call failed.  Before each of
 *     its launches the library consumes any HIP error left on the calling
 *     thread by earlier work, so such an error is never reported as this
 *     call's (and is no longer visible to the caller afterwards).
 */
#ifndef LORES_H
#define LORES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORES_SPEC_VERSION 8

/* Per-head state precision. */
enum {
    LORES_FP32 = 0, /* unquantized fp32 state (the full-precision reference path) */
    LORES_BF16 = 1, /* bfloat16 state, stochastic rounding from fp32               */
    LORES_INT8 = 2, /* int8 codes in [-127, 127] + one fp32 scale per value row     */
    LORES_INT4 = 3, /* int4 codes in [-7, 7]     + one fp32 scale per value row     */
    LORES_INT6 = 4, /* int6 codes in [-31, 31]   + one fp32 scale per value row     */
    LORES_FP8 = 5   /* E4M3 (OCP fp8) values     + one fp32 scale per value row     */
};
#define LORES_NUM_PREC 6

/* Rounding of the requantization (per state; lores_state_set_rounding). */
enum {
    LORES_ROUND_STOCHASTIC = 0, /* default: the counter-based draw n below              */
    LORES_ROUND_NEAREST = 1     /* the same quantizer with the draw fixed at n = 2^15 */
};

/* Scale grouping of the scaled classes (int8, int4, int6, fp8), fixed when
 * the state is allocated (lores_state_alloc_axis).  The pages compare one
 * scale per value row with one per key column ("Intra-State Quantization
 * (Section 4)", Scale Grouping and Proposition 1); value rows are their
 * choice and the default here. */
enum {
    LORES_SCALE_VALUE = 0, /* one fp32 scale per value row: s_i = max_j |S_ij| / r  */
    LORES_SCALE_KEY = 1    /* one fp32 scale per key column: s_j = max_i |S_ij| / r */
};

/* Status codes. */
enum {
    LORES_OK = 0,
    LORES_EINVAL = -1,      /* invalid argument (NULL, misaligned, out of range)  */
    LORES_EUNSUPPORTED = -2,/* valid but not built (kept for the ABI; no current case) */
    LORES_ESIZE = -3,       /* buffer too small                                     */
    LORES_EHIP = -4,        /* a HIP runtime call failed                           */
    LORES_ENOMEM = -5       /* host allocation failed                              */
};

/* Limits. */
#define LORES_MAX_HEADS 512 /* heads per state                                   */
#define LORES_MAX_DV 256    /* value rows per head                               */
#define LORES_ROW_BLOCK 64  /* value rows per stored row block (one wavefront)   */
#define LORES_MAX_WINDOW 16 /* steps per requantization window                   */

/* Opaque host handle: dimensions, per-head precision, layout and the bound
 * device buffer.  Created by lores_state_alloc, released by lores_state_free. */
typedef struct lores_state lores_state;

/*
 * Packed state layout (version LORES_SPEC_VERSION), for inspection, tests and
 * checkpointing.  The buffer holds one segment pair per precision class that
 * has at least one head, in class order fp32, bf16, int8, int4, int6, fp8,
 * each segment starting on a 256-byte boundary:
 *
 *   codes  [B][H_c][n_chunk][d_v_pad][16 bytes]
 *   scales [B][H_c][d_v_pad] fp32                 (int8, int4, int6, fp8 classes)
 *          [B][H_c][d_k] fp32                     (the same, key-column scales)
 *   window [B][H_c][unit_window_bytes]            (scaled classes of a windowed
 *                                                  state, window W > 1)
 *
 * H_c = heads of class c, ordered by head index (head_slot below).
 * d_v_pad = d_v rounded up to LORES_ROW_BLOCK; padding rows are never read
 * or written by a step.  A row is cut into 16-byte chunks of E elements
 * (E = 4 fp32, 8 bf16, 16 int8, 32 int4; n_chunk = d_k / E), stored
 * chunk-major so one wavefront's 64 rows of a chunk are 1 KiB contiguous.
 * Within a chunk, element e is:
 *   fp32: word e, IEEE binary32        bf16: halfword e, bfloat16 bits
 *   int8: byte e  = 128 + s code       (offset binary, 1..255)
 *   fp8:  byte e  = E4M3 byte (OCP: sign, 4 exponent bits with bias 7,
 *         3 mantissa bits; never the NaN pattern), value scale * E4M3 value
 *   int4: byte e/2, low nibble for even e, high nibble for odd e,
 *         nibble = 8 + s code          (offset binary, 1..15)
 * int6 rows are a little-endian bit stream over the row's chunks (chunk c
 * holds row bytes 16c .. 16c + 15): element j is bits 6j .. 6j + 5, value
 * 32 + s code (offset binary, 1..63); n_chunk = ceil(6 d_k / 128), the bits
 * after the last element are zero.
 * s = +1 in the even columns of a row and -1 in the odd ones: an int row
 * holds the codes of its odd columns negated (a column pair shares one
 * rounding draw, and the odd column is requantized as -U; see
 * lores_decode_step).
 * A row of d_k > 128 is stored as two half rows of d_k / 2 columns, each laid
 * out as above from its own first chunk (n_chunk = 2 n_chunk(d_k / 2): an
 * int4 or int6 half that ends inside a chunk is zero-padded to its end).
 * The value of an int element is scale[row] * code (scale[column] * code
 * with key-column scales).  A row of all-zero bytes with scale 0 also reads
 * as zero, so a zero-filled buffer is S = 0.
 * A unit's window block holds W - 1 token slots: g [W-1][d_v_pad] fp32 (the
 * write vector of the token), then k [W-1][d_k] fp32, then alpha [W-1][d_k]
 * fp32 (the token's decay per key channel; a scalar decay in element 0, the
 * others unused), the whole block padded to 16 bytes.  Slot tau - 1 holds
 * token tau of the current window (lores_state_alloc_window).
 */
typedef struct {
    int32_t B, H, d_k, d_v, d_v_pad;
    int32_t n_class[LORES_NUM_PREC];        /* heads per precision class        */
    int64_t codes_offset[LORES_NUM_PREC];   /* byte offset of class codes, -1   */
    int64_t scales_offset[LORES_NUM_PREC];  /* byte offset of class scales, -1  */
    int64_t unit_code_bytes[LORES_NUM_PREC];/* code bytes per (sequence, head)  */
    uint64_t total_bytes;      /* bytes the caller's buffer must hold           */
    int32_t scale_axis;        /* LORES_SCALE_VALUE or LORES_SCALE_KEY          */
    int32_t unit_scales;       /* fp32 scales per (sequence, head): d_v_pad or d_k */
    int32_t window;            /* W: steps per requantization (1: every step)   */
    int32_t window_fill;       /* tokens of the current window in the buffer    */
    int64_t window_offset[LORES_NUM_PREC];    /* byte offset of class windows, -1 */
    int64_t unit_window_bytes[LORES_NUM_PREC];/* window bytes per unit, 0       */
} lores_layout;

/*
 * lores_state_alloc - plan the packed layout and bind a caller-owned buffer.
 * The state of every (sequence, head) unit is S in R^{d_v x d_k} of the
 * general recurrence ("Introduction and Theoretical Foundation"), held in
 * the precision head_prec assigns to its head (decay-based mixed precision,
 * "Intra-State Quantization (Section 4)") with one scale per value row (the
 * same section, scale grouping), starting from S_0 = 0.
 *   B, H        sequences and heads (1 <= B <= 65535, 1 <= H <= LORES_MAX_HEADS)
 *   d_k, d_v    key and value dimensions; d_k a multiple of 32, at most 256
 *               (LORES_EINVAL otherwise), 1 <= d_v <= LORES_MAX_DV.
 *   head_prec   host [H] precision per head (LORES_FP32 .. LORES_FP8)
 *   d_buf       device buffer, 256-byte aligned, >= *bytes; or NULL
 *   bytes       host in/out.  d_buf == NULL: size query, writes the size and
 *               returns LORES_OK without creating a handle.  Otherwise *bytes
 *               is the buffer size (LORES_ESIZE if too small).
 *   stream      the buffer is cleared to S_0 = 0 asynchronously on it
 *   out         host out: the new handle (owned by the caller; free it with
 *               lores_state_free, which never touches device memory)
 */
int lores_state_alloc(int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                      const uint8_t *head_prec, void *d_buf, size_t *bytes,
                      void *stream, lores_state **out);

/*
 * lores_state_alloc_axis - lores_state_alloc with a choice of scale grouping
 * for every scaled head (int8, int4, int6, fp8): LORES_SCALE_VALUE is
 * lores_state_alloc itself; LORES_SCALE_KEY keeps one scale per key column,
 * s_j = fl(m_j / r) with m_j the maximum of |S_ij| over the unit's d_v rows,
 * and the same codes, rounding and draws otherwise (the comparison grouping
 * of "Intra-State Quantization (Section 4)", Scale Grouping and Proposition
 * 1).  A step then dequantizes S'_ij = fl(c_ij * fl(s_j * alpha_j)).
 * LORES_SCALE_KEY is built for every d_k and d_v that lores_state_alloc
 * accepts.  A key-column state runs one launch per precision class (no
 * fused pairs).  LORES_EINVAL for any other scale_axis.
 */
int lores_state_alloc_axis(int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                           const uint8_t *head_prec, int32_t scale_axis, void *d_buf,
                           size_t *bytes, void *stream, lores_state **out);

/*
 * lores_state_alloc_window - lores_state_alloc_axis for a state whose scaled
 * heads (int8, int4, int6, fp8) are requantized once per window of W steps
 * instead of every step, the window's tokens being kept at fp32
 * in a per-unit buffer (the reading of the PACE and LeapQuant abstracts:
 * rounding once every few tokens, with the tokens in between buffered, cuts
 * the error that accumulates in the state).  Windows are the steps
 * t = kW + 1 .. (k + 1) W.  Inside a window the stored state is the state at
 * the window start, X_0, and is not written; step t at position
 * p = (t - 1) mod W + 1 < W computes g, o from X_0 and the buffered tokens
 * and appends (g, k, alpha) to the buffer; the step at p = W rebuilds the
 * state by the fp32 recurrence (S'_1 = fl(c fl(s alpha_1)), then
 * U_tau = fma(g_tau, k_tau, S'_tau), S'_tau = fl(U_{tau-1} alpha_tau), with a
 * decay per key channel taken column by column), steps it and requantizes
 * it as lores_decode_step does.  W = 1 is
 * lores_state_alloc_axis.  fp32 and bf16 heads step every token as usual.
 * With key-column scales (PACE shares scales within a column), s_i above is
 * the column's s_j and the window's end takes the column maxima.
 *   scale_axis  LORES_SCALE_VALUE or LORES_SCALE_KEY (as lores_state_alloc_axis)
 *   window      W, 1 <= W <= LORES_MAX_WINDOW
 * Built for every d_k and d_v that lores_state_alloc_axis accepts.
 * Steps on a windowed state must come in order (t = 1, 2, ... from the
 * allocation or a lores_quant_state; the handle counts the buffered tokens
 * and lores_decode_step returns LORES_EINVAL for a step t whose window
 * position does not follow them).  The decay may be a scalar per head or
 * one value per key channel (alpha_per_channel), the same kind for every
 * token of a window: a step inside a window whose kind differs from the
 * buffered tokens' returns LORES_EINVAL.  Each scaled class runs one launch
 * per step.
 * The count is kept on the host: a captured graph of steps on a windowed
 * state replays correctly when it covers whole windows.
 */
int lores_state_alloc_window(int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                             const uint8_t *head_prec, int32_t scale_axis, int32_t window,
                             void *d_buf, size_t *bytes, void *stream, lores_state **out);

void lores_state_free(lores_state *st);

/* Copy the layout of `st` into host struct *out. */
int lores_state_layout(const lores_state *st, lores_layout *out);

/*
 * lores_state_set_rounding - rounding of every later requantization of `st`
 * (host only; takes effect for calls enqueued afterwards).
 *   LORES_ROUND_STOCHASTIC  stochastic rounding (the default), as described
 *                           at lores_decode_step
 *   LORES_ROUND_NEAREST     the same formula with u = 1/2 (n = 2^15): codes
 *                           s (floor(fl(s U * inv + bias + 1/2)) - bias), i.e.
 *                           round to nearest, ties upward in even and downward
 *                           in odd columns, after the fp32 rounding of the
 *                           sum; bf16 heads keep the high half of
 *                           f32bits(U) + 2^15 (nearest, ties away from zero)
 * Round-to-nearest is the deterministic baseline the stochastic rounding is
 * compared with ("Intra-State Quantization (Section 4)", Rounding and
 * Proposition 3).  LORES_EINVAL for any other mode.
 */
int lores_state_set_rounding(lores_state *st, int32_t mode);

/* Host arrays [H]: precision and slot (index among heads of that class). */
int lores_state_head_map(const lores_state *st, uint8_t *prec_out, int32_t *slot_out);

/*
 * lores_decay_stat - decay statistic per head for precision assignment:
 * stat[h] = mean over n rows and `width` channels of log(alpha), computed in
 * double.  Larger (closer to 0) means slower decay.
 *   alpha  host [n][H][width] fp32, every value > 0
 *   stat   host out [H] double
 * (Decay-based mixed precision: section "Intra-State Quantization (Section 4)".)
 */
int lores_decay_stat(const float *alpha, int64_t n, int32_t H, int32_t width,
                     double *stat);

/*
 * lores_assign_precision - decay-based mixed precision (same section): heads
 * are ranked slowest-decaying first (larger stat first, ties to the lower head
 * index) and dealt into tiers listed slowest first.  Tier k takes
 * floor(tier_frac[k] * H + 0.5) heads (never more than remain); the last tier
 * takes every remaining head.
 *   stat       host [H] double (e.g. from lores_decay_stat)
 *   tier_frac  host [n_tiers] double, each >= 0
 *   tier_prec  host [n_tiers] precision codes
 *   head_prec  host out [H]
 * Host only and synchronous.
 */
int lores_assign_precision(const double *stat, int32_t H, const double *tier_frac,
                           const uint8_t *tier_prec, int32_t n_tiers, uint8_t *head_prec);

/*
 * lores_decode_step - one decode step t for all B x H units, in place: the
 * general recurrence S_t = S_{t-1} diag(alpha_t)(I - delta beta_t k_t k_t^T)
 * + beta_t v_t k_t^T and the readout o_t = S_t q_t ("Introduction and
 * Theoretical Foundation"), on a state that is dequantized, updated and
 * requantized each step ("Intra-State Quantization Approach", property 3)
 * with a fresh scale per value row and stochastic rounding ("Intra-State
 * Quantization (Section 4)": scale grouping, Proposition 1, Rounding,
 * Proposition 3).
 *   q, k        device [B][H][d_k]; fp32, or bfloat16 if in_bf16 != 0
 *   v           device [B][H][d_v]; same dtype as q and k
 *   alpha       device fp32 decay: [B][H] (scalar per head) or, if
 *               alpha_per_channel != 0, [B][H][d_k] (one per key channel)
 *   beta        device [B][H] fp32 write gate
 *   delta       0 (no correction) or 1 (delta rule)
 *   seed, t     key the stochastic rounding; t >= 1 (S_{t-1} -> S_t)
 *   seq_base,   added to the local sequence and head index before keying the
 *   head_base   rounding, so a shard of a larger batch reproduces the
 *               unsharded result bit for bit
 *   o           device out [B][H][d_v] fp32, the readout S_t q_t taken from
 *               the updated state before requantization
 * q, k, alpha, beta and o must be 4-byte aligned and v aligned to its
 * element size (LORES_EINVAL otherwise).  Caller preconditions not
 * checked: |q| = |k| = 1, decay in (0, 1], beta in (0, 2) when delta = 1,
 * finite inputs.  Per element of an int head, with U the updated fp32 row:
 *   scale' = fl(m / r), m = max|U_row|, r = 127 (int8), 31 (int6) or 7 (int4);
 *   code'  = s (floor(fl(s U * inv + bias + u)) - bias), inv = the largest
 *            fp32 not above r / m (0 if m = 0), bias = 128 (int8), 160 (int6)
 *            or 136 (int4), s = +1 in even and -1 in odd columns, and the
 *            columns 2m, 2m + 1 of a row share one draw u (so the odd column
 *            rounds U with the antithetic draw 1 - u: still unbiased),
 * fp8 heads: scale' = fl(m / 448), y = fl(U * inv) with inv the largest fp32
 *            not above 448 / m; the E4M3 byte of y is the sign and the top
 *            7 magnitude bits of f32bits(fl(y * 2^-120)) + (n << 4), which
 *            rounds stochastically on the E4M3 grid (subnormals included),
 *            u = n * 2^-16 and n a 16-bit counter-based draw keyed on
 *            (seed, t, sequence, head, row, column) (int heads: on the
 *            column pair).
 */
int lores_decode_step(lores_state *st, const void *q, const void *k, const void *v,
                      int32_t in_bf16, const float *alpha, int32_t alpha_per_channel,
                      const float *beta, int32_t delta, uint64_t seed, uint64_t t,
                      int64_t seq_base, int64_t head_base, float *o, void *stream);

/*
 * lores_step_launches - kernel launches one lores_decode_step on `st`
 * enqueues (host out *n): one per precision class present, except that the
 * pairs (int8, int4), (int4, int6), (bf16, int8) and (bf16, int4) share a
 * single launch when the state keeps value-row scales.
 */
int lores_step_launches(const lores_state *st, int32_t *n);

/*
 * lores_dequant_state - packed state -> device out [B][H][d_v][d_k] fp32: the
 * dequantization step of "Intra-State Quantization Approach" (the state read
 * back at full precision between steps; for inspection, checkpoints and the
 * error measurements of "Intra-State Quantization (Section 4)"),
 * value = scale * code for int heads (the row's or the column's scale), the
 * stored value for bf16 / fp32 heads.  For a windowed state with buffered
 * tokens: the current state, the stored state followed by the buffered
 * tokens' fp32 recurrence (as lores_state_alloc_window describes).
 */
int lores_dequant_state(const lores_state *st, float *out, void *stream);

/*
 * lores_quant_state - fp32 state -> packed state of `st`, in place of its
 * contents: the requantization of lores_decode_step applied to X itself
 * (int heads: fresh row scale and codes; bf16 heads: rounded; fp32 heads:
 * copied; key-column states take the column maxima of X), with the state's
 * rounding mode and draws keyed on step index 0,
 * which lores_decode_step never uses (t >= 1).  This hands a state built
 * elsewhere (a prefill, a checkpoint) to decoding: S_0 = Q(X).
 * ("Intra-State Quantization Approach": the state is held quantized between
 * steps; "Intra-State Quantization (Section 4)", scale grouping and Rounding.)
 *   X          device [B][H][d_v][d_k] fp32, 16-byte aligned (the layout
 *              lores_dequant_state writes), finite
 *   seed, seq_base, head_base   as for lores_decode_step
 * LORES_EINVAL on a NULL or misaligned X or out-of-range bases; nothing is
 * launched then.  On a windowed state it also empties the window buffer: the
 * next step is a window's first (t = 1, W + 1, ...).
 */
int lores_quant_state(lores_state *st, const float *X, uint64_t seed, int64_t seq_base,
                      int64_t head_base, void *stream);

/* Thread-local description of the last error (empty string if none). */
const char *lores_last_error(void);

/* LORES_SPEC_VERSION of the library. */
int lores_spec_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LORES_H */
