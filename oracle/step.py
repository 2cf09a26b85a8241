"""The LoReS decode step, written out plainly.

General recurrence ([LoReS] "Introduction and Theoretical Foundation",
general recurrence form), per (sequence, head) unit:

    S_t = S_{t-1} diag(alpha_t) (I - delta * beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = S_t q_t

with S in R^{d_v x d_k}, decay alpha_t scalar or per key channel, write gate
beta_t and delta in {0, 1}.  LoReS stores S quantized and, every step,
dequantizes -> updates -> requantizes it ([LoReS] "Intra-State Quantization
Approach", property 3), with one scale per value row ([LoReS] Section 4,
scale grouping and Proposition 1: s_G = max |S_G| / r, r = 2^(b-1) - 1) and
stochastic rounding ([LoReS] Section 4, Rounding).  The comparison grouping
of the same section, one scale per key column (axis="key"), is the same
quantizer with the group G taken down a column instead of along a row; the
PACE abstract argues for it at four bits.

reference_step64 is the recurrence itself in fp64 matrix form.  decode_step
is the same recurrence in the row form a kernel evaluates, with every fp32
rounding the quantized path commits to (the readings are listed in the
repository's design notes):

  1  a_ij  = fl(s_i * alpha_j);  S'_ij = fl(c_ij * a_ij)          int heads
     S'_ij = fl(v_ij * a_ij), v_ij the E4M3 value                 fp8 heads
     (key-column scales: a_ij = fl(s_j * alpha_j), the same otherwise)
     S'_ij = fl(X_ij * alpha_j)                                   bf16 / fp32 heads
  2  delta = 1: r_i = fl(sum_j S'_ij k_j);  g_i = fl(beta * fl(v_i - r_i))
     delta = 0: g_i = fl(beta * v_i)
  3  U_ij = fma(g_i, k_j, S'_ij)
       (real arithmetic: U = S' - delta*beta (S'k) k^T + beta v k^T, which is
        S_{t-1} diag(alpha)(I - delta beta k k^T) + beta v k^T)
  4  o_i  = fl(sum_j U_ij q_j)             (readout of the pre-requant state)
  5  fp8 heads: s'_i = fl(m_i / 448), inv_i = largest fp32 <= 448 / m_i,
       y_ij = fl(U_ij * inv_i), bytes = e4m3_encode(y_ij, n_ij)
     int heads, r = 2^(b-1) - 1 = 127 (int8), 31 (int6) or 7 (int4), bias
     B = 128 (int8), 160 (int6) or 136 (int4):
       m_i = max_j |U_ij|;  s'_i = fl(m_i / r);  inv_i = largest fp32 <= r / m_i
       (inv_i = 0 for m_i = 0);  with s_j = +1 for even and -1 for odd j,
       z_ij = fl(s_j U_ij * inv_i + (B + n_ij 2^-16)) in one rounding;
       e_ij = floor(z_ij);  c'_ij = s_j (e_ij - B)  in [-r, r]
       (n_ij is shared by the columns 2m, 2m + 1, so the odd column rounds
        U_ij up with probability P(1 - u < frac): the antithetic draw)
     bf16 heads: bf16 bits of (f32bits(U_ij) + n_ij) >> 16   (rounding by noise)
     fp32 heads: X'_ij = U_ij
     (key-column scales: m_j = max_i |U_ij| over the unit's d_v rows, and
      s'_j, inv_j from m_j; the draws n_ij are the same)
The dot products in 2 and 4 are accumulated in fp64 and rounded once.
"""
import numpy as np

from . import exact
from .exact import F32, F64, f32, fma32
from .rng import noise16, noise16_iid, unit_key

PREC_FP32, PREC_BF16, PREC_INT8, PREC_INT4, PREC_INT6, PREC_FP8 = 0, 1, 2, 3, 4, 5
QMAX = {PREC_INT8: 127, PREC_INT4: 7, PREC_INT6: 31}
BIAS = {PREC_INT8: 128, PREC_INT4: 136, PREC_INT6: 160}
FP8_MAX = 448.0          # largest finite E4M3 value
AXES = ("value", "key")  # one scale per value row / per key column
SCALED = (PREC_INT8, PREC_INT4, PREC_INT6, PREC_FP8)


def _check_axis(axis):
    if axis not in AXES:
        raise ValueError(f"axis must be 'value' or 'key', got {axis!r}")


def _spread(scales, axis):
    """Scales [N, d_v] (value rows) or [N, d_k] (key columns) shaped to
    broadcast against states [N, d_v, d_k]."""
    _check_axis(axis)
    return scales[:, :, None] if axis == "value" else scales[:, None, :]


# ---------------------------------------------------------------------------
# E4M3 (OCP 8-bit floating point: 1 sign, 4 exponent bits with bias 7, 3
# mantissa bits; exponent 0 holds subnormals; S.1111.111 is NaN, so the
# largest finite magnitude is 1.75 * 2^8 = 448).  The pages compare this
# format with value-grouped INT8 ("Intra-State Quantization (Section 4)",
# Format).
# ---------------------------------------------------------------------------
def e4m3_decode(b):
    """E4M3 bytes -> fp32 values, from the format's definition."""
    b = np.asarray(b, np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(F64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return (sign * mag).astype(F32)


def e4m3_encode(y, n):
    """Stochastic rounding of fp32 values |y| <= 448 to E4M3 bytes with the
    16-bit draws n.  ys = fl(y * 2^-120) puts the E4M3 normal range on the
    fp32 normal range starting at 2^-126 and the E4M3 subnormals on fp32
    denormals, so in both ranges the E4M3 grid is the fp32 bit pattern with
    its low 20 bits dropped; the draw is added just below the kept bits
    (bits 4..19) before dropping them.  The byte is the sign and the next 7
    bits.  n = 2^15 for every element is round to nearest, ties upward in
    magnitude."""
    ys = (f32(y) * F32(2.0 ** -120)).astype(F32)
    t = exact.f32_bits(ys).astype(np.uint64) + (np.asarray(n, np.uint64) << np.uint64(4))
    u = (t >> np.uint64(20)) & np.uint64(0xFFF)
    return ((u & np.uint64(0x7F)) | ((u >> np.uint64(4)) & np.uint64(0x80))).astype(np.uint8)


# ---------------------------------------------------------------------------
# fp64 reference recurrence (the definition itself)
# ---------------------------------------------------------------------------
def reference_step64(S, q, k, v, alpha, beta, delta):
    """One step of the general recurrence in fp64 for one unit.

    S [dv, dk]; q, k [dk]; v [dv]; alpha scalar or [dk]; beta scalar.
    Returns (S_t, o_t).
    """
    S = np.asarray(S, F64)
    q, k, v = (np.asarray(a, F64) for a in (q, k, v))
    dk = k.shape[0]
    a = np.broadcast_to(np.asarray(alpha, F64), (dk,))
    A = np.diag(a) @ (np.eye(dk) - delta * float(beta) * np.outer(k, k))
    S_t = S @ A + float(beta) * np.outer(v, k)
    return S_t, S_t @ q


def transition64(k, alpha, beta, delta):
    """A_t = diag(alpha_t)(I - delta beta_t k_t k_t^T) in fp64 (error propagation)."""
    k = np.asarray(k, F64)
    dk = k.shape[0]
    a = np.broadcast_to(np.asarray(alpha, F64), (dk,))
    return np.diag(a) @ (np.eye(dk) - delta * float(beta) * np.outer(k, k))


# ---------------------------------------------------------------------------
# state containers
# ---------------------------------------------------------------------------
def zero_state(prec, n, dv, dk, axis="value"):
    _check_axis(axis)
    ns = dv if axis == "value" else dk
    if prec == PREC_FP8:
        return {"fp8": np.zeros((n, dv, dk), np.uint8), "scales": np.zeros((n, ns), F32)}
    if prec in QMAX:
        return {"codes": np.zeros((n, dv, dk), np.int32), "scales": np.zeros((n, ns), F32)}
    if prec == PREC_BF16:
        return {"bits": np.zeros((n, dv, dk), np.uint16)}
    return {"X": np.zeros((n, dv, dk), F32)}


def dequant(prec, state, axis="value"):
    """Stored state as fp32 values: fl(s_i * c_ij) for int heads, fl(s_i *
    E4M3 value) for fp8 heads (s_j with key-column scales), exact otherwise."""
    if prec == PREC_FP8:
        return (_spread(state["scales"], axis) * e4m3_decode(state["fp8"])).astype(F32)
    if prec in QMAX:
        return (_spread(state["scales"], axis) * state["codes"].astype(F32)).astype(F32)
    if prec == PREC_BF16:
        return exact.bf16_to_f32(state["bits"])
    return f32(state["X"]).copy()


# ---------------------------------------------------------------------------
# requantization
# ---------------------------------------------------------------------------
def quantize_rows(U, prec, n=None, rounding="sr", axis="value"):
    """Requantize U [N, dv, dk] (fp32) with one fresh scale per value row
    (axis="value") or per key column (axis="key": the maximum runs over the
    d_v rows of each column).

    n: noise draws [N, dv, dk] (uint32 < 2^16), needed for rounding="sr".
    Int classes: column j is rounded as z = fl(s_j U inv + bias + n 2^-16),
    code = s_j (floor(z) - bias), with s_j = +1 for even and -1 for odd j.
    rounding="nearest" is the same quantizer with every draw fixed at 2^15
    (u = 1/2): round to nearest, ties upward after the fp32 rounding of the
    sum (int odd columns: ties downward; bf16: ties away from zero) -- the
    library's round-to-nearest mode.
    rounding="rtn" is the textbook form: fl(U * inv) rounded to nearest, ties
    to even (bf16: ties to even), used by the error-propagation checks.
    Returns the new state dict.
    """
    U = f32(U)
    _check_axis(axis)
    gaxis = 2 if axis == "value" else 1           # the axis a scale group runs along
    if rounding == "nearest":
        n = np.full(U.shape, 1 << 15, dtype=np.uint32)
        rounding = "sr"
    if prec == PREC_FP8:
        # the row maximum maps to the largest E4M3 value
        if rounding != "sr":
            raise ValueError(rounding)
        m = np.max(np.abs(U), axis=gaxis)
        scales = exact.rn_div32(m, F32(FP8_MAX))
        inv = exact.rd_div32(F32(FP8_MAX), m)
        y = (U * _spread(inv, axis)).astype(F32)
        return {"fp8": e4m3_encode(y, n), "scales": scales}
    if prec in QMAX:
        r = QMAX[prec]
        m = np.max(np.abs(U), axis=gaxis)
        scales = exact.rn_div32(m, F32(r))
        inv = exact.rd_div32(F32(r), m)
        if rounding == "sr":
            # even columns round U, odd columns -U (each with its own draw
            # n; the int draws give a column pair one draw, so the odd
            # column rounds U with the antithetic draw 1 - u)
            sgn = np.where(np.arange(U.shape[-1]) % 2 == 0, 1, -1).astype(np.int32)
            bias = (F32(BIAS[prec]) + n.astype(F32) * F32(2.0 ** -16)).astype(F32)
            z = fma32((U * sgn.astype(F32)).astype(F32), _spread(inv, axis), bias)
            codes = sgn * (np.floor(z).astype(np.int32) - BIAS[prec])
        elif rounding == "rtn":
            y = (U * _spread(inv, axis)).astype(F32)
            codes = np.rint(y).astype(np.int32)
        else:
            raise ValueError(rounding)
        return {"codes": codes, "scales": scales}
    if prec == PREC_BF16:
        bits = exact.f32_bits(U).astype(np.uint64)
        if rounding == "sr":
            bits = (bits + n.astype(np.uint64)) & np.uint64(0xFFFFFFFF)
        elif rounding == "rtn":
            lsb = (bits >> np.uint64(16)) & np.uint64(1)
            bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFFFFFF)
        else:
            raise ValueError(rounding)
        return {"bits": (bits >> np.uint64(16)).astype(np.uint16)}
    return {"X": U.copy()}


# ---------------------------------------------------------------------------
# the decode step
# ---------------------------------------------------------------------------
def decode_step(prec, state, q, k, v, alpha, beta, delta, seed, t, b, h,
                rounding="sr", noise="weyl", axis="value"):
    """One decode step for N units of one precision class.

    q, k [N, dk] and v [N, dv]: fp32 values (bf16 inputs converted exactly);
    alpha [N] (scalar decay) or [N, dk] (per key channel); beta [N];
    b, h [N]: global sequence and head indices (they key the noise).
    axis: "value" (one scale per value row) or "key" (one per key column).
    Returns (new_state, o [N, dv]).
    """
    q, k, v, beta = f32(q), f32(k), f32(v), f32(beta)
    N, dk = k.shape
    dv = v.shape[1]
    alpha = f32(alpha)
    a_row = alpha[:, None, None] if alpha.ndim == 1 else alpha[:, None, :]

    # 1  dequantize and decay (key columns)
    if prec == PREC_FP8:
        a = (_spread(state["scales"], axis) * a_row).astype(F32)
        Sp = (e4m3_decode(state["fp8"]) * a).astype(F32)
    elif prec in QMAX:
        a = (_spread(state["scales"], axis) * a_row).astype(F32)
        Sp = (state["codes"].astype(F32) * a).astype(F32)
    else:
        Sp = (dequant(prec, state) * a_row).astype(F32)

    # 2  delta projection and write gate
    if delta:
        r = exact.dot_rn32(Sp, k)
        g = (beta[:, None] * (v - r).astype(F32)).astype(F32)
    else:
        g = (beta[:, None] * v).astype(F32)

    # 3  rank-one write
    U = fma32(g[:, :, None], k[:, None, :], Sp)

    # 4  readout from the updated state
    o = exact.dot_rn32(U, q)

    # 5  requantize with fresh scales
    n = None
    if prec != PREC_FP32 and rounding == "sr":  # "nearest" and "rtn" need no draws
        K = unit_key(seed, t, b, h)
        n = noise16(K, dv, dk, paired=prec in QMAX) if noise == "weyl" else noise16_iid(K, dv, dk)
    return quantize_rows(U, prec, n, rounding, axis), o


def quant_state(prec, X, seed, b, h, rounding="sr", axis="value"):
    """Quantize fp32 states X [N, dv, dk] of one precision class: the
    requantization of a decode step applied to X itself, with draws keyed on
    step index 0 (decode steps use t >= 1).  b, h [N]: global indices.

    The state is stored quantized between steps ("Intra-State Quantization
    Approach"); this is how a state built elsewhere enters that form."""
    X = f32(X)
    N, dv, dk = X.shape
    n = None
    if prec != PREC_FP32 and rounding == "sr":
        n = noise16(unit_key(seed, 0, b, h), dv, dk, paired=prec in QMAX)
    return quantize_rows(X, prec, n, rounding, axis)


def run_trajectory(prec, state, inputs, delta, seed, b, h, t0=1, rounding="sr",
                   noise="weyl", axis="value"):
    """Apply decode_step for t = t0, t0+1, ... over inputs' leading time axis.

    inputs: dict of arrays q [T, N, dk], k, v [T, N, dv], alpha [T, N(, dk)],
    beta [T, N].  Returns (final_state, o [T, N, dv]).
    """
    outs = []
    T = inputs["k"].shape[0]
    for s in range(T):
        state, o = decode_step(prec, state, inputs["q"][s], inputs["k"][s], inputs["v"][s],
                               inputs["alpha"][s], inputs["beta"][s], delta, seed, t0 + s,
                               b, h, rounding=rounding, noise=noise, axis=axis)
        outs.append(o)
    return state, np.stack(outs)
