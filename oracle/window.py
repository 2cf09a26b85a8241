"""Windowed requantization: the quantized state is rounded once per window of
W decode steps, with the window's updates held at high precision meanwhile.

Pages: [PACE] "PACE: Periodic and Channel-Aligned Encoding of Four-Bit
Recurrent States" (abstract: the state is rounded only once every few
generated tokens and the tokens in between are kept in a small buffer, which
reduces the error that accumulates in the state) and [LeapQuant] (abstract:
per-window quantization; inside a window the outputs come from the fixed
low-bit state together with the high-precision buffered updates).  The
recurrence and the quantizer are those of [LoReS] (oracle.step).

Reading (the pages give no more than this):
  * windows are the steps t = kW + 1 .. (k + 1)W; position p = (t - 1) mod W + 1;
  * the stored (quantized) state is the state at the window start, X_0; it is
    not rewritten inside the window;
  * the buffer holds, for each earlier token tau = 1 .. p - 1 of the window,
    its write vector g_tau (d_v), key k_tau (d_k) and decay alpha_tau: what
    the recurrence needs to rebuild S_{t-1} from X_0;
  * S_{t-1} is the recurrence from X_0 in fp32, exactly as the step computes
    it: token 1 of a window dequantizes and decays in one product,
    S'_1 = fl(c * fl(s * alpha_1)); later tokens S'_tau = fl(U_{tau-1} * alpha_tau);
    U_tau = fma(g_tau, k_tau, S'_tau);
  * each step computes r, g, U and o = U q like oracle.step.decode_step; at
    p = W it requantizes U with fresh scales and the draws of step t (the
    state is rounded once per window), otherwise it appends (g, k, alpha) to
    the buffer and leaves the stored state alone;
  * W = 1 is the per-step method itself.
Decay is a scalar per (sequence, head) (the gated delta rule's gate) or one
value per key channel (the diagonal decay of the recurrence), the same for
every token of a window; a channel decay scales key columns, so the
recurrence above holds with alpha_tau read column by column.  A buffer slot
keeps d_k decay values; a scalar decay is kept in the first.
"""
import numpy as np

from . import exact
from .exact import F32, f32, fma32
from .rng import noise16, unit_key
from . import step as ostep


def empty_buffer(n, W, dv, dk):
    """Buffer of W - 1 token slots per unit: the write vector g [d_v], the key
    [d_k] and the decay [d_k] of each token (a scalar decay in element 0,
    the rest unused)."""
    s = max(W - 1, 0)
    return {"g": np.zeros((n, s, dv), F32), "k": np.zeros((n, s, dk), F32),
            "alpha": np.ones((n, s, dk), F32)}


def _decay(a, per_channel):
    """A token's decay as a factor of the [N, d_v, d_k] state: a scalar per
    unit, or one value per key column."""
    return a[:, None, :] if per_channel else a[:, None, None]


def _slot_decay(buf, tau, per_channel):
    a = buf["alpha"][:, tau]
    return f32(a if per_channel else a[:, 0])


def position(t, W):
    """Window position p in 1 .. W of step t >= 1."""
    return (int(t) - 1) % int(W) + 1


def replay(prec, state, buf, n_tok, axis="value", per_channel=False):
    """S after the first n_tok buffered tokens of the window, from the stored
    state: the fp32 recurrence written out (n_tok = 0: the dequantized state).
    per_channel: the window's tokens carry one decay per key channel."""
    if n_tok == 0:
        return ostep.dequant(prec, state, axis=axis)
    X = None
    for tau in range(n_tok):
        a = _slot_decay(buf, tau, per_channel)
        if tau == 0:
            Sp = _first_decay(prec, state, a, axis, per_channel)
        else:
            Sp = (X * _decay(a, per_channel)).astype(F32)
        X = fma32(buf["g"][:, tau][:, :, None], buf["k"][:, tau][:, None, :], Sp)
    return X


def _first_decay(prec, state, a, axis, per_channel=False):
    """S' of a window's first token: dequantization and decay in one product,
    S'_ij = fl(c_ij * fl(s * alpha_j)) with s the row's or the column's scale
    (as oracle.step.decode_step)."""
    sc = state["scales"][:, :, None] if axis == "value" else state["scales"][:, None, :]
    f = (sc * _decay(a, per_channel)).astype(F32)
    if prec == ostep.PREC_FP8:
        return (ostep.e4m3_decode(state["fp8"]) * f).astype(F32)
    return (state["codes"].astype(F32) * f).astype(F32)


def window_step(prec, state, buf, q, k, v, alpha, beta, delta, seed, t, b, h, W,
                rounding="sr", axis="value"):
    """One decode step of N windowed units of one scaled class.

    state: the stored window-start state (codes / fp8 bytes and scales);
    buf: empty_buffer(...) holding tokens 1 .. p - 1 of the current window;
    alpha [N] (a scalar decay) or [N, d_k] (per key channel; then every
    token of the window is), beta [N]; the rest as
    oracle.step.decode_step.  Returns (state', buf', o [N, d_v])."""
    q, k, v, beta, alpha = f32(q), f32(k), f32(v), f32(beta), f32(alpha)
    N, dk = k.shape
    dv = v.shape[1]
    pc = alpha.ndim == 2
    p = position(t, W)
    if p == 1:
        Sp = _first_decay(prec, state, alpha, axis, pc)
    else:
        X = replay(prec, state, buf, p - 1, axis, pc)
        Sp = (X * _decay(alpha, pc)).astype(F32)
    if delta:
        r = exact.dot_rn32(Sp, k)
        g = (beta[:, None] * (v - r).astype(F32)).astype(F32)
    else:
        g = (beta[:, None] * v).astype(F32)
    U = fma32(g[:, :, None], k[:, None, :], Sp)
    o = exact.dot_rn32(U, q)
    if p == W:
        n = None
        if rounding == "sr":
            n = noise16(unit_key(seed, t, b, h), dv, dk, paired=prec in ostep.QMAX)
        return ostep.quantize_rows(U, prec, n, rounding, axis), empty_buffer(N, W, dv, dk), o
    nb = {kk: vv.copy() for kk, vv in buf.items()}
    nb["g"][:, p - 1] = g
    nb["k"][:, p - 1] = k
    if pc:
        nb["alpha"][:, p - 1] = alpha
    else:
        nb["alpha"][:, p - 1, 0] = alpha
    return {kk: vv.copy() for kk, vv in state.items()}, nb, o
