"""Pins for the oracle's windowed requantization (oracle.window).

The pages state only that the state is rounded once every few tokens while
the tokens in between are kept in a buffer at high precision ([PACE],
[LeapQuant] abstracts).  The checks follow from that and from the recurrence:
  * a hand-worked window of two tokens (tests/golden/window_case.json),
    including how it differs from rounding every step,
  * W = 1 is the per-step method itself (oracle.step.decode_step), bit for bit,
  * inside a window the stored state is untouched and the buffer holds the
    window's (g, k, alpha); with delta = 0 each g is fl(beta v) exactly,
  * the readouts inside a window follow the fp64 recurrence from the stored
    state to fp32 accuracy,
  * with alpha = 1 and delta = 0 the state at a window's end is the
    quantization of X_0 + sum_tau beta v k^T (one rounding per window),
  * the state changes only at window ends.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import step, window

F32 = np.float32
GOLD = os.path.join(os.path.dirname(__file__), "golden", "window_case.json")
SCALED = [step.PREC_INT8, step.PREC_INT4, step.PREC_INT6, step.PREC_FP8]


def _inputs(g, T, N, dv, dk, delta, per_channel=False):
    def unit(x):
        return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(F32)
    return {"q": unit(g.standard_normal((T, N, dk))), "k": unit(g.standard_normal((T, N, dk))),
            "v": g.standard_normal((T, N, dv)).astype(F32),
            "alpha": g.uniform(0.8, 1.0, (T, N, dk) if per_channel else (T, N)).astype(F32),
            "beta": (g.uniform(0.2, 1.5, (T, N)) if delta else g.uniform(0.1, 2.0, (T, N))).astype(F32)}


def _random_state(prec, N, dv, dk, g, axis="value"):
    ns = dv if axis == "value" else dk
    if prec == step.PREC_FP8:
        by = g.integers(0, 256, (N, dv, dk)).astype(np.uint8)
        by[(by & 0x7F) == 0x7F] ^= 1
        return {"fp8": by, "scales": np.exp(g.uniform(-5, -2, (N, ns))).astype(F32)}
    r = step.QMAX[prec]
    return {"codes": g.integers(-r, r + 1, (N, dv, dk)).astype(np.int32),
            "scales": np.exp(g.uniform(-5, -2, (N, ns))).astype(F32)}


def test_hand_worked_window():
    case = json.load(open(GOLD))
    s = F32(Fraction(1, 127))
    st = {"codes": np.array([case["state"]["codes"]], np.int32), "scales": np.array([[s]], F32)}
    buf = window.empty_buffer(1, case["W"], 1, 2)
    per = {k: v.copy() for k, v in st.items()}
    for i, tok in enumerate(case["tokens"]):
        t = i + 1
        args = (np.array([tok["q"]], F32), np.array([tok["k"]], F32), np.array([tok["v"]], F32),
                np.array([tok["alpha"]], F32), np.array([1.0], F32), 0, 0, t, np.array([0]),
                np.array([0]))
        st, buf, o = window.window_step(case["prec"], st, buf, *args, W=case["W"],
                                        rounding="nearest")
        per, _ = step.decode_step(case["prec"], per, *args[:7], t, args[8], args[9],
                                  rounding="nearest")
        want = case[f"expect_after_{t}"]
        assert st["codes"][0].tolist() == want["codes"], (t, st["codes"])
        assert o[0].tolist() == want["o"], (t, o)
        if "g" in want:
            assert buf["g"][0, 0].tolist() == want["g"]
    assert st["scales"][0].tolist() == [float(s)]
    assert per["codes"][0].tolist() == case["expect_per_step_after_2"]["codes"]


@pytest.mark.parametrize("prec", SCALED)
@pytest.mark.parametrize("delta", [0, 1])
@pytest.mark.parametrize("axis", ["value", "key"])
@pytest.mark.parametrize("per_channel", [False, True])
def test_window_one_is_the_per_step_method(prec, delta, axis, per_channel):
    g = np.random.default_rng(100 + prec + 10 * delta)
    N, dv, dk, T = 4, 24, 32, 5
    x = _inputs(g, T, N, dv, dk, delta, per_channel)
    st = _random_state(prec, N, dv, dk, g, axis)
    ref = {k: v.copy() for k, v in st.items()}
    buf = window.empty_buffer(N, 1, dv, dk)
    b, h = np.arange(N), np.full(N, 3)
    for t in range(1, T + 1):
        a = [x[k][t - 1] for k in ("q", "k", "v", "alpha", "beta")]
        st, buf, o = window.window_step(prec, st, buf, *a, delta, 9, t, b, h, W=1, axis=axis)
        ref, o_ref = step.decode_step(prec, ref, *a, delta, 9, t, b, h, axis=axis)
        for key in ref:
            assert np.array_equal(st[key], ref[key]), (t, key)
        assert np.array_equal(o, o_ref)


@pytest.mark.parametrize("prec", [step.PREC_INT8, step.PREC_INT4])
def test_inside_a_window_the_state_is_kept_and_the_buffer_fills(prec):
    g = np.random.default_rng(200 + prec)
    N, dv, dk, W = 3, 16, 32, 4
    x = _inputs(g, W, N, dv, dk, 0)
    st0 = _random_state(prec, N, dv, dk, g)
    st, buf = st0, window.empty_buffer(N, W, dv, dk)
    b, h = np.arange(N), np.zeros(N, np.int64)
    for t in range(1, W + 1):
        a = [x[k][t - 1] for k in ("q", "k", "v", "alpha", "beta")]
        st, buf, o = window.window_step(prec, st, buf, *a, 0, 1, t, b, h, W=W)
        if t < W:
            for key in st0:
                assert np.array_equal(st[key], st0[key])
            # delta = 0: the write vector is fl(beta v), exactly
            want = (x["beta"][t - 1][:, None] * x["v"][t - 1]).astype(F32)
            assert np.array_equal(buf["g"][:, t - 1], want)
            assert np.array_equal(buf["k"][:, t - 1], x["k"][t - 1])
            assert np.array_equal(buf["alpha"][:, t - 1, 0], x["alpha"][t - 1])
        else:
            assert not np.array_equal(st["codes"], st0["codes"])
            assert np.all(buf["g"] == 0)


@pytest.mark.parametrize("delta", [0, 1])
@pytest.mark.parametrize("axis,per_channel", [("value", False), ("value", True), ("key", True)])
def test_readouts_follow_the_fp64_recurrence(delta, axis, per_channel):
    g = np.random.default_rng(300 + delta)
    N, dv, dk, W = 4, 16, 32, 6
    x = _inputs(g, W, N, dv, dk, delta, per_channel)
    prec = step.PREC_INT8
    st = _random_state(prec, N, dv, dk, g, axis)
    S = step.dequant(prec, st, axis=axis).astype(np.float64)
    buf = window.empty_buffer(N, W, dv, dk)
    b, h = np.arange(N), np.zeros(N, np.int64)
    for t in range(1, W):                      # the readouts before the window's rounding
        a = [x[kk][t - 1] for kk in ("q", "k", "v", "alpha", "beta")]
        st, buf, o = window.window_step(prec, st, buf, *a, delta, 5, t, b, h, W=W, axis=axis)
        for n in range(N):
            S[n], o_ref = step.reference_step64(S[n], a[0][n], a[1][n], a[2][n], a[3][n],
                                                a[4][n], delta)
            scale = np.linalg.norm(S[n], axis=1).max()
            assert np.abs(o[n] - o_ref).max() <= 1e-5 * scale, (t, n)
        X = window.replay(prec, st, buf, t, axis, per_channel)
        assert np.abs(X - S).max() <= 1e-5 * np.abs(S).max()
        if per_channel:
            assert np.array_equal(buf["alpha"][:, t - 1], a[3])


def test_channel_decay_window_closed_form():
    """delta = 0, one decay per key channel: the state a window rebuilds is
    X_0 diag(prod alpha) + sum_tau beta_tau v_tau k_tau^T diag(prod of the
    later alphas), to fp32 accuracy; and a window whose decays are all equal
    per unit is the scalar-decay window, value for value."""
    g = np.random.default_rng(77)
    N, dv, dk, W = 3, 8, 32, 5
    x = _inputs(g, W, N, dv, dk, 0, per_channel=True)
    prec = step.PREC_INT4
    st = _random_state(prec, N, dv, dk, g)
    X0 = step.dequant(prec, st).astype(np.float64)
    buf = window.empty_buffer(N, W, dv, dk)
    b, h = np.arange(N), np.zeros(N, np.int64)
    for t in range(1, W):
        a = [x[kk][t - 1] for kk in ("q", "k", "v", "alpha", "beta")]
        st, buf, _ = window.window_step(prec, st, buf, *a, 0, 5, t, b, h, W=W)
    al = x["alpha"][:W - 1].astype(np.float64)                  # [tau, N, dk]
    want = X0 * np.prod(al, axis=0)[:, None, :]
    for tau in range(W - 1):
        later = np.prod(al[tau + 1:], axis=0) if tau + 1 < W - 1 else np.ones((N, dk))
        want += (x["beta"][tau][:, None, None] * x["v"][tau][:, :, None]
                 * x["k"][tau][:, None, :] * later[:, None, :])
    got = window.replay(prec, st, buf, W - 1, "value", True)
    assert np.abs(got - want).max() <= 1e-5 * np.abs(want).max()
    # equal decays per unit: the channel form reduces to the scalar one
    xs = _inputs(np.random.default_rng(78), W, N, dv, dk, 1)
    xc = dict(xs, alpha=np.repeat(xs["alpha"][:, :, None], dk, axis=2))
    s1 = s2 = _random_state(prec, N, dv, dk, np.random.default_rng(79))
    b1 = window.empty_buffer(N, W, dv, dk)
    b2 = window.empty_buffer(N, W, dv, dk)
    for t in range(1, W + 1):
        a1 = [xs[kk][t - 1] for kk in ("q", "k", "v", "alpha", "beta")]
        a2 = [xc[kk][t - 1] for kk in ("q", "k", "v", "alpha", "beta")]
        s1, b1, o1 = window.window_step(prec, s1, b1, *a1, 1, 5, t, b, h, W=W)
        s2, b2, o2 = window.window_step(prec, s2, b2, *a2, 1, 5, t, b, h, W=W)
        assert np.array_equal(o1, o2), t
        for kk in s1:
            assert np.array_equal(s1[kk], s2[kk]), (t, kk)


@pytest.mark.parametrize("prec", [step.PREC_INT8, step.PREC_INT4, step.PREC_INT6])
@pytest.mark.parametrize("axis", ["value", "key"])
def test_one_rounding_per_window(prec, axis):
    """alpha = 1, delta = 0: the window-end state is the quantization of the
    stored state plus every write of the window (nearest mode), and the
    codes move only at window ends; with key-column scales the scale of a
    column is its maximum over the rows."""
    g = np.random.default_rng(400 + prec)
    N, dv, dk, W, T = 3, 16, 32, 4, 12
    x = _inputs(g, T, N, dv, dk, 0)
    x["alpha"][:] = 1.0
    st = _random_state(prec, N, dv, dk, g, axis)
    gax = 2 if axis == "value" else 1
    buf = window.empty_buffer(N, W, dv, dk)
    b, h = np.arange(N), np.zeros(N, np.int64)
    r = step.QMAX[prec]
    for t in range(1, T + 1):
        a = [x[kk][t - 1] for kk in ("q", "k", "v", "alpha", "beta")]
        if (t - 1) % W == 0:
            X0 = step.dequant(prec, st, axis=axis).astype(np.float64)
            acc = X0.copy()
        acc += a[4][:, None, None].astype(np.float64) * a[2][:, :, None] * a[1][:, None, :]
        prev = st["codes"].copy()
        st, buf, _ = window.window_step(prec, st, buf, *a, 0, 2, t, b, h, W=W, rounding="nearest",
                                        axis=axis)
        if t % W:
            assert np.array_equal(st["codes"], prev)
        else:
            X = step.dequant(prec, st, axis=axis).astype(np.float64)
            sc = st["scales"].astype(np.float64)
            s = sc[:, :, None] if axis == "value" else sc[:, None, :]
            # nearest rounding of the exact window sum, up to fp32 rounding
            assert np.all(np.abs(X - acc) <= s * (0.5 + 1e-3)), t
            m = np.abs(acc).max(axis=gax)
            assert np.allclose(st["scales"], m / r, rtol=1e-5)
