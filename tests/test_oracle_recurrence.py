"""Pins for the oracle's recurrence ([LoReS] general recurrence form).

  * exact rational evaluation (Fractions) of the recurrence on tiny shapes,
    against the fp64 reference and the fp32 row-form step,
  * closed forms: delta = 0 with no decay (a sum of rank-one writes), the
    delta rule with beta = 1 and a repeated unit key (S_t k = v_t), decay only
    (S_t = S_0 diag(prod alpha)), and the general one-step identity
    S_t k_t = (1 - beta |k|^2) S' k_t + beta |k|^2 v_t,
  * the fp32 path free-running against the fp64 recurrence.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import step

F32, F64 = np.float32, np.float64


def _unit(g, n):
    x = g.standard_normal(n)
    return (x / np.linalg.norm(x)).astype(F32)


def _frac_step(S, q, k, v, alpha, beta, delta):
    """The recurrence in exact rationals, element by element."""
    dv, dk = len(S), len(k)
    a = alpha if isinstance(alpha, list) else [alpha] * dk
    # S diag(a)
    Sp = [[S[i][j] * a[j] for j in range(dk)] for i in range(dv)]
    # (I - delta beta k k^T)
    P = [[(1 if i == j else 0) - delta * beta * k[i] * k[j] for j in range(dk)] for i in range(dk)]
    out = [[sum(Sp[i][m] * P[m][j] for m in range(dk)) + beta * v[i] * k[j] for j in range(dk)]
           for i in range(dv)]
    o = [sum(out[i][j] * q[j] for j in range(dk)) for i in range(dv)]
    return out, o


def _fr(x):
    return Fraction(float(x))


@pytest.mark.parametrize("dv,dk,delta,per_channel", [(2, 2, 1, False), (3, 2, 0, False),
                                                      (2, 3, 1, True), (4, 4, 1, False),
                                                      (3, 4, 0, True)])
def test_exact_rational_recurrence(dv, dk, delta, per_channel):
    g = np.random.default_rng(dv * 10 + dk + delta)
    T = 6
    S_exact = [[Fraction(0)] * dk for _ in range(dv)]
    S64 = np.zeros((dv, dk))
    st = step.zero_state(step.PREC_FP32, 1, dv, dk)
    for t in range(T):
        q, k = _unit(g, dk), _unit(g, dk)
        v = g.standard_normal(dv).astype(F32)
        alpha = (g.uniform(0.5, 1.0, dk) if per_channel else g.uniform(0.5, 1.0, 1)).astype(F32)
        beta = F32(g.uniform(0.1, 1.9))
        a_ex = [_fr(x) for x in alpha] if per_channel else _fr(alpha[0])
        S_exact, o_exact = _frac_step(S_exact, [_fr(x) for x in q], [_fr(x) for x in k],
                                      [_fr(x) for x in v], a_ex, _fr(beta), delta)
        S64, o64 = step.reference_step64(S64, q, k, v, alpha if per_channel else alpha[0],
                                         beta, delta)
        st, o32 = step.decode_step(step.PREC_FP32, st, q[None], k[None], v[None],
                                   alpha[None] if per_channel else alpha, np.array([beta]),
                                   delta, 0, t + 1, [0], [0])
        ex = np.array([[float(x) for x in row] for row in S_exact])
        oex = np.array([float(x) for x in o_exact])
        scale = max(1.0, np.abs(ex).max())
        assert np.abs(S64 - ex).max() <= 1e-13 * scale
        assert np.abs(o64 - oex).max() <= 1e-13 * scale
        # fp32 path: a few roundings per step, compounded over <= 6 steps
        assert np.abs(st["X"][0].astype(F64) - ex).max() <= 64 * 2.0 ** -24 * scale * (t + 1)
        assert np.abs(o32[0].astype(F64) - oex).max() <= 64 * 2.0 ** -24 * scale * (t + 1)


def test_closed_form_no_delta_no_decay():
    g = np.random.default_rng(20)
    dv, dk, T = 16, 32, 40
    S0 = g.standard_normal((dv, dk)).astype(F32)
    st = {"X": S0[None].copy()}
    acc = S0.astype(F64)
    for t in range(T):
        k, q = _unit(g, dk), _unit(g, dk)
        v = g.standard_normal(dv).astype(F32)
        beta = F32(g.uniform(0.1, 3.0))
        st, _ = step.decode_step(step.PREC_FP32, st, q[None], k[None], v[None],
                                 np.ones(1, F32), np.array([beta]), 0, 0, t + 1, [0], [0])
        acc += float(beta) * np.outer(v.astype(F64), k.astype(F64))
    err = np.abs(st["X"][0] - acc).max() / np.abs(acc).max()
    assert err < T * 4 * 2.0 ** -24


def test_closed_form_delta_rule_repeated_key():
    g = np.random.default_rng(21)
    dv, dk = 16, 32
    k = _unit(g, dk)
    kk = float(np.dot(k.astype(F64), k.astype(F64)))
    st = {"X": g.standard_normal((1, dv, dk)).astype(F32)}
    for t in range(20):
        v = g.standard_normal(dv).astype(F32)
        st, _ = step.decode_step(step.PREC_FP32, st, k[None], k[None], v[None],
                                 np.ones(1, F32), np.ones(1, F32), 1, 0, t + 1, [0], [0])
        Sk = st["X"][0].astype(F64) @ k.astype(F64)
        assert np.abs(Sk - v).max() < 1e-5 + abs(1 - kk) * 10


def test_one_step_identity_general_beta():
    g = np.random.default_rng(22)
    dv, dk = 24, 48
    for trial in range(10):
        S = g.standard_normal((1, dv, dk)).astype(F32)
        k, q = _unit(g, dk), _unit(g, dk)
        v = g.standard_normal(dv).astype(F32)
        alpha = g.uniform(0.3, 1.0, dk).astype(F32)
        beta = F32(g.uniform(0.0, 2.0))
        st, _ = step.decode_step(step.PREC_FP32, {"X": S}, q[None], k[None], v[None],
                                 alpha[None], np.array([beta]), 1, 0, 1, [0], [0])
        k64 = k.astype(F64)
        Sp = S[0].astype(F64) * alpha.astype(F64)[None, :]
        kk = k64 @ k64
        want = (1 - float(beta) * kk) * (Sp @ k64) + float(beta) * kk * v.astype(F64)
        got = st["X"][0].astype(F64) @ k64
        assert np.abs(got - want).max() < 1e-5 * max(1.0, np.abs(Sp).max())


@pytest.mark.parametrize("per_channel", [False, True])
def test_closed_form_decay_only(per_channel):
    g = np.random.default_rng(23)
    dv, dk, T = 8, 16, 30
    S0 = g.standard_normal((1, dv, dk)).astype(F32)
    st = {"X": S0.copy()}
    prod = np.ones(dk)
    for t in range(T):
        alpha = g.uniform(0.9, 1.0, dk if per_channel else 1).astype(F32)
        k, q = _unit(g, dk), _unit(g, dk)
        st, _ = step.decode_step(step.PREC_FP32, st, q[None], k[None],
                                 np.zeros((1, dv), F32),
                                 alpha[None] if per_channel else alpha, np.zeros(1, F32), 1,
                                 0, t + 1, [0], [0])
        prod = prod * alpha.astype(F64)
    want = S0[0].astype(F64) * prod[None, :]
    assert np.abs(st["X"][0] - want).max() <= T * 2.0 ** -23 * np.abs(S0).max()


def test_readout_is_of_the_updated_state():
    g = np.random.default_rng(24)
    dv, dk = 8, 16
    S = g.standard_normal((1, dv, dk)).astype(F32)
    q, k = _unit(g, dk), _unit(g, dk)
    v = g.standard_normal(dv).astype(F32)
    st, o = step.decode_step(step.PREC_FP32, {"X": S}, q[None], k[None], v[None],
                             np.array([0.9], F32), np.array([0.7], F32), 1, 0, 1, [0], [0])
    want = st["X"][0].astype(F64) @ q.astype(F64)
    assert np.abs(o[0] - want).max() <= 1e-6 * np.abs(want).max()


@pytest.mark.parametrize("delta", [0, 1])
def test_fp32_path_tracks_fp64_recurrence(delta):
    g = np.random.default_rng(25 + delta)
    dv, dk, T = 32, 64, 64
    st = step.zero_state(step.PREC_FP32, 1, dv, dk)
    S64 = np.zeros((dv, dk))
    worst = 0.0
    for t in range(T):
        q, k = _unit(g, dk), _unit(g, dk)
        v = g.standard_normal(dv).astype(F32)
        alpha = F32(np.exp(-np.log1p(np.exp(g.normal(-3, 1)))))
        beta = F32(2 / (1 + np.exp(-g.standard_normal())))
        st, o = step.decode_step(step.PREC_FP32, st, q[None], k[None], v[None],
                                 np.array([alpha]), np.array([beta]), delta, 0, t + 1, [0], [0])
        S64, o64 = step.reference_step64(S64, q, k, v, alpha, beta, delta)
        # readout scale: max_i |S_t[i,:]|_2 bounds |o_i| for a unit q
        scale = np.linalg.norm(S64, axis=1).max()
        worst = max(worst, np.abs(o[0] - o64).max() / scale)
    assert worst < 1e-6, worst
