"""Pins for the oracle's key-column scale grouping (axis="key").

The pages compare two groupings of the state's scales: one per value row and
one per key column, s_G = max|S_G| / r ([LoReS] "Intra-State Quantization
(Section 4)", Scale Grouping and Proposition 1).  The checks follow from that
definition and from probability, not from the oracle's code:
  * hand-worked codes and scales of a 3 x 2 int8 state under both groupings
    (tests/golden/scale_axis_cases.json),
  * a rank-one state g k^T: with key-column scales every column holds the
    same codes up to the sign of k_j; with value-row scales every row holds
    the same codes up to the sign of g_i,
  * in nearest mode every nonzero column reaches a code of magnitude r,
    zero columns stay zero, and each value is within half a code of U,
  * quantizing a state by columns equals quantizing its transpose by rows
    (with the draws transposed; an int state's odd columns, which round -U,
    enter the transpose negated),
  * the mean over seeds is U (stochastic rounding is unbiased), and the
    readout error variance is sum_j q_j^2 C_j^2 / 6r^2 (the stochastic
    rounding counterpart of Proposition 1's key-axis formula) times
    (d_v - 1) / d_v, since each column's maximum is stored exactly,
  * a decode step from S_0 = 0 with alpha = 1 and delta = 0 stores beta v k^T
    to within one code of each column.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import rng, step

F32 = np.float32
QM = {step.PREC_INT8: 127, step.PREC_INT4: 7, step.PREC_INT6: 31}
INT = [step.PREC_INT8, step.PREC_INT4, step.PREC_INT6]
GOLD = os.path.join(os.path.dirname(__file__), "golden", "scale_axis_cases.json")


def _frac32(text):
    a, b = text.split("/")
    return F32(Fraction(int(a), int(b)))        # the correctly rounded fp32


@pytest.mark.parametrize("axis", ["key", "value"])
def test_hand_worked_cases(axis):
    for case in json.load(open(GOLD))["cases"]:
        U = np.array(case["U"], F32)[None]
        st = step.quantize_rows(U, case["prec"], rounding="nearest", axis=axis)
        want = case[axis]
        assert st["codes"][0].tolist() == want["codes"], (case["name"], axis, st["codes"][0])
        assert st["scales"][0].tolist() == [float(_frac32(s)) for s in want["scales"]]


def test_zero_state_shapes():
    assert step.zero_state(step.PREC_INT8, 3, 64, 128, axis="key")["scales"].shape == (3, 128)
    assert step.zero_state(step.PREC_INT8, 3, 64, 128)["scales"].shape == (3, 64)
    with pytest.raises(ValueError):
        step.zero_state(step.PREC_INT8, 1, 4, 4, axis="rows")


@pytest.mark.parametrize("prec", INT)
def test_rank_one_codes_follow_the_grouping(prec):
    g = np.random.default_rng(40 + prec)
    N, dv, dk = 8, 48, 64
    gv = g.standard_normal((N, dv)).astype(F32)
    kv = g.standard_normal((N, dk)).astype(F32)
    U = (gv[:, :, None] * kv[:, None, :]).astype(F32)
    key = step.quantize_rows(U, prec, rounding="nearest", axis="key")["codes"]
    # column j = sign(k_j) * the codes of round(r g_i / max|g|): compare |codes|
    # with the first column's and allow rare threshold crossings from the fp32
    # rounding of g_i k_j
    ref = np.abs(key[:, :, :1])
    assert np.mean(np.abs(key) != ref) < 1e-2
    assert np.all(np.abs(np.abs(key) - ref) <= 1)
    sgn = np.sign(kv)[:, None, :] * np.sign(gv)[:, :, None]
    nz = key != 0
    assert np.all(np.sign(key[nz]) == sgn[nz])
    val = step.quantize_rows(U, prec, rounding="nearest", axis="value")["codes"]
    refv = np.abs(val[:, :1, :])
    assert np.mean(np.abs(val) != refv) < 1e-2
    # the two groupings differ on such a state unless g or k is flat
    assert np.mean(key != val) > 0.3


@pytest.mark.parametrize("prec", INT)
def test_nearest_columns_reach_r_and_stay_within_half_a_code(prec):
    r = QM[prec]
    g = np.random.default_rng(50 + prec)
    U = (g.standard_normal((6, 40, 32)) * np.exp(g.uniform(-3, 3, (6, 1, 32)))).astype(F32)
    U[:, :, 5] = 0.0                                  # a zero column
    st = step.quantize_rows(U, prec, rounding="nearest", axis="key")
    c = st["codes"]
    assert c.min() >= -r and c.max() <= r
    colmax = np.abs(c).max(axis=1)
    assert np.all(colmax[:, 5] == 0) and np.all(st["scales"][:, 5] == 0)
    others = np.delete(colmax, 5, axis=1)
    assert np.all(others == r)
    X = step.dequant(prec, st, axis="key").astype(np.float64)
    s = st["scales"].astype(np.float64)[:, None, :]
    assert np.all(np.abs(X - U) <= s * (0.5 + 1e-5))


@pytest.mark.parametrize("prec", INT + [step.PREC_FP8])
def test_key_grouping_is_value_grouping_of_the_transpose(prec):
    g = np.random.default_rng(60 + prec)
    U = (g.standard_normal((4, 24, 40)) * np.exp(g.uniform(-2, 2, (4, 1, 40)))).astype(F32)
    n = g.integers(0, 1 << 16, U.shape).astype(np.uint32)
    a = step.quantize_rows(U, prec, n, axis="key")
    field = "fp8" if prec == step.PREC_FP8 else "codes"
    if prec == step.PREC_FP8:
        b = step.quantize_rows(np.ascontiguousarray(U.transpose(0, 2, 1)), prec,
                               np.ascontiguousarray(n.transpose(0, 2, 1)), axis="value")
        assert np.array_equal(a[field], b[field].transpose(0, 2, 1))
    else:
        # an int column j rounds sgn_j U (sgn_j = -1 for odd j): the value
        # rows of V[j, 2i] = sgn_j U[i, j] (zeros between, in the odd columns
        # of V, so that every V entry that counts is rounded as is) give the
        # key-column codes of U times sgn_j
        N, dv, dk = U.shape
        sgn = np.where(np.arange(dk) % 2 == 0, 1, -1)
        V = np.zeros((N, dk, 2 * dv), F32)
        V[:, :, 0::2] = U.transpose(0, 2, 1) * sgn[None, :, None].astype(F32)
        nv = np.zeros(V.shape, np.uint32)
        nv[:, :, 0::2] = n.transpose(0, 2, 1)
        b = step.quantize_rows(V, prec, nv, axis="value")
        assert np.array_equal(a[field], (b[field][:, :, 0::2] * sgn[None, :, None]).transpose(0, 2, 1))
    assert np.array_equal(a["scales"], b["scales"])


@pytest.mark.parametrize("prec", INT)
def test_key_grouping_mean_over_seeds_is_unbiased(prec):
    g = np.random.default_rng(70 + prec)
    U = (g.standard_normal((1, 16, 32)) * np.exp(g.uniform(-2, 2, (1, 1, 32)))).astype(F32)
    acc = np.zeros(U.shape, np.float64)
    acc2 = np.zeros(U.shape, np.float64)
    S = 3000
    for seed in range(S):
        n = rng.noise16(rng.unit_key(seed, 1, 0, 0), 16, 32, paired=True)
        X = step.dequant(prec, step.quantize_rows(U, prec, n, axis="key"), axis="key")
        acc += X
        acc2 += X.astype(np.float64) ** 2
    mean = acc / S
    var = np.maximum(acc2 / S - mean ** 2, 1e-30)
    z = (mean - U) / np.sqrt(var / S)
    # elements that always round the same way (each column's maximum) have
    # zero variance up to the cancellation in acc2 / S - mean^2
    nz = var > 1e-9 * U.astype(np.float64) ** 2
    assert np.abs(z[nz]).max() < 5.5, np.abs(z[nz]).max()


def test_key_grouping_sr_readout_error_variance():
    g = np.random.default_rng(80)
    N, dv, dk, r = 400, 32, 64, 127
    U = (g.standard_normal((N, dv, dk)) * np.exp(g.uniform(-2, 2, (N, dv, 1)))
         * np.exp(g.uniform(-1, 1, (N, 1, dk)))).astype(F32)
    q = g.standard_normal((N, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    C = np.max(np.abs(U), axis=1).astype(np.float64)
    n = rng.noise16(rng.unit_key(3, 1, np.arange(N), 0), dv, dk, paired=True)
    X = step.dequant(step.PREC_INT8, step.quantize_rows(U, step.PREC_INT8, n, axis="key"),
                     axis="key")
    e = np.einsum("nij,nj->ni", (X - U).astype(np.float64), q)
    # each column's maximum is stored exactly (its y is +-r), so one row in
    # d_v contributes no error to that column
    pred = np.einsum("nj,nj->n", q ** 2, C ** 2) / (6 * r * r) * (dv - 1) / dv
    ratio = np.mean(e ** 2) / np.mean(np.broadcast_to(pred[:, None], e.shape))
    assert abs(ratio - 1) < 0.05, ratio


@pytest.mark.parametrize("prec", INT)
def test_first_step_stores_the_write_to_one_code_per_column(prec):
    g = np.random.default_rng(90 + prec)
    N, dv, dk = 5, 40, 64
    q = g.standard_normal((N, dk)).astype(F32)
    k = g.standard_normal((N, dk)).astype(F32)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = g.standard_normal((N, dv)).astype(F32)
    beta = g.uniform(0.1, 2.0, N).astype(F32)
    st0 = step.zero_state(prec, N, dv, dk, axis="key")
    st1, o = step.decode_step(prec, st0, q, k, v, np.ones(N, F32), beta, 0, 7, 1,
                              np.arange(N), np.zeros(N, np.int64), axis="key")
    W = beta[:, None, None].astype(np.float64) * v[:, :, None] * k[:, None, :]
    X = step.dequant(prec, st1, axis="key").astype(np.float64)
    s = st1["scales"].astype(np.float64)[:, None, :]
    assert np.all(np.abs(X - W) <= s * (1 + 1e-5) + 1e-12)
    # the column scale is max_i |beta v_i k_j| / r
    want = np.abs(W).max(axis=1) / QM[prec]
    assert np.allclose(st1["scales"], want, rtol=1e-6, atol=0)
    # the readout is taken before requantization: o = (beta v k^T) q
    assert np.allclose(o, np.einsum("nij,nj->ni", W, q.astype(np.float64)), rtol=1e-5, atol=1e-6)
