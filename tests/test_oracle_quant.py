"""Pins for the oracle's requantizer (value-row scales, stochastic rounding).

What the pages fix: one scale per value row, s = max|row| / r with
r = 2^(b-1) - 1 ([LoReS] Section 4, scale grouping and Proposition 1), and
rounding that is stochastic so errors do not reinforce across steps ([LoReS]
Section 4, Rounding / Proposition 3).  The checks below follow from those
definitions and from probability, not from the oracle's code:
  * exhaustive enumeration of all 2^16 noise values, in an even and in an odd
    column (the odd column rounds -U with its draw): a value y rounds only to
    floor(y) or floor(y)+1, up with probability frac(y) (to the 2^-16 grid),
  * a column pair sharing one draw rounds antithetically: two equal values
    with fraction f both round up with probability max(0, 2f - 1) and both
    down with probability max(0, 1 - 2f),
  * bf16 rounding: the mean over all 2^16 noise values is the input, exactly,
  * zero rows, code range, one-step error bound, mean over seeds,
  * Proposition 1's readout-error variances for value-axis and key-axis
    scales under round-to-nearest (M_i^2 / 12r^2 and sum_j q_j^2 C_j^2 / 12r^2),
    and the stochastic-rounding analogue M_i^2 / 6r^2 (derived: the variance
    of a stochastic rounding with fraction f is f(1-f), mean 1/6),
  * the per-row Weyl noise gives the same readout error as one independent
    hash per element (within 10%).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import exact, rng, step

F32 = np.float32
QM = {step.PREC_INT8: 127, step.PREC_INT4: 7, step.PREC_INT6: 31}    # 2^(b-1) - 1


def _row_with_all_noise(x, m):
    """U [1, 1, 2 * 65536 + 2]: element 0 fixes the row max m, the rest all
    equal x; the odd columns 1, 3, ... and the even columns 2, 4, ... each
    see every draw once."""
    U = np.full((1, 1, 2 * 65536 + 2), x, F32)
    U[0, 0, 0] = m
    n = np.zeros(U.shape, np.uint32)
    n[0, 0, 1:-1:2] = np.arange(65536, dtype=np.uint32)
    n[0, 0, 2::2] = np.arange(65536, dtype=np.uint32)
    return U, n


@pytest.mark.parametrize("prec", [step.PREC_INT8, step.PREC_INT4, step.PREC_INT6])
def test_sr_exhaustive_probability(prec):
    r = QM[prec]
    g = np.random.default_rng(10 + prec)
    for trial in range(40):
        m = F32(np.exp(g.uniform(-8, 4)))
        x = F32(g.uniform(-1, 1) * m)
        if trial == 0:
            x = m                        # the row maximum itself
        if trial == 1:
            x = -m
        U, n = _row_with_all_noise(x, m)
        st = step.quantize_rows(U, prec, n)
        inv = exact.rd_div32(F32(r), np.array([m], F32))[0]
        y = Fraction(float(x)) * Fraction(float(inv))
        fl = y.numerator // y.denominator
        frac = y - fl
        for codes in (st["codes"][0, 0, 1:-1:2], st["codes"][0, 0, 2::2]):   # odd, even
            assert codes.size == 65536
            assert codes.min() >= -r and codes.max() <= r
            assert set(np.unique(codes).tolist()) <= {fl, fl + 1}
            p_up = Fraction(int((codes == fl + 1).sum()), 65536)
            assert abs(p_up - frac) <= Fraction(2, 65536), (x, m, float(p_up), float(frac))
            mean = Fraction(int(codes.astype(np.int64).sum()), 65536)
            assert abs(mean - y) <= Fraction(2, 65536)
        # the stored scale is the correctly rounded m / r
        assert st["scales"][0, 0] == exact.rn_div32(m, F32(r))


@pytest.mark.parametrize("prec", [step.PREC_INT8, step.PREC_INT4, step.PREC_INT6])
def test_column_pair_rounds_antithetically(prec):
    """Columns 2m and 2m + 1 share their draw; with equal values the two
    roundings are complementary: over all 2^16 draws, both round up with
    probability max(0, 2f - 1) and both down with max(0, 1 - 2f)."""
    r = QM[prec]
    g = np.random.default_rng(30 + prec)
    for trial in range(30):
        m = F32(np.exp(g.uniform(-6, 3)))
        x = F32(g.uniform(-1, 1) * m)
        U = np.full((1, 65536, 4), x, F32)
        U[:, :, 2] = m                    # the row maximum, in the second pair
        n = np.repeat(np.arange(65536, dtype=np.uint32)[:, None], 4, axis=1)[None]
        c = step.quantize_rows(U, prec, n)["codes"][0]
        inv = exact.rd_div32(F32(r), np.array([m], F32))[0]
        y = Fraction(float(x)) * Fraction(float(inv))
        fl = y.numerator // y.denominator
        f = y - fl
        up0, up1 = c[:, 0] == fl + 1, c[:, 1] == fl + 1
        both_up = Fraction(int((up0 & up1).sum()), 65536)
        both_down = Fraction(int((~up0 & ~up1).sum()), 65536)
        assert abs(both_up - max(0, 2 * f - 1)) <= Fraction(3, 65536), (trial, float(f), float(both_up))
        assert abs(both_down - max(0, 1 - 2 * f)) <= Fraction(3, 65536), (trial, float(f), float(both_down))


def test_bf16_rounding_exactly_unbiased():
    g = np.random.default_rng(11)
    xs = np.concatenate([(g.standard_normal(30) * np.exp2(g.integers(-20, 20, 30))),
                         [1.0, -1.0, 3.0e-39, 1e30, 0.0]]).astype(F32)
    for x in xs:
        U = np.full((1, 1, 65536), x, F32)
        n = np.arange(65536, dtype=np.uint32).reshape(1, 1, -1)
        vals = exact.bf16_to_f32(step.quantize_rows(U, step.PREC_BF16, n)["bits"])[0, 0]
        uniq, counts = np.unique(vals, return_counts=True)
        assert uniq.size <= 2
        mean = sum(Fraction(float(v)) * int(c) for v, c in zip(uniq, counts)) / 65536
        assert mean == Fraction(float(x)), x


@pytest.mark.parametrize("prec", [step.PREC_INT8, step.PREC_INT4, step.PREC_INT6, step.PREC_BF16])
def test_zero_rows_stay_zero(prec):
    U = np.zeros((2, 3, 64), F32)
    n = rng.noise16(rng.unit_key(0, 1, np.arange(2), 0), 3, 64)
    st = step.quantize_rows(U, prec, n)
    assert np.all(step.dequant(prec, st) == 0)
    if prec != step.PREC_BF16:
        assert np.all(st["codes"] == 0) and np.all(st["scales"] == 0)


@pytest.mark.parametrize("prec", [step.PREC_INT8, step.PREC_INT4, step.PREC_INT6])
def test_one_step_error_below_one_code(prec):
    r = QM[prec]
    g = np.random.default_rng(12)
    U = (g.standard_normal((8, 64, 128)) * np.exp(g.uniform(-5, 5, (8, 64, 1)))).astype(F32)
    U[0, 0, :] = 0
    U[1, 1, 5] = 1e30
    n = rng.noise16(rng.unit_key(5, 3, np.arange(8), 1), 64, 128)
    st = step.quantize_rows(U, prec, n)
    assert st["codes"].min() >= -r and st["codes"].max() <= r
    X = step.dequant(prec, st).astype(np.float64)
    s = st["scales"].astype(np.float64)[:, :, None]
    assert np.all(np.abs(X - U) <= s * (1 + 1e-5))


@pytest.mark.parametrize("prec", [step.PREC_INT8, step.PREC_INT4, step.PREC_INT6, step.PREC_BF16])
def test_mean_over_seeds_is_unbiased(prec):
    g = np.random.default_rng(13)
    U = (g.standard_normal((1, 16, 64))).astype(F32)
    acc = np.zeros(U.shape, np.float64)
    acc2 = np.zeros(U.shape, np.float64)
    S = 3000
    for seed in range(S):
        n = rng.noise16(rng.unit_key(seed, 1, 0, 0), 16, 64, paired=prec in QM)
        X = step.dequant(prec, step.quantize_rows(U, prec, n)).astype(np.float64)
        acc += X
        acc2 += X * X
    mean = acc / S
    var = np.maximum(acc2 / S - mean ** 2, 1e-30)
    z = (mean - U) / np.sqrt(var / S)
    nz = var > 1e-20
    assert np.abs(z[nz]).max() < 5.5, np.abs(z[nz]).max()


def test_proposition1_readout_error_variances():
    g = np.random.default_rng(14)
    N, dv, dk, r = 400, 32, 64, 127
    # rows and columns with different ranges, so the two groupings differ
    U = (g.standard_normal((N, dv, dk)) * np.exp(g.uniform(-2, 2, (N, dv, 1)))
         * np.exp(g.uniform(-1, 1, (N, 1, dk)))).astype(F32)
    q = g.standard_normal((N, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    M = np.max(np.abs(U), axis=2).astype(np.float64)            # row ranges
    C = np.max(np.abs(U), axis=1).astype(np.float64)            # column ranges

    val = step.dequant(step.PREC_INT8, step.quantize_rows(U, step.PREC_INT8, rounding="rtn"))
    e_val = np.einsum("nij,nj->ni", (val - U).astype(np.float64), q)
    ratio_val = np.mean(e_val ** 2) / np.mean(M ** 2 / (12 * r * r))
    assert abs(ratio_val - 1) < 0.05, ratio_val

    key = step.dequant(step.PREC_INT8, step.quantize_rows(U, step.PREC_INT8, rounding="rtn",
                                                          axis="key"), axis="key")
    e_key = np.einsum("nij,nj->ni", (key - U).astype(np.float64), q)
    pred_key = np.einsum("nj,nj->n", q ** 2, C ** 2)[:, None] / (12 * r * r)
    ratio_key = np.mean(e_key ** 2) / np.mean(np.broadcast_to(pred_key, e_key.shape))
    assert abs(ratio_key - 1) < 0.05, ratio_key

    n = rng.noise16(rng.unit_key(0, 1, np.arange(N), 0), dv, dk, paired=True)
    sr = step.dequant(step.PREC_INT8, step.quantize_rows(U, step.PREC_INT8, n))
    e_sr = np.einsum("nij,nj->ni", (sr - U).astype(np.float64), q)
    ratio_sr = np.mean(e_sr ** 2) / np.mean(M ** 2 / (6 * r * r))
    assert abs(ratio_sr - 1) < 0.05, ratio_sr


def _paired(K, dv, dk):
    """The int classes' draws: one Weyl draw per column pair."""
    return rng.noise16(K, dv, dk, paired=True)


@pytest.mark.parametrize("prec", [step.PREC_INT8, step.PREC_INT4, step.PREC_INT6])
def test_weyl_noise_matches_independent_noise_readout_error(prec):
    g = np.random.default_rng(15)
    N, dv, dk = 300, 32, 128
    U = (g.standard_normal((N, dv, dk)) * np.exp(g.uniform(-2, 2, (N, dv, 1)))).astype(F32)
    q = g.standard_normal((N, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    K = rng.unit_key(9, 4, np.arange(N), 2)
    errs = {}
    for name, fn in (("weyl", _paired), ("iid", rng.noise16_iid)):
        X = step.dequant(prec, step.quantize_rows(U, prec, fn(K, dv, dk)))
        e = np.einsum("nij,nj->ni", (X - U).astype(np.float64), q)
        errs[name] = float(np.mean(e ** 2))
    assert abs(errs["weyl"] / errs["iid"] - 1) < 0.10, errs


def _rank_one_states(g, N, dv, dk):
    """The state after one write from S_0 = 0: v k^T with a unit key."""
    k = g.standard_normal((N, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    return np.einsum("ni,nj->nij", g.standard_normal((N, dv)), k).astype(F32)


def _delta_rule_states(g, N, dv, dk, T):
    """States after T steps of the gated delta rule (scalar decay in [0.7, 1),
    beta = 2 sigmoid(N(0, 1)), unit keys, v ~ N(0, 1)) from S_0 = 0, in fp64:
    the low-rank rows the decode path carries."""
    S = np.zeros((N, dv, dk))
    for _ in range(T):
        k = g.standard_normal((N, dk))
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        v = g.standard_normal((N, dv))
        beta = 2.0 / (1.0 + np.exp(-g.standard_normal((N, 1))))
        S = S * g.uniform(0.7, 1.0, (N, 1, 1))
        r = np.einsum("nij,nj->ni", S, k)
        S = S + np.einsum("ni,nj->nij", beta * (v - r), k)
    return S.astype(F32)


@pytest.mark.parametrize("shape", ["rank_one", "delta_rule_4", "delta_rule_16"])
@pytest.mark.parametrize("prec", [step.PREC_INT8, step.PREC_INT4, step.PREC_INT6])
def test_weyl_noise_readout_error_on_recurrent_states(shape, prec):
    """The same gate on the structured rows of the recurrence (every row of a
    rank-one state is a multiple of the key, so its rounding fractions repeat
    from row to row), averaged over eight step keys."""
    g = np.random.default_rng(22)
    N, dv, dk = 300, 32, 128
    U = _rank_one_states(g, N, dv, dk) if shape == "rank_one" else \
        _delta_rule_states(g, N, dv, dk, int(shape.rsplit("_", 1)[1]))
    q = g.standard_normal((N, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    errs = {}
    for name, fn in (("weyl", _paired), ("iid", rng.noise16_iid)):
        tot = []
        for t in range(8):
            X = step.dequant(prec, step.quantize_rows(U, prec, fn(rng.unit_key(9, t + 1, np.arange(N), 2), dv, dk)))
            e = np.einsum("nij,nj->ni", (X - U).astype(np.float64), q)
            tot.append(np.mean(e ** 2))
        errs[name] = float(np.mean(tot))
    assert abs(errs["weyl"] / errs["iid"] - 1) < 0.10, errs


@pytest.mark.parametrize("prec", [step.PREC_INT8, step.PREC_INT4, step.PREC_INT6])
def test_nearest_mode_is_round_to_nearest(prec):
    """rounding="nearest" (the draw fixed at 2^15) rounds y = U * inv to the
    nearest code: |c - y| <= 1/2 (+ the 2^-16 rounding of the sum), and it
    agrees with the textbook ties-to-even rounding except within 2^-15 of a
    tie."""
    g = np.random.default_rng(41)
    U = (g.standard_normal((50, 16, 64)) * np.exp(g.uniform(-3, 3, (50, 16, 1)))).astype(F32)
    st = step.quantize_rows(U, prec, rounding="nearest")
    r = QM[prec]
    m = np.abs(U).max(axis=2)
    inv = exact.rd_div32(F32(r), m).astype(np.float64)
    y = U.astype(np.float64) * inv[:, :, None]
    c = st["codes"].astype(np.float64)
    assert np.all(np.abs(c - y) <= 0.5 + 2.0 ** -15)
    assert np.all(np.abs(c) <= r)
    rtn = step.quantize_rows(U, prec, rounding="rtn")["codes"]
    near_tie = np.abs(np.abs(y - np.floor(y)) - 0.5) <= 2.0 ** -15
    assert np.array_equal(st["codes"][~near_tie], rtn[~near_tie])
    # exact ties go up in even columns and down in odd ones (an odd column
    # rounds -y)
    U2 = np.zeros((1, 1, 6), F32)
    U2[0, 0] = [r, 0.5, 0.5, -0.5, -0.5, 0.0]          # y = U (inv = 1)
    c2 = step.quantize_rows(U2, prec, rounding="nearest")["codes"][0, 0]
    assert list(c2) == [r, 0, 1, -1, 0, 0]


def test_nearest_mode_bf16_is_round_to_nearest():
    g = np.random.default_rng(42)
    U = (g.standard_normal((4, 8, 256)) * np.exp(g.uniform(-20, 20, (4, 8, 1)))).astype(F32)
    near = step.quantize_rows(U, step.PREC_BF16, rounding="nearest")["bits"]
    rne = step.quantize_rows(U, step.PREC_BF16, rounding="rtn")["bits"]
    low = exact.f32_bits(U) & np.uint32(0xFFFF)
    tie = low == 0x8000
    assert np.array_equal(near[~tie], rne[~tie])
    # at a tie the magnitude rounds up (away from zero)
    x = np.array([[[exact.bits_f32(np.uint32(0x3F808000)), exact.bits_f32(np.uint32(0xBF818000))]]],
                 F32)
    got = step.quantize_rows(x, step.PREC_BF16, rounding="nearest")["bits"][0, 0]
    assert list(got) == [0x3F81, 0xBF82]


# ---------------------------------------------------------------------------
# E4M3 (fp8) heads
# ---------------------------------------------------------------------------
def _e4m3_values():
    """Every finite E4M3 byte and its value, enumerated from the format's
    definition (sign, 4-bit exponent with bias 7, 3-bit mantissa,
    exponent 0 = subnormal, S.1111.111 = NaN)."""
    out = {}
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            continue
        v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        out[b] = -v if s else v
    return out


def test_e4m3_decode_matches_the_format():
    table = _e4m3_values()
    got = step.e4m3_decode(np.arange(256))
    for b, v in table.items():
        assert Fraction(float(got[b])) == v, b
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert max(table.values()) == 448


def test_e4m3_encode_is_exact_on_the_grid_and_never_overflows():
    table = _e4m3_values()
    bytes_ = np.array(sorted(table), np.int64)
    vals = step.e4m3_decode(bytes_)
    for n in (0, 1 << 15, 65535):
        enc = step.e4m3_encode(vals, np.full(vals.shape, n, np.uint32))
        back = step.e4m3_decode(enc)
        assert np.array_equal(back, vals) or np.array_equal(np.abs(back), np.abs(vals))
    # the largest magnitude never rounds past 448, whatever the draw
    enc = step.e4m3_encode(np.array([448.0, -448.0, 447.99], np.float32), np.full(3, 65535, np.uint32))
    assert np.all(np.abs(step.e4m3_decode(enc)) <= 448)


def test_e4m3_sr_exhaustive_probability():
    """For values across the normal and subnormal ranges and the boundary,
    the 2^16 draws round to the two neighbouring grid values with P(up) equal
    to the position between them, within 2^-16."""
    grid = sorted(set(abs(v) for v in _e4m3_values().values()))
    g = np.random.default_rng(44)
    xs = [Fraction(1, 1024) * 3 + Fraction(1, 5000), Fraction(1, 64) - Fraction(1, 100000),
          Fraction(1, 64) + Fraction(1, 3000), Fraction(3, 7), Fraction(300, 1)]
    xs += [Fraction(float(x)) for x in g.uniform(0, 448, 6)]
    for x in xs:
        xf = np.float32(float(x))
        if float(xf) > 448:
            continue
        for sgn in (1, -1):
            y = np.full(65536, sgn * xf, np.float32)
            vals = step.e4m3_decode(step.e4m3_encode(y, np.arange(65536, dtype=np.uint32)))
            ax = Fraction(float(abs(xf)))
            lo = max(v for v in grid if v <= ax)
            hi = min(v for v in grid if v >= ax)
            got = set(Fraction(float(abs(v))) for v in np.unique(np.abs(vals)))
            assert got <= {lo, hi}, (x, got)
            if hi == lo:
                continue
            p_up = Fraction(int((np.abs(vals) == np.float32(float(hi))).sum()), 65536)
            assert abs(p_up - (ax - lo) / (hi - lo)) <= Fraction(2, 65536), (float(ax), float(p_up))
            assert np.all(np.sign(vals[vals != 0]) == sgn)


def test_fp8_rows_scale_to_448_and_round_to_nearest():
    g = np.random.default_rng(45)
    U = (g.standard_normal((20, 8, 64)) * np.exp(g.uniform(-5, 5, (20, 8, 1)))).astype(F32)
    st = step.quantize_rows(U, step.PREC_FP8, rounding="nearest")
    X = step.dequant(step.PREC_FP8, st)
    m = np.abs(U).max(axis=2)
    assert np.array_equal(st["scales"], exact.rn_div32(m, F32(448)))
    vals = step.e4m3_decode(st["fp8"]).astype(np.float64)
    inv = exact.rd_div32(F32(448), m).astype(np.float64)
    y = U.astype(np.float64) * inv[:, :, None]
    # nearest: within half of the local grid spacing (E4M3 keeps 3 mantissa bits)
    spacing = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(vals), 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(vals - y) <= 0.5 * spacing * (1 + 1e-6) + 2.0 ** -24 * np.abs(y))
    # every nonzero row reaches 448 (its maximum maps there)
    assert np.all(np.abs(vals).max(axis=2) == 448)
    assert X.dtype == np.float32
