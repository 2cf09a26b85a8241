"""GPU runs of the error-accumulation harness: the quantized state against an
fp32 twin through the same kernel over long horizons, checked for the trends
the pages derive (error propagation through the decay, Proposition 2; the
rounding comparison, Proposition 3; decay-based precision)."""
import numpy as np
import pytest
import torch

import quantized_linear_recurrence_amd as lores
from quantized_linear_recurrence_amd import error_harness as eh
from tests.parity import log

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SR, NEAR = lores.LORES_ROUND_STOCHASTIC, lores.LORES_ROUND_NEAREST


def _run(prec, lo, hi, rnd, T=1024, H=12):
    return eh.error_trajectory(prec if callable(prec) else [prec] * H, B=32, T=T, delta=0,
                               alpha_lo=lo, alpha_hi=hi, beta=0.5, drift=100.0, rounding=rnd,
                               seed=1)


def test_error_grows_with_decay_and_horizon():
    log("case: harness int4 stochastic, decay in [0.9, 1), T=1024")
    res = _run(3, 0.9, 1.0, SR)
    s = eh.summarize(res, bins=3)
    log(str([(round(r["alpha_range"][0], 3), round(r["rel_err_T"], 4)) for r in s]))
    # slower decay keeps more of every past local error
    assert s[2]["rel_err_T"] > 1.5 * s[0]["rel_err_T"]
    slowest = res["rel_err"][-1]
    assert slowest[-1] > 2.0 * slowest[0]                 # accumulated, not one step's error


def test_int8_error_far_below_int4():
    log("case: harness int8 vs int4 stochastic, decay in [0.9, 1), T=512")
    e8 = np.mean([e[-1] for e in _run(2, 0.9, 1.0, SR, T=512)["rel_err"]])
    e4 = np.mean([e[-1] for e in _run(3, 0.9, 1.0, SR, T=512)["rel_err"]])
    log(f"int8 {e8:.4f} int4 {e4:.4f}")
    assert e8 < e4 / 8                                    # 127 vs 7 levels per sign


def test_nearest_rounding_stagnates_on_slow_heads():
    log("case: harness int4 stochastic vs nearest, decay in [0.99, 1), T=2048")
    s_sr = eh.summarize(_run(3, 0.99, 1.0, SR, T=2048), bins=3)[-1]
    s_nr = eh.summarize(_run(3, 0.99, 1.0, NEAR, T=2048), bins=3)[-1]
    log(f"stochastic {s_sr['rel_err_T']:.3f} (x{s_sr['growth_T4_to_T']:.2f} from T/4), "
        f"nearest {s_nr['rel_err_T']:.3f} (x{s_nr['growth_T4_to_T']:.2f})")
    assert s_nr["rel_err_T"] > 1.15 * s_sr["rel_err_T"]
    assert s_nr["growth_T4_to_T"] > s_sr["growth_T4_to_T"]


def test_decay_assigned_mixed_precision_sits_between():
    log("case: harness decay-assigned int8 (slowest half) + int4 vs uniform, T=512")
    H = 12
    mixed = _run(eh.decay_assigned(H, [(0.5, 2), (0.5, 3)]), 0.9, 1.0, SR, T=512)
    assert mixed["head_prec"] == [3] * 6 + [2] * 6       # heads are sorted fastest first
    assert abs(eh.effective_bits(mixed["head_prec"]) - 6.25) < 1e-9
    em = np.mean([e[-1] for e in mixed["rel_err"]])
    e8 = np.mean([e[-1] for e in _run(2, 0.9, 1.0, SR, T=512)["rel_err"]])
    e4 = np.mean([e[-1] for e in _run(3, 0.9, 1.0, SR, T=512)["rel_err"]])
    log(f"int8 {e8:.4f} mixed {em:.4f} int4 {e4:.4f}")
    assert e8 < em < e4


def test_int6_and_the_five_bit_mix():
    """int6 sits between int8 and int4, and promoting the slowest-decaying
    half of int4 heads to int6 (5.25 effective bits) recovers most of the
    int4 error on the slow heads, where it accumulates."""
    log("case: harness int6, int4 and the decay-assigned int6 + int4 mix, T=512")
    H = 12
    e = {}
    for name, prec in (("int8", 2), ("int6", 4), ("int4", 3),
                       ("mix", eh.decay_assigned(H, [(0.5, 4), (0.5, 3)]))):
        res = _run(prec, 0.9, 1.0, SR, T=512)
        e[name] = res
    mean = {k: float(np.mean([x[-1] for x in r["rel_err"]])) for k, r in e.items()}
    log(str({k: round(v, 4) for k, v in mean.items()}))
    assert mean["int8"] < mean["int6"] < mean["mix"] < mean["int4"]
    assert abs(eh.effective_bits(e["mix"]["head_prec"]) - 5.25) < 1e-9
    slow = slice(6, 12)                                  # heads sorted fastest first
    slow_mix = np.mean([x[-1] for x in e["mix"]["rel_err"][slow]])
    slow_int4 = np.mean([x[-1] for x in e["int4"]["rel_err"][slow]])
    assert slow_mix < slow_int4 / 2


def test_int8_beats_e4m3_at_the_same_bits():
    """Value-row-scaled int8 keeps a uniform grid down to zero; E4M3 spends
    bits on an exponent, so its grid is coarse at the large values a row
    scale maps near 448.  Over the horizon int8 accumulates less error."""
    log("case: harness int8 vs E4M3, stochastic, decay in [0.9, 1), T=512")
    e8 = np.mean([e[-1] for e in _run(2, 0.9, 1.0, SR, T=512)["rel_err"]])
    ef = np.mean([e[-1] for e in _run(5, 0.9, 1.0, SR, T=512)["rel_err"]])
    log(f"int8 {e8:.4f} fp8 {ef:.4f}")
    assert e8 < ef


@pytest.mark.parametrize("prec", [2, 4])
def test_grouping_readout_error_follows_proposition1(prec):
    """One quantization under value-row and key-column scales: the measured
    readout error matches Proposition 1's formula for each grouping, and the
    grouping that wins follows the outlier structure (value rows with row
    outliers, key columns with column outliers)."""
    log(f"case: Proposition 1 value rows vs key columns, prec={prec}")
    rows = eh.grouping_readout_error(prec, row_spread=2.0, col_spread=0.0, seed=3)
    cols = eh.grouping_readout_error(prec, row_spread=0.0, col_spread=2.0, seed=3)
    for res in (rows, cols):
        for name in ("value", "key"):
            ratio = res[name]["mean_e2"] / res[name]["prop1"]
            log(f"  spread rows={res['row_spread']} cols={res['col_spread']} {name}: "
                f"measured/Prop1 = {ratio:.3f}")
            assert 0.85 < ratio < 1.05, (res, name, ratio)
    assert rows["value"]["mean_e2"] < 0.5 * rows["key"]["mean_e2"], rows
    assert cols["key"]["mean_e2"] < 0.5 * cols["value"]["mean_e2"], cols


def test_windowed_requantization_accumulates_less_error():
    """Rounding once per window of W steps (the buffer holding the window's
    tokens at fp32) leaves the state with less accumulated error than
    rounding every step, under stochastic and nearest rounding (the PACE
    abstract's claim), and the error falls as W grows."""
    log("case: windowed int4 vs per-step int4, slow decay, 1024 steps")
    errs = {}
    for rnd in (SR, NEAR):
        for W in (1, 4, 16):
            res = eh.error_trajectory([3] * 12, B=32, T=1024, delta=0, alpha_lo=0.99, alpha_hi=1.0,
                                      beta=0.5, drift=100.0, rounding=rnd, seed=1, window=W)
            errs[(rnd, W)] = float(np.mean([e[-1] for e in res["rel_err"]]))
            log(f"  rounding={rnd} W={W}: rel err {errs[(rnd, W)]:.4f}")
    for rnd in (SR, NEAR):
        assert errs[(rnd, 4)] < 0.75 * errs[(rnd, 1)], errs
        assert errs[(rnd, 16)] < errs[(rnd, 4)], errs


def _oracle_series(rec, head_prec, T, dk, dv, delta, seed, rounding, axis, window):
    """The harness's two statistics recomputed by the oracle from the inputs
    the harness recorded: per head and step, the mean over sequences of
    ||S_q - S_f||_F / ||S_f||_F and of |o_q - o_f| / |o_f|, with S_q the
    quantized state (its current value: inside a window the stored state
    plus the buffered tokens) and S_f the fp32 state."""
    from oracle import step as ostep
    from oracle import window as owin
    B, H = rec["alpha"].shape
    rnd = "sr" if rounding == SR else "nearest"
    rel = np.zeros((H, T))
    orel = np.zeros((H, T))
    for h in range(H):
        c = head_prec[h]
        bs, hs = np.arange(B), np.full(B, h)
        sq = ostep.zero_state(c, B, dv, dk, axis=axis)
        sf = ostep.zero_state(0, B, dv, dk)
        buf = owin.empty_buffer(B, window, dv, dk)
        al, be = rec["alpha"][:, h], rec["beta"][:, h]
        for t in range(1, T + 1):
            q, k, v = (rec[n][t - 1][:, h] for n in ("q", "k", "v"))
            if window > 1 and c in ostep.SCALED:
                sq, buf, oq = owin.window_step(c, sq, buf, q, k, v, al, be, delta, seed, t, bs, hs,
                                               window, rounding=rnd, axis=axis)
                p = owin.position(t, window)
                Xq = owin.replay(c, sq, buf, 0 if p == window else p, axis)
            else:
                sq, oq = ostep.decode_step(c, sq, q, k, v, al, be, delta, seed, t, bs, hs,
                                           rounding=rnd, axis=axis)
                Xq = ostep.dequant(c, sq, axis=axis)
            sf, of = ostep.decode_step(0, sf, q, k, v, al, be, delta, seed, t, bs, hs)
            Xf = sf["X"].astype(np.float64)
            num = ((Xq.astype(np.float64) - Xf) ** 2).sum(axis=(1, 2))
            rel[h, t - 1] = np.sqrt(num / np.maximum((Xf ** 2).sum(axis=(1, 2)), 1e-300)).mean()
            of64 = of.astype(np.float64)
            orel[h, t - 1] = (np.linalg.norm(oq.astype(np.float64) - of64, axis=-1)
                              / np.maximum(np.linalg.norm(of64, axis=-1), 1e-300)).mean()
    return rel, orel


@pytest.mark.parametrize("axis,window", [("value", 1), ("key", 1), ("value", 4), ("key", 4)])
@pytest.mark.parametrize("rounding", [SR, NEAR])
def test_harness_statistics_equal_the_oracle(axis, window, rounding):
    """The harness's reported statistics against the oracle on the same
    inputs: with delta = 0 (the harness's setting) no dot product enters the
    state, so the GPU's quantized and fp32 trajectories are the oracle's bit
    for bit in either rounding mode, and the relative state errors agree to
    the rounding of the fp64 reductions; the readout errors differ only by the
    summation order of o."""
    head_prec = [2, 3, 4, 5]                   # int8, int4, int6, E4M3
    T, d = 64, 64
    log(f"case: harness vs oracle, B=2 H=4 d=64 T={T}, {axis} scales, window {window}, "
        f"rounding {rounding}")
    rec = {}
    res = eh.error_trajectory(head_prec, B=2, d_k=d, d_v=d, T=T, delta=0, alpha_lo=0.9,
                              alpha_hi=1.0, beta=0.5, drift=100.0, rounding=rounding, seed=3,
                              points=list(range(1, T + 1)), scale_axis=lores.LORES_SCALE_KEY
                              if axis == "key" else lores.LORES_SCALE_VALUE, window=window,
                              record=rec)
    rel, orel = _oracle_series(rec, head_prec, T, d, d, 0, 3, rounding, axis, window)
    got_rel = np.array(res["rel_err"])
    got_orel = np.array(res["o_rel_err"])
    # inside the first window from S_0 = 0 nothing has been rounded yet: both
    # sides report a zero state error there
    nz = rel > 0
    log(f"  final rel err per head: harness {np.round(got_rel[:, -1], 5).tolist()} "
        f"oracle {np.round(rel[:, -1], 5).tolist()}; worst relative difference "
        f"{np.max(np.abs(got_rel - rel)[nz] / rel[nz]):.2e} (state), worst readout difference "
        f"{np.max(np.abs(got_orel - orel)):.2e}")
    assert np.all(rel[:, -1] > 0)
    assert np.array_equal(got_rel[~nz], rel[~nz])
    np.testing.assert_allclose(got_rel, rel, rtol=1e-9, atol=0)
    np.testing.assert_allclose(got_orel, orel, rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("rounding", [SR, NEAR])
def test_harness_statistics_track_the_oracle_with_the_delta_rule(rounding):
    """With delta = 1 the projection r = S k is summed in a different order on
    the two sides, so a rare code decides differently and the trajectories
    part; the statistics still agree closely (free-running, 64 steps)."""
    head_prec = [2, 3, 4, 5]
    T, d = 64, 64
    log(f"case: harness vs oracle, delta rule, B=2 H=4 d=64 T={T}, rounding {rounding}")
    rec = {}
    res = eh.error_trajectory(head_prec, B=2, d_k=d, d_v=d, T=T, delta=1, alpha_lo=0.9,
                              alpha_hi=1.0, beta=0.5, drift=100.0, rounding=rounding, seed=4,
                              points=list(range(1, T + 1)), record=rec)
    rel, orel = _oracle_series(rec, head_prec, T, d, d, 1, 4, rounding, "value", 1)
    got_rel = np.array(res["rel_err"])
    worst = float(np.max(np.abs(got_rel - rel) / rel))
    log(f"  final rel err per head: harness {np.round(got_rel[:, -1], 5).tolist()} "
        f"oracle {np.round(rel[:, -1], 5).tolist()}; worst relative difference {worst:.2e}")
    assert worst < 0.05
