"""GPU-versus-oracle parity harness (test infrastructure).

Protocol: the oracle runs its own trajectory from its own initial state.
Before every GPU step the oracle's current state of the compared units is
written into the device buffer (the oracle never receives GPU data); the GPU
step then runs over the whole batch in the production launch shape, and its
outputs for the compared units are set against the oracle's step from the
same state and inputs.  Units not compared keep whatever the GPU computed.

Tolerances (per compared step):
  codes   at most 1e-4 of codes differ, each by at most 1 (a different dot
          product summation order can move a pre-rounding value across a
          rounding threshold)
  scales  relative difference <= 2^-20
  fp8     at most 1e-4 of bytes differ, each value within one E4M3 step
          (1/8 of the larger magnitude, or the subnormal step) of the
          oracle's, plus 2^-16 of the row's absolute maximum
  bf16    at most 1e-4 of values differ, each by one bf16 ulp, or, where the
          update cancelled to a value far below its row's magnitude (a bf16
          ulp there is tiny), by at most one ulp plus 2^-16 of the row's
          absolute maximum: a different summation order of r moves g by a
          few fp32 ulps and U by about 2^-19 of the row's magnitude
  o       per unit, max_i |o_i - o_ref_i| <= 1e-3 * max_i |o_ref_i| (1e-5 for
          fp32 heads): "relative" to the unit's largest readout.  Where a
          unit's readout is itself about zero (below 1e-6 of its readout
          scale, max_i |S_ref[i, :]|_2, which bounds |o_i| for a unit-norm q)
          that floor takes its place.  The error relative to the readout
          scale is reported beside it.
  fp32    max |X - X_ref| <= 1e-5 * max_i |X_ref[i, :]|_2

Only the compared units' bytes, inputs and readouts cross between host and
device each step, so full-size batches are compared over many steps.
"""
import sys

import numpy as np
import torch

import quantized_linear_recurrence_amd as lores
from oracle import assign as oassign
from oracle import step as ostep
from tests import layout_codec as lc
from workloads import make_inputs

F32 = np.float32


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def head_precisions(w, inputs, calib_steps=32):
    """Decay-based precision per head (library) checked against the oracle."""
    if len(w.tiers) == 1:
        return [w.tiers[0][1]] * w.H
    a = inputs["alpha"][:calib_steps].float().cpu().numpy()
    a = a.reshape(a.shape[0] * a.shape[1], w.H, -1)
    stat = lores.lores_decay_stat(a)
    frac = [f for f, _ in w.tiers]
    prec = [p for _, p in w.tiers]
    got = lores.lores_assign_precision(stat, frac, prec)
    want = oassign.assign_precision(oassign.decay_stat(a), frac, prec)
    assert got == want, (got, want)
    return got


def random_unit_state(c, dv, dk, g, axis="value"):
    ns = dv if axis == "value" else dk
    if c == 5:
        by = g.integers(0, 256, (dv, dk)).astype(np.uint8)
        by[(by & 0x7F) == 0x7F] ^= 0x01                  # no NaN patterns
        return {"fp8": by, "scales": np.exp(g.uniform(-7, -2, ns)).astype(F32)}
    if c in (2, 3, 4):
        r = {2: 127, 3: 7, 4: 31}[c]
        return {"codes": g.integers(-r, r + 1, (dv, dk)).astype(np.int32),
                "scales": np.exp(g.uniform(-7, -2, ns)).astype(F32)}
    X = (g.standard_normal((dv, dk)) * 0.05).astype(F32)
    if c == 1:
        return {"bits": (X.view(np.uint32) >> 16).astype(np.uint16)}
    return {"X": X}


def _stack(states):
    return {k: np.stack([s[k] for s in states]) for k in states[0]}


def _unstack(st, n):
    return [{k: v[i] for k, v in st.items()} for i in range(n)]


class Stats:
    def __init__(self):
        self.codes = self.code_diff = 0
        self.max_dc = 0
        self.scale_rel = 0.0
        self.bf16 = self.bf16_diff = 0
        self.max_dbits = 0
        self.fp8 = self.fp8_diff = 0
        self.fp8_excess = 0.0           # worst excess over one E4M3 step / row max
        self.bf16_far = 0               # differing by more than one ulp
        self.bf16_far_rel = 0.0         # their worst excess over one ulp / row max
        self.far_at = []                # (step, b, h, row, col) of the first far elements
        self.o_err_q = 0.0
        self.o_err_f = 0.0
        self.o_err_scale = 0.0          # the same errors over the readout scale
        self.x_err_f = 0.0
        self.steps = 0

    def summary(self):
        return (f"steps={self.steps} code_flip={self.code_diff}/{self.codes} max|dc|={self.max_dc} "
                f"scale_rel={self.scale_rel:.2e} bf16_flip={self.bf16_diff}/{self.bf16} "
                f"max|dbits|={self.max_dbits} far={self.bf16_far} "
                f"far_rel={self.bf16_far_rel:.2e} fp8_flip={self.fp8_diff}/{self.fp8} "
                f"fp8_excess={self.fp8_excess:.2e} o_err_q={self.o_err_q:.2e} "
                f"o_err_f32={self.o_err_f:.2e} (over the readout scale {self.o_err_scale:.2e}) "
                f"x_err_f32={self.x_err_f:.2e}"
                + (f" far_at(t,b,h,row,col)={self.far_at}" if self.far_at else ""))

    def check(self):
        assert self.max_dc <= 1, self.summary()
        assert self.code_diff <= max(1e-4 * self.codes, 0), self.summary()
        assert self.scale_rel <= 2.0 ** -20, self.summary()
        assert self.bf16_far_rel <= 2.0 ** -16, self.summary()
        assert self.fp8_diff <= 1e-4 * self.fp8, self.summary()
        assert self.fp8_excess <= 2.0 ** -16, self.summary()
        assert self.bf16_diff <= 1e-4 * self.bf16, self.summary()
        assert self.o_err_q <= 1e-3, self.summary()
        assert self.o_err_f <= 1e-5, self.summary()
        assert self.x_err_f <= 1e-5, self.summary()


def bf16_values(bits):
    return (np.asarray(bits, np.uint32) << np.uint32(16)).view(F32)


def _readout_scale(X):
    return np.maximum(np.linalg.norm(X.astype(np.float64), axis=-1).max(axis=-1), 1e-30)


def o_errors(o, o_ref, X_ref):
    """Per unit: (max_i |o - o_ref| / max_i |o_ref|, with a floor of 1e-6 of
    the readout scale where the readout is about zero; the same error over
    the readout scale)."""
    scale = _readout_scale(X_ref)
    err = np.abs(np.asarray(o, np.float64) - o_ref).max(axis=1)
    den = np.maximum(np.abs(np.asarray(o_ref, np.float64)).max(axis=1), 1e-6 * scale)
    return err / den, err / scale


class Mirror:
    """Host copy of a state buffer of which only the given byte ranges move:
    pull() reads them back from the device, push() writes them to it, each
    as one gather / scatter."""

    def __init__(self, buf, ranges):
        self.buf = buf
        self.host = buf.cpu().numpy()
        idx = np.concatenate([np.arange(a, a + n, dtype=np.int64) for a, n in ranges if n]) \
            if ranges else np.zeros(0, np.int64)
        self.idx = idx
        self.idx_dev = torch.from_numpy(idx).to(buf.device)

    def pull(self):
        self.host[self.idx] = self.buf[self.idx_dev].cpu().numpy()

    def push(self):
        self.buf[self.idx_dev] = torch.from_numpy(self.host[self.idx]).to(self.buf.device)


def _gather_inputs(x, bs_dev, hs_dev):
    """The compared units' inputs of one step, on the host, in unit order."""
    return {k: v[bs_dev, hs_dev].float().cpu().numpy() for k, v in x.items()}


def run_parity(w, T, B=None, units=None, seed=0, head_prec=None, init="zero", inputs=None,
               device="cuda", rounding="sr", axis="value"):
    """Run T GPU steps with per-step resync to the oracle; returns Stats.

    units: list of (b, h) to compare (default: all).  init: "zero" (S_0 = 0),
    "random" (random codes and scales, or random bf16 / fp32 values) or a
    function (prec, dv, dk, numpy Generator) -> one unit's state.
    rounding: "sr" (stochastic, the default) or "nearest" (the library's
    round-to-nearest mode, set on the state through the C ABI).
    axis: "value" (value-row scales) or "key" (key-column scales, allocated
    with LORES_SCALE_KEY).
    """
    B = w.B if B is None else B
    if inputs is None:
        inputs = make_inputs(w, seed, device, T=T, B=B)
    if head_prec is None:
        head_prec = head_precisions(w, inputs)
    st = lores.lores_state_alloc(B, w.H, w.dk, w.dv, head_prec, device=device,
                                 scale_axis=lores.LORES_SCALE_KEY if axis == "key"
                                 else lores.LORES_SCALE_VALUE)
    if rounding == "nearest":
        lores.lores_state_set_rounding(st, lores.LORES_ROUND_NEAREST)
    lay = lores.lores_state_layout(st)
    hprec, hslot = lores.lores_state_head_map(st)
    assert list(hprec) == list(head_prec)
    if units is None:
        units = [(b, h) for b in range(B) for h in range(w.H)]
    g = np.random.default_rng(1234 + seed)
    # oracle state per compared unit
    ost = {}
    for (b, h) in units:
        c = head_prec[h]
        if callable(init):
            s = init(c, w.dv, w.dk, g)
        elif init == "zero":
            s = {k: v[0] for k, v in ostep.zero_state(c, 1, w.dv, w.dk, axis=axis).items()}
        else:
            s = random_unit_state(c, w.dv, w.dk, g, axis)
        ost[(b, h)] = s
    by_class = {}
    for (b, h) in units:
        by_class.setdefault(head_prec[h], []).append((b, h))
    unit_no = {u: i for i, u in enumerate(units)}
    bs_dev = torch.tensor([b for b, _ in units], device=st.buf.device)
    hs_dev = torch.tensor([h for _, h in units], device=st.buf.device)
    ranges = []
    for (b, h) in units:
        cs, cl, ss, sl = lc.unit_ranges(lay, head_prec[h], b * lay["n_class"][head_prec[h]] + hslot[h])
        ranges += [(cs, cl), (ss, sl)]
    mirror = Mirror(st.buf, ranges)
    stats = Stats()
    for t in range(1, T + 1):
        # resync: install the oracle's state of the compared units
        for (b, h), s in ost.items():
            c = head_prec[h]
            lc.write_unit(mirror.host, lay, c, b * lay["n_class"][c] + hslot[h], s)
        mirror.push()
        x = {k: v[t - 1] for k, v in inputs.items()}
        o = lores.lores_decode_step(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], w.delta,
                                    seed, t)
        torch.cuda.synchronize()
        mirror.pull()
        o_sel = o[bs_dev, hs_dev].cpu().numpy()
        xsel = _gather_inputs(x, bs_dev, hs_dev)
        for c, us in by_class.items():
            rows = np.array([unit_no[u] for u in us])
            bs = np.array([b for b, _ in us])
            hs = np.array([h for _, h in us])
            prev = _stack([ost[u] for u in us])
            q, k, v = xsel["q"][rows], xsel["k"][rows], xsel["v"][rows]
            al, be = xsel["alpha"][rows], xsel["beta"][rows]
            new, o_ref = ostep.decode_step(c, prev, q, k, v, al, be, w.delta, seed, t, bs, hs,
                                           rounding=rounding, axis=axis)
            X_ref = ostep.dequant(c, new, axis=axis)
            scale = _readout_scale(X_ref)
            o_rel, o_sc = o_errors(o_sel[rows], o_ref, X_ref)
            o_err = float(o_rel.max())
            stats.o_err_scale = max(stats.o_err_scale, float(o_sc.max()))
            gpu = _stack([lc.read_unit(mirror.host, lay, c, b * lay["n_class"][c] + hslot[h])
                          for (b, h) in us])
            if c in (2, 3, 4):
                d = np.abs(gpu["codes"].astype(np.int64) - new["codes"])
                stats.codes += d.size
                stats.code_diff += int((d > 0).sum())
                stats.max_dc = max(stats.max_dc, int(d.max()))
                rel = np.abs(gpu["scales"].astype(np.float64) - new["scales"]) / \
                    np.maximum(np.abs(new["scales"]).astype(np.float64), 1e-38)
                rel[(new["scales"] == 0) & (gpu["scales"] == 0)] = 0
                stats.scale_rel = max(stats.scale_rel, float(rel.max()))
                stats.o_err_q = max(stats.o_err_q, float(o_err))
            elif c == 5:
                # E4M3 has a value-relative grid like bf16: a differing value
                # must lie within one E4M3 step of the oracle's value, plus the
                # cancellation allowance of the bf16 rule
                Xg = ostep.dequant(c, gpu, axis=axis).astype(np.float64)
                Xr = X_ref.astype(np.float64)
                diff = gpu["fp8"] != new["fp8"]
                stats.fp8 += diff.size
                stats.fp8_diff += int(diff.sum())
                if diff.any():
                    # the maximum of the scale group (row, or key column)
                    rowmax = np.abs(Xr).max(axis=2 if axis == "value" else 1, keepdims=True)
                    step = np.maximum(np.abs(Xr), np.abs(Xg)) / 8 + rowmax / 448 * 2.0 ** -9
                    excess = (np.abs(Xg - Xr) - step) / np.maximum(rowmax, 1e-300)
                    stats.fp8_excess = max(stats.fp8_excess, float(excess[diff].max()))
                rel = np.abs(gpu["scales"].astype(np.float64) - new["scales"]) / \
                    np.maximum(np.abs(new["scales"]).astype(np.float64), 1e-38)
                rel[(new["scales"] == 0) & (gpu["scales"] == 0)] = 0
                stats.scale_rel = max(stats.scale_rel, float(rel.max()))
                stats.o_err_q = max(stats.o_err_q, float(o_err))
            elif c == 1:
                d = np.abs(gpu["bits"].astype(np.int64) - new["bits"].astype(np.int64))
                stats.bf16 += d.size
                stats.bf16_diff += int((d > 0).sum())
                stats.max_dbits = max(stats.max_dbits, int(d.max()))
                far = d > 1
                if far.any():
                    xg = bf16_values(gpu["bits"]).astype(np.float64)
                    xr = X_ref.astype(np.float64)
                    ulp = np.abs(bf16_values(new["bits"] | np.uint16(1)).astype(np.float64)
                                 - bf16_values(new["bits"] & np.uint16(0xFFFE)).astype(np.float64))
                    rowmax = np.abs(xr).max(axis=2, keepdims=True)
                    excess = (np.abs(xg - xr) - ulp) / np.maximum(rowmax, 1e-300)
                    stats.bf16_far += int(far.sum())
                    for (i, r, col) in np.argwhere(far)[:8 - len(stats.far_at)]:
                        stats.far_at.append((t, us[i][0], us[i][1], int(r), int(col)))
                    stats.bf16_far_rel = max(stats.bf16_far_rel, float(excess[far].max()))
                stats.o_err_q = max(stats.o_err_q, float(o_err))
            else:
                xe = (np.abs(gpu["X"].astype(np.float64) - new["X"]).max(axis=(1, 2)) / scale).max()
                stats.x_err_f = max(stats.x_err_f, float(xe))
                stats.o_err_f = max(stats.o_err_f, float(o_err))
            for i, u in enumerate(us):
                ost[u] = {kk: vv[i] for kk, vv in new.items()}
        stats.steps += 1
    return stats


def run_free_fp32(w, T, B=None, seed=0, device="cuda"):
    """All heads fp32, no resync: the GPU trajectory against the oracle's over T steps.
    Returns the worst o error relative to the unit's largest readout (the
    stated bar, o_errors) and the worst relative to the readout scale."""
    B = w.B if B is None else B
    inputs = make_inputs(w, seed, device, T=T, B=B)
    st = lores.lores_state_alloc(B, w.H, w.dk, w.dv, [0] * w.H, device=device)
    bs = np.repeat(np.arange(B), w.H)
    hs = np.tile(np.arange(w.H), B)
    ost = ostep.zero_state(0, B * w.H, w.dv, w.dk)
    worst = worst_scale = 0.0
    for t in range(1, T + 1):
        x = {k: v[t - 1] for k, v in inputs.items()}
        o = lores.lores_decode_step(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], w.delta, 0, t)
        xin = {k: v.float().cpu().numpy() for k, v in x.items()}
        q = xin["q"].reshape(B * w.H, -1)
        k = xin["k"].reshape(B * w.H, -1)
        v = xin["v"].reshape(B * w.H, -1)
        al = xin["alpha"].reshape(B * w.H, -1) if w.per_channel else xin["alpha"].reshape(-1)
        be = xin["beta"].reshape(-1)
        ost, o_ref = ostep.decode_step(0, ost, q, k, v, al, be, w.delta, 0, t, bs, hs)
        rel, sc = o_errors(o.cpu().numpy().reshape(B * w.H, -1), o_ref, ost["X"])
        worst = max(worst, float(rel.max()))
        worst_scale = max(worst_scale, float(sc.max()))
    return worst, worst_scale


def run_window_parity(w, T, W, head_prec, B=None, units=None, seed=0, init="random", inputs=None,
                      device="cuda", rounding="sr", axis="value"):
    """Windowed states (lores_state_alloc_window): T steps with per-step
    resync of the stored state and of the window buffer to the oracle's
    (oracle.window).  Checked per step: o (1e-3 of the unit's largest readout,
    o_errors), the stored state unchanged inside a window and requantized
    at window ends (the code rules of Stats), the buffered token (g within
    1e-5 of |v_i| + the readout scale, times beta; k and alpha exact).
    Returns Stats."""
    from oracle import window as owin
    B = w.B if B is None else B
    if inputs is None:
        inputs = make_inputs(w, seed, device, T=T, B=B)
    st = lores.lores_state_alloc(B, w.H, w.dk, w.dv, head_prec, device=device, window=W,
                                 scale_axis=lores.LORES_SCALE_KEY if axis == "key"
                                 else lores.LORES_SCALE_VALUE)
    if rounding == "nearest":
        lores.lores_state_set_rounding(st, lores.LORES_ROUND_NEAREST)
    lay = lores.lores_state_layout(st)
    assert lay["window"] == W
    _, hslot = lores.lores_state_head_map(st)
    if units is None:
        units = [(b, h) for b in range(B) for h in range(w.H)]
    g = np.random.default_rng(4321 + seed)
    ost, obuf = {}, {}
    for (b, h) in units:
        c = head_prec[h]
        if init == "zero":
            ost[(b, h)] = {k: v[0] for k, v in ostep.zero_state(c, 1, w.dv, w.dk, axis=axis).items()}
        else:
            ost[(b, h)] = random_unit_state(c, w.dv, w.dk, g, axis)
        obuf[(b, h)] = {k: v[0] for k, v in owin.empty_buffer(1, W, w.dv, w.dk).items()}
    by_class = {}
    for (b, h) in units:
        by_class.setdefault(head_prec[h], []).append((b, h))
    unit_no = {u: i for i, u in enumerate(units)}
    bs_dev = torch.tensor([b for b, _ in units], device=st.buf.device)
    hs_dev = torch.tensor([h for _, h in units], device=st.buf.device)
    ranges = []
    for (b, h) in units:
        c = head_prec[h]
        unit = b * lay["n_class"][c] + hslot[h]
        cs, cl, ss, sl = lc.unit_ranges(lay, c, unit)
        ranges += [(cs, cl), (ss, sl)]
        wr = lc.window_ranges(lay, c, unit)
        if wr is not None:
            ranges.append(wr)
    mirror = Mirror(st.buf, ranges)
    buf_host = mirror.host
    stats = Stats()
    stats.g_err = 0.0
    for t in range(1, T + 1):
        p = owin.position(t, W)
        assert lores.lores_state_layout(st)["window_fill"] == p - 1
        for (b, h), s in ost.items():
            c = head_prec[h]
            unit = b * lay["n_class"][c] + hslot[h]
            lc.write_unit(buf_host, lay, c, unit, s)
            if lc.window_ranges(lay, c, unit) is not None:
                lc.write_window(buf_host, lay, c, unit, obuf[(b, h)])
        mirror.push()
        x = {k: v[t - 1] for k, v in inputs.items()}
        o = lores.lores_decode_step(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], w.delta,
                                    seed, t)
        torch.cuda.synchronize()
        mirror.pull()
        o_sel = o[bs_dev, hs_dev].cpu().numpy()
        xsel = _gather_inputs(x, bs_dev, hs_dev)
        for c, us in by_class.items():
            rows = np.array([unit_no[u] for u in us])
            bs = np.array([b for b, _ in us])
            hs = np.array([h for _, h in us])
            prev = _stack([ost[u] for u in us])
            pbuf = _stack([obuf[u] for u in us])
            new, nbuf, o_ref = owin.window_step(
                c, prev, pbuf, xsel["q"][rows], xsel["k"][rows], xsel["v"][rows],
                xsel["alpha"][rows], xsel["beta"][rows], w.delta, seed, t, bs, hs, W,
                rounding=rounding, axis=axis)
            Xcur = owin.replay(c, new, nbuf, 0 if p == W else p, axis, xsel["alpha"].ndim == 2)
            scale = _readout_scale(Xcur)
            o_rel, o_sc = o_errors(o_sel[rows], o_ref, Xcur)
            stats.o_err_q = max(stats.o_err_q, float(o_rel.max()))
            stats.o_err_scale = max(stats.o_err_scale, float(o_sc.max()))
            units_idx = [b * lay["n_class"][c] + hslot[h] for (b, h) in us]
            gpu = _stack([lc.read_unit(buf_host, lay, c, u) for u in units_idx])
            field = "fp8" if c == 5 else "codes"
            if p < W:
                # the stored state is not written inside a window
                assert np.array_equal(gpu[field], prev[field]), (t, c)
                assert np.array_equal(gpu["scales"].view(np.uint32), prev["scales"].view(np.uint32))
                gw = _stack([lc.read_window(buf_host, lay, c, u) for u in units_idx])
                assert np.array_equal(gw["k"][:, p - 1], nbuf["k"][:, p - 1]), (t, c)
                # a scalar decay is kept in element 0 of the slot's d_k values
                na = xsel["alpha"].ndim == 1
                assert np.array_equal(gw["alpha"][:, p - 1, :1] if na else gw["alpha"][:, p - 1],
                                      nbuf["alpha"][:, p - 1, :1] if na else nbuf["alpha"][:, p - 1]), (t, c)
                bound = (np.abs(xsel["v"][rows]) + scale[:, None]) * np.abs(xsel["beta"][rows])[:, None]
                ge = np.abs(gw["g"][:, p - 1].astype(np.float64) - nbuf["g"][:, p - 1]) / \
                    np.maximum(bound, 1e-30)
                stats.g_err = max(stats.g_err, float(ge.max()))
            elif c == 5:
                Xg = ostep.dequant(c, gpu, axis=axis).astype(np.float64)
                Xr = ostep.dequant(c, new, axis=axis).astype(np.float64)
                diff = gpu["fp8"] != new["fp8"]
                stats.fp8 += diff.size
                stats.fp8_diff += int(diff.sum())
                if diff.any():
                    rowmax = np.abs(Xr).max(axis=2 if axis == "value" else 1, keepdims=True)
                    step = np.maximum(np.abs(Xr), np.abs(Xg)) / 8 + rowmax / 448 * 2.0 ** -9
                    excess = (np.abs(Xg - Xr) - step) / np.maximum(rowmax, 1e-300)
                    stats.fp8_excess = max(stats.fp8_excess, float(excess[diff].max()))
            else:
                d = np.abs(gpu["codes"].astype(np.int64) - new["codes"])
                stats.codes += d.size
                stats.code_diff += int((d > 0).sum())
                stats.max_dc = max(stats.max_dc, int(d.max()))
            if p == W:
                rel = np.abs(gpu["scales"].astype(np.float64) - new["scales"]) / \
                    np.maximum(np.abs(new["scales"]).astype(np.float64), 1e-38)
                rel[(new["scales"] == 0) & (gpu["scales"] == 0)] = 0
                stats.scale_rel = max(stats.scale_rel, float(rel.max()))
            for i, u in enumerate(us):
                ost[u] = {kk: vv[i] for kk, vv in new.items()}
                obuf[u] = {kk: vv[i] for kk, vv in nbuf.items()}
        stats.steps += 1
    assert stats.g_err <= 1e-5, stats.g_err
    return stats
