"""Error accumulation of the quantized state over long decode trajectories.

A second workload on the same decode-step kernel: one state stored at the
chosen precisions and an unquantized (fp32) twin are stepped through the C ABI
on identical synthetic inputs from S_0 = 0, and the relative state error
||Q-state - fp32 state||_F / ||fp32 state||_F and readout error are sampled
along the horizon.  This measures at kernel speed what the pages analyse:

  - errors enter as one local rounding error per step and propagate through
    the decay ("Introduction and Theoretical Foundation", error propagation;
    "Intra-State Quantization (Section 4)", Proposition 2: a decay-weighted
    sum of local errors, so slowly decaying heads accumulate the most);
  - stochastic rounding makes the local errors zero-mean and uncorrelated
    across steps, so they add in quadrature, while round-to-nearest errors
    are deterministic and can add up coherently: once a slowly decaying
    state is large next to each write, nearest rounding drops the part of a
    write below half a code every step (same section, Rounding and
    Proposition 3);
  - value-row scales at 8 or 4 bits set the size of the local error (same
    section, scale grouping and Proposition 1).

Inputs: per head a decay alpha_h fixed over time (drawn in [alpha_lo,
alpha_hi), sorted so head index follows decay), q_t fresh unit vectors, and
k_t = unit(k0 + drift * n_t), v_t = v0 + drift * n'_t.  A small drift keeps
the writes aligned with the state (rank one, nothing accumulates); a large
one gives independent random writes, with which a slowly decaying state
random-walks, each write shrinks relative to the state, and round-to-nearest
starts to drop writes smaller than half a code.  All inputs are generated on
the device; nothing here is on the decode path.
"""
import math

import numpy as np

from . import (LORES_FP32, LORES_ROUND_NEAREST, LORES_ROUND_STOCHASTIC, LORES_SCALE_KEY,
               LORES_SCALE_VALUE, lores_decode_step, lores_dequant_state, lores_quant_state,
               lores_state_alloc, lores_state_set_rounding)


def sample_points(T, n=24):
    """About n log-spaced step indices in [1, T], always including T."""
    pts = sorted({int(round(x)) for x in np.geomspace(1, T, n)} | {T})
    return [p for p in pts if 1 <= p <= T]


def error_trajectory(head_prec, B=32, d_k=128, d_v=128, T=1024, delta=0, alpha_lo=0.9,
                     alpha_hi=0.999, beta=0.5, drift=0.05, rounding=LORES_ROUND_STOCHASTIC,
                     seed=0, points=None, device="cuda", scale_axis=LORES_SCALE_VALUE, window=1,
                     record=None):
    """Run T steps of a state with per-head precisions `head_prec` (a list,
    or a function of the per-head decays giving one; scales per value row or,
    with scale_axis = LORES_SCALE_KEY, per key column; requantized every step
    or, with window = W > 1, once per window of W steps) and of its fp32 twin;
    return {"t": [...], "rel_err": [H lists], "o_rel_err": [H lists],
    "alpha": [H], "head_prec": [H]} with errors averaged over the B
    sequences at each sampled t.  A dict passed as `record` receives the
    inputs of every step on the host ("q", "k", "v": lists of [B, H, d]
    arrays; "alpha", "beta": [B, H]), for recomputing the statistics
    elsewhere.
    """
    import torch

    H = len(head_prec) if not callable(head_prec) else int(head_prec(None))
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed) * 1000003 + 17)
    f32 = torch.float32

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)

    alpha_h = torch.sort(alpha_lo + (alpha_hi - alpha_lo) * torch.rand(H, generator=g, device=dev,
                                                                       dtype=f32))[0]
    alpha = alpha_h.view(1, H).expand(B, H).contiguous()
    beta_t = torch.full((B, H), float(beta), dtype=f32, device=dev)
    k0 = torch.randn(B, H, d_k, generator=g, device=dev, dtype=f32)
    v0 = torch.randn(B, H, d_v, generator=g, device=dev, dtype=f32)

    if callable(head_prec):
        head_prec = head_prec(alpha_h.cpu().numpy())
    if record is not None:
        record["alpha"] = alpha.cpu().numpy()
        record["beta"] = beta_t.cpu().numpy()
    sq = lores_state_alloc(B, H, d_k, d_v, list(head_prec), device=dev, scale_axis=scale_axis,
                           window=window)
    lores_state_set_rounding(sq, rounding)
    sf = lores_state_alloc(B, H, d_k, d_v, [LORES_FP32] * H, device=dev)
    oq = torch.empty((B, H, d_v), dtype=f32, device=dev)
    of = torch.empty_like(oq)
    pts = set(points if points is not None else sample_points(T))
    out = {"t": [], "rel_err": [], "o_rel_err": [], "alpha": alpha_h.cpu().tolist(),
           "head_prec": list(head_prec)}
    for t in range(1, T + 1):
        q = unit(torch.randn(B, H, d_k, generator=g, device=dev, dtype=f32))
        k = unit(k0 + drift * torch.randn(B, H, d_k, generator=g, device=dev, dtype=f32))
        v = v0 + drift * torch.randn(B, H, d_v, generator=g, device=dev, dtype=f32)
        lores_decode_step(sq, q, k, v, alpha, beta_t, delta, seed, t, o=oq)
        lores_decode_step(sf, q, k, v, alpha, beta_t, delta, seed, t, o=of)
        if record is not None:
            for name, x in (("q", q), ("k", k), ("v", v)):
                record.setdefault(name, []).append(x.cpu().numpy())
        if t in pts:
            Xq = lores_dequant_state(sq).double()
            Xf = lores_dequant_state(sf).double()
            num = (Xq - Xf).pow(2).sum(dim=(2, 3))
            den = Xf.pow(2).sum(dim=(2, 3)).clamp_min(1e-300)
            rel = (num / den).sqrt().mean(dim=0)                     # [H]
            onum = (oq.double() - of.double()).norm(dim=-1)
            oden = of.double().norm(dim=-1).clamp_min(1e-300)
            orel = (onum / oden).mean(dim=0)
            out["t"].append(t)
            out["rel_err"].append(rel.cpu().tolist())
            out["o_rel_err"].append(orel.cpu().tolist())
    # transpose to per-head series
    out["rel_err"] = [list(x) for x in zip(*out["rel_err"])]
    out["o_rel_err"] = [list(x) for x in zip(*out["o_rel_err"])]
    return out


def summarize(res, bins=3):
    """Final-step relative state error and its growth from t_mid to T, by
    decay bin (heads sorted by alpha, split into `bins` equal groups)."""
    H = len(res["alpha"])
    t = res["t"]
    i_end = len(t) - 1
    i_mid = min(range(len(t)), key=lambda i: abs(t[i] - t[-1] / 4))
    groups = np.array_split(np.arange(H), bins)
    rows = []
    for gi in groups:
        e_end = float(np.mean([res["rel_err"][h][i_end] for h in gi]))
        e_mid = float(np.mean([res["rel_err"][h][i_mid] for h in gi]))
        o_end = float(np.mean([res["o_rel_err"][h][i_end] for h in gi]))
        rows.append({"alpha_range": [float(res["alpha"][gi[0]]), float(res["alpha"][gi[-1]])],
                     "rel_err_T": e_end, "rel_err_T_over_4": e_mid,
                     "growth_T4_to_T": e_end / e_mid if e_mid > 0 else math.inf,
                     "o_rel_err_T": o_end})
    return rows


# bits per stored element including the fp32 row scale (d_k = 128)
def effective_bits(head_prec, d_k=128):
    per = {LORES_FP32: 32.0, 1: 16.0, 2: 8.0 + 32.0 / d_k, 3: 4.0 + 32.0 / d_k,
           4: 6.0 + 32.0 / d_k, 5: 8.0 + 32.0 / d_k}
    return float(np.mean([per[p] for p in head_prec]))


def decay_assigned(H, tiers):
    """Per-head precision from the decays through lores_assign_precision
    (tiers slowest first, as [(fraction, precision), ...]); called with None
    it returns H."""
    from . import lores_assign_precision

    def f(alpha):
        if alpha is None:
            return H
        stat = np.log(np.asarray(alpha, np.float64))
        return lores_assign_precision(stat, [fr for fr, _ in tiers], [p for _, p in tiers])
    return f


def grouping_readout_error(prec, B=64, H=8, d_k=128, d_v=128, row_spread=2.0, col_spread=2.0,
                           seed=0, device="cuda"):
    """Readout error of one quantization of synthetic states under value-row
    and key-column scales, against Proposition 1 ("Intra-State Quantization
    (Section 4)"): with round to nearest and a uniform rounding error,
    E[e_i^2] = M_i^2 / 12 r^2 (value rows; M_i the row range, |q| = 1) and
    sum_j q_j^2 C_j^2 / 12 r^2 (key columns; C_j the column range).  States
    S_ij = g_ij exp(a_i) exp(b_j) with a_i ~ U(-row_spread, row_spread),
    b_j ~ U(-col_spread, col_spread): the row spread favours value rows, the
    column spread key columns.  Quantized by lores_quant_state (nearest mode)
    and read back by lores_dequant_state; returns measured and predicted mean
    e_i^2 per grouping."""
    import torch

    r = {2: 127, 3: 7, 4: 31}[prec]
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    f64 = torch.float64
    a = (2 * torch.rand(B, H, d_v, 1, generator=g, device=dev) - 1) * row_spread
    b = (2 * torch.rand(B, H, 1, d_k, generator=g, device=dev) - 1) * col_spread
    X = (torch.randn(B, H, d_v, d_k, generator=g, device=dev) * a.exp() * b.exp()).float().contiguous()
    q = torch.randn(B, H, d_k, generator=g, device=dev, dtype=f64)
    q = q / q.norm(dim=-1, keepdim=True)
    Xd = X.double()
    M = Xd.abs().amax(dim=3)                                     # [B, H, d_v]
    C = Xd.abs().amax(dim=2)                                     # [B, H, d_k]
    pred = {"value": (M ** 2).mean().item() / (12 * r * r),
            "key": ((q ** 2 * C ** 2).sum(-1, keepdim=True).expand(B, H, d_v)).mean().item()
            / (12 * r * r)}
    out = {"prec": prec, "row_spread": row_spread, "col_spread": col_spread}
    for name, axis in (("value", LORES_SCALE_VALUE), ("key", LORES_SCALE_KEY)):
        st = lores_state_alloc(B, H, d_k, d_v, [prec] * H, device=dev, scale_axis=axis)
        lores_state_set_rounding(st, LORES_ROUND_NEAREST)
        lores_quant_state(st, X, seed)
        E = lores_dequant_state(st).double() - Xd
        e = (E @ q.unsqueeze(-1)).squeeze(-1)                    # [B, H, d_v]
        out[name] = {"mean_e2": (e ** 2).mean().item(), "prop1": pred[name]}
    return out


def run_suite(T=2048, B=32, H=12, d=128, seed=1, device="cuda"):
    """The harness's report: random writes (drift 100), scalar decay, delta
    = 0, two decay regimes; int8, E4M3, int6 and int4 states, int8 and int4
    with key-column scales, int8 and int4 requantized once per window of 4 or
    16 steps (int4 also over key columns), and the decay-assigned mixes that keep the slowest half of the
    heads at 8 or 6 bits (6.25 and 5.25 effective bits); stochastic and
    nearest rounding.  Then Proposition 1's value-row versus key-column
    readout error on states with row or column outliers."""
    names = {0: "stochastic", 1: "nearest"}
    rows = []
    for lo, hi in ((0.9, 1.0), (0.99, 1.0)):
        V = LORES_SCALE_VALUE
        for label, prec, axis, win in (
                ("int8", [2] * H, V, 1), ("fp8 (E4M3)", [5] * H, V, 1),
                ("int6", [4] * H, V, 1), ("int4", [3] * H, V, 1),
                ("int8, key columns", [2] * H, LORES_SCALE_KEY, 1),
                ("int4, key columns", [3] * H, LORES_SCALE_KEY, 1),
                ("int8, window 4", [2] * H, V, 4), ("int4, window 4", [3] * H, V, 4),
                ("int4, window 16", [3] * H, V, 16),
                ("int4, key columns, window 4", [3] * H, LORES_SCALE_KEY, 4),
                ("int8 slowest half + int4", decay_assigned(H, [(0.5, 2), (0.5, 3)]), V, 1),
                ("int6 slowest half + int4", decay_assigned(H, [(0.5, 4), (0.5, 3)]), V, 1)):
            for rnd in (LORES_ROUND_STOCHASTIC, LORES_ROUND_NEAREST):
                res = error_trajectory(prec, B=B, d_k=d, d_v=d, T=T, delta=0, alpha_lo=lo,
                                       alpha_hi=hi, beta=0.5, drift=100.0, rounding=rnd, seed=seed,
                                       device=device, scale_axis=axis, window=win)
                rows.append({"decay": [lo, hi], "state": label, "rounding": names[rnd], "window": win,
                             "effective_bits": effective_bits(res["head_prec"], d),
                             "mean_rel_err_T": float(np.mean([e[-1] for e in res["rel_err"]])),
                             "by_decay_bin": summarize(res, bins=3)})
    for prec in (2, 4):
        for rs, cs in ((2.0, 0.0), (0.0, 2.0), (1.0, 1.0)):
            rows.append({"grouping": grouping_readout_error(prec, row_spread=rs, col_spread=cs,
                                                            seed=seed, device=device)})
    return rows
