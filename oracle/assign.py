"""Decay-based per-head precision assignment.

[LoReS] abstract and "Intra-State Quantization (Section 4)", decay-based mixed
precision: slowly decaying heads keep their errors longest (Proposition 2's
bound weights old errors by powers of the decay), so they are the ones given
more bits; promoting the slowest-decaying half of the heads recovers most of
the INT4-to-INT6 gap.

Reading used here: the decay statistic of head h is the mean of log(alpha)
over every sampled (step, sequence) and, for per-channel decay, every key
channel.  A larger (less negative) mean is a slower decay.  Heads are ranked
slowest first (ties: lower head index first) and dealt into tiers listed
slowest first; tier k takes floor(frac_k * H + 0.5) heads, never more than
remain, and the last tier takes all that remain.

Pinned by hand-worked cases in tests/test_oracle_assign.py.
"""
import math

import numpy as np


def decay_stat(alpha):
    """Mean log(alpha) per head; alpha [n, H] or [n, H, width], any float dtype."""
    a = np.asarray(alpha, dtype=np.float64)
    if a.ndim == 2:
        a = a[:, :, None]
    H = a.shape[1]
    return np.array([np.mean(np.log(a[:, h, :])) for h in range(H)], dtype=np.float64)


def assign_precision(stat, tier_frac, tier_prec):
    """Precision code per head (list of ints), slowest-decaying heads in the first tier."""
    H = len(stat)
    order = sorted(range(H), key=lambda h: (-float(stat[h]), h))
    out = [None] * H
    pos = 0
    for n, (frac, prec) in enumerate(zip(tier_frac, tier_prec)):
        if n == len(tier_frac) - 1:
            count = H - pos
        else:
            count = min(int(math.floor(float(frac) * H + 0.5)), H - pos)
        for h in order[pos:pos + count]:
            out[h] = int(prec)
        pos += count
    return out
