"""The pages' error analysis, checked on the oracle's quantized trajectories.

[LoReS] "Introduction and Theoretical Foundation", error propagation:
    E_t = E_{t-1} diag(alpha_t)(I - delta beta_t k_t k_t^T) + eps_t
[LoReS] Section 4, Proposition 2: with every decay at most alpha < 1,
    ||E_t||_F <= sum_tau alpha^(t - tau) ||eps_tau||_F
[LoReS] Section 4, Proposition 3 (scalar decay, delta = 0,
    gamma_{tau,t} = prod_{j = tau+1..t} alpha_j): E_t = sum_tau gamma eps_tau, so
    ||E_t||^2 has cross terms 2 sum gamma gamma <eps_tau, eps_s>, which stochastic
    rounding removes in expectation and round-to-nearest does not.

Here E_t is the quantized state (dequantized, exact in fp64) minus the fp64
unquantized trajectory, and eps_t = S^q_t - (S^q_{t-1} A_t + beta_t v_t k_t^T)
in fp64.  The identity then holds by algebra, so checking it to ~1e-12 pins
that the quantized step and the reference apply the same A_t and write term;
the size of eps_t (at most about one code step per element) pins that the
quantized step is the recurrence plus a requantization and nothing else.
"""
import numpy as np
import pytest

from oracle import step

F32, F64 = np.float32, np.float64


def _unit(g, n):
    x = g.standard_normal(n)
    return (x / np.linalg.norm(x)).astype(F32)


def _trajectory(prec, T, dv, dk, delta, seed, rounding="sr", alpha_range=(0.8, 0.98),
                per_channel=False, inputs_seed=0, slow_inputs=False):
    g = np.random.default_rng(inputs_seed)
    st = step.zero_state(prec, 1, dv, dk)
    S64 = np.zeros((dv, dk))
    Sq_prev = np.zeros((dv, dk))
    Es, eps, As, scales = [], [], [], []
    k0, v0 = _unit(g, dk), g.standard_normal(dv).astype(F32)
    for t in range(T):
        if slow_inputs:    # slowly varying inputs: rounding errors line up under RTN
            k = (0.98 * k0 + 0.02 * _unit(g, dk)).astype(F32)
            k = (k / np.linalg.norm(k.astype(F64))).astype(F32)
            v = (v0 + 0.02 * g.standard_normal(dv)).astype(F32)
        else:
            k = _unit(g, dk)
            v = g.standard_normal(dv).astype(F32)
        q = _unit(g, dk)
        alpha = g.uniform(*alpha_range, dk if per_channel else 1).astype(F32)
        beta = F32(g.uniform(0.2, 1.5))
        a_in = alpha[None] if per_channel else alpha
        st, _ = step.decode_step(prec, st, q[None], k[None], v[None], a_in, np.array([beta]),
                                 delta, seed, t + 1, [0], [0], rounding=rounding)
        Sq = step.dequant(prec, st)[0].astype(F64)
        A = step.transition64(k, alpha if per_channel else alpha[0], beta, delta)
        Bw = float(beta) * np.outer(v.astype(F64), k.astype(F64))
        S64 = S64 @ A + Bw
        e = Sq - (Sq_prev @ A + Bw)
        Es.append(Sq - S64)
        eps.append(e)
        As.append(A)
        if prec in step.QMAX:
            scales.append(st["scales"][0].astype(F64))
        Sq_prev = Sq
    return Es, eps, As, scales


@pytest.mark.parametrize("prec,delta,per_channel", [(step.PREC_INT8, 1, False),
                                                    (step.PREC_INT4, 1, False),
                                                    (step.PREC_INT8, 0, True),
                                                    (step.PREC_BF16, 1, True)])
def test_error_propagation_identity_and_local_error(prec, delta, per_channel):
    Es, eps, As, scales = _trajectory(prec, 40, 16, 32, delta, seed=3, per_channel=per_channel)
    E_prev = np.zeros_like(Es[0])
    for t in range(len(Es)):
        pred = E_prev @ As[t] + eps[t]
        assert np.abs(pred - Es[t]).max() <= 1e-10 * max(1.0, np.abs(Es[t]).max())
        if scales:
            # one requantization moves an element by at most one code step (plus fp32 slop)
            bound = scales[t][:, None] * 1.001 + 1e-6 * np.abs(Es[t]).max()
            assert np.all(np.abs(eps[t]) <= bound + 1e-12)
        E_prev = Es[t]


@pytest.mark.parametrize("prec", [step.PREC_INT8, step.PREC_INT4])
def test_proposition2_decaying_error_bound(prec):
    Es, eps, As, _ = _trajectory(prec, 60, 16, 32, 1, seed=4, alpha_range=(0.5, 0.9))
    for t in range(len(Es)):
        bound = 0.0
        for tau in range(t + 1):
            rho = 1.0
            for j in range(tau + 1, t + 1):
                rho *= np.linalg.norm(As[j], 2)       # <= max alpha_j for beta|k|^2 in [0,2]
            bound += rho * np.linalg.norm(eps[tau])
        assert np.linalg.norm(Es[t]) <= bound * (1 + 1e-9) + 1e-12
    # the pages' form: ||A_j||_2 <= max alpha_j, so alpha^(t - tau) bounds hold too
    for A in As:
        assert np.linalg.norm(A, 2) <= 0.9 * (1 + 1e-6)


def test_proposition3_identity_and_sr_cross_terms():
    T, dv, dk = 24, 8, 16
    cross_sr = []
    cross_rtn = None
    for seed in range(96):
        Es, eps, As, _ = _trajectory(step.PREC_INT8, T, dv, dk, 0, seed=seed,
                                     alpha_range=(0.9, 0.99), inputs_seed=1, slow_inputs=True)
        gam = [As[j][0, 0] for j in range(T)]            # scalar decay: A_j = alpha_j I
        # E_T = sum_tau gamma_{tau,T} eps_tau
        acc = np.zeros_like(Es[0])
        for tau in range(T):
            acc += np.prod(gam[tau + 1:]) * eps[tau]
        assert np.abs(acc - Es[-1]).max() <= 1e-10 * max(1.0, np.abs(Es[-1]).max())
        c = 0.0
        for tau in range(T):
            for s in range(tau + 1, T):
                c += np.prod(gam[tau + 1:]) * np.prod(gam[s + 1:]) * np.sum(eps[tau] * eps[s])
        cross_sr.append(2 * c)
    Es, eps, As, _ = _trajectory(step.PREC_INT8, T, dv, dk, 0, seed=0, rounding="rtn",
                                 alpha_range=(0.9, 0.99), inputs_seed=1, slow_inputs=True)
    gam = [As[j][0, 0] for j in range(T)]
    diag = sum(np.prod(gam[tau + 1:]) ** 2 * np.sum(eps[tau] ** 2) for tau in range(T))
    cross_rtn = float(np.sum(Es[-1] ** 2) - diag)
    cross_sr = np.array(cross_sr)
    m, se = cross_sr.mean(), cross_sr.std(ddof=1) / np.sqrt(cross_sr.size)
    # SR: cross terms vanish in expectation
    assert abs(m) < 5 * se, (m, se)
    # RTN on slowly varying inputs: errors line up step after step (a demonstration)
    assert cross_rtn > 5 * se, (cross_rtn, se)
