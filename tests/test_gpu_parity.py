"""GPU parity of the HIP decode step against the CPU oracle (through the C ABI).

Every case prints its name before touching the GPU.  See tests/parity.py for
the protocol and the tolerances.
"""
import numpy as np
import pytest
import torch

import quantized_linear_recurrence_amd as lores
from tests.parity import log, run_free_fp32, run_parity
from workloads import get_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

C1 = get_workload("C1")


def _sample_units(B, H, n, seed=0):
    g = np.random.default_rng(seed)
    idx = g.choice(B * H, size=min(n, B * H), replace=False)
    return sorted((int(i // H), int(i % H)) for i in idx)


def test_c1_all_steps_int8():
    log("case: C1 tiny gated delta rule, int8, all 128 steps, all units")
    s = run_parity(C1, T=C1.T)
    log(s.summary())
    s.check()


@pytest.mark.parametrize("prec", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("delta", [0, 1])
def test_small_each_precision(prec, delta):
    w = C1.scaled(B=2, H=3, T=12, delta=delta)
    log(f"case: small B=2 H=3 d=64 prec={prec} delta={delta}, random initial state")
    s = run_parity(w, T=w.T, head_prec=[prec] * w.H, init="random")
    log(s.summary())
    s.check()


@pytest.mark.parametrize("dk,dv", [(96, 100), (32, 1), (128, 65), (64, 128), (256, 100),
                                   (256, 33), (160, 70), (192, 100), (224, 33)])
@pytest.mark.parametrize("decay", ["softplus_step", "kda_channel"])
def test_ragged_mixed_precisions(dk, dv, decay):
    w = C1.scaled(B=3, H=6, dk=dk, dv=dv, T=5, decay=decay)
    log(f"case: ragged mixed B=3 H=6 dk={dk} dv={dv} decay={decay} "
        "heads fp32/bf16/int8/int4/int6/fp8")
    s = run_parity(w, T=w.T, head_prec=[0, 1, 2, 3, 4, 5], init="random")
    log(s.summary())
    s.check()


@pytest.mark.parametrize("prec", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("delta", [0, 1])
@pytest.mark.parametrize("dk", [256, 160, 224])
def test_split_rows_each_precision(prec, delta, dk):
    """d_k > 128: each row split across a lane pair (r, o and the row maximum
    combined across the pair, the second lane's draws from column d_k / 2;
    at 160 and 224 the int4 and int6 half rows end inside a chunk)."""
    w = C1.scaled(B=2, H=3, dk=dk, dv=70, T=8, delta=delta)
    log(f"case: split rows B=2 H=3 d_k={dk} d_v=70 prec={prec} delta={delta}, random initial state")
    s = run_parity(w, T=w.T, head_prec=[prec] * w.H, init="random")
    log(s.summary())
    s.check()


@pytest.mark.parametrize("mix", [[2, 3, 2, 2, 3], [3, 4, 4, 3, 3], [1, 2, 2, 1, 2],
                                 [3, 1, 3, 3, 1]])
@pytest.mark.parametrize("decay", ["softplus_step", "kda_channel"])
@pytest.mark.parametrize("dk", [256, 160, 192, 224])
def test_split_rows_fused_pairs(mix, decay, dk):
    """d_k > 128 with two classes in one launch: int8 + int4 and int4 + int6
    through the pair work queue (unequal class sizes, so the unpaired rest of
    one class runs after the pairs), bf16 + int8 and bf16 + int4 side by
    side; d_v = 70 gives three 32-row tasks per unit, the last one ragged."""
    w = C1.scaled(B=3, H=len(mix), dk=dk, dv=70, T=6, decay=decay)
    log(f"case: split-row pair B=3 H={w.H} d_k={dk} d_v=70 heads {mix} decay={decay}")
    st = lores.lores_state_alloc(w.B, w.H, dk, w.dv, mix, device=torch.device("cuda:0"))
    assert lores.lores_step_launches(st) == 1
    s = run_parity(w, T=w.T, head_prec=mix, init="random")
    log(s.summary())
    s.check()


def test_split_rows_sampled_batch():
    """d_k = 256 at a large batch (int8 + int4 in one fused launch), sampled units."""
    w = get_workload("C5").scaled(B=256, dk=256, T=8)
    units = _sample_units(w.B, w.H, 48, seed=256)
    log(f"case: split rows B={w.B} H={w.H} d_k=256 d_v=128 int8 + int4, {len(units)} units, "
        f"{w.T} steps")
    s = run_parity(w, T=w.T, units=units)
    log(s.summary())
    s.check()


@pytest.mark.parametrize("delta", [0, 1])
def test_nearest_rounding_each_precision(delta):
    w = C1.scaled(B=3, H=6, dk=128, dv=80, T=6, delta=delta, decay="kda_channel")
    log(f"case: round-to-nearest mode B=3 H=6 d_k=128 d_v=80 delta={delta}, "
        "heads fp32/bf16/int8/int4/int6/fp8")
    s = run_parity(w, T=w.T, head_prec=[0, 1, 2, 3, 4, 5], init="random", rounding="nearest")
    log(s.summary())
    s.check()


def test_nearest_rounding_fused_pair_full_size():
    w = get_workload("C5")
    log("case: round-to-nearest mode, C5 full batch (fused int8 + int4), 32 sampled units, 2 steps")
    s = run_parity(w, T=2, units=_sample_units(w.B, w.H, 32, seed=5), init="random",
                   rounding="nearest")
    log(s.summary())
    s.check()


@pytest.mark.parametrize("B,n8,n4,dv", [
    (300, 7, 4, 128),     # paired tasks plus an int8 remainder; several sequence strides per group
    (300, 3, 9, 100),     # an int4 remainder, ragged row blocks
    (5, 5, 5, 64),        # pairs only, one sequence per group
])
def test_fused_pair_work_queue(B, n8, n4, dv):
    # heads interleaved, so each class's head list is not contiguous
    prec = ([2, 3] * max(n8, n4))
    head_prec, c8, c4 = [], 0, 0
    for p in prec:
        if (p == 2 and c8 < n8) or (p == 3 and c4 < n4):
            head_prec.append(p)
            c8 += p == 2
            c4 += p == 3
    w = C1.scaled(B=B, H=n8 + n4, dk=128, dv=dv, T=3)
    log(f"case: fused int8 + int4 work queue B={B} int8 heads {n8} int4 heads {n4} d_v={dv}")
    units = None
    if B * w.H > 200:
        units = _sample_units(B, w.H, 64, seed=B + n8)
        units = sorted(set(units + [(0, 0), (B - 1, w.H - 1), (B - 1, 0), (0, w.H - 1)]))
    s = run_parity(w, T=w.T, units=units, head_prec=head_prec, init="random")
    log(s.summary())
    s.check()


def test_bf16_inputs_small():
    w = C1.scaled(B=2, H=4, T=8, in_bf16=True)
    log("case: bf16 q/k/v inputs, mixed precisions")
    s = run_parity(w, T=w.T, head_prec=[2, 3, 1, 0], init="random")
    log(s.summary())
    s.check()


@pytest.mark.parametrize("key,T,n_units", [("C2", 16, 64), ("C3", 16, 64), ("C4", 16, 64),
                                           ("C5", 64, 64), ("C5i6", 16, 64)])
def test_full_size_sampled_units(key, T, n_units):
    w = get_workload(key)
    log(f"case: {key} full batch B={w.B} H={w.H} d_v={w.dv} d_k={w.dk}, {n_units} sampled units, "
        f"{T} steps")
    s = run_parity(w, T=T, units=_sample_units(w.B, w.H, n_units), init="random")
    log(s.summary())
    s.check()


@pytest.mark.parametrize("seed", get_workload("C5").seeds)
def test_c5_seed_sweep(seed):
    w = get_workload("C5")
    log(f"case: C5 seed {seed}, 64 sampled units, all {w.T} steps")
    s = run_parity(w, T=w.T, units=_sample_units(w.B, w.H, 64, seed=seed), seed=seed,
                   init="random")
    log(s.summary())
    s.check()


@pytest.mark.parametrize("delta,decay,dk", [(1, "softplus_step", 64), (0, "softplus_step", 64),
                                            (1, "kda_channel", 64), (1, "kda_channel", 256)])
def test_fp32_path_free_running(delta, decay, dk):
    w = C1.scaled(B=2, H=2, dk=dk, T=128, delta=delta, decay=decay)
    log(f"case: fp32 heads free-running 128 steps delta={delta} decay={decay} d_k={dk}")
    worst, worst_scale = run_free_fp32(w, T=w.T)
    log(f"worst o error / largest readout = {worst:.2e} (over the readout scale {worst_scale:.2e})")
    assert worst <= 1e-5


@pytest.mark.parametrize("B,H,dk,dv,prec", [
    (65535, 1, 128, 64, [2]),                                  # the largest batch (grid y limit)
    (3, 512, 128, 256, [0, 1, 2, 3, 4] * 102 + [2, 3]),        # the most heads, the tallest state
    (3, 512, 256, 256, [0, 1, 2, 3, 4, 5] * 85 + [2, 3]),      # and the widest
])
def test_maximum_sizes(B, H, dk, dv, prec):
    w = C1.scaled(B=B, H=H, dk=dk, dv=dv, T=2)
    log(f"case: maximum sizes B={B} H={H} d_v={dv} d_k={dk}, sampled units")
    units = _sample_units(B, H, 40, seed=B + H)
    units += [(B - 1, H - 1), (0, 0), (B - 1, 0), (0, H - 1)]
    s = run_parity(w, T=w.T, units=sorted(set(units)), head_prec=prec, init="random")
    log(s.summary())
    s.check()
