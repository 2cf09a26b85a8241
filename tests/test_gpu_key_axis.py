"""GPU parity of the key-column scale grouping (LORES_SCALE_KEY) against the
oracle's axis="key", through the C ABI.

Key-column scales make the requantization of a unit depend on all of its d_v
rows, so the cases cover one, two and four row blocks per unit (d_v = 64,
100, 200, 256), ragged row blocks, both d_k built (64, 128), every scaled
class with fp32 / bf16 heads beside them, per-channel decay, bf16 inputs,
nearest rounding, the quantize / dequantize entries, and full-size batches in
the launch shape the bench times.  Tolerances: tests/parity.py.
Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import quantized_linear_recurrence_amd as lores
from oracle import step as ostep
from tests import layout_codec as lc
from tests.parity import log, run_parity
from workloads import get_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

C1 = get_workload("C1")
DEV = "cuda"


def _sample_units(B, H, n, seed=0):
    g = np.random.default_rng(seed)
    idx = g.choice(B * H, size=min(n, B * H), replace=False)
    return sorted((int(i // H), int(i % H)) for i in idx)


@pytest.mark.parametrize("prec", [2, 3, 4, 5])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 100), (64, 256), (128, 200), (128, 150),
                                   (64, 192), (32, 64), (96, 100), (32, 200), (96, 150),
                                   (256, 100), (256, 256), (256, 33), (256, 160), (160, 100),
                                   (192, 70), (224, 256)])
def test_each_scaled_class(prec, dk, dv):
    w = C1.scaled(B=3, H=4, dk=dk, dv=dv, T=4, delta=1)
    log(f"case: key columns prec={prec} B=3 H=4 dk={dk} dv={dv} delta=1, random initial state")
    s = run_parity(w, T=w.T, head_prec=[prec] * w.H, init="random", axis="key")
    log(s.summary())
    s.check()


@pytest.mark.parametrize("delta", [0, 1])
@pytest.mark.parametrize("decay", ["softplus_step", "kda_channel"])
@pytest.mark.parametrize("dk", [128, 256, 160])
def test_mixed_heads_from_zero(delta, decay, dk):
    w = C1.scaled(B=2, H=6, dk=dk, dv=128, T=10, delta=delta, decay=decay)
    log(f"case: key columns, heads fp32/bf16/int8/int4/int6/fp8, from S_0 = 0, delta={delta} "
        f"decay={decay} dk={dk}")
    s = run_parity(w, T=w.T, head_prec=[0, 1, 2, 3, 4, 5], init="zero", axis="key")
    log(s.summary())
    s.check()


def test_bf16_inputs_nearest_rounding():
    w = C1.scaled(B=3, H=4, dk=64, dv=72, T=5, in_bf16=True, decay="kda_channel")
    log("case: key columns, bf16 q/k/v, per-channel decay, nearest rounding, dv=72")
    s = run_parity(w, T=w.T, head_prec=[2, 3, 4, 5], init="random", axis="key",
                   rounding="nearest")
    log(s.summary())
    s.check()


def test_c1_all_steps_int8_key():
    log("case: C1 tiny gated delta rule, int8 key columns, all 128 steps")
    s = run_parity(C1, T=C1.T, axis="key")
    log(s.summary())
    s.check()


@pytest.mark.parametrize("name", ["C2", "C5"])
def test_full_size_sampled(name):
    w = get_workload(name)
    log(f"case: key columns, {name} full batch B={w.B} H={w.H}, 64 sampled units, 8 steps")
    s = run_parity(w, T=8, units=_sample_units(w.B, w.H, 64, seed=11), init="random", axis="key")
    log(s.summary())
    s.check()


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 200), (64, 1), (128, 160), (32, 70),
                                   (96, 256), (256, 100), (256, 256), (224, 100), (160, 33)])
def test_quant_and_dequant_match_oracle(dk, dv):
    """lores_quant_state with key columns equals the oracle bit for bit (the
    column maxima span every row block of a unit), and lores_dequant_state
    reads it back as the oracle's s_j * c_ij."""
    B, head_prec = 3, [0, 2, 3, 4, 5, 1]
    H = len(head_prec)
    log(f"case: key columns quant/dequant B={B} dk={dk} dv={dv} precisions {head_prec}")
    g = np.random.default_rng(dk + dv)
    X = (g.standard_normal((B, H, dv, dk)) * np.exp(g.uniform(-5, 5, (B, H, 1, dk)))).astype(np.float32)
    X[0, :, :, 3] = 0.0                                    # a zero column
    st = lores.lores_state_alloc(B, H, dk, dv, head_prec, device=DEV,
                                 scale_axis=lores.LORES_SCALE_KEY)
    lay = lores.lores_state_layout(st)
    assert lay["scale_axis"] == 1 and lay["unit_scales"] == dk
    seed, sb, hb = 5, 2, 3
    lores.lores_quant_state(st, torch.from_numpy(X).to(DEV), seed, seq_base=sb, head_base=hb)
    torch.cuda.synchronize()
    _, slot = lores.lores_state_head_map(st)
    buf = st.buf.cpu().numpy()
    out = lores.lores_dequant_state(st).cpu().numpy()
    for h, c in enumerate(head_prec):
        want = ostep.quant_state(c, X[:, h], seed, np.arange(B) + sb, np.full(B, h + hb), axis="key")
        for b in range(B):
            got = lc.read_unit(buf, lay, c, b * lay["n_class"][c] + slot[h])
            for key, val in got.items():
                assert np.array_equal(np.asarray(val).view(np.uint8),
                                      np.ascontiguousarray(want[key][b]).astype(val.dtype).view(np.uint8)), \
                    (b, h, key)
        Xq = ostep.dequant(c, want, axis="key")
        assert np.array_equal(out[:, h].view(np.uint32), Xq.view(np.uint32)), h


def test_key_and_value_states_differ_and_launch_per_class():
    """The same inputs through a value-row and a key-column state give
    different codes; a key-column state with int8 and int4 heads runs one
    launch per class."""
    w = C1.scaled(B=2, H=2, dk=128, dv=128, T=1)
    log("case: key vs value grouping on the same inputs, launch count")
    sv = lores.lores_state_alloc(2, 2, 128, 128, [2, 3], device=DEV)
    sk = lores.lores_state_alloc(2, 2, 128, 128, [2, 3], device=DEV, scale_axis=lores.LORES_SCALE_KEY)
    assert lores.lores_step_launches(sv) == 1 and lores.lores_step_launches(sk) == 2
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    q = torch.nn.functional.normalize(torch.randn(2, 2, 128, device=DEV, generator=g), dim=-1)
    k = torch.nn.functional.normalize(torch.randn(2, 2, 128, device=DEV, generator=g), dim=-1)
    v = torch.randn(2, 2, 128, device=DEV, generator=g)
    a = torch.full((2, 2), 0.9, device=DEV)
    b = torch.full((2, 2), 0.5, device=DEV)
    for st in (sv, sk):
        for t in (1, 2, 3):
            lores.lores_decode_step(st, q, k, v, a, b, 1, 0, t)
    torch.cuda.synchronize()
    Xv = lores.lores_dequant_state(sv)
    Xk = lores.lores_dequant_state(sk)
    assert not torch.equal(Xv, Xk)
    # both are within a few codes of each other (same recurrence)
    assert (Xv - Xk).abs().max().item() < 0.2 * Xv.abs().max().item()
