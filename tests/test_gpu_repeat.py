"""Run-to-run identity of full-size launches.

The step is deterministic: the same state and inputs give the same bytes.  A
dependence the hardware does not interlock (a missing wait state between two
instructions) shows as a few lanes of a few launches differing from the other
launches, at a rate the sampled-unit parity tests catch only by chance.  Each
case repeats one full-size launch many times from the same state and requires
every byte of the state and every readout to equal those of the first repeat,
over all units.
"""
import pytest
import torch

import quantized_linear_recurrence_amd as lores
from tests.parity import head_precisions, log
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu

# (workload, scale axis, repeats): every launch kind of the benchmarked shapes
# (single class with bf16 inputs, single class, bf16 + int8 side by side, the
# fused int8 + int4 pair with its work queue, key-column scales)
CASES = [("C2", "value", 60), ("C3", "value", 40), ("C4", "value", 60), ("C5", "value", 16),
         ("C5", "key", 16)]


@pytest.mark.parametrize("key,axis,reps", CASES)
def test_full_launch_repeats(key, axis, reps):
    w = get_workload(key)
    log(f"case: {key} ({axis} scales) B={w.B} H={w.H}, one step repeated {reps} times")
    inputs = make_inputs(w, 0, "cuda", T=2, B=w.B)
    hp = head_precisions(w, inputs)
    st = lores.lores_state_alloc(w.B, w.H, w.dk, w.dv, hp, device="cuda",
                                 scale_axis=lores.LORES_SCALE_KEY if axis == "key"
                                 else lores.LORES_SCALE_VALUE)
    x = [{k: v[i] for k, v in inputs.items()} for i in range(2)]
    # a first step from S_0 = 0 gives every unit content
    lores.lores_decode_step(st, x[0]["q"], x[0]["k"], x[0]["v"], x[0]["alpha"], x[0]["beta"],
                            w.delta, 7, 1)
    start = st.buf.clone()
    ref_state = ref_o = None
    bad = []
    for r in range(reps):
        st.buf.copy_(start)
        o = lores.lores_decode_step(st, x[1]["q"], x[1]["k"], x[1]["v"], x[1]["alpha"],
                                    x[1]["beta"], w.delta, 7, 2)
        if r == 0:
            ref_state, ref_o = st.buf.clone(), o.clone()
            continue
        if not (torch.equal(st.buf, ref_state) and torch.equal(o, ref_o)):
            bad.append((r, int((st.buf != ref_state).sum()), int((o != ref_o).sum())))
    torch.cuda.synchronize()
    assert not torch.equal(ref_state, start), "the step left the state unchanged"
    log(f"{reps} repeats, {len(bad)} differing (repeat, state bytes, readouts): {bad[:8]}")
    assert not bad
