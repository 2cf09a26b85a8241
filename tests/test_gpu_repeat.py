"""Run-to-run identity of full-size launches.

The step is deterministic: the same state and inputs give the same bytes.  A
dependence the hardware does not interlock (a missing wait state between two
instructions) shows as a few lanes of a few launches differing from the other
launches, at a rate the sampled-unit parity tests catch only by chance.  Each
case runs the first steps of a full-size state many times from S_0 = 0 and
requires every byte of the state and every readout of the last step to equal
those of the first run, over all units.
"""
import pytest
import torch

import quantized_linear_recurrence_amd as lores
from tests.parity import head_precisions, log
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu

# (workload, scale axis, window, steps per run, runs): every launch kind of
# the benchmarked shapes (single class with bf16 inputs, single class, bf16 +
# int8 side by side, the fused int8 + int4 and int6 + int4 pairs with their
# work queue, key-column scales, and windowed states inside a window and at
# its end)
CASES = [("C2", "value", 1, 2, 60), ("C3", "value", 1, 2, 40), ("C4", "value", 1, 2, 60),
         ("C5", "value", 1, 2, 16), ("C5", "key", 1, 2, 16), ("C5i6", "value", 1, 2, 16),
         ("C5", "value", 4, 2, 16), ("C5", "value", 4, 4, 16), ("C5", "key", 4, 4, 8)]


@pytest.mark.parametrize("key,axis,window,t_rep,reps", CASES)
def test_full_launch_repeats(key, axis, window, t_rep, reps):
    w = get_workload(key)
    log(f"case: {key} ({axis} scales, window {window}) B={w.B} H={w.H}, steps 1..{t_rep} "
        f"repeated {reps} times")
    inputs = make_inputs(w, 0, "cuda", T=t_rep, B=w.B)
    hp = head_precisions(w, inputs)
    x = [{k: v[i] for k, v in inputs.items()} for i in range(t_rep)]
    ref_state = ref_o = None
    bad = []
    for r in range(reps):
        # a fresh state (S_0 = 0; a windowed state's token count at zero) and
        # steps 1 .. t_rep, the last one compared
        st = lores.lores_state_alloc(w.B, w.H, w.dk, w.dv, hp, device="cuda",
                                     scale_axis=lores.LORES_SCALE_KEY if axis == "key"
                                     else lores.LORES_SCALE_VALUE, window=window)
        for t in range(1, t_rep + 1):
            xi = x[t - 1]
            o = lores.lores_decode_step(st, xi["q"], xi["k"], xi["v"], xi["alpha"], xi["beta"],
                                        w.delta, 7, t)
        if r == 0:
            ref_state, ref_o = st.buf.clone(), o.clone()
            assert bool(ref_state.any()), "the steps left the state at zero"
        elif not (torch.equal(st.buf, ref_state) and torch.equal(o, ref_o)):
            bad.append((r, int((st.buf != ref_state).sum()), int((o != ref_o).sum())))
        del st
    torch.cuda.synchronize()
    log(f"{reps} repeats, {len(bad)} differing (repeat, state bytes, readouts): {bad[:8]}")
    assert not bad
