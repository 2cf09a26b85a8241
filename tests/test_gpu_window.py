"""GPU parity of windowed requantization (lores_state_alloc_window) against
the oracle's oracle.window, through the C ABI, and the windowed state's
contract: in-order steps, scalar decay, the buffer's dequantization, W = 1.

Tolerances: tests/parity.py (run_window_parity).  Every case prints its
name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import quantized_linear_recurrence_amd as lores
from oracle import step as ostep
from oracle import window as owin
from tests import layout_codec as lc
from tests.parity import head_precisions, log, random_unit_state, run_window_parity
from workloads import get_workload, make_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

C1 = get_workload("C1")
DEV = "cuda"


@pytest.mark.parametrize("prec", [2, 3, 4, 5])
@pytest.mark.parametrize("W,dk,dv,delta", [(2, 64, 64, 1), (4, 128, 100, 1), (3, 128, 128, 0),
                                           (3, 256, 100, 1), (4, 256, 33, 0), (3, 160, 100, 1),
                                           (4, 224, 70, 0),
                                           (5, 64, 200, 1), (3, 32, 70, 1), (4, 96, 128, 1)])
def test_each_scaled_class(prec, W, dk, dv, delta):
    w = C1.scaled(B=3, H=4, dk=dk, dv=dv, T=2 * W + 1, delta=delta)
    log(f"case: window W={W} prec={prec} B=3 H=4 dk={dk} dv={dv} delta={delta}, "
        f"{w.T} steps from a random state")
    s = run_window_parity(w, T=w.T, W=W, head_prec=[prec] * w.H)
    log(s.summary())
    s.check()


@pytest.mark.parametrize("prec", [2, 3, 4, 5])
@pytest.mark.parametrize("W,dk,dv,decay", [(4, 128, 100, "softplus_step"), (3, 256, 70, "softplus_step"),
                                           (4, 128, 100, "kda_channel"), (3, 224, 70, "kda_channel")])
def test_bf16_inputs(prec, W, dk, dv, decay):
    """Windows fed bf16 q, k and v (the window-end kernels with bf16 inputs)."""
    w = C1.scaled(B=3, H=4, dk=dk, dv=dv, T=2 * W + 1, decay=decay, in_bf16=True)
    log(f"case: window W={W} prec={prec} B=3 H=4 dk={dk} dv={dv} decay={decay}, bf16 inputs")
    s = run_window_parity(w, T=w.T, W=W, head_prec=[prec] * w.H)
    log(s.summary())
    s.check()


@pytest.mark.parametrize("prec,dk,dv", [(2, 128, 128), (3, 64, 1)])
def test_longest_window(prec, dk, dv):
    """W = LORES_MAX_WINDOW (15 buffered tokens replayed at the window end),
    and a single value row."""
    W = lores.LORES_MAX_WINDOW
    w = C1.scaled(B=2, H=2, dk=dk, dv=dv, T=W + 2, delta=1)
    log(f"case: window W={W} prec={prec} dk={dk} dv={dv}, {w.T} steps")
    s = run_window_parity(w, T=w.T, W=W, head_prec=[prec] * w.H)
    log(s.summary())
    s.check()


@pytest.mark.parametrize("prec", [2, 3, 4, 5])
@pytest.mark.parametrize("W,dk,dv", [(3, 64, 64), (4, 128, 100), (4, 64, 256), (3, 128, 180),
                                    (4, 32, 100), (3, 96, 200), (3, 256, 100), (4, 256, 200),
                                    (3, 192, 100), (4, 160, 70)])
def test_key_column_windows(prec, W, dk, dv):
    """Windows over key-column scales (the PACE combination): the window end
    takes the column maxima of the replayed state."""
    w = C1.scaled(B=3, H=4, dk=dk, dv=dv, T=2 * W + 1, delta=1)
    log(f"case: key-column window W={W} prec={prec} dk={dk} dv={dv}, {w.T} steps")
    s = run_window_parity(w, T=w.T, W=W, head_prec=[prec] * w.H, axis="key")
    log(s.summary())
    s.check()


def test_mixed_heads_from_zero_nearest():
    w = C1.scaled(B=2, H=4, dk=128, dv=128, T=9, delta=1)
    log("case: window W=4, heads int8/int4/int6/fp8 from S_0 = 0, nearest rounding")
    s = run_window_parity(w, T=w.T, W=4, head_prec=[2, 3, 4, 5], init="zero",
                          rounding="nearest")
    log(s.summary())
    s.check()


def test_unscaled_heads_step_every_token():
    """fp32 and bf16 heads of a windowed state step every token, exactly as
    in a plain state (their segments come first, so the bytes line up)."""
    w = C1.scaled(B=2, H=3, dk=64, dv=64, T=5)
    log("case: fp32 / bf16 heads of a windowed state match a plain state's")
    x = make_inputs(w, 2, DEV, T=w.T)
    a = lores.lores_state_alloc(w.B, w.H, w.dk, w.dv, [0, 1, 2], device=DEV)
    b = lores.lores_state_alloc(w.B, w.H, w.dk, w.dv, [0, 1, 2], device=DEV, window=4)
    for t in range(1, w.T + 1):
        xs = {k: v[t - 1] for k, v in x.items()}
        oa = lores.lores_decode_step(a, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], 1, 4, t)
        ob = lores.lores_decode_step(b, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], 1, 4, t)
        assert torch.equal(oa[:, :2], ob[:, :2])
    la, lb = lores.lores_state_layout(a), lores.lores_state_layout(b)
    for c in (0, 1):
        assert la["codes_offset"][c] == lb["codes_offset"][c]
        s0, n = la["codes_offset"][c], la["unit_code_bytes"][c] * w.B
        assert torch.equal(a.buf[s0:s0 + n], b.buf[s0:s0 + n])


def test_full_size_c2_window8():
    w = get_workload("C2")
    g = np.random.default_rng(3)
    idx = g.choice(w.B * w.H, size=16, replace=False)
    units = sorted((int(i // w.H), int(i % w.H)) for i in idx)
    log("case: window W=8 on the full C2 batch (bf16 inputs), 16 sampled units, 9 steps")
    s = run_window_parity(w, T=9, W=8, head_prec=[2] * w.H, units=units)
    log(s.summary())
    s.check()


@pytest.mark.parametrize("axis", ["value", "key"])
def test_full_size_c5_window4(axis):
    # the benchmarked windowed launch shape: the C5 batch, decay-assigned
    # int8 + int4 heads, three whole windows
    w = get_workload("C5")
    inputs = make_inputs(w, 0, DEV, T=12)
    head_prec = head_precisions(w, inputs)
    g = np.random.default_rng(5)
    idx = g.choice(w.B * w.H, size=64, replace=False)
    units = sorted((int(i // w.H), int(i % w.H)) for i in idx)
    log(f"case: window W=4 on the full C5 batch, {axis} scales, 64 sampled units, 12 steps")
    s = run_window_parity(w, T=12, W=4, head_prec=head_prec, units=units, inputs=inputs,
                          axis=axis)
    log(s.summary())
    s.check()


@pytest.mark.parametrize("prec", [2, 3, 4, 5])
@pytest.mark.parametrize("W,dk,dv,delta,axis", [(3, 64, 64, 1, "value"), (4, 128, 100, 1, "value"),
                                               (4, 128, 128, 0, "value"), (3, 128, 100, 1, "key"),
                                               (5, 64, 200, 1, "key"), (3, 96, 64, 1, "value"),
                                               (4, 32, 128, 1, "value"), (3, 96, 100, 1, "key"),
                                               (4, 32, 64, 0, "key"), (3, 256, 70, 1, "value"),
                                               (3, 256, 100, 1, "key"), (3, 224, 70, 1, "key"),
                                               (4, 160, 100, 1, "value"), (3, 224, 70, 1, "value"),
                                               (4, 192, 100, 0, "value")])
def test_channel_decay_windows(prec, W, dk, dv, delta, axis):
    """Windows whose tokens carry one decay per key channel (the diagonal
    decay of the recurrence): the in-window readouts from the stored state
    and the buffer, the buffered (g, k, alpha), and the window end's replay
    and requantization."""
    w = C1.scaled(B=3, H=4, dk=dk, dv=dv, T=2 * W + 1, delta=delta, decay="kda_channel")
    log(f"case: channel-decay window W={W} prec={prec} dk={dk} dv={dv} delta={delta} "
        f"{axis} scales, {w.T} steps")
    s = run_window_parity(w, T=w.T, W=W, head_prec=[prec] * w.H, axis=axis)
    log(s.summary())
    s.check()


def test_full_size_c4_window4():
    # the KDA-style workload (per-channel decay, 8 bf16 + 24 int8 heads): its
    # int8 heads windowed, its bf16 heads stepping every token
    w = get_workload("C4")
    inputs = make_inputs(w, 0, DEV, T=8)
    head_prec = head_precisions(w, inputs)
    g = np.random.default_rng(6)
    scaled = [h for h in range(w.H) if head_prec[h] == 2]   # the windowed heads
    units = sorted({(int(g.integers(w.B)), int(g.choice(scaled))) for _ in range(64)})
    log(f"case: window W=4 on the full C4 batch (per-channel decay), {len(units)} sampled "
        "int8 units, 8 steps")
    s = run_window_parity(w, T=8, W=4, head_prec=head_prec, units=units, inputs=inputs)
    log(s.summary())
    s.check()


def test_window_one_is_the_plain_state():
    w = C1.scaled(B=2, H=4, dk=128, dv=96, T=4)
    log("case: lores_state_alloc_window(W = 1) steps like lores_state_alloc")
    x = make_inputs(w, 0, DEV, T=w.T)
    a = lores.lores_state_alloc(w.B, w.H, w.dk, w.dv, [2, 3, 4, 5], device=DEV)
    b = lores.lores_state_alloc(w.B, w.H, w.dk, w.dv, [2, 3, 4, 5], device=DEV, window=1)
    for t in range(1, w.T + 1):
        xs = {k: v[t - 1] for k, v in x.items()}
        oa = lores.lores_decode_step(a, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], 1, 4, t)
        ob = lores.lores_decode_step(b, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], 1, 4, t)
        assert torch.equal(oa, ob)
    assert torch.equal(a.buf, b.buf)


@pytest.mark.parametrize("prec", [2, 3, 4, 5])
@pytest.mark.parametrize("axis,decay", [("value", "softplus_step"), ("key", "softplus_step"),
                                        ("value", "kda_channel"), ("key", "kda_channel")])
@pytest.mark.parametrize("dk", [128, 96, 256, 160, 224])
def test_dequant_replays_the_buffer(prec, axis, decay, dk):
    """Inside a window lores_dequant_state returns the current state: the
    stored state followed by the buffered tokens' fp32 recurrence, bit for
    bit against the oracle's replay of the same (oracle-written) buffer, for
    scalar and per-channel decays."""
    W, B, H, dv, n = 6, 2, 3, 72, 3
    pc = decay == "kda_channel"
    w = C1.scaled(B=B, H=H, dk=dk, dv=dv, T=n, decay=decay)
    log(f"case: window dequant after {n} buffered tokens, prec={prec} axis={axis} decay={decay} "
        f"dk={dk}")
    st = lores.lores_state_alloc(B, H, dk, dv, [prec] * H, device=DEV, window=W,
                                 scale_axis=lores.LORES_SCALE_KEY if axis == "key" else 0)
    x = make_inputs(w, 1, DEV, T=n)
    for t in range(1, n + 1):           # the handle now counts n buffered tokens
        xs = {k: v[t - 1] for k, v in x.items()}
        lores.lores_decode_step(st, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], 1, 0, t)
    torch.cuda.synchronize()
    lay = lores.lores_state_layout(st)
    assert lay["window_fill"] == n
    _, slot = lores.lores_state_head_map(st)
    g = np.random.default_rng(prec)
    host = st.buf.cpu().numpy()
    want = np.zeros((B, H, dv, dk), np.float32)
    for b in range(B):
        for h in range(H):
            s = random_unit_state(prec, dv, dk, g, axis)
            win = {"g": g.standard_normal((W - 1, dv)).astype(np.float32),
                   "k": (g.standard_normal((W - 1, dk)) / np.sqrt(dk)).astype(np.float32),
                   "alpha": g.uniform(0.8, 1.0, (W - 1, dk)).astype(np.float32)}
            u = b * lay["n_class"][prec] + slot[h]
            lc.write_unit(host, lay, prec, u, s)
            lc.write_window(host, lay, prec, u, win)
            want[b, h] = owin.replay(prec, {k: v[None] for k, v in s.items()},
                                     {k: v[None] for k, v in win.items()}, n, axis, pc)[0]
    st.buf.copy_(torch.from_numpy(host))
    got = lores.lores_dequant_state(st).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_windowed_state_contract():
    log("case: windowed state errors: the decay kind inside a window, out-of-order t, "
        "quant_state resets")
    w = C1.scaled(B=2, H=2, dk=64, dv=64, T=3)
    x = make_inputs(w, 0, DEV, T=3)
    st = lores.lores_state_alloc(2, 2, 64, 64, [2, 3], device=DEV, window=4)
    xs = {k: v[0] for k, v in x.items()}
    pc = torch.full((2, 2, 64), 0.9, device=DEV)
    with pytest.raises(lores.LoresError, match="EINVAL"):
        lores.lores_decode_step(st, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], 1, 0, 2)
    lores.lores_decode_step(st, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], 1, 0, 1)
    assert lores.lores_state_layout(st)["window_fill"] == 1
    # the window's tokens share one kind of decay
    with pytest.raises(lores.LoresError, match="EINVAL"):
        lores.lores_decode_step(st, xs["q"], xs["k"], xs["v"], pc, xs["beta"], 1, 0, 2)
    assert lores.lores_state_layout(st)["window_fill"] == 1
    X = torch.zeros(2, 2, 64, 64, device=DEV)
    lores.lores_quant_state(st, X, 0)
    assert lores.lores_state_layout(st)["window_fill"] == 0
    with pytest.raises(lores.LoresError, match="EINVAL"):
        lores.lores_decode_step(st, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], 1, 0, 2)
    lores.lores_decode_step(st, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], 1, 0, 5)
    torch.cuda.synchronize()


@pytest.mark.parametrize("axis", ["value", "key"])
def test_shard_invariance_of_windowed_states(axis):
    """Sequence and head shards of a windowed state (seq_base / head_base key
    the rounding at window ends) reproduce the whole batch bit for bit: the
    readouts of every step and the current state after two windows and a
    half."""
    B, head_prec, dk, dv, W = 10, [2, 3, 4, 5], 128, 96, 4
    H = len(head_prec)
    w = C1.scaled(B=B, H=H, dk=dk, dv=dv, T=2 * W + 2)
    log(f"case: windowed shard invariance axis={axis} B={B} H={H} W={W}")
    sa = lores.LORES_SCALE_KEY if axis == "key" else lores.LORES_SCALE_VALUE
    inp = make_inputs(w, 5, DEV)
    full = lores.lores_state_alloc(B, H, dk, dv, head_prec, device=DEV, window=W, scale_axis=sa)
    cuts = [(0, 4, 0, 2), (0, 4, 2, 4), (4, 10, 0, 4)]
    shards = [(b0, b1, h0, h1, lores.lores_state_alloc(b1 - b0, h1 - h0, dk, dv, head_prec[h0:h1],
                                                       device=DEV, window=W, scale_axis=sa))
              for b0, b1, h0, h1 in cuts]
    for t in range(1, w.T + 1):
        x = {k: v[t - 1] for k, v in inp.items()}
        o_full = lores.lores_decode_step(full, x["q"], x["k"], x["v"], x["alpha"], x["beta"], 1, 8, t)
        for b0, b1, h0, h1, st in shards:
            xs = {k: v[b0:b1, h0:h1].contiguous() for k, v in x.items()}
            o_s = lores.lores_decode_step(st, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], 1,
                                          8, t, seq_base=b0, head_base=h0)
            assert torch.equal(o_s, o_full[b0:b1, h0:h1]), (t, b0, h0)
    X = lores.lores_dequant_state(full)
    for b0, b1, h0, h1, st in shards:
        assert torch.equal(lores.lores_dequant_state(st), X[b0:b1, h0:h1])


@pytest.mark.parametrize("axis", ["value", "key"])
def test_windowed_graph_replays_match_eager(axis):
    """A captured graph of two whole windows replays the eager steps' bytes
    and readouts exactly, three times over, with eager work between."""
    B, head_prec, W = 48, [2, 3] * 4, 4
    w = C1.scaled(B=B, H=8, dk=128, dv=128, T=2 * W)
    log(f"case: windowed graph replays axis={axis} B={B} H=8 W={W}")
    sa = lores.LORES_SCALE_KEY if axis == "key" else lores.LORES_SCALE_VALUE
    inp = make_inputs(w, 6, DEV)
    st = lores.lores_state_alloc(B, 8, 128, 128, head_prec, device=DEV, window=W, scale_axis=sa)
    warm = {k: v[0] for k, v in inp.items()}
    for t in range(1, W + 1):           # a first window, so the stored state is not zero
        lores.lores_decode_step(st, warm["q"], warm["k"], warm["v"], warm["alpha"], warm["beta"],
                                1, 2, t)
    torch.cuda.synchronize()
    init = st.buf.clone()
    outs = [torch.empty((B, 8, 128), dtype=torch.float32, device=DEV) for _ in range(w.T)]

    def steps():
        for t in range(1, w.T + 1):
            x = {k: v[t - 1] for k, v in inp.items()}
            lores.lores_decode_step(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], 1, 3,
                                    W + t, o=outs[t - 1])

    steps()
    torch.cuda.synchronize()
    ref_buf, ref_o = st.buf.clone(), [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    st.buf.copy_(init)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        steps()
    torch.cuda.synchronize()
    for rep in range(3):
        st.buf.copy_(init)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.buf, ref_buf), rep
        assert all(torch.equal(a, b) for a, b in zip(outs, ref_o)), rep
