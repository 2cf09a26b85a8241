"""GPU tests of the C-ABI contract beyond step parity: launch grouping, shard
invariance of the rounding keys, repeatability (eager and graph replays),
dequantization of a packed state, error paths on a live handle, and states at
the ends of the fp32 range.

Every case prints its name before touching the GPU.
"""
import ctypes

import numpy as np
import pytest
import torch

import quantized_linear_recurrence_amd as lores
from oracle import step as ostep
from quantized_linear_recurrence_amd import _lib
from tests import layout_codec as lc
from tests.parity import log, random_unit_state, run_parity
from workloads import get_workload, make_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

C1 = get_workload("C1")
DEV = "cuda"


def _install(st, states):
    """Write {(b, h): unit state} into the device buffer of `st` through the codec."""
    lay = lores.lores_state_layout(st)
    _, slot = lores.lores_state_head_map(st)
    buf = st.buf.cpu().numpy().copy()
    for (b, h), s in states.items():
        c = st.head_prec[h]
        lc.write_unit(buf, lay, c, b * lay["n_class"][c] + slot[h], s)
    st.buf.copy_(torch.from_numpy(buf))


def _random_states(B, head_prec, dv, dk, seed):
    g = np.random.default_rng(seed)
    return {(b, h): random_unit_state(c, dv, dk, g)
            for b in range(B) for h, c in enumerate(head_prec)}


def _unit_bytes(st, buf_host, b, h):
    """Raw code bytes and scales of one unit (bytes, for bit comparisons)."""
    lay = lores.lores_state_layout(st)
    _, slot = lores.lores_state_head_map(st)
    c = st.head_prec[h]
    cs, cl, ss, sl = lc.unit_ranges(lay, c, b * lay["n_class"][c] + slot[h])
    out = [buf_host[cs:cs + cl]]
    if ss is not None:
        out.append(buf_host[ss:ss + sl])
    return np.concatenate(out)


@pytest.mark.parametrize("prec,n", [([2, 2], 1), ([0], 1), ([2, 3], 1), ([1, 2], 1),
                                    ([3, 1], 1), ([0, 2], 2), ([0, 1], 2), ([1, 2, 3], 3),
                                    ([0, 1, 2, 3], 4), ([4], 1), ([4, 3], 1), ([2, 4], 2),
                                    ([0, 1, 2, 3, 4], 5), ([5], 1), ([5, 2], 2)])
def test_step_launches(prec, n):
    log(f"case: launches per step for precisions {prec}")
    st = lores.lores_state_alloc(2, len(prec), 64, 64, prec, device=DEV)
    assert lores.lores_step_launches(st) == n


@pytest.mark.parametrize("B,head_prec,dk,dv,seq_cuts,head_cuts", [
    (6, [0, 1, 2, 3, 2, 3], 128, 96, [0, 2, 6], [0, 3, 6]),
    (160, [2, 3] * 4, 128, 128, [0, 40, 160], [0, 4, 8]),
    (9, [1, 2, 1, 2], 64, 33, [0, 1, 9], [0, 1, 4]),
    (130, [4, 3] * 4, 128, 96, [0, 66, 130], [0, 2, 8]),
])
def test_shard_invariance(B, head_prec, dk, dv, seq_cuts, head_cuts):
    """A shard of sequences and heads, keyed with seq_base / head_base, gives
    the unsharded result bit for bit (state bytes and o); the shards also run
    in other launch shapes than the whole batch."""
    H = len(head_prec)
    w = C1.scaled(B=B, H=H, dk=dk, dv=dv, T=3)
    log(f"case: shard invariance B={B} H={H} dk={dk} dv={dv} precisions {head_prec} "
        f"seq cuts {seq_cuts} head cuts {head_cuts}")
    inp = make_inputs(w, 3, DEV)
    init = _random_states(B, head_prec, dv, dk, seed=11)
    full = lores.lores_state_alloc(B, H, dk, dv, head_prec, device=DEV)
    _install(full, init)
    shards = []
    for b0, b1 in zip(seq_cuts[:-1], seq_cuts[1:]):
        for h0, h1 in zip(head_cuts[:-1], head_cuts[1:]):
            st = lores.lores_state_alloc(b1 - b0, h1 - h0, dk, dv, head_prec[h0:h1], device=DEV)
            _install(st, {(b - b0, h - h0): init[(b, h)]
                          for b in range(b0, b1) for h in range(h0, h1)})
            shards.append((b0, b1, h0, h1, st))
    for t in range(1, w.T + 1):
        x = {k: v[t - 1] for k, v in inp.items()}
        o_full = lores.lores_decode_step(full, x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                                         w.delta, 21, t)
        for b0, b1, h0, h1, st in shards:
            xs = {k: v[b0:b1, h0:h1].contiguous() for k, v in x.items()}
            o_s = lores.lores_decode_step(st, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"],
                                          w.delta, 21, t, seq_base=b0, head_base=h0)
            assert torch.equal(o_s, o_full[b0:b1, h0:h1]), (t, b0, h0)
    torch.cuda.synchronize()
    fh = full.buf.cpu().numpy()
    for b0, b1, h0, h1, st in shards:
        sh = st.buf.cpu().numpy()
        for b in range(b0, b1):
            for h in range(h0, h1):
                assert np.array_equal(_unit_bytes(st, sh, b - b0, h - h0),
                                      _unit_bytes(full, fh, b, h)), (b, h)


def test_key_changes_the_rounding():
    """Another seed, step or base index moves the stochastic rounding: the
    keys reach the noise (a sanity check against a constant key)."""
    w = C1.scaled(B=2, H=2, dk=128, dv=64, T=1)
    log("case: rounding keys, B=2 H=2 int8")
    x = {k: v[0] for k, v in make_inputs(w, 0, DEV).items()}
    init = _random_states(2, [2, 2], 64, 128, seed=5)
    results = []
    for seed, t, sb, hb in [(0, 1, 0, 0), (1, 1, 0, 0), (0, 2, 0, 0), (0, 1, 7, 0), (0, 1, 0, 7)]:
        st = lores.lores_state_alloc(2, 2, 128, 64, [2, 2], device=DEV)
        _install(st, init)
        lores.lores_decode_step(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], 1, seed, t,
                                seq_base=sb, head_base=hb)
        results.append(st.buf.cpu().numpy())
    for r in results[1:]:
        assert not np.array_equal(r, results[0])


def test_nearest_rounding_ignores_the_keys():
    """In round-to-nearest mode the seed, step and base indices no longer
    reach the result; an invalid mode is rejected."""
    w = C1.scaled(B=2, H=3, dk=128, dv=64, T=1)
    log("case: nearest mode is key-independent, B=2 H=3 int8/int4/bf16")
    x = {k: v[0] for k, v in make_inputs(w, 0, DEV).items()}
    prec = [2, 3, 1]
    init = _random_states(2, prec, 64, 128, seed=6)
    results = []
    for seed, t, sb, hb in [(0, 1, 0, 0), (1, 1, 0, 0), (0, 2, 0, 0), (0, 1, 7, 0), (0, 1, 0, 7)]:
        st = lores.lores_state_alloc(2, 3, 128, 64, prec, device=DEV)
        lores.lores_state_set_rounding(st, lores.LORES_ROUND_NEAREST)
        _install(st, init)
        lores.lores_decode_step(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], 1, seed, t,
                                seq_base=sb, head_base=hb)
        results.append(st.buf.cpu().numpy())
    for r in results[1:]:
        assert np.array_equal(r, results[0])
    with pytest.raises(lores.LoresError, match="EINVAL"):
        lores.lores_state_set_rounding(st, 2)


def test_repeatable_eager_and_graph():
    """The same steps from the same state give the same bytes: twice eagerly,
    and over several replays of a captured graph with eager work between."""
    B, head_prec = 96, [2, 3] * 16
    w = get_workload("C5").scaled(B=B, T=4)
    log(f"case: repeatability B={B} H=32 d=128 int8/int4, 4 steps, eager x2 and graph x3")
    inp = make_inputs(w, 0, DEV)
    st = lores.lores_state_alloc(B, 32, 128, 128, head_prec, device=DEV)
    _install(st, _random_states(B, head_prec, 128, 128, seed=2))
    init = st.buf.clone()
    outs = [torch.empty((B, 32, 128), dtype=torch.float32, device=DEV) for _ in range(w.T)]

    def steps():
        for t in range(1, w.T + 1):
            x = {k: v[t - 1] for k, v in inp.items()}
            lores.lores_decode_step(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], w.delta,
                                    4, t, o=outs[t - 1])

    steps()
    torch.cuda.synchronize()
    ref_buf = st.buf.clone()
    ref_o = [o.clone() for o in outs]
    st.buf.copy_(init)
    steps()
    torch.cuda.synchronize()
    assert torch.equal(st.buf, ref_buf)
    assert all(torch.equal(a, b) for a, b in zip(outs, ref_o))

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


def test_two_states_on_two_streams():
    """Two independent states stepped concurrently on two streams give the
    bytes and outputs of the same steps run one after the other: the library
    keeps no state outside its handles and launches on the stream it is given."""
    log("case: two states, two streams, 6 steps each, int8/int4 and bf16/int6")
    cfg = [(64, [2, 3] * 8, 128, 128), (48, [1, 4] * 6, 64, 96)]
    runs = {}
    for mode in ("sequential", "concurrent"):
        states, outs, inps = [], [], []
        for i, (B, prec, dk, dv) in enumerate(cfg):
            w = C1.scaled(B=B, H=len(prec), dk=dk, dv=dv, T=6)
            inps.append(make_inputs(w, 10 + i, DEV))
            st = lores.lores_state_alloc(B, len(prec), dk, dv, prec, device=DEV)
            _install(st, _random_states(B, prec, dv, dk, seed=20 + i))
            states.append((st, w))
            outs.append([torch.empty((B, len(prec), dv), device=DEV) for _ in range(w.T)])
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]

        def run(i):
            st, w = states[i]
            for t in range(1, w.T + 1):
                x = {k: v[t - 1] for k, v in inps[i].items()}
                lores.lores_decode_step(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], 1,
                                        3, t, o=outs[i][t - 1], stream=streams[i])
        if mode == "sequential":
            run(0)
            torch.cuda.synchronize()
            run(1)
        else:
            run(0)
            run(1)
        torch.cuda.synchronize()
        runs[mode] = ([st.buf.clone() for st, _ in states], [[o.clone() for o in oo] for oo in outs])
    for i in range(2):
        assert torch.equal(runs["sequential"][0][i], runs["concurrent"][0][i]), i
        assert all(torch.equal(a, b) for a, b in zip(runs["sequential"][1][i], runs["concurrent"][1][i]))


@pytest.mark.parametrize("dk,dv", [(128, 128), (96, 65), (32, 1), (64, 200)])
def test_dequant_matches_oracle(dk, dv):
    """lores_dequant_state of a packed state (written through the codec)
    equals the oracle's dequantization bit for bit."""
    B, head_prec = 3, [0, 1, 2, 3, 3, 2, 4, 5]
    log(f"case: dequant B={B} dk={dk} dv={dv} precisions {head_prec}")
    st = lores.lores_state_alloc(B, len(head_prec), dk, dv, head_prec, device=DEV)
    zero = lores.lores_dequant_state(st)
    torch.cuda.synchronize()
    assert torch.count_nonzero(zero).item() == 0
    states = _random_states(B, head_prec, dv, dk, seed=dk + dv)
    _install(st, states)
    out = lores.lores_dequant_state(st).cpu().numpy()
    for (b, h), s in states.items():
        want = ostep.dequant(head_prec[h], {k: v[None] for k, v in s.items()})[0]
        assert np.array_equal(out[b, h].view(np.uint32), want.view(np.uint32)), (b, h)


def test_error_paths_live_handle():
    """Invalid calls on a live handle fail with the documented code and
    launch nothing."""
    w = C1.scaled(B=2, H=2, dk=64, dv=64, T=1, in_bf16=True)
    log("case: error paths on a live handle")
    x = {k: v[0] for k, v in make_inputs(w, 0, DEV).items()}
    st = lores.lores_state_alloc(2, 2, 64, 64, [2, 3], device=DEV)
    _install(st, _random_states(2, [2, 3], 64, 64, seed=9))
    before = st.buf.clone()
    args = (x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    with pytest.raises(lores.LoresError, match="EINVAL"):
        lores.lores_decode_step(st, *args, 1, 0, 0)                # t = 0
    assert "t must be" in lores.lores_last_error()
    with pytest.raises(lores.LoresError, match="EINVAL"):
        lores.lores_decode_step(st, *args, 2, 0, 1)                # delta = 2
    with pytest.raises(lores.LoresError, match="EINVAL"):
        lores.lores_decode_step(st, *args, 1, 0, 1, seq_base=(1 << 32) - 1)
    with pytest.raises(ValueError):
        lores.lores_decode_step(st, x["q"][:1], *args[1:], 1, 0, 1)   # wrong size (binding)

    # misaligned bf16 q through the C ABI directly (2 bytes past an element pair)
    L = _lib.lib()
    o = torch.empty((2, 2, 64), dtype=torch.float32, device=DEV)
    qq = torch.empty(2 * 2 * 64 + 1, dtype=torch.bfloat16, device=DEV)
    vp = ctypes.c_void_p
    rc = L.lores_decode_step(vp(st.handle), vp(qq.data_ptr() + 2), vp(x["k"].data_ptr()),
                             vp(x["v"].data_ptr()), 1, vp(x["alpha"].data_ptr()), 0,
                             vp(x["beta"].data_ptr()), 1, 0, 1, 0, 0, vp(o.data_ptr()),
                             vp(torch.cuda.current_stream().cuda_stream))
    assert rc == -1 and "aligned" in lores.lores_last_error()
    rc = L.lores_decode_step(vp(st.handle), vp(x["q"].data_ptr()), vp(x["k"].data_ptr()),
                             vp(x["v"].data_ptr()), 1, vp(x["alpha"].data_ptr()), 0,
                             vp(x["beta"].data_ptr()), 1, 0, 1, 0, 0, vp(None),
                             vp(torch.cuda.current_stream().cuda_stream))
    assert rc == -1
    torch.cuda.synchronize()
    assert torch.equal(st.buf, before)

    # buffers: too small, misaligned
    need = lores.lores_state_alloc(2, 2, 64, 64, [2, 3])
    with pytest.raises(lores.LoresError, match="ESIZE"):
        lores.lores_state_alloc(2, 2, 64, 64, [2, 3],
                                buf=torch.empty(need - 16, dtype=torch.uint8, device=DEV))
    big = torch.empty(need + 512, dtype=torch.uint8, device=DEV)
    with pytest.raises(lores.LoresError, match="EINVAL"):
        lores.lores_state_alloc(2, 2, 64, 64, [2, 3], buf=big[16:16 + need])
    with pytest.raises(lores.LoresError, match="EUNSUPPORTED|EINVAL"):
        lores.lores_state_alloc(2, 2, 48, 64, [2, 3], device=DEV)


@pytest.mark.parametrize("dk,dv,rounding", [(128, 128, "sr"), (96, 65, "sr"), (32, 1, "sr"),
                                             (64, 200, "nearest"), (128, 64, "nearest"),
                                             (256, 100, "sr"), (256, 33, "nearest"),
                                             (160, 70, "sr"), (192, 100, "nearest"),
                                             (224, 33, "sr")])
def test_quant_state_matches_oracle(dk, dv, rounding):
    """lores_quant_state equals the oracle's quantization of the same fp32
    state bit for bit (no summation is involved), for every precision, with
    zero rows and rows of very different magnitude; base indices key it."""
    B, head_prec = 3, [0, 1, 2, 3, 3, 2, 4, 5]
    H = len(head_prec)
    log(f"case: quant state B={B} dk={dk} dv={dv} rounding={rounding} precisions {head_prec}")
    g = np.random.default_rng(dk * 7 + dv)
    X = (g.standard_normal((B, H, dv, dk)) * np.exp(g.uniform(-6, 6, (B, H, dv, 1)))).astype(np.float32)
    X[0, :, 0, :] = 0.0                                    # zero rows
    st = lores.lores_state_alloc(B, H, dk, dv, head_prec, device=DEV)
    if rounding == "nearest":
        lores.lores_state_set_rounding(st, lores.LORES_ROUND_NEAREST)
    seed, sb, hb = 77, 5, 9
    lores.lores_quant_state(st, torch.from_numpy(X).to(DEV), seed, seq_base=sb, head_base=hb)
    torch.cuda.synchronize()
    lay = lores.lores_state_layout(st)
    _, slot = lores.lores_state_head_map(st)
    buf = st.buf.cpu().numpy()
    for h, c in enumerate(head_prec):
        bs = np.arange(B)
        want = ostep.quant_state(c, X[:, h], seed, bs + sb, np.full(B, h + hb), rounding=rounding)
        for b in range(B):
            got = lc.read_unit(buf, lay, c, b * lay["n_class"][c] + slot[h])
            for key, val in got.items():
                assert np.array_equal(np.asarray(val).view(np.uint8),
                                      np.ascontiguousarray(want[key][b]).astype(val.dtype).view(np.uint8)), \
                    (b, h, key)
    # the round trip through lores_dequant_state is the oracle's dequantization
    out = lores.lores_dequant_state(st).cpu().numpy()
    for h, c in enumerate(head_prec):
        want = ostep.dequant(c, ostep.quant_state(c, X[:, h], seed, np.arange(B) + sb,
                                                  np.full(B, h + hb), rounding=rounding))
        assert np.array_equal(out[:, h].view(np.uint32), want.view(np.uint32)), h
    with pytest.raises(lores.LoresError, match="EINVAL"):
        lores.lores_quant_state(st, torch.from_numpy(X).to(DEV), seed, seq_base=-1)


def test_quant_state_then_step():
    """A state handed over by lores_quant_state steps on like any other: the
    GPU's quantize-then-step matches the oracle's (quantization bit-exact,
    the step to the parity tolerances)."""
    B, H, dk, dv, prec, seed = 2, 6, 128, 64, [0, 1, 2, 3, 4, 5], 11
    w = C1.scaled(B=B, H=H, dk=dk, dv=dv, T=1)
    log("case: quant state, then one decode step, precisions fp32/bf16/int8/int4")
    g = np.random.default_rng(3)
    X = (g.standard_normal((B, H, dv, dk)) * 0.1).astype(np.float32)
    x = {k: v[0] for k, v in make_inputs(w, 4, DEV).items()}
    st = lores.lores_state_alloc(B, H, dk, dv, prec, device=DEV)
    lores.lores_quant_state(st, torch.from_numpy(X).to(DEV), seed)
    o = lores.lores_decode_step(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], 1, seed, 1)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    xin = {k: v.float().cpu().numpy() for k, v in x.items()}
    lay = lores.lores_state_layout(st)
    _, slot = lores.lores_state_head_map(st)
    buf = st.buf.cpu().numpy()
    bs = np.arange(B)
    for h, c in enumerate(prec):
        s0 = ostep.quant_state(c, X[:, h], seed, bs, np.full(B, h))
        new, o_ref = ostep.decode_step(c, s0, xin["q"][:, h], xin["k"][:, h], xin["v"][:, h],
                                       xin["alpha"][:, h], xin["beta"][:, h], 1, seed, 1, bs,
                                       np.full(B, h))
        X_ref = ostep.dequant(c, new).astype(np.float64)
        scale = np.linalg.norm(X_ref, axis=-1).max(axis=-1)
        tol = 1e-5 if c == 0 else 1e-3
        assert np.all(np.abs(o[:, h] - o_ref).max(axis=1) <= tol * scale), h
        gpu = [lc.read_unit(buf, lay, c, b * lay["n_class"][c] + slot[h]) for b in range(B)]
        X_gpu = np.stack([ostep.dequant(c, {k: v[None] for k, v in u.items()})[0] for u in gpu])
        # one code (or one bf16 ulp plus the cancellation allowance) per element
        err = np.abs(X_gpu.astype(np.float64) - X_ref)
        rowmax = np.abs(X_ref).max(axis=2, keepdims=True)
        if c in (2, 3, 4):
            step_size = rowmax / {2: 127, 3: 7, 4: 31}[c]
            assert np.all(err <= step_size * (1 + 1e-6)), h
            d = np.abs(np.stack([u["codes"] for u in gpu]).astype(np.int64) - new["codes"])
            assert d.max() <= 1 and (d > 0).sum() <= max(1, 1e-4 * d.size), h
        elif c == 1:
            assert np.all(err <= np.abs(X_ref) * 2.0 ** -7 + rowmax * 2.0 ** -16), h
        elif c == 5:
            assert np.all(err <= np.maximum(np.abs(X_ref), np.abs(X_gpu)) / 8
                          + rowmax / 448 * 2.0 ** -9 + rowmax * 2.0 ** -16), h
        else:
            assert np.all(err <= 1e-5 * rowmax), h


def _scaled_state(lo, hi):
    """Unit states with int scales exp(U(lo, hi)) and bf16 / fp32 values of that size."""
    def init(c, dv, dk, g):
        if c in (2, 3, 4):
            r = {2: 127, 3: 7, 4: 31}[c]
            return {"codes": g.integers(-r, r + 1, (dv, dk)).astype(np.int32),
                    "scales": np.exp(g.uniform(lo, hi, dv)).astype(np.float32)}
        X = (g.standard_normal((dv, dk)) * np.exp(g.uniform(lo, hi, (dv, 1)))).astype(np.float32)
        if c == 1:
            return {"bits": (X.view(np.uint32) >> 16).astype(np.uint16)}
        return {"X": X}
    return init


@pytest.mark.parametrize("name,lo,hi,v_scale", [
    ("huge", 60.0, 78.0, 1.0),            # scales ~1e26..1e34, |U| up to ~1e36
    ("tiny", -90.0, -84.0, 1e-37),        # r / m above the fp32 range for some rows
    ("subnormal", -100.0, -95.0, 1e-41),  # scales and values below the normal range
])
def test_extreme_magnitudes(name, lo, hi, v_scale):
    w = C1.scaled(B=2, H=4, dk=128, dv=64, T=3)
    log(f"case: extreme magnitudes ({name}) B=2 H=4 precisions fp32/bf16/int8/int4")
    inp = make_inputs(w, 1, DEV)
    inp["v"] = inp["v"] * v_scale
    s = run_parity(w, T=w.T, head_prec=[0, 1, 2, 3], init=_scaled_state(lo, hi), inputs=inp)
    log(s.summary())
    s.check()


def test_zero_rows():
    """Rows that stay zero (zero state, zero write) keep scale 0 and code 0."""
    w = C1.scaled(B=2, H=2, dk=64, dv=64, T=2)
    log("case: zero rows, int8 / int4")
    inp = make_inputs(w, 0, DEV)
    inp["v"] = torch.zeros_like(inp["v"])
    st = lores.lores_state_alloc(2, 2, 64, 64, [2, 3], device=DEV)
    for t in (1, 2):
        x = {k: v[t - 1] for k, v in inp.items()}
        o = lores.lores_decode_step(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], 1, 0, t)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0
    assert torch.count_nonzero(lores.lores_dequant_state(st)).item() == 0
    lay = lores.lores_state_layout(st)
    buf = st.buf.cpu().numpy()
    for c in (2, 3):
        for u in range(2):
            s = lc.read_unit(buf, lay, c, u)
            assert not s["codes"].any() and not s["scales"].any()
