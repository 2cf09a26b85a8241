"""Host codec of the packed state layout documented in include/lores.h.

Test infrastructure: it converts the oracle's state (signed codes and scales,
bf16 bit patterns, fp32 values per unit) to the bytes of a device buffer and
back, using only the offsets lores_state_layout reports and the layout rules
the header states.  It holds none of the method's arithmetic.

Units of class c are ordered [B][H_c]; slot s of class c is the s-th head of
that class in head order.
"""
import numpy as np

E = {0: 4, 1: 8, 2: 16, 3: 32}       # elements per 16-byte chunk (int6: a bit stream, below)
OFFSET = {2: 128, 3: 8, 4: 32}       # offset-binary code offset
QMAX = {2: 127, 3: 7, 4: 31}
INT_CLASSES = (2, 3, 4)
SCALED_CLASSES = (2, 3, 4, 5)        # classes with fp32 scales (per value row or key column)


def _col_sign(dk):
    """+1 for the even columns, -1 for the odd ones: an int row stores the
    code of an odd column negated."""
    return np.where(np.arange(dk) % 2 == 0, 1, -1).astype(np.int32)


def n_chunks(c, dk):
    """16-byte chunks per row: d_k elements of 32, 16, 8, 4 or 6 bits, the
    last chunk zero-padded; a row of d_k > 128 is two halves of d_k / 2
    columns, each padded to whole chunks."""
    if dk > 128:
        return 2 * n_chunks(c, dk // 2)
    bits = {0: 32, 1: 16, 2: 8, 3: 4, 4: 6, 5: 8}[c]
    return (dk * bits + 127) // 128


def _halves(state_unit, h, dk):
    """The columns [h dk/2, (h + 1) dk/2) of a unit's per-element arrays."""
    sl = slice(h * (dk // 2), (h + 1) * (dk // 2))
    out = {k: np.asarray(v)[:, sl] for k, v in state_unit.items() if k != "scales"}
    if "scales" in state_unit:                   # stored once, by the caller
        out["scales"] = np.zeros(next(iter(out.values())).shape[0], np.float32)
    return out


def _pack6(vals):
    """[dv, dk] values 0..63 -> [dv, n_bytes] bytes of the little-endian bit
    stream: value j at bits [6j, 6j + 6)."""
    dv, dk = vals.shape
    bits = ((vals[:, :, None].astype(np.uint16) >> np.arange(6)) & 1).astype(np.uint8)
    return np.packbits(bits.reshape(dv, dk * 6), axis=1, bitorder="little")


def _unpack6(rows, dk):
    dv = rows.shape[0]
    bits = np.unpackbits(rows, axis=1, bitorder="little")[:, :dk * 6].reshape(dv, dk, 6)
    return (bits.astype(np.int32) << np.arange(6)).sum(axis=2)


def unit_index(b, slot, Hc):
    return b * Hc + slot


def class_units(head_prec, B, c):
    """(b, h) of every unit of class c, in storage order."""
    heads = [h for h, p in enumerate(head_prec) if p == c]
    return [(b, h) for b in range(B) for h in heads]


def pack_unit(c, dk, dv, dv_pad, state_unit, key=False):
    """One unit's state -> (code bytes [n_chunk*dv_pad*16] uint8, scales | None).

    state_unit: {"codes": int [dv, dk], "scales": f32 [dv]} (int classes),
                {"bits": uint16 [dv, dk]} (bf16) or {"X": f32 [dv, dk]} (fp32).
    The stored scales are [dv_pad] (value rows) or, with key=True, the
    unit's [dk] key-column scales.
    """
    if dk > 128:
        if c == 5:
            fp8 = np.asarray(state_unit["fp8"], np.uint8).reshape(dv, dk)
            su = dict(state_unit, fp8=fp8)
        else:
            su = state_unit
        parts = [pack_unit(c, dk // 2, dv, dv_pad, _halves(su, h, dk), key=False)[0]
                 .reshape(-1, dv_pad, 16) for h in (0, 1)]
        sc = None
        if c in SCALED_CLASSES:
            ns, nv = (dk, dk) if key else (dv_pad, dv)
            sc = np.zeros(ns, np.float32)
            sc[:nv] = state_unit["scales"]
        return np.concatenate(parts, axis=0).reshape(-1), sc
    n_chunk = n_chunks(c, dk)
    out = np.zeros((n_chunk, dv_pad, 16), np.uint8)
    sc = None
    ns, nv = (dk, dk) if key else (dv_pad, dv)
    if c == 5:
        sc = np.zeros(ns, np.float32)
        sc[:nv] = state_unit["scales"]
        by = np.asarray(state_unit["fp8"], np.uint8)
        out[:, :dv, :] = by.reshape(dv, n_chunk, 16).transpose(1, 0, 2)
    elif c in INT_CLASSES:
        codes = np.asarray(state_unit["codes"], np.int64)
        assert codes.min() >= -QMAX[c] and codes.max() <= QMAX[c]
        sc = np.zeros(ns, np.float32)
        sc[:nv] = state_unit["scales"]
        # odd columns hold the negated code (include/lores.h)
        off = (codes * _col_sign(codes.shape[1]) + OFFSET[c]).astype(np.uint8)   # [dv, dk]
        if c == 2:
            out[:, :dv, :] = off.reshape(dv, n_chunk, 16).transpose(1, 0, 2)
        elif c == 4:
            row = np.zeros((dv, n_chunk * 16), np.uint8)
            packed = _pack6(off)
            row[:, :packed.shape[1]] = packed
            out[:, :dv, :] = row.reshape(dv, n_chunk, 16).transpose(1, 0, 2)
        else:
            padded = np.zeros((dv, n_chunk * 32), np.uint8)     # a half chunk at the end stays 0
            padded[:, :dk] = off
            pairs = padded.reshape(dv, n_chunk, 16, 2)
            by = (pairs[..., 0] | (pairs[..., 1] << 4)).astype(np.uint8)
            out[:, :dv, :] = by.transpose(1, 0, 2)
    elif c == 1:
        bits = np.asarray(state_unit["bits"], np.uint16).reshape(dv, n_chunk, 8)
        out[:, :dv, :] = bits.view(np.uint8).reshape(dv, n_chunk, 16).transpose(1, 0, 2)
    else:
        X = np.ascontiguousarray(np.asarray(state_unit["X"], np.float32)).reshape(dv, n_chunk, 4)
        out[:, :dv, :] = X.view(np.uint8).reshape(dv, n_chunk, 16).transpose(1, 0, 2)
    return out.reshape(-1), sc


def unpack_unit(c, dk, dv, dv_pad, code_bytes, scales=None, key=False):
    """Inverse of pack_unit."""
    if dk > 128:
        nh = n_chunks(c, dk // 2)
        raw = np.asarray(code_bytes, np.uint8).reshape(2 * nh, dv_pad, 16)
        halves = [unpack_unit(c, dk // 2, dv, dv_pad, raw[h * nh:(h + 1) * nh].reshape(-1), scales)
                  for h in (0, 1)]
        out = {}
        for k in halves[0]:
            if k == "scales":
                continue
            out[k] = np.concatenate([halves[0][k], halves[1][k]], axis=1)
        if c in SCALED_CLASSES:
            nv = dk if key else dv
            out["scales"] = np.asarray(scales, np.float32)[:nv].copy()
        return out
    n_chunk = n_chunks(c, dk)
    nv = dk if key else dv
    raw = np.asarray(code_bytes, np.uint8).reshape(n_chunk, dv_pad, 16)[:, :dv, :]
    rows = np.ascontiguousarray(raw.transpose(1, 0, 2)).reshape(dv, n_chunk * 16)
    if c == 2:
        return {"codes": (rows.astype(np.int32) - 128) * _col_sign(dk),
                "scales": np.asarray(scales, np.float32)[:nv].copy()}
    if c == 5:
        return {"fp8": rows.copy(), "scales": np.asarray(scales, np.float32)[:nv].copy()}
    if c == 4:
        return {"codes": (_unpack6(rows, dk) - 32) * _col_sign(dk),
                "scales": np.asarray(scales, np.float32)[:nv].copy()}
    if c == 3:
        lo = (rows & 0x0F).astype(np.int32)
        hi = (rows >> 4).astype(np.int32)
        codes = (np.stack([lo, hi], axis=-1).reshape(dv, -1)[:, :dk] - 8) * _col_sign(dk)
        return {"codes": codes, "scales": np.asarray(scales, np.float32)[:nv].copy()}
    if c == 1:
        return {"bits": rows.view(np.uint16).reshape(dv, dk).copy()}
    return {"X": rows.view(np.float32).reshape(dv, dk).copy()}


def unit_ranges(layout, c, unit):
    """Byte ranges (code_start, code_len, scale_start | None, scale_len) of a unit."""
    ub = layout["unit_code_bytes"][c]
    cs = layout["codes_offset"][c] + unit * ub
    if c in SCALED_CLASSES:
        ns = layout["unit_scales"]
        return cs, ub, layout["scales_offset"][c] + unit * ns * 4, ns * 4
    return cs, ub, None, 0


def read_unit(buf_host, layout, c, unit):
    """Decode unit `unit` of class c from a host copy (uint8 numpy) of the buffer."""
    cs, cl, ss, sl = unit_ranges(layout, c, unit)
    sc = buf_host[ss:ss + sl].view(np.float32) if ss is not None else None
    return unpack_unit(c, layout["d_k"], layout["d_v"], layout["d_v_pad"], buf_host[cs:cs + cl], sc,
                       key=layout["scale_axis"] == 1)


def write_unit(buf_host, layout, c, unit, state_unit):
    cs, cl, ss, sl = unit_ranges(layout, c, unit)
    code_bytes, sc = pack_unit(c, layout["d_k"], layout["d_v"], layout["d_v_pad"], state_unit,
                               key=layout["scale_axis"] == 1)
    buf_host[cs:cs + cl] = code_bytes
    if ss is not None:
        buf_host[ss:ss + sl] = sc.view(np.uint8)


def window_ranges(layout, c, unit):
    """(start, length) of a unit's window block, or None."""
    off = layout["window_offset"][c]
    if off < 0:
        return None
    ub = layout["unit_window_bytes"][c]
    return off + unit * ub, ub


def read_window(buf_host, layout, c, unit):
    """A unit's window buffer as {"g": [W-1, d_v], "k": [W-1, d_k], "alpha": [W-1, d_k]}:
    slots of g [W-1][d_v_pad], then k [W-1][d_k], then alpha [W-1][d_k] (fp32;
    a scalar decay in element 0)."""
    W, dvp, dk, dv = layout["window"], layout["d_v_pad"], layout["d_k"], layout["d_v"]
    s, n = window_ranges(layout, c, unit)
    f = buf_host[s:s + n].view(np.float32)
    ns = W - 1
    g = f[:ns * dvp].reshape(ns, dvp)[:, :dv].copy()
    k = f[ns * dvp:ns * (dvp + dk)].reshape(ns, dk).copy()
    a = f[ns * (dvp + dk):ns * (dvp + 2 * dk)].reshape(ns, dk).copy()
    return {"g": g, "k": k, "alpha": a}


def write_window(buf_host, layout, c, unit, win):
    W, dvp, dk, dv = layout["window"], layout["d_v_pad"], layout["d_k"], layout["d_v"]
    s, n = window_ranges(layout, c, unit)
    f = np.zeros(n // 4, np.float32)
    ns = W - 1
    g = np.zeros((ns, dvp), np.float32)
    g[:, :dv] = win["g"]
    f[:ns * dvp] = g.reshape(-1)
    f[ns * dvp:ns * (dvp + dk)] = np.asarray(win["k"], np.float32).reshape(-1)
    f[ns * (dvp + dk):ns * (dvp + 2 * dk)] = np.asarray(win["alpha"], np.float32).reshape(-1)
    buf_host[s:s + n] = f.view(np.uint8)
