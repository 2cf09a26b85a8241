"""The host codec of the packed layout: exhaustive round trips over every code
value and every byte / nibble / halfword position (CPU only)."""
import numpy as np
import pytest

from tests import layout_codec as lc


@pytest.mark.parametrize("c,r", [(2, 127), (3, 7), (4, 31)])
@pytest.mark.parametrize("dk,dv", [(32, 1), (64, 64), (96, 70), (128, 128), (160, 33),
                                   (192, 70), (224, 1), (256, 100)])
def test_int_roundtrip_every_code_every_position(c, r, dk, dv):
    dv_pad = (dv + 63) // 64 * 64
    vals = np.arange(-r, r + 1)
    codes = np.resize(vals, dv * dk).reshape(dv, dk)
    codes = np.roll(codes, 3, axis=1)                 # every value reaches every column
    scales = np.linspace(0.5, 2, dv).astype(np.float32)
    by, sc = lc.pack_unit(c, dk, dv, dv_pad, {"codes": codes, "scales": scales})
    bits = {2: 8, 3: 4, 4: 6}[c]
    row_chunks = 2 * -(-(dk // 2 * bits) // 128) if dk > 128 else -(-(dk * bits) // 128)
    assert by.size == dv_pad * 16 * row_chunks
    back = lc.unpack_unit(c, dk, dv, dv_pad, by, sc)
    assert np.array_equal(back["codes"], codes) and np.array_equal(back["scales"], scales)


def test_int8_byte_positions():
    dk, dv = 32, 2
    codes = np.zeros((dv, dk), np.int64)
    codes[1, 16] = -127                               # row 1, chunk 1, byte 0
    codes[1, 17] = -127                               # byte 1: an odd column, stored negated
    by, _ = lc.pack_unit(2, dk, dv, 64, {"codes": codes, "scales": np.ones(dv, np.float32)})
    chunk = by.reshape(2, 64, 16)
    assert chunk[1, 1, 0] == 1 and chunk[1, 1, 1] == 255 and chunk[0, 0, 0] == 128


def test_int4_nibble_positions():
    dk, dv = 32, 1
    codes = np.zeros((dv, dk), np.int64)
    codes[0, 4] = 7                                   # byte 2, low nibble
    codes[0, 5] = 7                                   # byte 2, high nibble (odd: 8 - 7)
    by, _ = lc.pack_unit(3, dk, dv, 64, {"codes": codes, "scales": np.ones(dv, np.float32)})
    assert by.reshape(1, 64, 16)[0, 0, 2] == (15 | (1 << 4))


def test_bf16_and_fp32_roundtrip():
    g = np.random.default_rng(0)
    for dk, dv in [(32, 3), (128, 65)]:
        bits = g.integers(0, 65536, (dv, dk), dtype=np.uint16)
        by, _ = lc.pack_unit(1, dk, dv, (dv + 63) // 64 * 64, {"bits": bits})
        assert np.array_equal(lc.unpack_unit(1, dk, dv, (dv + 63) // 64 * 64, by)["bits"], bits)
        X = g.standard_normal((dv, dk)).astype(np.float32)
        by, _ = lc.pack_unit(0, dk, dv, (dv + 63) // 64 * 64, {"X": X})
        assert np.array_equal(lc.unpack_unit(0, dk, dv, (dv + 63) // 64 * 64, by)["X"], X)


def test_int6_bit_positions():
    """Element j occupies bits 6j .. 6j + 5 of the row's little-endian bytes,
    across 16-byte chunk boundaries; the padding bits stay zero."""
    dk, dv = 96, 1                                    # 576 bits: 4.5 chunks -> 5
    codes = np.full((dv, dk), -32 + 32, np.int64)     # stored 32 everywhere ...
    codes[0, 21] = -31                                # bits 126..131: straddles chunks 0 and 1
    codes[0, 5] = 31                                  # bits 30..35: straddles words 0 and 1
    # (both odd columns: stored negated, 32 + 31 = 63 and 32 - 31 = 1)
    by, _ = lc.pack_unit(4, dk, dv, 64, {"codes": codes, "scales": np.ones(dv, np.float32)})
    row = by.reshape(5, 64, 16)[:, 0, :].reshape(-1)  # the row's 80 bytes, chunk after chunk
    bits = np.unpackbits(row, bitorder="little")
    val = lambda j: int(sum(int(bits[6 * j + i]) << i for i in range(6)))
    assert val(21) == 63 and val(5) == 1 and val(0) == 32 and val(95) == 32
    assert not bits[576:].any()


def test_fp8_bytes_roundtrip():
    dk, dv = 64, 70
    g = np.random.default_rng(3)
    by = g.integers(0, 256, (dv, dk)).astype(np.uint8)
    sc = np.linspace(0.1, 3, dv).astype(np.float32)
    packed, psc = lc.pack_unit(5, dk, dv, 128, {"fp8": by, "scales": sc})
    assert packed.size == 128 * dk
    back = lc.unpack_unit(5, dk, dv, 128, packed, psc)
    assert np.array_equal(back["fp8"], by) and np.array_equal(back["scales"], sc)
    assert packed.reshape(dk // 16, 128, 16)[1, 3, 5] == by[3, 16 + 5]   # chunk 1, row 3, byte 5


def test_split_row_halves_start_on_a_chunk():
    """Above d_k = 128 a row is two half rows, the second starting on its own
    chunk: int4 at d_k = 160 keeps 80 columns per half, so half 0 fills 2.5
    chunks (the rest of its third chunk zero) and column 80 is the low nibble
    of byte 0 of chunk 3."""
    dk, dv = 160, 1
    codes = np.zeros((dv, dk), np.int64)
    codes[0, 79] = -7                                 # half 0, last column: chunk 2, byte 7, high nibble
    #                                                   (odd: stored negated, 8 + 7)
    codes[0, 80] = -7                                 # half 1, first column: chunk 3, byte 0, low nibble
    by, _ = lc.pack_unit(3, dk, dv, 64, {"codes": codes, "scales": np.ones(dv, np.float32)})
    ch = by.reshape(6, 64, 16)[:, 0, :]
    assert ch[2, 7] == (8 | (15 << 4)) and (ch[2, 8:] == 0).all()
    assert ch[3, 0] == (1 | (8 << 4))


def test_split_row_roundtrip_float_and_fp8():
    g = np.random.default_rng(5)
    for dk, dv in [(160, 3), (224, 65), (256, 64)]:
        dvp = (dv + 63) // 64 * 64
        bits = g.integers(0, 65536, (dv, dk), dtype=np.uint16)
        by, _ = lc.pack_unit(1, dk, dv, dvp, {"bits": bits})
        assert np.array_equal(lc.unpack_unit(1, dk, dv, dvp, by)["bits"], bits)
        X = g.standard_normal((dv, dk)).astype(np.float32)
        by, _ = lc.pack_unit(0, dk, dv, dvp, {"X": X})
        assert np.array_equal(lc.unpack_unit(0, dk, dv, dvp, by)["X"], X)
        f8 = g.integers(0, 256, (dv, dk)).astype(np.uint8)
        sc = np.linspace(0.1, 3, dk).astype(np.float32)         # key-column scales
        by, psc = lc.pack_unit(5, dk, dv, dvp, {"fp8": f8, "scales": sc}, key=True)
        back = lc.unpack_unit(5, dk, dv, dvp, by, psc, key=True)
        assert np.array_equal(back["fp8"], f8) and np.array_equal(back["scales"], sc)
