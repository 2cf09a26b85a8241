"""Counter-based rounding noise for stochastic rounding.

The pages require stochastic rounding of the state at every requantization
([LoReS] abstract; "Intra-State Quantization (Section 4)", Rounding and
Proposition 3) but fix no generator.  The noise here is a pure function of
(seed, step t, global sequence b, global head h, row i, column j), so any
order of evaluation, launch shape or sharding gives the same draws.

Building blocks (published definitions, restated):
  mix64  : the SplitMix64 output finalizer (Steele, Lea and Flood, "Fast
           splittable pseudorandom number generators", OOPSLA 2014):
             z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
             z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31   (mod 2^64)
  fmix32 : the MurmurHash3 32-bit finalizer (A. Appleby, public domain):
             x ^= x >> 16; x *= 0x85EBCA6B; x ^= x >> 13;
             x *= 0xC2B2AE35; x ^= x >> 16                         (mod 2^32)

Keying and draws (this implementation's definition):
  unit key  K = lo32(z) ^ hi32(z),
            z = mix64(mix64(mix64(seed) ^ t) ^ ((b << 32) | h))      once per unit
  row word  w_i = fmix32(K ^ i)
  noise     n_ij = (lo16(w_i) + j * 0x9E37) mod 2^16             (bf16, E4M3)
            n_ij = (lo16(w_i) + floor(j / 2) * 0x9E37) mod 2^16  (int classes)
  n_ij is a 16-bit integer; the int quantizer uses u_ij = n_ij * 2^-16 in
  [0, 1) and the bf16 rounding adds n_ij below the kept bits.  The int
  classes take one draw per pair of columns (2m, 2m + 1): the even column
  rounds U with it, the odd column rounds -U with it, which is rounding U
  with the antithetic draw 1 - u (step.quantize_rows), so each column is
  still rounded without bias and one draw serves two columns.

Each n_ij is exactly uniform on {0, ..., 65535} when w_i is, so every
element's rounding is unbiased on its own; within a row the draws form a
16-bit Weyl sequence with the golden-ratio step 0x9E37 (about 0.618 * 2^16)
rather than independent draws.  noise16_iid is the reference with one hash
per element, kept to check that this choice does not change the readout
error statistics.

PARITY UNPINNED by the pages (they fix no generator): mix64 and fmix32 are
pinned by published test vectors; the keying and the draws only by
distribution tests.
"""
import numpy as np

U32 = np.uint32
U64 = np.uint64
PSI16 = U32(0x9E37)


def mix64(z):
    z = np.asarray(z, dtype=U64).copy()
    with np.errstate(over="ignore"):
        z ^= z >> U64(30)
        z *= U64(0xBF58476D1CE4E5B9)
        z ^= z >> U64(27)
        z *= U64(0x94D049BB133111EB)
        z ^= z >> U64(31)
    return z


def fmix32(x):
    x = np.asarray(x, dtype=U32).copy()
    with np.errstate(over="ignore"):
        x ^= x >> U32(16)
        x *= U32(0x85EBCA6B)
        x ^= x >> U32(13)
        x *= U32(0xC2B2AE35)
        x ^= x >> U32(16)
    return x


def unit_key(seed, t, b, h):
    """32-bit key of unit (b, h) at step t; arguments broadcast."""
    seed, t, b, h = (np.asarray(a, dtype=U64) for a in (seed, t, b, h))
    z = mix64(mix64(mix64(seed) ^ t) ^ ((b << U64(32)) | (h & U64(0xFFFFFFFF))))
    return ((z & U64(0xFFFFFFFF)) ^ (z >> U64(32))).astype(U32)


def noise16(K, dv, dk, paired=False):
    """Draws n_ij for keys K [N]: uint32 array [N, dv, dk] with values < 2^16.
    paired: one draw per pair of columns (the int classes' draws)."""
    K = np.asarray(K, dtype=U32).reshape(-1)
    i = np.arange(dv, dtype=U32)
    w = fmix32(K[:, None] ^ i[None, :])                       # [N, dv]
    j = np.arange(dk, dtype=U32)
    if paired:
        j = j >> U32(1)
    with np.errstate(over="ignore"):
        x = (w[:, :, None] & U32(0xFFFF)) + j[None, None, :] * PSI16
    return (x & U32(0xFFFF)).astype(U32)


def noise16_iid(K, dv, dk):
    """Reference draws with one fmix32 per element: high 16 bits of fmix32(K ^ (i*dk + j))."""
    K = np.asarray(K, dtype=U32).reshape(-1)
    e = (np.arange(dv, dtype=U32)[:, None] * U32(dk) + np.arange(dk, dtype=U32)[None, :])
    return (fmix32(K[:, None, None] ^ e[None]) >> U32(16)).astype(U32)
