"""Correctly rounded fp32 primitives in NumPy.

The quantized step takes its rounding decisions in fp32, so the oracle must
reproduce fp32 results exactly where a decision depends on them.  NumPy's
float32 add, subtract, multiply and divide are IEEE single-precision
operations (one round-to-nearest-even each); what NumPy lacks is a fused
multiply-add and a division rounded downward, supplied here.

fma32: a*b is exact in fp64 (24 + 24 significant bits <= 53).  The sum
p + c is formed in fp64 together with its exact error (Knuth's TwoSum), the
fp64 result is rounded to odd (if inexact and its last bit is even, step one
fp64 ulp toward the exact value), and that is rounded to fp32.  Rounding to
odd at a precision of at least 24 + 2 bits followed by a round to nearest
gives the correctly rounded result (Boldo and Melquiond, "Emulation of FMA
and correctly rounded sums: proved algorithms using rounding to odd", IEEE
Trans. Computers, 2008).

Pinned by tests/test_oracle_exact.py against exact rational arithmetic.
"""
import numpy as np

F32 = np.float32
F64 = np.float64


def f32(x):
    return np.asarray(x, dtype=F32)


def fma32(a, b, c):
    """Correctly rounded fp32 value of a*b + c (one rounding), elementwise."""
    a, b, c = np.broadcast_arrays(f32(a), f32(b), f32(c))
    p = a.astype(F64) * b.astype(F64)          # exact
    cd = c.astype(F64)
    s = p + cd
    bp = s - p
    err = (p - (s - bp)) + (cd - bp)            # s + err == p + c exactly
    with np.errstate(invalid="ignore"):
        fix = (err != 0) & ((s.view(np.uint64) & np.uint64(1)) == 0)
        toward = np.where(err > 0, np.inf, -np.inf)
        s = np.where(fix, np.nextafter(s, toward), s)
    return s.astype(F32)


def rn_div32(num, den):
    """fp32 num / den rounded to nearest even (IEEE single division)."""
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        return (f32(num) / f32(den)).astype(F32)


def rd_div32(num, den):
    """Largest fp32 value not above num / den, for num > 0 and den >= 0.

    den == 0 gives 0 (the quantizer's zero-row convention).  A quotient above
    the largest finite fp32 gives that largest finite value.
    """
    num = f32(num)
    den = f32(den)
    q = rn_div32(num, den)
    with np.errstate(invalid="ignore", over="ignore"):
        over = q.astype(F64) * den.astype(F64) > num.astype(F64)   # exact product
    q = np.where(over, np.nextafter(q, F32(0)), q).astype(F32)
    return np.where(den == 0, F32(0), q).astype(F32)


def f32_bits(x):
    return np.ascontiguousarray(f32(x)).view(np.uint32)


def bits_f32(u):
    return np.ascontiguousarray(np.asarray(u, dtype=np.uint32)).view(F32)


def bf16_to_f32(h):
    """bfloat16 bit patterns (uint16) to fp32 values (exact)."""
    return bits_f32(np.asarray(h, dtype=np.uint32) << np.uint32(16))


def dot_rn32(A, x):
    """fl32 of sum_j A[..., i, j] * x[..., j]: fp64 accumulation, one final rounding."""
    return np.einsum("...ij,...j->...i", f32(A).astype(F64), f32(x).astype(F64)).astype(F32)
