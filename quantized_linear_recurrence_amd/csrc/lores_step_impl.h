// Fused LoReS decode step for gfx950: dequantize -> decay -> delta projection
// -> rank-one write -> readout -> fresh row scale -> stochastic requantize ->
// pack, in one pass over the state.
//
// Method: "Quantizing Recurrent Language Models Is Easier Than You Think",
// general recurrence form (section "Introduction and Theoretical Foundation")
//   S_t = S_{t-1} diag(alpha)(I - delta beta k k^T) + beta v k^T,  o_t = S_t q_t
// evaluated row by row: with S' = S_{t-1} diag(alpha) and r_i = S'_i . k,
//   U_i = S'_i + g_i k^T,  g_i = beta (v_i - r_i) (delta = 1) or beta v_i,
// so every value row is independent once its own r_i is known.  The state is
// requantized each step with one scale per value row and stochastic rounding
// (section "Intra-State Quantization (Section 4)": scale grouping,
// Proposition 1, Rounding, Proposition 3).
//
// Mapping: one wavefront per (sequence, head, block of 64 value rows); lane i
// owns row i of the block for the whole step.  All lanes walk the key columns
// in lock-step, so k_j, q_j and a per-channel alpha_j are wave-uniform: they
// are held as 16-lane row vectors and broadcast by the DPP modifier of the
// FMA that consumes them, so value-row states need no LDS, no barriers and no
// cross-lane reductions (key-column states add one column reduction and an
// LDS exchange per task).  Codes are stored chunk-major (16-byte column
// chunks of 64 consecutive rows), so each chunk load or store of a wavefront
// is one contiguous 1 KiB access.  The updated row U lives in d_k VGPRs
// between the passes (dequant+r, update+readout+max, quantize+store).  A
// wavefront walks two sequences (a fused int pair: a work queue of them),
// loading the next task while the current one computes.
//
// Arithmetic (must match the CPU oracle bit for bit where it decides codes):
//   int heads   a = fl(s * alpha); S' = fl(c * a), computed as
//               fma(c + off, a, -off * a) with the stored offset-binary code
//               c + off (exact: the fma's exact value is c * a, and off * a
//               is exact as off is a power of two)
//   r, o        fp32 fma chains (summation order is free; the oracle rounds
//               an fp64 sum once, and per-step parity absorbs the difference)
//   g           fl(beta * fl(v - r))            (contraction disabled)
//   U           fma(g, k_j, S'_j)
//   s'          fl(m / r) (IEEE division);  inv = the largest fp32 <= r / m
//   code        e = floor(fma(U, inv, bias + n 2^-16)): the addend register
//               holds bias + n 2^-16 (n in its low 16 mantissa bits) and steps
//               to the next column's draw with one packed 16-bit add; e is the
//               stored offset-binary byte (int8) or, mod 16, the offset-binary
//               nibble (int4, bias 136 = 128 + 8), or the 6-bit field (int6)
//   bf16        bits of U plus the 16-bit draw, truncated to the high half
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lores_internal.h"

namespace lores {

// ---------------------------------------------------------------------------
// counter-based noise: SplitMix64 finalizer (Steele, Lea, Flood 2014) and
// MurmurHash3 32-bit finalizer (Appleby), as published.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

__device__ __forceinline__ uint32_t fmix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x85EBCA6Bu;
    x ^= x >> 13;
    x *= 0xC2B2AE35u;
    x ^= x >> 16;
    return x;
}

// Key of unit (b, h) at step t: fold of a three-level SplitMix64 chain.
__device__ __forceinline__ uint32_t unit_key(uint64_t seed, uint64_t t, uint64_t b, uint64_t h) {
    uint64_t z = mix64(mix64(mix64(seed) ^ t) ^ ((b << 32) | (h & 0xFFFFFFFFull)));
    return (uint32_t)z ^ (uint32_t)(z >> 32);
}

// The draws of row i: n_ij = (lo16(w_i) + j * kPsi16) mod 2^16, a 16-bit
// Weyl sequence with the golden-ratio step.
constexpr uint32_t kPsi16 = 0x9E37u;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte chunk

// ---------------------------------------------------------------------------
// precision traits: elements per 16-byte chunk, quantizer constants
// ---------------------------------------------------------------------------
template <int PREC> struct Prec;
template <> struct Prec<LORES_FP32> { static constexpr int E = 4, BITS = 32; };
template <> struct Prec<LORES_BF16> { static constexpr int E = 8, BITS = 16; };
template <> struct Prec<LORES_INT8> {
    static constexpr int E = 16, BITS = 8;
    static constexpr float R = 127.0f;        // 2^(8-1) - 1
    static constexpr float OFF = 128.0f;      // stored byte = code + 128
    static constexpr uint32_t FBASE = 0x43000000u;  // 128.0f: mantissa takes n * 2^-16
};
template <> struct Prec<LORES_INT4> {
    static constexpr int E = 32, BITS = 4;
    static constexpr float R = 7.0f;          // 2^(4-1) - 1
    static constexpr float OFF = 8.0f;        // stored nibble = code + 8
    static constexpr uint32_t FBASE = 0x43080000u;  // 136.0f = 128 + 8
};
// int6 rows are a bit stream (element j at bits 6j .. 6j + 5), not E
// elements per chunk; the stored field is floor(z) - 128 = code + 32.
template <> struct Prec<LORES_INT6> {
    static constexpr int E = 0, BITS = 6;
    static constexpr float R = 31.0f;         // 2^(6-1) - 1
    static constexpr float OFF = 32.0f;       // stored field = code + 32
    static constexpr uint32_t FBASE = 0x43200000u;  // 160.0f = 128 + 32
};

// E4M3 (OCP fp8) values with a value-row scale: the row maximum maps to
// 448, the largest finite E4M3 value.
template <> struct Prec<LORES_FP8> {
    static constexpr int E = 16, BITS = 8;
    static constexpr float R = 448.0f;
};

template <int PREC> constexpr bool is_int() {
    return PREC == LORES_INT8 || PREC == LORES_INT4 || PREC == LORES_INT6;
}

// classes stored with one fp32 scale per value row
template <int PREC> constexpr bool has_scale() { return is_int<PREC>() || PREC == LORES_FP8; }

// E4M3 byte `sel` of w as fp32 (hardware decode; gfx950 decodes the OCP
// E4M3 format).  sel is a constant once the callers' loops are unrolled; the
// bytes are decoded in pairs (v_cvt_pk_f32_fp8, bytes 0-1 or 2-3), and the
// two calls of a pair share one instruction.
__device__ __forceinline__ float fp8_value(uint32_t w, int sel) {
    const auto p = sel >= 2 ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
                            : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    return (sel & 1) ? p[1] : p[0];
}

// 16-byte chunks per stored row of d_k elements
template <int DK, int PREC> constexpr int row_chunks() {
    return (DK * Prec<PREC>::BITS + 127) / 128;
}

// Field j (6 bits) of an int6 row held in chunk registers cw.
__device__ __forceinline__ uint32_t int6_field(const u32x4 *cw, int j) {
    const int bit = 6 * j, w = bit >> 5, o = bit & 31;
    const uint32_t lo = cw[w >> 2][w & 3];
    if (o <= 26) return __builtin_amdgcn_ubfe(lo, o, 6);
    const uint32_t hi = cw[(w + 1) >> 2][(w + 1) & 3];
    return __builtin_amdgcn_alignbit(hi, lo, o) & 63u;
}

// For each word w of an int6 row: the sum, over the fields that touch w, of
// the bit 7 that each stored byte floor(z) carries (floor(z) = 128 + field),
// shifted like the field.  Packing adds floor(z) << offset and subtracts it.
template <int DK>
struct Int6Stray {
    uint32_t k[4 * ((6 * DK + 127) / 128)];   // the row's words
    constexpr Int6Stray() : k{} {
        for (int j = 0; j < DK; ++j) {
            const int bit = 6 * j, w = bit >> 5, o = bit & 31;
            k[w] += 128u << o;
            if (o > 26) k[w + 1] += 128u >> (32 - o);
        }
    }
};

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));


// Both 16-bit halves of x advanced by those of inc, each mod 2^16 (one
// v_pk_add_u16): the noise sequence steps in the low half while the high
// half, the sign, exponent and top mantissa bits of the bias, is kept.
__device__ __forceinline__ uint32_t step16(uint32_t x, uint32_t inc) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, x) + __builtin_bit_cast(u16x2, inc));
}

// A wave-uniform constant the compiler cannot see through: with it as the
// step, the noise stays one add per column instead of every column being
// re-derived from the first with a constant of its own.
__device__ __forceinline__ uint32_t opaque_uniform(uint32_t v) {
    uint32_t r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "s"(v));
    return r;
}

// x & m through an opaque VALU op: the compiler then keeps the byte structure
// of the result and converts its bytes with v_cvt_f32_ubyte{0..3} instead of
// re-deriving each nibble with a bit-field extract.
__device__ __forceinline__ uint32_t and_opaque(uint32_t x, uint32_t m) {
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(m));
    return r;
}

// (float)(int8_t) of byte k of w, in one SDWA conversion with sign extension.
// With w = stored bytes ^ 0x80808080 this is the int8 code (byte - 128).
__device__ __forceinline__ float cvt_sbyte(uint32_t w, int k) {
    float r;
    switch (k) {
        case 0:
            asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0"
                : "=v"(r) : "v"(w));
            break;
        case 1:
            asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1"
                : "=v"(r) : "v"(w));
            break;
        case 2:
            asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2"
                : "=v"(r) : "v"(w));
            break;
        default:
            asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3"
                : "=v"(r) : "v"(w));
            break;
    }
    return r;
}

// fl(x * A + B) where x is the f16 number held in the low (hi = 0) or high
// (hi = 1) half of h, in one rounding (v_fma_mix_f32: the f16 operand is
// widened exactly).  A half whose pattern P is below 2048 is the number
// P 2^-24 exactly (an f16 subnormal below 1024; exponent field 1 above), so
// with P an offset-binary code, A = a 2^24 and B = -off a the result is
// fl((P - off) a): code and dequantization in one instruction.
__device__ __forceinline__ float mix_f16(uint32_t h, int hi, float A, float B) {
    float r;
    if (hi)
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
            : "=v"(r) : "v"(h), "v"(A), "v"(B));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]"
            : "=v"(r) : "v"(h), "v"(A), "v"(B));
    return r;
}

// The same for an odd column, whose stored code is negated: -(h A + B), both
// products negated by the instruction's neg modifiers.
__device__ __forceinline__ float mix_f16n(uint32_t h, int hi, float A, float B) {
    float r;
    if (hi)
        asm("v_fma_mix_f32 %0, %1, -%2, -%3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
            : "=v"(r) : "v"(h), "v"(A), "v"(B));
    else
        asm("v_fma_mix_f32 %0, %1, -%2, -%3 op_sel:[0,0,0] op_sel_hi:[1,0,0]"
            : "=v"(r) : "v"(h), "v"(A), "v"(B));
    return r;
}

// Bytes 1 and 3 of w into the low bytes of its two halves, the high bytes 0.
__device__ __forceinline__ uint32_t odd_bytes(uint32_t w) {
    return __builtin_amdgcn_perm(w, w, 0x0c030c01u);
}

template <bool B> struct Flag { static constexpr bool value = B; };

// Uses of v and of the k and q row vectors: every load of them has completed
// here (forces the compiler's wait for them at this point).
template <int NV>
__device__ __forceinline__ void pin_inputs(float v, const float (&kv)[NV], const float (&qv)[NV]) {
    asm volatile("" ::"v"(v));
#pragma unroll
    for (int i = 0; i < NV; ++i) asm volatile("" ::"v"(kv[i]), "v"(qv[i]));
}

// Byte 2 of the fp32 patterns of z[0..3] into bytes 0..3 (three v_perm_b32).
__device__ __forceinline__ uint32_t gather_byte2(const float *z) {
    // selector bytes: 0-3 pick the second operand's bytes, 4-7 the first's,
    // 0x0c gives zero
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(z[1]), __float_as_uint(z[0]), 0x0c0c0602u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(z[3]), __float_as_uint(z[2]), 0x0c0c0602u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Byte K of `word` := truncation of z (0 <= z < 256) to an integer; the other
// bytes are kept.  One SDWA convert per element packs the codes for free.
template <int K>
__device__ __forceinline__ void cvt_u8_into(uint32_t &word, float z) {
    if constexpr (K == 0) {
        asm("v_cvt_u32_f32_sdwa %0, %1 dst_sel:BYTE_0 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
            : "+v"(word) : "v"(z));
    } else if constexpr (K == 1) {
        asm("v_cvt_u32_f32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
            : "+v"(word) : "v"(z));
    } else if constexpr (K == 2) {
        asm("v_cvt_u32_f32_sdwa %0, %1 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
            : "+v"(word) : "v"(z));
    } else {
        asm("v_cvt_u32_f32_sdwa %0, %1 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
            : "+v"(word) : "v"(z));
    }
}

// m / R correctly rounded, for an int class's R (7, 31 or 127) and every
// finite m >= 0: Markstein's correction step with the rounded reciprocal,
// one product and two fused multiply-adds in place of an IEEE division
// (checked against the IEEE quotient for every finite non-negative fp32 m on
// the host).  A non-finite m gives NaN rather than inf.
template <int PREC>
__device__ __forceinline__ float div_by_r(float m) {
    static_assert(is_int<PREC>(), "checked for the int classes' R only");
    constexpr float R = Prec<PREC>::R;
    constexpr float z = 1.0f / R;
    const float y = m * z;
    return __builtin_fmaf(__builtin_fmaf(-y, R, m), z, y);
}

// Largest fp32 not above r / m (0 for m = 0).
__device__ __forceinline__ float rd_div(float r, float m) {
    float q = r / m;                               // IEEE, correctly rounded
    if (__builtin_fmaf(q, m, -r) > 0.0f) q = __uint_as_float(__float_as_uint(q) - 1u);
    return m == 0.0f ? 0.0f : q;
}

// ---------------------------------------------------------------------------
// k, q and a per-channel alpha as "row vectors": register i of a wavefront
// holds element 16*i + (lane % 16) in every lane, so each 16-lane row holds
// 16 consecutive elements, and DPP row_newbcast:e hands element 16*i + e to
// all lanes as the first multiplicand of a v_fmac / v_mul at no extra cost.
// Each block opens with s_nop 1: a DPP source read needs two wait states
// after a VALU write of that register, which a copy the compiler might place
// just before the block would otherwise violate.
// ---------------------------------------------------------------------------
#define LORES_V16(P) "v"(P[0]), "v"(P[1]), "v"(P[2]), "v"(P[3]), "v"(P[4]), "v"(P[5]), \
    "v"(P[6]), "v"(P[7]), "v"(P[8]), "v"(P[9]), "v"(P[10]), "v"(P[11]), "v"(P[12]), \
    "v"(P[13]), "v"(P[14]), "v"(P[15])
#define LORES_PV16(P) "+v"(P[0]), "+v"(P[1]), "+v"(P[2]), "+v"(P[3]), "+v"(P[4]), \
    "+v"(P[5]), "+v"(P[6]), "+v"(P[7]), "+v"(P[8]), "+v"(P[9]), "+v"(P[10]), "+v"(P[11]), \
    "+v"(P[12]), "+v"(P[13]), "+v"(P[14]), "+v"(P[15])

// r += sum_e x[e] * row element e of kv
__device__ __forceinline__ void dot16(float &r, const float *x, float kv) {
    asm("s_nop 1\n"
        "v_fmac_f32_dpp %0, %17, %1 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %2 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %3 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %4 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %5 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %6 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %7 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %8 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %9 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %10 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %11 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %12 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %13 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %14 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %15 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %17, %16 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        : "+v"(r)
        : LORES_V16(x), "v"(kv));
}

// Forces the 16 values into registers at this point of the program; as a
// volatile statement it also keeps later memory accesses after it.
__device__ __forceinline__ void pin16(float *x) {
    asm volatile("" : LORES_PV16(x));
}

// u[e] += g * row element e of kv, then o += u[e] * row element e of qv
__device__ __forceinline__ void upd16(float *u, float &o, float g, float kv, float qv) {
    asm("s_nop 1\n"
        "v_fmac_f32_dpp %0, %18, %17 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %0 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %18, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %1 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %18, %17 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %2 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %18, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %3 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %4, %18, %17 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %4 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %5, %18, %17 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %5 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %6, %18, %17 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %6 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %7, %18, %17 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %7 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %8, %18, %17 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %9, %18, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %10, %18, %17 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %11, %18, %17 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %12, %18, %17 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %12 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %13, %18, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %14, %18, %17 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %14 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %15, %18, %17 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %16, %19, %15 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        : LORES_PV16(u), "+v"(o)
        : "v"(g), "v"(kv), "v"(qv));
}

// y[e] = row element e of av * x
__device__ __forceinline__ void scale16(float *y, float x, float av) {
    asm("s_nop 1\n"
        "v_mul_f32_dpp %0, %17, %16 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %1, %17, %16 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %2, %17, %16 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %3, %17, %16 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %4, %17, %16 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %5, %17, %16 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %6, %17, %16 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %7, %17, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %8, %17, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %9, %17, %16 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %10, %17, %16 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %11, %17, %16 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %12, %17, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %13, %17, %16 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %14, %17, %16 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %15, %17, %16 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        : "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]), "=&v"(y[4]), "=&v"(y[5]),
          "=&v"(y[6]), "=&v"(y[7]), "=&v"(y[8]), "=&v"(y[9]), "=&v"(y[10]), "=&v"(y[11]),
          "=&v"(y[12]), "=&v"(y[13]), "=&v"(y[14]), "=&v"(y[15])
        : "v"(x), "v"(av));
}

// x[e] *= row element e of av
__device__ __forceinline__ void mul16(float *x, float av) {
    asm("s_nop 1\n"
        "v_mul_f32_dpp %0, %16, %0 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %1, %16, %1 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %2, %16, %2 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %3, %16, %3 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %4, %16, %4 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %5, %16, %5 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %6, %16, %6 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %7, %16, %7 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %8, %16, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %9, %16, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %10, %16, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %11, %16, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %12, %16, %12 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %13, %16, %13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %14, %16, %14 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %15, %16, %15 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        : LORES_PV16(x)
        : "v"(av));
}

// x[e] *= s_e times row element e of av, s_e = +1 for even e and -1 for odd
// e (the negated codes of an int row's odd columns)
__device__ __forceinline__ void mul16n(float *x, float av) {
    asm("s_nop 1\n"
        "v_mul_f32_dpp %0, %16, %0 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %1, %16, -%1 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %2, %16, %2 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %3, %16, -%3 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %4, %16, %4 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %5, %16, -%5 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %6, %16, %6 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %7, %16, -%7 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %8, %16, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %9, %16, -%9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %10, %16, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %11, %16, -%11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %12, %16, %12 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %13, %16, -%13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %14, %16, %14 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %15, %16, -%15 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        : LORES_PV16(x)
        : "v"(av));
}

// ---------------------------------------------------------------------------
// key-column scales: one scale per key column of a (sequence, head) unit,
// s_j = max_i |U_ij| / r over all d_v rows, the comparison grouping of the
// pages' scale-grouping section.  The column maximum of a wavefront's 64
// rows is a butterfly across lanes; the unit's row blocks (wavefronts of one
// work-group) then combine theirs through LDS.  The column factors (s_j
// alpha_j for the dequantization, r / m_j for the requantization) are row
// vectors like k and q, consumed through DPP row_newbcast.
// ---------------------------------------------------------------------------

// z[e] += row element E0 + e of inv * s_e u[e] for e < 4 (one rounding each),
// s_e = +1 for the even and -1 for the odd elements (E0 is even): an int row's
// odd columns are requantized negated
#define LORES_FMAC4(E0, E1, E2, E3)                                                          \
    asm("s_nop 1\n"                                                                          \
        "v_fmac_f32_dpp %0, %4, %5 row_newbcast:" #E0 " row_mask:0xf bank_mask:0xf\n"        \
        "v_fmac_f32_dpp %1, %4, -%6 row_newbcast:" #E1 " row_mask:0xf bank_mask:0xf\n"       \
        "v_fmac_f32_dpp %2, %4, %7 row_newbcast:" #E2 " row_mask:0xf bank_mask:0xf\n"        \
        "v_fmac_f32_dpp %3, %4, -%8 row_newbcast:" #E3 " row_mask:0xf bank_mask:0xf\n"       \
        : "+v"(z[0]), "+v"(z[1]), "+v"(z[2]), "+v"(z[3])                                    \
        : "v"(inv), "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]))
__device__ __forceinline__ void fmac4_col(float *z, float inv, const float *u, int e0) {
    switch (e0) {
        case 0: LORES_FMAC4(0, 1, 2, 3); break;
        case 4: LORES_FMAC4(4, 5, 6, 7); break;
        case 8: LORES_FMAC4(8, 9, 10, 11); break;
        default: LORES_FMAC4(12, 13, 14, 15); break;
    }
}
#undef LORES_FMAC4

// y[e] = row element E0 + e of inv * u[e] for e < 4
#define LORES_MUL4(E0, E1, E2, E3)                                                           \
    asm("s_nop 1\n"                                                                          \
        "v_mul_f32_dpp %0, %4, %5 row_newbcast:" #E0 " row_mask:0xf bank_mask:0xf\n"         \
        "v_mul_f32_dpp %1, %4, %6 row_newbcast:" #E1 " row_mask:0xf bank_mask:0xf\n"         \
        "v_mul_f32_dpp %2, %4, %7 row_newbcast:" #E2 " row_mask:0xf bank_mask:0xf\n"         \
        "v_mul_f32_dpp %3, %4, %8 row_newbcast:" #E3 " row_mask:0xf bank_mask:0xf\n"         \
        : "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3])                                \
        : "v"(inv), "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]))
__device__ __forceinline__ void mul4_col(float *y, float inv, const float *u, int e0) {
    switch (e0) {
        case 0: LORES_MUL4(0, 1, 2, 3); break;
        case 4: LORES_MUL4(4, 5, 6, 7); break;
        case 8: LORES_MUL4(8, 9, 10, 11); break;
        default: LORES_MUL4(12, 13, 14, 15); break;
    }
}
#undef LORES_MUL4

// max(|x|, |z|) (values are finite: no NaN quieting needed)
__device__ __forceinline__ float absmax(float x, float z) {
    float y;
    asm("v_max_f32_e64 %0, |%1|, |%2|" : "=v"(y) : "v"(x), "v"(z));
    return y;
}

// y[p] = max(|s[p]|, |o[p] of the partner lane|) for p < 8; the partner is
// lane ^ 7 within 8 (row_half_mirror), lane ^ 1 (quad_perm [1,0,3,2]),
// lane ^ 2 (quad_perm [2,3,0,1]) or lane ^ 8 (row_ror:8)
#define LORES_DPP_HALF_MIRROR "row_half_mirror"
#define LORES_DPP_XOR1 "quad_perm:[1,0,3,2]"
#define LORES_DPP_XOR2 "quad_perm:[2,3,0,1]"
#define LORES_DPP_XOR8 "row_ror:8"
#define LORES_XMAX8(CTRL)                                                                     \
    asm("s_nop 1\n"                                                                           \
        "v_max_f32_dpp %0, |%8|, |%16| " CTRL " row_mask:0xf bank_mask:0xf\n"                 \
        "v_max_f32_dpp %1, |%9|, |%17| " CTRL " row_mask:0xf bank_mask:0xf\n"                 \
        "v_max_f32_dpp %2, |%10|, |%18| " CTRL " row_mask:0xf bank_mask:0xf\n"                \
        "v_max_f32_dpp %3, |%11|, |%19| " CTRL " row_mask:0xf bank_mask:0xf\n"                \
        "v_max_f32_dpp %4, |%12|, |%20| " CTRL " row_mask:0xf bank_mask:0xf\n"                \
        "v_max_f32_dpp %5, |%13|, |%21| " CTRL " row_mask:0xf bank_mask:0xf\n"                \
        "v_max_f32_dpp %6, |%14|, |%22| " CTRL " row_mask:0xf bank_mask:0xf\n"                \
        "v_max_f32_dpp %7, |%15|, |%23| " CTRL " row_mask:0xf bank_mask:0xf\n"                \
        : "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]), "=&v"(y[4]), "=&v"(y[5]),      \
          "=&v"(y[6]), "=&v"(y[7])                                                            \
        : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]), "v"(o[5]), "v"(o[6]),        \
          "v"(o[7]), "v"(s[0]), "v"(s[1]), "v"(s[2]), "v"(s[3]), "v"(s[4]), "v"(s[5]),        \
          "v"(s[6]), "v"(s[7]))
#define LORES_XMAX1(CTRL)                                                                     \
    asm("s_nop 1\n"                                                                           \
        "v_max_f32_dpp %0, |%1|, |%2| " CTRL " row_mask:0xf bank_mask:0xf\n"                  \
        : "=&v"(y) : "v"(o), "v"(s))

// One level of the column-maximum butterfly for one pair of registers (a, b):
// lanes whose bit `mask` is clear keep column a, the others column b, each
// combined with the partner lane across that bit.
template <int LEVEL>
__device__ __forceinline__ float xmax_pair(float a, float b, bool hi) {
    const float s = hi ? b : a, o = hi ? a : b;
    float y;
    if constexpr (LEVEL == 4) LORES_XMAX1(LORES_DPP_XOR1);
    else if constexpr (LEVEL == 5) LORES_XMAX1(LORES_DPP_XOR2);
    else LORES_XMAX1(LORES_DPP_XOR8);
    return y;
}

// Column maxima of |U| over the 64 rows (lanes) of a wavefront.  Six
// levels, each pairing registers (2p, 2p + 1) and lanes across one bit:
// lane ^ 7 within 8 (bit 2 selects), lane ^ 32 and lane ^ 16 (v_permlane32 /
// v_permlane16 swaps; bits 5, 4), lane ^ 1, lane ^ 2, lane ^ 8 (bits 0, 1, 3).
// Depth first, 16 columns at a time, so only a few partial results are live.
// Register t of lane L then holds the maximum of column key_col(t, L).
template <int DK> constexpr int key_groups() { return (DK + 63) / 64; }
// LDS of the key-column launches: floats per wavefront slot (64 per maximum
// register of a lane) and wavefront slots per buffer (the largest group)
template <int DK> constexpr int key_slot() { return DK > 128 ? 256 : 64 * key_groups<DK>(); }
template <int DK> constexpr int key_lds_waves() {
    return DK > 128 ? kMaxKeyGroupWaves : kWavesPerGroup;
}

__device__ __forceinline__ int key_col(int t, int L) {
    return 64 * t + ((L >> 3) & 1) * 32 + ((L >> 1) & 1) * 16 + (L & 1) * 8 +
           ((L >> 4) & 1) * 4 + ((L >> 5) & 1) * 2 + ((L >> 2) & 1);
}

// With d_k = 32 or 96 the last group holds 32 columns; its other 32 read as
// zeros, which leaves every real column's maximum as it is.
template <int DK>
__device__ __forceinline__ void col_absmax(const float (&U)[DK], float (&cm)[key_groups<DK>()]) {
    static_assert(DK % 32 == 0, "key-column scales need d_k a multiple of 32");
    const int lane = threadIdx.x & 63;
    const bool h0 = lane & 1, h1 = lane & 2, h2 = lane & 4, h3 = lane & 8;
    const float zeros[16] = {};
#pragma unroll
    for (int t = 0; t < key_groups<DK>(); ++t) {
        float g[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float *u = 64 * t + 16 * q < DK ? &U[64 * t + 16 * q] : zeros;
            float s[8], o[8], y[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                s[p] = h2 ? u[2 * p + 1] : u[2 * p];
                o[p] = h2 ? u[2 * p] : u[2 * p + 1];
            }
            LORES_XMAX8(LORES_DPP_HALF_MIRROR);
            float y2[4], y3[2];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(y[2 * p]),
                                                                 __float_as_uint(y[2 * p + 1]),
                                                                 false, false);
                y2[p] = absmax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(y2[2 * p]),
                                                                 __float_as_uint(y2[2 * p + 1]),
                                                                 false, false);
                y3[p] = absmax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            g[q] = xmax_pair<4>(y3[0], y3[1], h0);
        }
        cm[t] = xmax_pair<6>(xmax_pair<5>(g[0], g[1], h1), xmax_pair<5>(g[2], g[3], h1), h3);
    }
}
// The same over the 32 rows of a split-row task (d_k = 256: lane L and
// L + 32 hold the two halves of one row, so lane bit 5 is not a row bit):
// U holds the lane's 128 columns, the levels across lane bits 2, 4, 0, 1
// and 3 leave two registers per 64-column group, and register 2 t + s of
// lane L holds the maximum of column key_col_split(2 t + s, L).
// With CPL < 128 columns per half (d_k = 160, 192, 224) the columns past
// CPL read as zeros and their maxima go to the stage slots past d_k.
template <int CPL>
__device__ __forceinline__ int key_col_split(int j, int L) {
    const int t = j >> 1, s = j & 1, half = (L >> 5) & 1;
    const int c = 64 * t + ((L >> 3) & 1) * 32 + ((L >> 1) & 1) * 16 + s * 8 + (L & 1) * 4 +
                  ((L >> 4) & 1) * 2 + ((L >> 2) & 1);
    return c < CPL ? half * CPL + c : 2 * CPL + half * (128 - CPL) + (c - CPL);
}

template <int CPL>
__device__ __forceinline__ void col_absmax_split(const float (&U)[CPL], float (&cm)[4]) {
    const int lane = threadIdx.x & 63;
    const bool h0 = lane & 1, h1 = lane & 2, h2 = lane & 4, h3 = lane & 8;
    const float zeros[16] = {};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float g[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float *u = 64 * t + 16 * q < CPL ? &U[64 * t + 16 * q] : zeros;
            float s[8], o[8], y[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                s[p] = h2 ? u[2 * p + 1] : u[2 * p];
                o[p] = h2 ? u[2 * p] : u[2 * p + 1];
            }
            LORES_XMAX8(LORES_DPP_HALF_MIRROR);
            float y2[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(y[2 * p]),
                                                                 __float_as_uint(y[2 * p + 1]),
                                                                 false, false);
                y2[p] = absmax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) g[q][p] = xmax_pair<4>(y2[2 * p], y2[2 * p + 1], h0);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)
            cm[2 * t + p] = xmax_pair<6>(xmax_pair<5>(g[0][p], g[1][p], h1),
                                         xmax_pair<5>(g[2][p], g[3][p], h1), h3);
    }
}
#undef LORES_XMAX8
#undef LORES_XMAX1

// x of lane L combined with x of lane L ^ 32 (v_permlane32_swap gives each
// lane both halves' values; the operations commute, so both lanes of a pair
// hold the same result).
__device__ __forceinline__ float pair_sum(float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                     false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float pair_max(float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                     false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// s_barrier after this wavefront's LDS writes have landed; later memory
// accesses stay after it, loads already in flight are not waited for.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Column scales of a unit from its wavefronts' column maxima.  Wavefront wv
// (row block rb of n_rb; the unit's blocks are wavefronts wv - rb ..
// wv - rb + n_rb - 1 of the work-group) publishes its NCM maxima per lane in
// part[wv][.] and, after the barrier, combines the unit's: register j of
// lane L then holds column col_of(j, L) of snew = fl(m / r) and of inv = the
// largest fp32 <= r / m (0 for a zero column).  inv goes through the
// wavefront's own slot of `stage` to the row-vector form the requantization
// reads: register i of invrow holds column c0 + 16 i + lane % 16.  Each
// wavefront's slots hold 64 NCM values.
template <int NCM, int NVR, class ColOf>
__device__ __forceinline__ void key_scales(const float (&cm)[NCM], float *part, float *stage,
                                           int wv, int rb, int n_rb, float R,
                                           float (&snew)[NCM], float (&invrow)[NVR],
                                           ColOf &&col_of, int c0 = 0) {
    constexpr int SLOT = 64 * NCM;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < NCM; ++t) part[wv * SLOT + 64 * t + lane] = cm[t];
    // a unit of one row block reads back only its own maxima
    if (n_rb > 1) lds_barrier();
    else asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const float *base = part + (wv - rb) * SLOT + lane;
    float *mine = stage + wv * SLOT;
#pragma unroll
    for (int t = 0; t < NCM; ++t) {
        float m = base[64 * t];
        for (int w = 1; w < n_rb; ++w) m = fmaxf(m, base[w * SLOT + 64 * t]);
        snew[t] = m / R;
        mine[col_of(t, lane)] = rd_div(R, m);
    }
    // this wavefront's own writes, read back by its other lanes: LDS keeps a
    // wavefront's accesses in order, the compiler must not reorder them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < NVR; ++i) invrow[i] = mine[c0 + 16 * i + (lane & 15)];
}

// u[e] = fma(g, row element e of kv, u[e]) for e < 16
__device__ __forceinline__ void axpy16(float *u, float g, float kv) {
    asm("s_nop 1\n"
        "v_fmac_f32_dpp %0, %17, %16 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %17, %16 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %17, %16 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %17, %16 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %4, %17, %16 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %5, %17, %16 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %6, %17, %16 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %7, %17, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %8, %17, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %9, %17, %16 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %10, %17, %16 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %11, %17, %16 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %12, %17, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %13, %17, %16 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %14, %17, %16 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %15, %17, %16 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        : LORES_PV16(u)
        : "v"(g), "v"(kv));
}

template <bool BF16IN>
__device__ __forceinline__ float in_scalar(const void *__restrict__ p, long idx) {
    if constexpr (BF16IN) {
        return __uint_as_float((uint32_t)((const uint16_t *)p)[idx] << 16);
    } else {
        return ((const float *)p)[idx];
    }
}

// Prefetched inputs: a bf16 element is held as its 16 bits (zero-extended)
// until the task that uses it widens it, so nothing waits for the load
// where it is issued.
template <bool BF16IN>
__device__ __forceinline__ float in_raw(const void *__restrict__ p, long idx) {
    if constexpr (BF16IN) {
        return __uint_as_float((uint32_t)((const uint16_t *)p)[idx]);
    } else {
        return ((const float *)p)[idx];
    }
}
template <bool BF16IN>
__device__ __forceinline__ float from_raw(float x) {
    if constexpr (BF16IN) return __uint_as_float(__float_as_uint(x) << 16);
    else return x;
}

// ---------------------------------------------------------------------------
// A unit's code rows through a buffer resource: chunk c of a lane's row is at
// byte voff + c * cstride of the unit's codes (voff = 16 row, cstride =
// 16 d_v_pad), so a load takes the lane's offset from one VGPR and the
// chunk's from an SGPR, with no per-access address arithmetic in the vector
// ALU (a store adds the two in a VGPR, below).  The resource's size is the
// unit's code bytes: an access outside it reads zeros and writes nothing.
// ---------------------------------------------------------------------------
struct CodeRows {
    __amdgpu_buffer_rsrc_t rsrc;
    int voff, cstride;

    // raw (untyped) 32-bit data format, the buffer-resource word 3 of gfx9 parts
    static constexpr int kRawFormat = 0x00020000;
    static constexpr int kNT = 2;                  // nontemporal

    // c0: the lane's first chunk of the row (a lane holding the second half
    // of a split row starts there)
    __device__ __forceinline__ CodeRows(const uint8_t *unit_codes, long unit_bytes, int row,
                                        long dv_pad, int c0 = 0)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(unit_codes), 0,
                                                 (int)unit_bytes, kRawFormat)),
          voff(row * 16 + c0 * (int)dv_pad * 16), cstride((int)dv_pad * 16) {}
    __device__ __forceinline__ u32x4 load(int c) const {
        return __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, c * cstride, kNT);
    }
    // A store of more than 64 bits needs one wait state before a VALU
    // instruction rewrites its data registers; the compiler inserts it for a
    // buffer store only when the store's SGPR offset field holds no register.
    // With the chunk's offset there, the next chunk's first packed word has
    // been seen to overwrite dword 0 of a store in flight (in lanes 12..15
    // of each row), so a store takes its whole offset from the VGPR.
    __device__ __forceinline__ void store(int c, u32x4 v) const {
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, voff + c * cstride, 0, kNT);
    }
};

// ---------------------------------------------------------------------------
// requantization of one row (one lane): fresh scale, rounding, packing and
// store of the row's 16-byte chunks (chunk c through `io`).  Shared by
// the step and by the fp32 -> packed state entry.
// ---------------------------------------------------------------------------
// KEY: key-column scales; invrow holds r / m_j as row vectors (register i,
// column 16 i + lane % 16), m and scale_out are unused (the caller stores
// the column scales).  col0: the row's column of U[0] (a split row's second
// lane: its draws continue the row's, and the other lane stores the scale).
template <int DK, int PREC, bool KEY = false>
__device__ __forceinline__ void requantize_row(const float (&U)[DK], float m, const StepMeta &meta,
                                               int b, int h, int row, bool active,
                                               const CodeRows &io, float *scale_out,
                                               const float *invrow = nullptr, int col0 = 0) {
    constexpr int E = Prec<PREC>::E;
    constexpr int NCH = row_chunks<DK, PREC>();
    static_assert(!KEY || has_scale<PREC>(), "key-column scales belong to scaled classes");
    float inv = 0.0f;
    if constexpr (has_scale<PREC>() && !KEY) {
        float snew;
        if constexpr (is_int<PREC>()) snew = div_by_r<PREC>(m);
        else snew = m / Prec<PREC>::R;
        inv = rd_div(Prec<PREC>::R, m);
        if (active && col0 == 0) *scale_out = snew;
    }
    // int: x holds the fma addend bias + n_ij * 2^-16 of the current
    // column (in [128, 256), where one fp32 ulp is 2^-16: the draw is the
    // low 16 mantissa bits); bf16: x holds the draws of columns 0 and 1.
    // Round-to-nearest is the constant draw 2^15 (first draw 2^15, step 0).
    const bool nearest = meta.rounding == LORES_ROUND_NEAREST;
    uint32_t x = 0;
    if constexpr (PREC != LORES_FP32) {
        const uint32_t K = unit_key(meta.seed, meta.t, (uint64_t)(meta.seq_base + b),
                                    (uint64_t)(meta.head_base + h));
        uint32_t n0 = fmix32(K ^ (uint32_t)row) & 0xFFFFu;
        // int classes: one draw per column pair (col0 is even)
        n0 = nearest ? 0x8000u
                     : (n0 + (uint32_t)(is_int<PREC>() ? col0 >> 1 : col0) * kPsi16) & 0xFFFFu;
        const uint32_t n1 = nearest ? n0 : (n0 + kPsi16) & 0xFFFFu;
        if constexpr (is_int<PREC>()) x = (Prec<PREC>::FBASE & 0xFFFF0000u) | n0;
        else if constexpr (PREC == LORES_BF16) x = n0 | (n1 << 16);
        else x = n0;                                     // fp8: the draw alone
    }
    const uint32_t psi = opaque_uniform(nearest ? 0u : kPsi16);
    const uint32_t psi2 = opaque_uniform(nearest ? 0u : ((2 * kPsi16) & 0xFFFFu) * 0x00010001u);
    if constexpr (PREC == LORES_INT6) {
        // floor(z) = 128 + field; add it shifted into place and take the
        // fields' bit 7 back out with one constant per word (folded into the
        // initial value), so no field needs a mask.  Chunk by chunk: a chunk
        // is stored as soon as its four words are complete, and the draw
        // register is pinned after each store, so the compiler cannot compute
        // every element's sum up front and hold them all.
        constexpr Int6Stray<DK> stray;
        int j = 0;
        uint32_t carry = 0;                  // high bits of a field crossing into the next chunk
        float zb[4];                         // key columns: sums of columns j & ~3 .. (j & ~3) + 3
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            uint32_t acc[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = 0u - stray.k[4 * c + k];
            acc[0] += carry;
            carry = 0;
#pragma unroll
            for (; j < DK && 6 * j < 128 * (c + 1); ++j) {
                float z;
                if constexpr (KEY) {
                    if ((j & 3) == 0) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            zb[e] = __uint_as_float(x);
                            if (e & 1) x = step16(x, psi);
                        }
                        fmac4_col(zb, invrow[j >> 4], &U[j], j & 15);
                    }
                    z = zb[j & 3];
                } else {
                    // an odd column rounds -U with its pair's draw
                    z = __builtin_fmaf((j & 1) ? -U[j] : U[j], inv, __uint_as_float(x));
                    if (j & 1) x = step16(x, psi);
                }
                const uint32_t e = (uint32_t)z;
                const int bit = 6 * j - 128 * c, w = bit >> 5, o = bit & 31;
                acc[w] += e << o;
                if (o > 26) {
                    if (w < 3) acc[w + 1] += e >> (32 - o);
                    else carry = e >> (32 - o);
                }
            }
            if (active)
                io.store(c, u32x4{acc[0], acc[1], acc[2], acc[3]});
            asm volatile("" : "+v"(x));
        }
    } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            uint32_t ow[4];
            if constexpr (PREC == LORES_INT8) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int j = c * E + q4 * 4;
                    float z[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // an odd column rounds -U with its pair's draw
                        if constexpr (KEY) z[e] = __uint_as_float(x);
                        else z[e] = __builtin_fmaf((e & 1) ? -U[j + e] : U[j + e], inv, __uint_as_float(x));
                        if (e & 1) x = step16(x, psi);
                    }
                    if constexpr (KEY) fmac4_col(z, invrow[j >> 4], &U[j], j & 15);
                    const float z0 = z[0], z1 = z[1], z2 = z[2], z3 = z[3];
                    uint32_t word = (uint32_t)z0;           // 1 <= z < 256: bytes 1..3 are 0
                    cvt_u8_into<1>(word, z1);
                    cvt_u8_into<2>(word, z2);
                    cvt_u8_into<3>(word, z3);
                    ow[q4] = word;
                }
            } else if constexpr (PREC == LORES_INT4) {
                // floor(z) in [129, 143]: floor(z) - 128 is the offset-binary code c + 8
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int j = c * E + q4 * 8;
                    if (j >= DK) {                   // the padding of a half chunk
                        ow[q4] = 0u;
                        continue;
                    }
                    float ze[4], zo[4];
                    if constexpr (KEY) {
                        float z[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            z[e] = __uint_as_float(x);
                            if (e & 1) x = step16(x, psi);
                        }
                        fmac4_col(z, invrow[j >> 4], &U[j], j & 15);
                        fmac4_col(z + 4, invrow[j >> 4], &U[j + 4], (j + 4) & 15);
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            ze[p] = z[2 * p];
                            zo[p] = z[2 * p + 1];
                        }
                    } else {
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            // the odd column rounds -U with the pair's draw
                            ze[p] = __builtin_fmaf(U[j + 2 * p], inv, __uint_as_float(x));
                            zo[p] = __builtin_fmaf(-U[j + 2 * p + 1], inv, __uint_as_float(x));
                            x = step16(x, psi);
                        }
                    }
                    // z lies in [128, 256), where bits 16..22 of its fp32
                    // pattern are floor(z) - 128 = code + 8 (<= 15) and bit
                    // 23 is 0: byte 2 of each z is its stored nibble
                    const uint32_t ev = gather_byte2(ze);
                    const uint32_t od = gather_byte2(zo);
                    ow[q4] = ev | (od << 4);
                }
            } else if constexpr (PREC == LORES_FP8) {
                // y = U * inv in [-448, 448]; fl(y * 2^-120) puts the E4M3
                // grid on the fp32 pattern with its low 20 bits dropped (E4M3
                // subnormals on fp32 denormals): add the draw at bits 4..19,
                // keep the sign (bit 31) and the next 7 bits (20..26; bits
                // 27..30 are 0 since |y| <= 448).  Two elements at a time:
                // their high halves side by side, shifted right by 4 in each
                // half (v_pk_lshrrev_b16) for bits 20..26, merged (v_bfi)
                // with their top bytes for the signs.
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int j = c * E + q4 * 4;
                    uint32_t t[4], pr[2];
                    float yk[4];
                    if constexpr (KEY) mul4_col(yk, invrow[j >> 4], &U[j], j & 15);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float y;
                        if constexpr (KEY) y = yk[e];
                        else y = U[j + e] * inv;
                        t[e] = __float_as_uint(y * 0x1p-120f) + (x << 4);
                        x = step16(x, psi);
                    }
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const uint32_t hi = __builtin_amdgcn_perm(t[2 * h2 + 1], t[2 * h2], 0x07060302u);
                        const uint32_t sg = __builtin_amdgcn_perm(t[2 * h2 + 1], t[2 * h2], 0x0c070c03u);
                        const uint32_t pl = __builtin_bit_cast(
                            uint32_t, __builtin_bit_cast(u16x2, hi) >> (u16x2){4, 4});
                        pr[h2] = (pl & 0x007F007Fu) | (sg & ~0x007F007Fu);
                    }
                    // byte 0 of each half: elements 0..3 into bytes 0..3
                    ow[q4] = __builtin_amdgcn_perm(pr[1], pr[0], 0x06040200u);
                }
            } else if constexpr (PREC == LORES_BF16) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int j = c * E + q4 * 2;
                    // draws of columns j, j + 1: those of columns 0, 1 plus
                    // (j / 2) * 2 psi in each half (one v_pk_mad_u16)
                    const u16x2 kk = {(unsigned short)(j >> 1), (unsigned short)(j >> 1)};
                    const uint32_t xj = __builtin_bit_cast(
                        uint32_t, __builtin_bit_cast(u16x2, x) + kk * __builtin_bit_cast(u16x2, psi2));
                    const uint32_t b0 = __float_as_uint(U[j]) + (xj & 0xFFFFu);
                    const uint32_t b1 = __float_as_uint(U[j + 1]) + (xj >> 16);
                    ow[q4] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
                }
            } else {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) ow[q4] = __float_as_uint(U[c * E + q4]);
            }
            if (active) io.store(c, u32x4{ow[0], ow[1], ow[2], ow[3]});
            // key-column rows: keep the next chunk's draws after this store
            // (unpinned, the cheap, input-independent chain may be computed
            // up front and held in registers)
            if constexpr (KEY) asm volatile("" : "+v"(x));
        }
    }
}

// ---------------------------------------------------------------------------
// one (class, head slot, row block) stream of tasks
// ---------------------------------------------------------------------------
// A wavefront owns one (head slot, row block) of a class and walks the
// sequences b = blockIdx.y, blockIdx.y + gridDim.y, ...  `issue` starts the
// loads of one task: its chunks, row scale and v, alpha and beta, and k and
// q (and a per-channel alpha) as row vectors; `run` computes and stores the
// task and calls `mid` right after pass 1, when the chunk registers are free,
// so the caller can start the next task's loads there.
constexpr int kMaxPrefetchChunks = 8;    // int8 and int4 rows of d_k <= 128

// Per-task values loaded ahead of the task, besides its chunks: the row
// scale and v of this lane's row, beta and a scalar alpha, and k, q and a
// per-channel alpha as row vectors (NV registers each).  With bf16 inputs, v,
// k and q hold the raw 16 bits (from in_raw) until `run` widens them.
// With key-column scales, sl and al hold the unit's column scales and a
// per-channel alpha in lane form (lane L: columns 64 t + L), two registers
// each at d_k = 128 (one per 64 columns, the last one padded with zeros at
// d_k = 32, 96); the row vectors of their product are built at the start of
// the task.
// WPC: the end of a window whose tokens carry one decay per key channel:
// av (al with key-column scales) holds the window's first token's decays and
// avt this step's, as row vectors.
template <int NV, bool KEY = false, bool WPC = false, int KG = 1>
struct TaskSide {
    float s = 0.0f, v = 0.0f, alpha = 1.0f, beta = 0.0f;
    float alpha_t = 1.0f;              // window end: this step's decay (alpha is token 1's)
    float kv[NV], qv[NV], av[KEY ? 1 : NV];
    float sl[KEY ? KG : 1], al[KEY ? KG : 1];   // KG: 64-column groups of the row
    float avt[WPC ? NV : 1];
};

// KEY: key-column scales (d_k per unit); the unit's row blocks are the
// wavefronts wv - rb .. wv - rb + n_rb - 1 of one work-group, and `lds`
// holds two buffers of kWavesPerGroup x DK column maxima (tasks alternate
// between them) and a kWavesPerGroup x DK staging area.
// WEND: the last step of a window of a windowed state: pass 1
// dequantizes with the window's first decay, then the window buffer's
// tokens are replayed on U before this step's token.
// SPLIT (d_k > 128): a row of d_k fp32 values does not fit one lane's
// registers beside the rest, so two lanes share it: lane L < 32 holds
// columns [0, d_k / 2) of row 32 rb + L and lane L + 32 the other half
// (each half of a stored row starts on a chunk: the layout pads each half to
// whole 16-byte chunks).  Each lane runs the per-lane code on its
// CPL = d_k / 2 columns (an int4 half of 80 or 112 columns ends inside its
// last chunk); r, o and the row maximum are combined across the pair with
// one v_permlane32_swap each (in the same order in both lanes, so both hold
// the same values), and the second lane's draws start at column CPL.
template <int DK, int PREC, bool PC, bool DELTA, bool BF16IN, bool KEY = false, bool WEND = false>
struct TaskStream {
    static constexpr bool SPLIT = DK > 128;
    static constexpr int CPL = SPLIT ? DK / 2 : DK;   // columns per lane
    static constexpr int RPW = SPLIT ? 32 : 64;       // rows per wavefront task
    static_assert(DK % 32 == 0 && DK <= 256, "d_k a multiple of 32, at most 256");
    static constexpr int E = Prec<PREC>::E;
    static constexpr int NCH = row_chunks<CPL, PREC>();   // chunks of the lane's columns
    static_assert(PREC == LORES_INT6 || CPL % E == 0 || (PREC == LORES_INT4 && CPL % 16 == 0),
                  "a lane's columns end on a chunk (int4 halves: on a half chunk)");

    const void *__restrict__ qp;
    const void *__restrict__ kp;
    const void *__restrict__ vp;
    const float *__restrict__ alphap;
    const float *__restrict__ betap;
    float *__restrict__ op;
    uint8_t *__restrict__ codes;
    float *__restrict__ scales;
    const StepMeta &meta;
    int Hc, slot, h, row, lrow, rb, half;
    long unit_bytes;
    bool active;
    float *lds;
    const float *win;                  // window buffers of the class (WEND)

    __device__ __forceinline__ TaskStream(const void *q, const void *k, const void *v,
                                          const float *alpha, const float *beta, float *o,
                                          uint8_t *c, float *sc, const StepMeta &m,
                                          const ClassDesc &cd, int task, float *lds_ = nullptr,
                                          const float *win_ = nullptr)
        : qp(q), kp(k), vp(v), alphap(alpha), betap(beta), op(o), codes(c), scales(sc), meta(m),
          lds(lds_), win(win_) {
        const int n_rb = m.n_rb;
        slot = n_rb == 1 ? task : n_rb == 2 ? task >> 1 : n_rb == 4 ? task >> 2 : task / n_rb;
        rb = task - slot * n_rb;
        Hc = cd.Hc;
        unit_bytes = cd.unit_bytes;
        h = (int)m.heads[cd.head_off + slot];
        half = SPLIT ? (int)(threadIdx.x & 63) >> 5 : 0;
        row = rb * RPW + (threadIdx.x & (RPW - 1));
        active = row < m.dv;
        // padding rows (row >= d_v) load row d_v - 1 and store nothing, so
        // they repeat a real row (and leave column maxima unchanged)
        lrow = active ? row : m.dv - 1;
    }

    static constexpr int NV = CPL / 16;           // row-vector registers per vector
    using Side = TaskSide<NV, KEY, WEND && PC, key_groups<DK>()>;

    // Loads of task b: chunks [C0, C1) and, with C0 = 0, the per-task values.
    template <int C0 = 0, int C1 = NCH>
    __device__ __forceinline__ void issue(int b, u32x4 *cw, Side &in) const {
        const long dv_pad = meta.dv_pad;
        const long unit = (long)b * Hc + slot;
        const long bh = (long)b * meta.H + h;
        const CodeRows io(codes + unit * unit_bytes, unit_bytes, lrow, dv_pad, half * NCH);
#pragma unroll
        for (int c = C0; c < C1; ++c) cw[c] = io.load(c);
        if constexpr (C0 != 0) return;
        // window end with channel decays: pass 1 decays with the window's
        // first token's, held in slot 0 of the unit's window buffer
        const float *wa1 = nullptr;
        if constexpr (WEND && PC)
            wa1 = win + unit * window_unit_floats(meta.window, meta.dv_pad, DK) +
                  (long)(meta.window - 1) * (meta.dv_pad + DK);
        if constexpr (KEY) {
#pragma unroll
            for (int t = 0; t < key_groups<DK>(); ++t) {
                const int col = 64 * t + (threadIdx.x & 63);
                in.sl[t] = 0.0f;
                in.al[t] = 1.0f;
                if (64 * t + 64 <= DK || col < DK) {
                    in.sl[t] = scales[unit * DK + col];
                    if constexpr (PC && WEND) in.al[t] = wa1[col];
                    else if constexpr (PC) in.al[t] = alphap[bh * DK + col];
                }
            }
        } else if constexpr (has_scale<PREC>()) {
            in.s = scales[unit * dv_pad + lrow];
        }
        in.v = in_raw<BF16IN>(vp, bh * meta.dv + lrow);
        in.beta = betap[bh];
        in.alpha = PC ? 1.0f : alphap[bh];
        if constexpr (WEND && !PC) {
            // pass 1 decays with the window's first token's alpha
            in.alpha_t = in.alpha;
            in.alpha = win[unit * window_unit_floats(meta.window, meta.dv_pad, DK) +
                           (long)(meta.window - 1) * (meta.dv_pad + DK)];
        }
        // row vectors: register i holds element 16 i + lane % 16 (of the
        // lane's half of the columns with SPLIT)
        const long kb = bh * DK + half * CPL + (threadIdx.x & 15);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            in.kv[i] = in_raw<BF16IN>(kp, kb + 16 * i);
            in.qv[i] = in_raw<BF16IN>(qp, kb + 16 * i);
            if constexpr (PC && WEND) {
                in.avt[i] = alphap[kb + 16 * i];
                if constexpr (!KEY) in.av[i] = wa1[half * CPL + 16 * i + (threadIdx.x & 15)];
            } else if constexpr (PC && !KEY) {
                in.av[i] = alphap[kb + 16 * i];
            }
        }
    }

    template <class Mid>
    __device__ __forceinline__ void run(int b, const u32x4 *cw, const Side &in,
                                        Mid &&mid, int buf = 0) const {
        const float s = in.s, vi = from_raw<BF16IN>(in.v);
        float kv[NV], qv[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            kv[i] = from_raw<BF16IN>(in.kv[i]);
            qv[i] = from_raw<BF16IN>(in.qv[i]);
        }
        const long dv_pad = meta.dv_pad;
        const long unit = (long)b * Hc + slot;
        const long bh = (long)b * meta.H + h;           // index into [B][H] inputs
        const CodeRows io(codes + unit * unit_bytes, unit_bytes, row, dv_pad, half * NCH);

        const float beta = in.beta;
        const float alpha_s = in.alpha;
        float a = 0.0f, na = 0.0f;
        // key columns: sig_j = fl(s_j * alpha_j), turned into row vectors
        // through this wavefront's staging slot
        float sig[KEY ? NV : 1];
        if constexpr (KEY) {
            const int lane = threadIdx.x & 63;
            constexpr int SLOT = key_slot<DK>(), LW = key_lds_waves<DK>();
            float *mine = lds + 2 * LW * SLOT + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * SLOT;
#pragma unroll
            for (int t = 0; t < key_groups<DK>(); ++t)
                mine[64 * t + lane] = in.sl[t] * (PC ? in.al[t] : alpha_s);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int i = 0; i < NV; ++i) sig[i] = mine[half * CPL + 16 * i + (lane & 15)];
        } else if constexpr (is_int<PREC>() && !PC) {
            a = s * alpha_s;
            na = a * -Prec<PREC>::OFF;
        } else if constexpr (PREC == LORES_FP8 && !PC) {
            a = s * alpha_s;
        }

        // ---- pass 1: dequantize, decay, delta projection r = S'_i . k
        float U[CPL];
        float r = 0.0f;
        float aj[16];                                    // s * alpha_j of one group (int, per channel)
        // after each group of 16 columns: per-channel decay of float heads,
        // then the group's share of r
        auto group_done = [&](int j) {
            if constexpr (PC && !has_scale<PREC>()) mul16(&U[j - 15], in.av[j >> 4]);
            if constexpr (KEY) {
                if constexpr (is_int<PREC>()) mul16n(&U[j - 15], sig[j >> 4]);   // odd columns negated
                else mul16(&U[j - 15], sig[j >> 4]);
            }
            if constexpr (DELTA && !WEND) dot16(r, &U[j - 15], kv[j >> 4]);
            // without the projection nothing orders pass 1 before the
            // next task's loads; materialize the group here so the
            // chunk registers are free when `mid` reuses them
            else pin16(&U[j - 15]);
        };
        // Value-row int8, int4 and int6 codes under a scalar decay take the
        // code and the dequantization in one v_fma_mix_f32 (MIX): the code's
        // bits as an f16 half times a 2^24, plus -off a (an int6 field is
        // extracted into the low bits of a dword first; int6 only on lanes of
        // 128 columns, where it measured faster: elsewhere it did not).
        // a 2^24 must be finite, so a wavefront with a row scale near the top
        // of the fp32 range takes the conversion and fma instead (the same
        // values).
        constexpr bool kMixable =
            (PREC == LORES_INT8 || PREC == LORES_INT4 || (PREC == LORES_INT6 && CPL == 128)) &&
            !KEY && !PC;
        // Key-column int4 rows take the bare code the same way,
        // fma_mix(P 2^-24, 2^24, -off) = P - off, exact, in place of a
        // conversion and a subtraction; the column factor (and the odd
        // column's sign) follows per group of 16 (mul16n).  int8 keeps its
        // one-instruction sign-extending conversion; key-column int6 rows
        // compiled this way spilled 46 registers and ran 61 % slower.
        constexpr bool kKeyMix = KEY && PREC == LORES_INT4;
        if constexpr (kKeyMix) {
            a = 1.0f;
            na = -Prec<PREC>::OFF;
        }
        const float A0 = a * 0x1p24f, A1 = a * 0x1p20f;
        auto pass1 = [&](auto mix_flag) {
        constexpr bool MIX = decltype(mix_flag)::value;
        if constexpr (PREC == LORES_INT6) {
            // MIX reads the chunks through an opaque copy, so that the two
            // forms' field extracts are not shared and hoisted above the
            // branch between them (which would hold every field at once)
            u32x4 cv[NCH];
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                cv[c] = cw[c];
                if constexpr (MIX) asm volatile("" : "+v"(cv[c]));
            }
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                if constexpr (PC && !KEY) {
                    if ((j & 15) == 0) scale16(aj, s, in.av[j >> 4]);
                }
                // an odd column's stored code is negated
                if constexpr (MIX) {
                    // (key columns: the sign comes with the column factor)
                    U[j] = (!KEY && (j & 1)) ? mix_f16n(int6_field(cv, j), 0, A0, na)
                                             : mix_f16(int6_field(cv, j), 0, A0, na);
                    if ((j & 15) == 15) group_done(j);
                    continue;
                }
                const float ub = (float)int6_field(cv, j);
                if constexpr (KEY) U[j] = ub - Prec<PREC>::OFF;     // times +-sig_j per group
                else if constexpr (PC) U[j] = ((j & 1) ? -(ub - Prec<PREC>::OFF) : ub - Prec<PREC>::OFF) * aj[j & 15];
                else U[j] = (j & 1) ? __builtin_fmaf(ub, -a, -na) : __builtin_fmaf(ub, a, na);
                if ((j & 15) == 15) group_done(j);
            }
        } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const uint32_t wd[4] = {cw[c].x, cw[c].y, cw[c].z, cw[c].w};
            // MIX: the codes of each dword spread over f16 halves, each half
            // holding one code in its low bits.  int8: bytes 0, 2 and bytes
            // 1, 3.  int4 (nibble k = element 8 d + k): nibbles 0, 4 and
            // 1, 5 (the latter times 16, so read with a 2^20), then the same
            // of bytes 1 and 3.
            uint32_t hv[4][4] = {};
            if constexpr (MIX && PREC == LORES_INT8) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    hv[d][0] = wd[d] & 0x00FF00FFu;
                    hv[d][1] = odd_bytes(wd[d]);
                }
            } else if constexpr (MIX && PREC == LORES_INT4) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t t = odd_bytes(wd[d]);
                    hv[d][0] = wd[d] & 0x000F000Fu;
                    hv[d][1] = wd[d] & 0x00F000F0u;
                    hv[d][2] = t & 0x000F000Fu;
                    hv[d][3] = t & 0x00F000F0u;
                }
            }
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int j = c * E + e;
                if (j >= CPL) break;                     // the padding of a half chunk
                if constexpr (PC && has_scale<PREC>() && !KEY) {
                    if ((j & 15) == 0) scale16(aj, s, in.av[j >> 4]);
                }
                float sp;
                if constexpr (PREC == LORES_FP8) {
                    // the E4M3 value (hardware decode of byte e & 3), times s * alpha
                    const float v = fp8_value(wd[e >> 2], e & 3);
                    if constexpr (KEY) sp = v;                       // times sig_j per group
                    else if constexpr (PC) sp = v * aj[j & 15];
                    else sp = v * a;
                } else if constexpr (MIX && PREC == LORES_INT8) {
                    // an odd column's stored code is negated
                    sp = (e & 1) ? mix_f16n(hv[e >> 2][e & 1], (e >> 1) & 1, A0, na)
                                 : mix_f16(hv[e >> 2][e & 1], (e >> 1) & 1, A0, na);
                } else if constexpr (MIX && PREC == LORES_INT4) {
                    // (key columns: the sign comes with the column factor)
                    sp = (!KEY && (e & 1)) ? mix_f16n(hv[e >> 3][e & 3], (e >> 2) & 1, A1, na)
                                           : mix_f16(hv[e >> 3][e & 3], (e >> 2) & 1,
                                                     (e & 1) ? A1 : A0, na);
                } else if constexpr (PREC == LORES_INT8 || PREC == LORES_INT4) {
                    float ub;
                    if constexpr (PREC == LORES_INT8 && (KEY || PC)) {
                        // the code itself (byte - 128), for a product with a
                        // per-column factor
                        ub = cvt_sbyte(wd[e >> 2] ^ 0x80808080u, e & 3);
                    } else if constexpr (PREC == LORES_INT8) {
                        ub = (float)((wd[e >> 2] >> (8 * (e & 3))) & 0xFFu);
                    } else {
                        // low nibbles (even elements) and high nibbles (odd) as bytes
                        const uint32_t w = wd[e >> 3];
                        const uint32_t nib = (e & 1) ? and_opaque(w >> 4, 0x0F0F0F0Fu)
                                                     : and_opaque(w, 0x0F0F0F0Fu);
                        ub = (float)((nib >> (8 * ((e & 7) >> 1))) & 0xFFu);
                    }
                    constexpr float OFF = PREC == LORES_INT8 && (KEY || PC) ? 0.0f : Prec<PREC>::OFF;
                    // an odd column's stored code is negated
                    if constexpr (KEY) sp = ub - OFF;               // times +-sig_j per group
                    else if constexpr (PC) sp = ((e & 1) ? -(ub - OFF) : ub - OFF) * aj[j & 15];
                    else sp = (e & 1) ? __builtin_fmaf(ub, -a, -na) : __builtin_fmaf(ub, a, na);
                } else if constexpr (PREC == LORES_BF16) {
                    const uint32_t w = wd[e >> 1];
                    sp = __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
                    if constexpr (!PC) sp = sp * alpha_s;
                } else {
                    sp = __uint_as_float(wd[e]);
                    if constexpr (!PC) sp = sp * alpha_s;
                }
                U[j] = sp;
                if ((j & 15) == 15) group_done(j);
            }
        }
        }
        };
        if constexpr (kKeyMix) {
            pass1(Flag<true>{});
        } else if constexpr (kMixable) {
            if (__builtin_amdgcn_ballot_w64(!(a < 0x1p100f)) == 0) pass1(Flag<true>{});
            else pass1(Flag<false>{});
            // Both branches have waited for this task's loads, but the
            // structurized branch leaves a path around them in the compiler's
            // graph: without these uses the next task's loads would be
            // followed by waits for themselves in pass 2.
            pin_inputs<NV>(vi, kv, qv);
        } else {
            pass1(Flag<false>{});
        }

        mid();                                           // the chunks are consumed

        if constexpr (WEND) {
            // the window's buffered tokens: U = fma(g_tau, k_tau, S'_tau), then
            // the next token's S' = fl(U alpha); the slots of token tau + 1 load
            // while token tau is applied
            const int nslot = meta.window - 1;
            const float *ub = win + unit * window_unit_floats(meta.window, meta.dv_pad, DK);
            const float *gs = ub + lrow,
                        *ks = ub + (long)nslot * dv_pad + half * CPL + (threadIdx.x & 15);
            const float *as = ub + (long)nslot * (dv_pad + DK);
            float gt = gs[0], kt[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) kt[i] = ks[16 * i];
            for (int tau = 1; tau <= nslot; ++tau) {
                // the next token's decay: from slot tau, or this step's own
                float gn = 0.0f, kn[NV], an = in.alpha_t, anv[PC ? NV : 1];
                if constexpr (PC) {
#pragma unroll
                    for (int i = 0; i < NV; ++i) anv[i] = in.avt[i];
                }
                if (tau < nslot) {
                    gn = gs[(long)tau * dv_pad];
#pragma unroll
                    for (int i = 0; i < NV; ++i) kn[i] = ks[(long)tau * DK + 16 * i];
                    if constexpr (PC) {
#pragma unroll
                        for (int i = 0; i < NV; ++i)
                            anv[i] = as[(long)tau * DK + half * CPL + 16 * i + (threadIdx.x & 15)];
                    } else {
                        an = as[(long)tau * DK];
                    }
                }
#pragma unroll
                for (int gi = 0; gi < NV; ++gi) axpy16(&U[16 * gi], gt, kt[gi]);
                if constexpr (PC) {
#pragma unroll
                    for (int gi = 0; gi < NV; ++gi) mul16(&U[16 * gi], anv[gi]);
                } else {
#pragma unroll
                    for (int j = 0; j < CPL; ++j) U[j] = U[j] * an;
                }
                gt = gn;
#pragma unroll
                for (int i = 0; i < NV; ++i) kt[i] = kn[i];
            }
            if constexpr (DELTA) {
#pragma unroll
                for (int gi = 0; gi < NV; ++gi) dot16(r, &U[16 * gi], kv[gi]);
            }
        }

        if constexpr (SPLIT && DELTA) r = pair_sum(r);

        // ---- write gate
        const float g = DELTA ? beta * (vi - r) : beta * vi;

        // ---- pass 2: rank-one write, readout, row abs-max
        float o = 0.0f, m = 0.0f;
#pragma unroll
        for (int gi = 0; gi < NV; ++gi) {
            upd16(&U[16 * gi], o, g, kv[gi], qv[gi]);
            if constexpr (!KEY) {
#pragma unroll
                for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(U[16 * gi + e]));
            }
        }
        if constexpr (SPLIT) {
            o = pair_sum(o);
            m = pair_max(m);
        }
        if (active && half == 0) op[bh * meta.dv + row] = o;

        // ---- pass 3: requantize and store in place
        if constexpr (KEY) {
            // column maxima of the unit's rows, fresh column scales
            constexpr int SLOT = key_slot<DK>(), LW = key_lds_waves<DK>();
            constexpr int NCM = SPLIT ? 4 : key_groups<DK>();
            float cm[NCM], snew[NCM], inv[NV];
            if constexpr (SPLIT) col_absmax_split(U, cm);
            else col_absmax<DK>(U, cm);
            auto col_of = [](int j, int L) {
                if constexpr (SPLIT) return key_col_split<CPL>(j, L);
                else return key_col(j, L);
            };
            const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
            key_scales(cm, lds + buf * (LW * SLOT), lds + 2 * LW * SLOT, wv, rb, meta.n_rb,
                       Prec<PREC>::R, snew, inv, col_of, half * CPL);
            if (rb == 0) {
#pragma unroll
                for (int t = 0; t < NCM; ++t) {
                    const int col = col_of(t, threadIdx.x & 63);
                    if (col < DK) scales[unit * DK + col] = snew[t];
                }
            }
            requantize_row<CPL, PREC, true>(U, 0.0f, meta, b, h, row, active, io, nullptr,
                                            inv, half * CPL);
        } else {
            requantize_row<CPL, PREC>(U, m, meta, b, h, row, active, io,
                                      has_scale<PREC>() ? scales + unit * dv_pad + row : nullptr,
                                      nullptr, half * CPL);
        }
    }
};

// One stream over its sequences (at most kSeqPerWave of them unless the
// batch exceeds the grid's y limit).  Right after pass 1 of a task (when
// the chunk registers are free) the next sequence's per-task values and
// first chunks are loaded: all of an int row, the first kMaxPrefetchChunks
// of a bf16 row (the rest are loaded as that task starts), none of an fp32
// row.  The loop body holds two tasks, so the prefetched per-task values
// alternate between two register sets instead of being copied.
template <int DK, int PREC, bool PC, bool DELTA, bool BF16IN, bool KEY, bool WEND>
__device__ __forceinline__ void run_single(
    const TaskStream<DK, PREC, PC, DELTA, BF16IN, KEY, WEND> &ts) {
    using TS = TaskStream<DK, PREC, PC, DELTA, BF16IN, KEY, WEND>;
    // fp32 rows (32 chunks at d_k = 128) leave no registers for a prefetch
    // beside U: only their per-task values are loaded ahead.  A window end
    // with channel decays holds the replay's row vectors as well, so its
    // 8-chunk rows (int8, E4M3) prefetch half their chunks, which leaves
    // room for two wavefronts per SIMD.
    constexpr int P = WEND && PC && TS::NCH == 8 ? 4
                    : TS::NCH <= kMaxPrefetchChunks ? TS::NCH
                    : PREC == LORES_BF16 ? kMaxPrefetchChunks : 0;
    const int bstep = gridDim.y;
    u32x4 cw[TS::NCH];
    typename TS::Side in0, in1;
    int b = blockIdx.y;
    ts.issue(b, cw, in0);
    while (true) {
        int bn = b + bstep;
        ts.run(b, cw, in0, [&] {
            if (bn < ts.meta.B) ts.template issue<0, P>(bn, cw, in1);
        }, 0);
        if (bn >= ts.meta.B) break;
        b = bn;
        bn = b + bstep;
        if constexpr (P < TS::NCH) ts.template issue<P, TS::NCH>(b, cw, in1);
        ts.run(b, cw, in1, [&] {
            if (bn < ts.meta.B) ts.template issue<0, P>(bn, cw, in0);
        }, 1);
        if (bn >= ts.meta.B) break;
        b = bn;
        if constexpr (P < TS::NCH) ts.template issue<P, TS::NCH>(b, cw, in0);
    }
}

// ---------------------------------------------------------------------------
// Work queue of a work-group (launches of a fused int pair).  Wavefronts do
// not progress at the same rate: of two wavefronts sharing a SIMD the older
// one is issued first, so with a fixed share of tasks per wavefront one of
// them finishes long before the other.  A fused-pair launch runs one
// kPairWavesPerGroup-wavefront group per CU whose items are handed out by an
// LDS counter: item n is task slot task_base + n % kPairWavesPerGroup and
// sequence blockIdx.y + (n / kPairWavesPerGroup) gridDim.y, and a wavefront
// takes its next item as it starts a task (slots past the class's last task
// are skipped).
// ---------------------------------------------------------------------------
struct WorkQueue {
    int *counter;                      // LDS, zeroed before the group's first take
    int task_base, n_tasks, total;

    __device__ __forceinline__ WorkQueue(int *c, int base, int n, int B)
        : counter(c), task_base(base), n_tasks(n) {
        const int nb = (B - (int)blockIdx.y + (int)gridDim.y - 1) / (int)gridDim.y;
        total = kPairWavesPerGroup * (nb > 0 ? nb : 0);
    }
    // the next valid item, or -1 when the group's items are used up
    __device__ __forceinline__ int take() const {
        while (true) {
            int n = 0;
            if ((threadIdx.x & 63) == 0)
                n = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            n = __builtin_amdgcn_readfirstlane(n);
            if (n >= total) return -1;
            if (task_base + n % kPairWavesPerGroup < n_tasks) return n;
        }
    }
    __device__ __forceinline__ int task(int n) const { return task_base + n % kPairWavesPerGroup; }
    __device__ __forceinline__ int seq(int n) const {
        return (int)blockIdx.y + (n / kPairWavesPerGroup) * (int)gridDim.y;
    }
};

// One class through the work queue; `make(task)` builds the task's stream.
// Loads are prefetched as in run_single: the next item's per-task values and
// chunks right after pass 1 of the current one.
template <class Make>
__device__ __forceinline__ void run_queue(const WorkQueue &wq, Make &&make) {
    using TS = decltype(make(0));
    constexpr int P = TS::NCH;                   // whole rows are prefetched
    static_assert(P <= kMaxPrefetchChunks, "queued streams hold prefetchable rows");
    u32x4 cw[TS::NCH];
    typename TS::Side in0, in1;
    int n = wq.take();
    if (n < 0) return;
    make(wq.task(n)).issue(wq.seq(n), cw, in0);
    while (true) {
        int nn = wq.take();
        {
            const TS cur = make(wq.task(n));
            const TS nxt = make(wq.task(nn >= 0 ? nn : n));
            cur.run(wq.seq(n), cw, in0, [&] {
                if (nn >= 0) nxt.template issue<0, P>(wq.seq(nn), cw, in1);
            }, 0);
            if (nn < 0) break;
        }
        n = nn;
        nn = wq.take();
        {
            const TS cur = make(wq.task(n));
            const TS nxt = make(wq.task(nn >= 0 ? nn : n));
            cur.run(wq.seq(n), cw, in1, [&] {
                if (nn >= 0) nxt.template issue<0, P>(wq.seq(nn), cw, in0);
            }, 1);
            if (nn < 0) break;
        }
        n = nn;
    }
}

// A fused pair of int classes through the work queue: an item is task p of
// class 0 then task p of class 1 for one sequence, alternating in one
// wavefront, so every SIMD carries the same mix of the VALU-heavier and the
// HBM-heavier class; each task's pass 1 is followed by the loads of the other
// stream's next task.
template <class Make0, class Make1>
__device__ __forceinline__ void run_queue_paired(const WorkQueue &wq, Make0 &&make0, Make1 &&make1) {
    using T0 = decltype(make0(0));
    using T1 = decltype(make1(0));
    static_assert(T0::NCH <= kMaxPrefetchChunks && T1::NCH <= kMaxPrefetchChunks,
                  "paired streams need prefetchable rows");
    u32x4 cw[kMaxPrefetchChunks];
    typename T0::Side in0;
    typename T1::Side in1;
    int n = wq.take();
    if (n < 0) return;
    make0(wq.task(n)).issue(wq.seq(n), cw, in0);
    while (true) {
        const int nn = wq.take();
        const int b = wq.seq(n);
        const T0 a = make0(wq.task(n));
        const T1 c = make1(wq.task(n));
        a.run(b, cw, in0, [&] { c.issue(b, cw, in1); });
        const T0 an = make0(wq.task(nn >= 0 ? nn : n));
        c.run(b, cw, in1, [&] {
            if (nn >= 0) an.issue(wq.seq(nn), cw, in0);
        });
        if (nn < 0) break;
        n = nn;
    }
}

// ---------------------------------------------------------------------------
// the step kernel: one class (P1 < 0) or a fused pair of classes
// ---------------------------------------------------------------------------
// Grid x, single class: groups of kWavesPerGroup tasks of class 0.  Two
// classes side by side (bf16 with an int class): the groups of class 0, then
// those of class 1.  Fused int pair (both classes prefetchable int classes),
// in groups of kPairWavesPerGroup: first the paired groups (task p of class 0
// with task p of class 1), then the remaining tasks of class 0, then those of
// class 1; meta.cls[i].groups then counts the groups of the unpaired
// remainder of class i and the paired groups number
// ceil(min(n0, n1) / kPairWavesPerGroup).
template <int P0, int P1, int DK>
constexpr bool pairable() {
    if constexpr (P1 < 0 || !is_int<P0>() || !is_int<P1>()) {
        return false;
    } else {
        constexpr int C = DK > 128 ? DK / 2 : DK;       // a lane's columns (split rows: half)
        return row_chunks<C, P0>() <= kMaxPrefetchChunks && row_chunks<C, P1>() <= kMaxPrefetchChunks;
    }
}

// Wavefronts per work-group of a launch: fused int pairs run one queued
// group per CU.
template <int P0, int P1, int DK, bool KEY = false>
constexpr int group_waves() {
    return pairable<P0, P1, DK>()   ? kPairWavesPerGroup
           : KEY && DK > 128        ? kMaxKeyGroupWaves
                                    : kWavesPerGroup;
}

// Wavefronts per SIMD the compiler must leave room for.  Left to itself it
// gives the window ends and the per-channel key-column steps up to 294
// registers, so one wavefront per SIMD; held to 256 (two per SIMD) they
// spill 0-32 registers and measured 1-30 % faster.  Everything else keeps
// the compiler's own choice (bf16 rows at d_k = 256 take 259-270 registers
// and measured the same at one or two wavefronts per SIMD).
template <bool KEY, bool WEND>
constexpr int min_waves_per_simd() {
    return KEY || WEND ? 2 : 1;
}

template <int DK, bool PC, bool DELTA, bool BF16IN, int P0, int P1, bool KEY = false,
          bool WEND = false>
__global__ void __launch_bounds__((64 * group_waves<P0, P1, DK, KEY>()))
__attribute__((amdgpu_waves_per_eu(min_waves_per_simd<KEY, WEND>())))
lores_step_kernel(const void *__restrict__ qp, const void *__restrict__ kp,
                  const void *__restrict__ vp, const float *__restrict__ alphap,
                  const float *__restrict__ betap, float *__restrict__ op,
                  uint8_t *__restrict__ codes0, float *__restrict__ scales0,
                  uint8_t *__restrict__ codes1, float *__restrict__ scales1,
                  const float *__restrict__ win0, const StepMeta meta) {
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int gx = blockIdx.x;
    const int n_rb = meta.n_rb;
    static_assert(!WEND || P1 < 0, "window ends run one class per launch");
    if constexpr (WEND && !KEY) {
        // the last step of a window: one scaled class
        const int task = gx * kWavesPerGroup + wv;
        if (task >= meta.cls[0].Hc * n_rb) return;
        run_single(TaskStream<DK, P0, PC, DELTA, BF16IN, false, true>(
            qp, kp, vp, alphap, betap, op, codes0, scales0, meta, meta.cls[0], task, nullptr,
            win0));
    } else if constexpr (KEY) {
        // one class (a step, or with WEND a window's end); the n_rb row
        // blocks of a unit are consecutive tasks, so whole units share a
        // work-group (key_group_waves).  A wave past
        // the last task still takes part in the work-group's barriers: one
        // per sequence of its stride, as a working wave does (units of one
        // row block take no barrier at all).
        static_assert(P1 < 0, "key-column scales run one class per launch");
        __shared__ float cmax[3 * key_lds_waves<DK>() * key_slot<DK>()];  // two maxima buffers, staging
        const int task = gx * key_group_waves(n_rb) + wv;
        if (task >= meta.cls[0].Hc * n_rb) {
            if (n_rb > 1)
                for (int b = blockIdx.y; b < meta.B; b += gridDim.y) lds_barrier();
            return;
        }
        run_single(TaskStream<DK, P0, PC, DELTA, BF16IN, true, WEND>(
            qp, kp, vp, alphap, betap, op, codes0, scales0, meta, meta.cls[0], task, cmax, win0));
    } else if constexpr (P1 < 0) {
        const int task = gx * kWavesPerGroup + wv;
        if (task >= meta.cls[0].Hc * n_rb) return;
        run_single(TaskStream<DK, P0, PC, DELTA, BF16IN>(qp, kp, vp, alphap, betap, op, codes0,
                                                         scales0, meta, meta.cls[0], task));
    } else if constexpr (pairable<P0, P1, DK>()) {
        // fused int pair: the paired tasks, then the rest of either class,
        // each group through its work queue
        __shared__ int counter;
        if (threadIdx.x == 0) counter = 0;
        __syncthreads();
        auto make0 = [&](int task) {
            return TaskStream<DK, P0, PC, DELTA, BF16IN>(qp, kp, vp, alphap, betap, op, codes0,
                                                         scales0, meta, meta.cls[0], task);
        };
        auto make1 = [&](int task) {
            return TaskStream<DK, P1, PC, DELTA, BF16IN>(qp, kp, vp, alphap, betap, op, codes1,
                                                         scales1, meta, meta.cls[1], task);
        };
        const int n0 = meta.cls[0].Hc * n_rb, n1 = meta.cls[1].Hc * n_rb;
        const int paired = n0 < n1 ? n0 : n1;
        const int pg = (paired + kPairWavesPerGroup - 1) / kPairWavesPerGroup;
        if (gx < pg)
            run_queue_paired(WorkQueue(&counter, gx * kPairWavesPerGroup, paired, meta.B), make0,
                             make1);
        else if (gx - pg < meta.cls[0].groups)
            run_queue(WorkQueue(&counter, paired + (gx - pg) * kPairWavesPerGroup, n0, meta.B),
                      make0);
        else
            run_queue(WorkQueue(&counter,
                                paired + (gx - pg - meta.cls[0].groups) * kPairWavesPerGroup, n1,
                                meta.B),
                      make1);
    } else {
        // two classes side by side (bf16 with an int class): groups of class 0, then of class 1
        const int n0 = meta.cls[0].Hc * n_rb, n1 = meta.cls[1].Hc * n_rb;
        const int paired = 0;
        if (gx < meta.cls[0].groups) {
            const int task = paired + gx * kWavesPerGroup + wv;
            if (task >= n0) return;
            run_single(TaskStream<DK, P0, PC, DELTA, BF16IN>(qp, kp, vp, alphap, betap, op,
                                                             codes0, scales0, meta, meta.cls[0],
                                                             task));
        } else {
            const int task = paired + (gx - meta.cls[0].groups) * kWavesPerGroup + wv;
            if (task >= n1) return;
            run_single(TaskStream<DK, P1, PC, DELTA, BF16IN>(qp, kp, vp, alphap, betap, op,
                                                             codes1, scales1, meta, meta.cls[1],
                                                             task));
        }
    }
}

// ---------------------------------------------------------------------------
// launcher: the grid holds every (class, head slot, row block) group along x
// and along y as many sequence strides as fit on the device at once, or, for
// launches without a work queue, enough that no wavefront gets more than
// kSeqPerWave sequences
// ---------------------------------------------------------------------------
// Sequences per wavefront of the launches without a work queue (the second
// prefetched behind the first).
constexpr long kSeqPerWave = 2;

// A failed query here falls back to a default and must not leave its error
// behind for the launch's own check: it is consumed.
inline int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cached[dev] = n;
    }
    return cached[dev];
}

template <int DK, bool PC, bool DELTA, bool BF16IN, int P0, int P1, bool KEY = false,
          bool WEND = false>
hipError_t launch_one(const StepPtrs &p, const StepMeta &m, hipStream_t s) {
    auto kern = lores_step_kernel<DK, PC, DELTA, BF16IN, P0, P1, KEY, WEND>;
    const int W = KEY ? key_group_waves(m.n_rb) : group_waves<P0, P1, DK>();
    static int per_cu_of[kMaxKeyGroupWaves + 1] = {0};   // resident work-groups per CU, by W
    int &per_cu = per_cu_of[W <= kMaxKeyGroupWaves ? W : 0];
    if (!per_cu) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(kern),
                                                         64 * W, 0) != hipSuccess ||
            n <= 0) {
            (void)hipGetLastError();                // not the launch's error
            n = 1;
        }
        per_cu = n;
    }
    int gx = m.cls[0].groups + (P1 < 0 ? 0 : m.cls[1].groups);
    if constexpr (pairable<P0, P1, DK>()) {
        const int n0 = m.cls[0].Hc * m.n_rb, n1 = m.cls[1].Hc * m.n_rb;
        const int paired = n0 < n1 ? n0 : n1;
        gx = (paired + W - 1) / W + (n0 - paired + W - 1) / W + (n1 - paired + W - 1) / W;
    }
    long resident = (long)per_cu * device_cu_count();
    long gy = resident / gx;
    if (gy < 1) gy = 1;
    if constexpr (!pairable<P0, P1, DK>()) {
        // at most kSeqPerWave sequences per wavefront: the grid's further
        // rows are started by the dispatcher as earlier work-groups finish,
        // which balances the CUs better than long fixed streams (a fused
        // pair balances through its work queue instead)
        const long gmin = (m.B + kSeqPerWave - 1) / kSeqPerWave;
        if (gy < gmin) gy = gmin;
    }
    if (gy > 65535) gy = 65535;                     // grid y limit
    if (gy > m.B) gy = m.B;
    hipLaunchKernelGGL(kern, dim3(gx, (unsigned)gy), dim3(64 * W), 0, s, p.q, p.k,
                       p.v, p.alpha, p.beta, p.o, p.codes[0], p.scales[0], p.codes[1],
                       p.scales[1], p.win[0], m);
    return hipGetLastError();
}

template <int DK, int P0, int P1, bool KEY = false>
hipError_t launch_dk(bool pc, bool delta, bool bf16, const StepPtrs &p, const StepMeta &m,
                     hipStream_t s) {
    if (pc) {
        if (delta) return bf16 ? launch_one<DK, true, true, true, P0, P1, KEY>(p, m, s)
                               : launch_one<DK, true, true, false, P0, P1, KEY>(p, m, s);
        return bf16 ? launch_one<DK, true, false, true, P0, P1, KEY>(p, m, s)
                    : launch_one<DK, true, false, false, P0, P1, KEY>(p, m, s);
    }
    if (delta) return bf16 ? launch_one<DK, false, true, true, P0, P1, KEY>(p, m, s)
                           : launch_one<DK, false, true, false, P0, P1, KEY>(p, m, s);
    return bf16 ? launch_one<DK, false, false, true, P0, P1, KEY>(p, m, s)
                : launch_one<DK, false, false, false, P0, P1, KEY>(p, m, s);
}

template <int P0, int P1>
hipError_t launch_classes(int dk, bool pc, bool delta, bool bf16, const StepPtrs &p,
                          const StepMeta &m, hipStream_t s) {
    switch (dk) {
        case 32: return launch_dk<32, P0, P1>(pc, delta, bf16, p, m, s);
        case 64: return launch_dk<64, P0, P1>(pc, delta, bf16, p, m, s);
        case 96: return launch_dk<96, P0, P1>(pc, delta, bf16, p, m, s);
        case 128: return launch_dk<128, P0, P1>(pc, delta, bf16, p, m, s);
        case 160: return launch_dk<160, P0, P1>(pc, delta, bf16, p, m, s);
        case 192: return launch_dk<192, P0, P1>(pc, delta, bf16, p, m, s);
        case 224: return launch_dk<224, P0, P1>(pc, delta, bf16, p, m, s);
        case 256: return launch_dk<256, P0, P1>(pc, delta, bf16, p, m, s);
        default: return hipErrorInvalidValue;
    }
}

// key-column scales: one class per launch
template <int P0>
hipError_t launch_classes_key(int dk, bool pc, bool delta, bool bf16, const StepPtrs &p,
                              const StepMeta &m, hipStream_t s) {
    switch (dk) {
        case 32: return launch_dk<32, P0, -1, true>(pc, delta, bf16, p, m, s);
        case 64: return launch_dk<64, P0, -1, true>(pc, delta, bf16, p, m, s);
        case 96: return launch_dk<96, P0, -1, true>(pc, delta, bf16, p, m, s);
        case 128: return launch_dk<128, P0, -1, true>(pc, delta, bf16, p, m, s);
        case 160: return launch_dk<160, P0, -1, true>(pc, delta, bf16, p, m, s);
        case 192: return launch_dk<192, P0, -1, true>(pc, delta, bf16, p, m, s);
        case 224: return launch_dk<224, P0, -1, true>(pc, delta, bf16, p, m, s);
        case 256: return launch_dk<256, P0, -1, true>(pc, delta, bf16, p, m, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lores
