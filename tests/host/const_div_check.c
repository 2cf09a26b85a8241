/* Exhaustive check of the step kernel's division of a row maximum by a
 * quantizer constant R (2^(b-1) - 1 for b = 4, 6, 8): for every finite
 * non-negative fp32 m,
 *     y = RN(m * z),  q = RN(RN(m - y * R) * z + y),  z = RN(1 / R)
 * (a product and two fused multiply-adds: Markstein's correction step) must
 * equal the IEEE quotient RN(m / R) bit for bit.  Prints the number of
 * mismatches per R; exit status 0 when there are none.
 *
 * The reference RN(m / R) is the float quotient of the host's IEEE
 * division; fmaf is the C library's fused multiply-add (one rounding).  Build
 * with -ffp-contract=off so no other product is fused. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t to_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }

static long mismatches(float R) {
    const float z = 1.0f / R;
    long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(dynamic, 1 << 20)
    for (long p = 0; p < 0x7F800000L; ++p) {          /* +0 up to the largest finite */
        const float m = from_bits((uint32_t)p);
        const float y = m * z;
        const float q = fmaf(fmaf(-y, R, m), z, y);
        if (to_bits(q) != to_bits(m / R)) ++bad;
    }
    return bad;
}

int main(void) {
    const float Rs[] = {7.0f, 31.0f, 127.0f};
    int ok = 1;
    for (int i = 0; i < 3; ++i) {
        const long bad = mismatches(Rs[i]);
        printf("R=%g mismatches=%ld\n", Rs[i], bad);
        if (bad) ok = 0;
    }
    if (ok) printf("const div ok\n");
    return ok ? 0 : 1;
}
