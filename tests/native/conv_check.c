/* Exhaustive host check of the oracle's storage conversions
 * (oracle/oracle.c, compiled into this program): for every binary32 bit
 * pattern, binary32 -> binary16 equals the x86 F16C conversion (hardware
 * IEEE round to nearest even, subnormals kept), and binary32 -> bfloat16
 * equals the bfloat16 neighbour nearer to x in exact binary64 arithmetic
 * (the even one on a tie, +-infinity past the midpoint towards 2^128); a NaN
 * must give a NaN.  Prints "ok" and exits 0 on success. */
#include <immintrin.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint16_t oracle_f32_to_bf16(float f);
uint16_t oracle_f32_to_f16(float f);

static float f32_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bfloat16 from the definition: the two neighbours of |x| among bfloat16
 * magnitudes, the exact midpoint between them in binary64, and the side x
 * lies on. */
static uint16_t bf16_nearest(float x)
{
    uint32_t u; memcpy(&u, &x, 4);
    const uint32_t sign = u & 0x80000000u, a = u & 0x7fffffffu;
    if (a == 0x7f800000u) return (uint16_t)((sign | a) >> 16);
    const uint32_t lo = a & 0xffff0000u, hi = lo + 0x10000u;
    const double vlo = (double)f32_of(lo);
    const double vhi = hi == 0x7f800000u ? ldexp(1.0, 128) : (double)f32_of(hi);
    const double mid = (vlo + vhi) / 2.0, ax = fabs((double)x);
    uint32_t r = ax < mid ? lo : ax > mid ? hi : (((lo >> 16) & 1u) ? hi : lo);
    return (uint16_t)((sign | r) >> 16);
}

int main(void)
{
    const int f16c = __builtin_cpu_supports("f16c");
    long bad_h = 0, bad_b = 0;
#pragma omp parallel for schedule(static, 1 << 20) reduction(+ : bad_h, bad_b)
    for (int64_t i = 0; i < (int64_t)1 << 32; ++i) {
        const float x = f32_of((uint32_t)i);
        const uint16_t b = oracle_f32_to_bf16(x);
        const uint16_t h = oracle_f32_to_f16(x);
        if (x != x) {
            bad_b += !((b & 0x7f80u) == 0x7f80u && (b & 0x7fu));
            bad_h += !((h & 0x7c00u) == 0x7c00u && (h & 0x3ffu));
            continue;
        }
        bad_b += b != bf16_nearest(x);
        if (f16c) bad_h += h != (uint16_t)_cvtss_sh(x, _MM_FROUND_TO_NEAREST_INT);
    }
    printf("%s bf16_bad=%ld f16_bad=%ld%s\n", (bad_h || bad_b) ? "FAIL" : "ok", bad_b, bad_h,
           f16c ? "" : " (no F16C on this CPU: binary16 not checked)");
    return (bad_h || bad_b) ? 1 : 0;
}
