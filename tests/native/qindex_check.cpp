// Host check of the 8-bit quantizer of the library
// (optimizer_update_amd/csrc/qmap.hpp), composed as the kernels compose it:
// the key of the binary64 estimate |v| * r + 2^-27, the key table's est, and one
// exact comparison est + (bound[est] * A < |v|); the signed code adds bit 7
// for v < 0.  The expected index is that of the magnitude nearest to |v| / A
// in exact arithmetic, ties to the smaller: the number of midpoints of
// neighbouring magnitudes that lie below |v| / A, found by a walk over the
// midpoints formed here in x87 extended precision (64-bit significands, so
// the midpoints, their products with A and the comparisons are exact) and
// sharing nothing with the key tables or count_below.
//
// For each absmax A of a set spanning the binary32 range (subnormal, around
// 1, near the largest), every binary32 v with A * 2^-26 <= |v| <= A (every
// v <= A for subnormal A) is checked, together with a sample below that,
// and the reciprocal r is taken three ways: 1/A rounded to binary64, and
// that value moved by 2^-21 relative either way, the widest error the
// kernels' reciprocal can have (qmap.hpp).  NaN values and the blocks with
// absmax 0 or +inf are checked as well.  Prints "ok" and exits 0 on success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "qmap.hpp"

using namespace ou;

static float from_bits(uint32_t u)
{
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

static uint32_t bits(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
}

// The kernels' composition for one state value.
static uint32_t kernel_index(bool is_signed, float v, double r, double A)
{
    const QTables& T = kQTablesHost;
    const QKeys& K = kQKeysHost;
    const uint32_t t = qkey(qestimate(v, r)) - kQKeyFirst;
    if (t >= static_cast<uint32_t>(kQKeys)) return 0xffffffffu;   // outside the table: an error
    if (is_signed) return qsigned(v, qindex(K.s[t], T.sbound, A, v));
    return qindex(K.u[t], T.ubound, A, v);
}

int main()
{
    const QTables& T = kQTablesHost;
    // midpoints in extended precision, from the magnitudes alone
    std::vector<long double> smid, umid;
    for (int k = 0; k + 1 < 128; ++k) smid.push_back(((long double)T.smag[k] + (long double)T.smag[k + 1]) / 2);
    for (int k = 0; k + 1 < 256; ++k) umid.push_back(((long double)T.umag[k] + (long double)T.umag[k + 1]) / 2);

    const float absmaxes[] = {1.0f, 0.75f, from_bits(0x3f7fffff), 1.234567e-3f, 3.0e-20f,
                              0x1p-126f, from_bits(0x00000003), from_bits(0x007fffff),
                              0x1.8p-140f, 3.3e38f, from_bits(0x7f7fffff), 0x1.5p100f};
    long bad = 0, checked = 0;
    for (const float A : absmaxes) {
        const double Ad = A;
        const double r0 = 1.0 / Ad;
        const double rs[3] = {r0, r0 * (1.0 - 0x1p-21), r0 * (1.0 + 0x1p-21)};
        const uint32_t top = bits(A);
        const float low = A * 0x1p-26f;
        const uint32_t first = (low > 0.0f && low >= 0x1p-126f) ? bits(low) : 0u;
        const int64_t lo = first, hi = top;
        constexpr int64_t kChunk = 1 << 18;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad, checked)
        for (int64_t c0 = lo; c0 <= hi; c0 += kChunk) {
            const int64_t c1 = c0 + kChunk - 1 < hi ? c0 + kChunk - 1 : hi;
            // indices at the chunk's first value by a scan, then a walk
            const long double A_l = A;
            uint32_t is = 0, iu = 0;
            const long double v0 = from_bits(static_cast<uint32_t>(c0));
            while (is < smid.size() && smid[is] * A_l < v0) ++is;
            while (iu < umid.size() && umid[iu] * A_l < v0) ++iu;
            for (int64_t u = c0; u <= c1; ++u) {
                const float v = from_bits(static_cast<uint32_t>(u));
                const long double vl = v;
                while (is < smid.size() && smid[is] * A_l < vl) ++is;
                while (iu < umid.size() && umid[iu] * A_l < vl) ++iu;
                for (const double r : rs) {
                    bad += kernel_index(true, v, r, Ad) != is;
                    bad += kernel_index(true, -v, r, Ad) != (v > 0.0f ? (is | 0x80u) : is);
                    bad += kernel_index(false, v, r, Ad) != iu;
                    checked += 3;
                }
            }
        }
        // below A * 2^-26 every index is 0 (a sample of the patterns)
        for (uint32_t u = 0; u < first; u += 4099u) {
            const float v = from_bits(u);
            for (const double r : rs) {
                bad += kernel_index(true, v, r, Ad) != 0u;
                bad += kernel_index(true, -v, r, Ad) != (v > 0.0f ? 0x80u : 0u);
                bad += kernel_index(false, v, r, Ad) != 0u;
                checked += 3;
            }
        }
        // NaN values (every payload's class: quiet, both signs)
        for (const uint32_t u : {0x7fc00000u, 0xffc00000u, 0x7fffffffu, 0xffc12345u}) {
            bad += kernel_index(true, from_bits(u), r0, Ad) != 0u;
            bad += kernel_index(false, from_bits(u), r0, Ad) != 0u;
        }
    }
    // absmax 0 (every value +-0 or NaN) and +inf (finite values have ratio
    // 0, infinite ones NaN): the kernels' reciprocal is 0 there
    const double inf = __builtin_huge_val();
    for (const float v : {0.0f, -0.0f, from_bits(0x7fc00000u)}) {
        bad += kernel_index(true, v, 0.0, 0.0) != 0u;
        bad += kernel_index(false, v, 0.0, 0.0) != 0u;
    }
    for (const float v : {0.0f, 1.0f, 3.0e38f, -2.0f, static_cast<float>(inf), -static_cast<float>(inf)}) {
        bad += kernel_index(true, v, 0.0, inf) != (v < 0.0f ? 0x80u : 0u);
        bad += kernel_index(false, std::fabs(v), 0.0, inf) != 0u;
    }
    std::printf("%s bad=%ld checked=%ld\n", bad == 0 ? "ok" : "FAIL", bad, checked);
    return bad == 0 ? 0 : 1;
}
