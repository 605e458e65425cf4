// qmap.hpp -- the 8-bit dynamic data type of block-wise quantized optimizer
// states, built at compile time.
//
// The page "Investigate a 256-thread SM103 path for small 32-bit optimizer
// tensors" names the 8-bit optimizers only (AdamW8bit with min_8bit_size,
// section "B300 benchmark and acceptance").  The type follows the published
// description of dynamic tree quantization (Dettmers 2016) as used for
// 8-bit optimizer states (Dettmers, Lewis, Shleifer & Zettlemoyer 2022,
// section 2):
//
//   signed code   (first moments): bit 7 = sign, bits 0..6 = magnitude index
//   unsigned code (second moment): bits 0..7 = magnitude index
//
// With P payload bits (7 signed, 8 unsigned), index 0 is zero and the
// others run through the decades 10^-E for E = P-1 down to 0: a value with E
// leading zero bits and F = P-1-E fraction bits is the centre of one of 2^F
// equal bins of [0.1, 1], scaled by 10^-E,
//     fl32( (0.1 + ((j + 1/2) * 0.9) / 2^F) / 10^E ),  j = 0 .. 2^F - 1,
// evaluated in binary64 and rounded once.  The largest magnitude is set to
// 1 so that a block's largest state (normalised to +-1) is kept exactly.
//
// Quantizing: a state value v in a block whose largest |state| is A takes
// the magnitude nearest to |v| / A in exact arithmetic, a ratio exactly
// halfway between two magnitudes going to the smaller one: its index is the
// number of exact midpoints mid[k] = (mag[k] + mag[k+1]) / 2 lying strictly
// below |v| / A, i.e. with mid[k] * A < |v|.  A midpoint of two neighbouring
// binary32 magnitudes has at most 26 significant bits, so mid[k] * A is
// exact in binary64 and the comparison is exact.  The signed code adds bit
// 7 for v < 0.
#pragma once

#include <stdint.h>

namespace ou {

constexpr int kQBlock = 256;   // elements per quantization block (one wave x 4)

struct QTables {
    double sbound[128];  // signed type: exact midpoints 0..126; entry 127 = +inf
    double ubound[256];  // unsigned type: exact midpoints 0..254; entry 255 = +inf
    float smag[128];     // signed type: magnitudes by index
    float umag[256];     // unsigned type
    float svalue[256];   // signed type: value of each code byte (sign bit 7)
};
static_assert(sizeof(QTables) == 384 * 8 + 640 * 4, "QTables layout");

constexpr void build_magnitudes(float* mag, int payload)
{
    int k = 0;
    mag[k++] = 0.0f;
    for (int E = payload - 1; E >= 0; --E) {
        const int F = payload - 1 - E;
        const double bins = static_cast<double>(1 << F);
        double decade = 1.0;
        for (int e = 0; e < E; ++e) decade *= 10.0;
        for (int j = 0; j < (1 << F); ++j) {
            const double centre = 0.1 + ((static_cast<double>(j) + 0.5) * 0.9) / bins;
            mag[k++] = static_cast<float>(centre / decade);
        }
    }
    mag[k - 1] = 1.0f;
}

// Exact midpoints (two binary32 values within a factor 16 of each other sum
// exactly in binary64) and the +inf sentinel that stops the count.
constexpr void build_bounds(const float* mag, double* bound, int count)
{
    for (int k = 0; k + 1 < count; ++k)
        bound[k] = (static_cast<double>(mag[k]) + static_cast<double>(mag[k + 1])) * 0.5;
    bound[count - 1] = __builtin_huge_val();
}

// Significant bits of a positive binary64 value.
constexpr int significant_bits(double x)
{
    while (x < 4503599627370496.0) x *= 2.0;   // scale to [2^52, ...): an integer
    while (x >= 9007199254740992.0) x *= 0.5;  // exact: back into [2^52, 2^53)
    uint64_t m = static_cast<uint64_t>(x);
    int bits = 53;
    while ((m & 1u) == 0) {
        m >>= 1;
        --bits;
    }
    return bits;
}

constexpr QTables make_qtables()
{
    QTables t{};
    build_magnitudes(t.smag, 7);
    build_magnitudes(t.umag, 8);
    build_bounds(t.smag, t.sbound, 128);
    build_bounds(t.umag, t.ubound, 256);
    for (int c = 0; c < 256; ++c) t.svalue[c] = (c & 0x80) ? -t.smag[c & 0x7f] : t.smag[c & 0x7f];
    return t;
}

inline constexpr QTables kQTablesHost = make_qtables();

constexpr bool midpoints_fit(const double* bound, int count)
{
    for (int k = 0; k + 1 < count; ++k)
        if (!(bound[k] > 0x1p-26) || significant_bits(bound[k]) > 29) return false;
    return true;
}
static_assert(midpoints_fit(kQTablesHost.sbound, 128) && midpoints_fit(kQTablesHost.ubound, 256),
              "mid * absmax is exact in binary64 (at most 29 + 24 bits) and every midpoint lies above 2^-26");

// Finding the index without a search.  The kernels estimate the ratio as
// y = fl64(|v| * r + 2^-27) (one binary64 fused multiply-add), with r the
// block's reciprocal 1 / A (within 2^-22 relative, see the kernels); the
// added 2^-27 keeps y at or above 2^-27 without a comparison.  The key of y
// is bits 13..24 of its upper word: the low 5 exponent bits and the top 7
// fraction bits.  For y in [2^-27, 2) (its exponent field 996..1023) that
// is 512 + t, where t numbers the 3,584 buckets [s_t, s_t+1) of width 2^-7
// of a binade from s_0 = 2^-27.  A value y in bucket t means a ratio
// X = |v| / A in
//     [(s_t (1 - 2^-53) - 2^-27) / (1 + 2^-22),
//      (s_t+1 (1 + 2^-53) - 2^-27) / (1 - 2^-22)),
// which the tables widen to [lo_t, hi_t] below (about 2^-20 relative, plus
// an absolute 2^-80).  The key table holds est[t] = #{k : mid[k] < lo_t},
// and every widened bucket holds at most one midpoint (checked below),
// which is then mid[est[t]].  So the index of |v| / A is
// est[t] + (mid[est[t]] * A < |v|): below that midpoint est[t], above it
// est[t] + 1, and with no midpoint in the widened bucket mid[est[t]] lies
// above the ratio.  A ratio never exceeds 1, so a finite y stays below
// 1 + 2^-20; the buckets from 1.5 up are reached only by a NaN y (a NaN
// state, or an infinite one in a block with absmax +inf, where r = 0):
// every quiet NaN has exponent field 2047 and the top fraction bit set, so
// its key lies in those buckets, whose entry is 0, and the comparison with
// a NaN is false.  The +inf sentinel stops the count at the top.
constexpr int kQKeys = 28 << 7;       // binades 2^-27 .. 2^0, 128 buckets each
constexpr int kQKeyFirst = 4 << 7;    // key of 2^-27: (996 & 31) << 7
constexpr int kQKeyNaN = (27 << 7) + 64;   // first bucket from 1.5 (t): NaN keys only
constexpr double kQOffset = 0x1p-27;
constexpr double kQMargin = 0x1p-20;

constexpr double bucket_start(int t)
{
    double s = 1.0 + static_cast<double>(t % 128) / 128.0;
    for (int e = t / 128; e < 27; ++e) s *= 0.5;   // exact
    return s;
}

// The widened ratio range of bucket t (s_t - 2^-27 is exact: both are
// multiples of 2^-34 below 2).
constexpr double bucket_lo(int t)
{
    const double s = bucket_start(t);
    const double x = (s - kQOffset - s * 0x1p-52) * (1.0 - kQMargin) - 0x1p-80;
    return x > 0.0 ? x : 0.0;
}
constexpr double bucket_hi(int t)
{
    const double s = t + 1 < kQKeys ? bucket_start(t + 1) : 2.0;
    return (s - kQOffset + s * 0x1p-52) * (1.0 + kQMargin) + 0x1p-80;
}

constexpr uint32_t count_below(const double* bound, int count, double a)
{
    int lo = 0, hi = count - 1;   // bound[0 .. count-2] sorted
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (bound[mid] < a) lo = mid + 1; else hi = mid;
    }
    return static_cast<uint32_t>(lo);
}

struct QKeys {
    uint8_t s[kQKeys];   // signed type: est of each bucket
    uint8_t u[kQKeys];   // unsigned type
};

constexpr QKeys make_qkeys(const QTables& t)
{
    QKeys k{};
    for (int i = 0; i < kQKeyNaN; ++i) {
        k.s[i] = static_cast<uint8_t>(count_below(t.sbound, 128, bucket_lo(i)));
        k.u[i] = static_cast<uint8_t>(count_below(t.ubound, 256, bucket_lo(i)));
    }
    return k;   // buckets from kQKeyNaN on stay 0
}

inline constexpr QKeys kQKeysHost = make_qkeys(kQTablesHost);

constexpr bool one_midpoint_per_bucket(const double* bound, int count)
{
    for (int i = 0; i < kQKeyNaN; ++i)
        if (count_below(bound, count, bucket_hi(i)) - count_below(bound, count, bucket_lo(i)) > 1) return false;
    return true;
}
static_assert(one_midpoint_per_bucket(kQTablesHost.sbound, 128) &&
                  one_midpoint_per_bucket(kQTablesHost.ubound, 256),
              "a widened key bucket holds at most one midpoint");
static_assert(bucket_lo(kQKeyNaN) > 1.25, "finite ratio estimates stay below the NaN buckets");

// The ratio estimate of a state v (binary32) for reciprocal r >= 0: one
// binary64 fused multiply-add.  A constexpr template so that the kernels
// and the host check compile the same code (constexpr functions are callable
// on both sides; a fused multiply-add has no constant evaluation, which the
// compiler accepts in a template).
template <class Float>
constexpr double qestimate(Float v, double r)
{
    static_assert(sizeof(Float) == 4, "a binary32 state");
    return __builtin_fma(static_cast<double>(__builtin_fabsf(v)), r, kQOffset);
}

// Key of an estimate y (>= 2^-27, or a quiet NaN): bits 13..24 of the
// upper word; kQKeyFirst for y in the first bucket, kQKeyFirst + kQKeys - 1
// at most for y < 2 and for every quiet NaN.
constexpr uint32_t qkey(double y)
{
    const uint32_t hi = static_cast<uint32_t>(__builtin_bit_cast(uint64_t, y) >> 32);
    return (hi >> 13) & 0xfffu;
}
static_assert(qkey(kQOffset) == kQKeyFirst && qkey(0x1.fffffffffffffp0) == kQKeyFirst + kQKeys - 1 &&
                  qkey(bucket_start(1000)) == kQKeyFirst + 1000 &&
                  qkey(1.5) == kQKeyFirst + kQKeyNaN &&
                  qkey(__builtin_nan("")) >= kQKeyFirst + kQKeyNaN,
              "key layout");

// Magnitude index of |v| / A from est = the key table's entry.
constexpr uint32_t qindex(uint32_t est, const double* bound, double A, float v)
{
    return est + ((bound[est] * A < static_cast<double>(__builtin_fabsf(v))) ? 1u : 0u);
}

// Signed code: the sign bit for v < 0 (not for -0 or NaN).
constexpr uint32_t qsigned(float v, uint32_t idx) { return (v < 0.0f) ? (idx | 0x80u) : idx; }

}  // namespace ou
