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
// Decision points: bound[k] = fl32((mag[k] + mag[k+1]) / 2) (exact in
// binary64, rounded once).  A magnitude a quantizes to #{k : bound[k] < a}:
// the nearest magnitude, a value exactly on a decision point going to the
// smaller one.
#pragma once

#include <stdint.h>

namespace ou {

constexpr int kQBlock = 256;   // elements per quantization block (one wave x 4)

struct QTables {
    float smag[128];     // signed type: magnitudes by index
    float sbound[128];   // decision points 0..126; entry 127 = +inf
    float umag[256];     // unsigned type
    float ubound[256];   // decision points 0..254; entry 255 = +inf
    float svalue[256];   // signed type: value of each code byte (sign bit 7)
};
static_assert(sizeof(QTables) == 1024 * 4, "QTables layout");

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

constexpr void build_bounds(const float* mag, float* bound, int count)
{
    for (int k = 0; k + 1 < count; ++k)
        bound[k] = static_cast<float>((static_cast<double>(mag[k]) + static_cast<double>(mag[k + 1])) * 0.5);
    bound[count - 1] = __builtin_huge_valf();   // no value lies above it
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

// Quantizing without a search.  The magnitude index of a >= 0 is
// #{k : bound[k] < a}.  The binary32 pattern of a, shifted right by 16 (sign,
// exponent, top 7 mantissa bits), names a bucket [s, s') of width at most
// 2^-7 of its binade; for a in [2^-27, 2) the key is that number, and
// larger a clamp to the last key (kQKeyBase + kQKeys - 1).  A bucket never
// holds more than one decision point, so with est = the index of the
// bucket's start s (the key table's entry key - kQKeyBase), the index of any
// a in the bucket is est + (bound[est] < a).  Every magnitude below 2^-27
// has index 0 (both types' first decision points lie above 2^-26), so the
// quantizer raises smaller magnitudes to 2^-27 (qmagnitude), which changes
// no index and keeps every key at or above kQKeyBase; a >= 2 (infinity,
// after a reciprocal that overflowed) takes the largest index, where the
// +inf sentinel stops the count.  The test suite checks the composition
// below against the definition for every binary32 input.
constexpr int kQKeyBase = 100 << 7;   // bits >> 16 of 2^-27
constexpr int kQKeys = 28 << 7;       // binades 2^-27 .. 2^0

constexpr uint32_t count_below(const float* bound, int count, float a)
{
    int lo = 0, hi = count - 1;   // bound[0 .. count-2] sorted
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (bound[mid] < a) lo = mid + 1; else hi = mid;
    }
    return static_cast<uint32_t>(lo);
}

struct QKeys {
    uint8_t s[kQKeys];   // signed type: index of each bucket's start
    uint8_t u[kQKeys];   // unsigned type
};

constexpr QKeys make_qkeys(const QTables& t)
{
    QKeys k{};
    for (int i = 0; i < kQKeys; ++i) {
        const float start = __builtin_bit_cast(float, static_cast<uint32_t>(i + kQKeyBase) << 16);
        k.s[i] = static_cast<uint8_t>(count_below(t.sbound, 128, start));
        k.u[i] = static_cast<uint8_t>(count_below(t.ubound, 256, start));
    }
    return k;
}

inline constexpr QKeys kQKeysHost = make_qkeys(kQTablesHost);

// The magnitude the quantizer classifies: |x| raised to at least 2^-27,
// with NaN mapped to 2^-27 (maxNum returns the number when one operand is a
// quiet NaN), so a NaN takes index 0.  x is a product (a state times its
// block's reciprocal), never a signaling NaN.
constexpr float kQFloor = 0x1p-27f;
static_assert(__builtin_bit_cast(uint32_t, kQFloor) >> 16 == kQKeyBase, "floor is the first key");
static_assert(kQTablesHost.sbound[0] > 0x1p-26f && kQTablesHost.ubound[0] > 0x1p-26f,
              "magnitudes below 2^-26 have index 0");
constexpr float qmagnitude(float x) { return __builtin_fmaxf(__builtin_fabsf(x), kQFloor); }

// Key of a = qmagnitude(x) (so a >= 2^-27): bits >> 16, at most
// kQKeyBase + kQKeys - 1.
constexpr uint32_t qkey(float a)
{
    const uint32_t k = __builtin_bit_cast(uint32_t, a) >> 16;
    constexpr uint32_t hi = kQKeyBase + kQKeys - 1;
    return k > hi ? hi : k;
}

// Magnitude index of a from est = the key table's entry for qkey(a).
constexpr uint32_t qindex(uint32_t est, const float* bound, float a)
{
    return est + ((bound[est] < a) ? 1u : 0u);
}

// Signed code: the sign bit for x < 0 (not for -0 or NaN, whose magnitude
// index is 0).
constexpr uint32_t qsigned(float x, uint32_t idx) { return (x < 0.0f) ? (idx | 0x80u) : idx; }

}  // namespace ou
