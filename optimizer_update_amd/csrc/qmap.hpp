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
    float sbound[128];   // decision points 0..126 (entry 127 unused)
    float umag[256];     // unsigned type
    float ubound[256];   // decision points 0..254 (entry 255 unused)
};
static_assert(sizeof(QTables) == 768 * 4, "QTables layout");

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
    bound[count - 1] = 2.0f;   // never compared
}

constexpr QTables make_qtables()
{
    QTables t{};
    build_magnitudes(t.smag, 7);
    build_magnitudes(t.umag, 8);
    build_bounds(t.smag, t.sbound, 128);
    build_bounds(t.umag, t.ubound, 256);
    return t;
}

inline constexpr QTables kQTablesHost = make_qtables();

}  // namespace ou
