// Exhaustive host check of the 8-bit quantizer of the library
// (optimizer_update_amd/csrc/qmap.hpp), composed as the kernels compose it:
// a = qmagnitude(x), est = key table entry of qkey(a), idx = qindex(est,
// bound, a), and for the signed type qsigned(x, idx).  For every binary32
// x (both signs, infinities, every NaN) the codes must equal the
// definition: the index of |x| is #{k : bound[k] < |x|} over the decision
// points (the +inf sentinel excluded), the signed code adds bit 7 for
// x < 0, and a NaN quantizes to 0.  The kernels quantize products (a state
// times the block's reciprocal), so each pattern is passed as x * 1, which
// is exact for every number and quiets a signaling NaN.  The expected
// indices come from a walk over the sorted decision points, not from the
// key tables or count_below.  Prints "ok" and exits 0 on success.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "qmap.hpp"

using namespace ou;

static volatile float g_one = 1.0f;

static float from_bits(uint32_t u)
{
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// #{k < count-1 : bound[k] < a}, by a linear scan
static uint32_t scan(const float* bound, int count, float a)
{
    uint32_t c = 0;
    for (int k = 0; k + 1 < count; ++k) c += bound[k] < a ? 1u : 0u;
    return c;
}

int main()
{
    const QTables& T = kQTablesHost;
    const QKeys& K = kQKeysHost;
    long bad = 0;
    // non-negative non-NaN patterns in increasing order (0 .. +inf), chunked;
    // each chunk starts from a linear scan and walks the decision points
    constexpr int64_t kTop = 0x7f800000LL;
    constexpr int64_t kChunk = 1 << 20;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t c0 = 0; c0 <= kTop; c0 += kChunk) {
        const int64_t c1 = c0 + kChunk - 1 < kTop ? c0 + kChunk - 1 : kTop;
        uint32_t is = scan(T.sbound, 128, from_bits(static_cast<uint32_t>(c0)));
        uint32_t iu = scan(T.ubound, 256, from_bits(static_cast<uint32_t>(c0)));
        for (int64_t u = c0; u <= c1; ++u) {
            const float a = from_bits(static_cast<uint32_t>(u));
            while (is < 127 && T.sbound[is] < a) ++is;
            while (iu < 255 && T.ubound[iu] < a) ++iu;
            for (const float y : {a, -a}) {
                const float x = y * g_one;
                const float m = qmagnitude(x);
                const uint32_t ks = qkey(m) - kQKeyBase;
                const uint32_t got_s = qsigned(x, qindex(K.s[ks], T.sbound, m));
                const uint32_t got_u = qindex(K.u[ks], T.ubound, m);
                const uint32_t want_s = (x < 0.0f) ? (is | 0x80u) : is;
                bad += (got_s != want_s) + (got_u != iu);
            }
        }
    }
    // every NaN, both signs: code 0
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad)
    for (int64_t u = kTop + 1; u <= 0x7fffffffLL; ++u) {
        for (const uint32_t sign : {0u, 0x80000000u}) {
            const float x = from_bits(static_cast<uint32_t>(u) | sign) * g_one;
            const float m = qmagnitude(x);
            const uint32_t ks = qkey(m) - kQKeyBase;
            bad += (qsigned(x, qindex(K.s[ks], T.sbound, m)) != 0u) + (qindex(K.u[ks], T.ubound, m) != 0u);
        }
    }
    std::printf("%s bad=%ld\n", bad == 0 ? "ok" : "FAIL", bad);
    return bad == 0 ? 0 : 1;
}
