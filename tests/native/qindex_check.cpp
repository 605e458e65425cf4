// Exhaustive host check of the 8-bit quantizer of the library
// (optimizer_update_amd/csrc/qmap.hpp): for every binary32 value a in
// [0, 2], for +infinity and for NaN, the key-table qindex<P> equals the
// definition #{k : bound[k] < a} (clamped to the largest index, NaN -> 0).
// Prints "ok" and exits 0 on success.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "qmap.hpp"

using namespace ou;

static uint32_t definition(const float* bound, int count, float a)
{
    if (a != a) return 0;
    uint32_t c = count_below(bound, count, a);
    return c;
}

int main()
{
    const QTables& T = kQTablesHost;
    const QKeys& K = kQKeysHost;
    long bad = 0;
#pragma omp parallel for schedule(static, 1 << 20) reduction(+ : bad)
    for (int64_t u = 0; u <= 0x40000000LL; ++u) {
        float a;
        const uint32_t bits = static_cast<uint32_t>(u);
        std::memcpy(&a, &bits, 4);
        if (qindex<7>(K.s, T.sbound, a) != definition(T.sbound, 128, a)) ++bad;
        if (qindex<8>(K.u, T.ubound, a) != definition(T.ubound, 256, a)) ++bad;
    }
    for (uint32_t bits : {0x7f800000u, 0x7fc00000u, 0x7f7fffffu, 0x00000001u}) {
        float a;
        std::memcpy(&a, &bits, 4);
        if (qindex<7>(K.s, T.sbound, a) != definition(T.sbound, 128, a)) ++bad;
        if (qindex<8>(K.u, T.ubound, a) != definition(T.ubound, 256, a)) ++bad;
    }
    std::printf("%s bad=%ld\n", bad == 0 ? "ok" : "FAIL", bad);
    return bad == 0 ? 0 : 1;
}
