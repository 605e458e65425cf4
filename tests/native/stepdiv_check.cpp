// Host check of the library's division by a per-step constant
// (optimizer_update_amd/csrc/stepdiv.hpp): for bias corrections b formed as
// the library forms them, fl32(1 - fl64(beta^t)), and for the ends of
// [2^-24, 1], div_step_constant(x, step_reciprocal(b)) equals the
// correctly rounded binary32 quotient x / b bitwise (a NaN equals a NaN).
// Every binary32 x for the first divisors; for the others every 61st bit
// pattern plus all subnormals, the smallest normals and the values near
// the overflow threshold.  Prints "ok <checked>" and exits 0 on success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "stepdiv.hpp"

using namespace ou;

static float from_bits(uint32_t u)
{
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

static uint32_t to_bits(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
}

static float bias_correction(float beta, int t)
{
    return static_cast<float>(1.0 - std::pow(static_cast<double>(beta), static_cast<double>(t)));
}

// one x: 1 if the two quotients differ
static int differs(float x, float b, double rb)
{
    const float want = x / b;
    const float got = div_step_constant(x, rb);
    if (want != want) return got == got;
    return to_bits(want) != to_bits(got);
}

static long check(float b, uint64_t stride, uint64_t* checked)
{
    const double rb = step_reciprocal(b);
    long bad = 0;
    uint64_t count = 0;
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad, count)
    for (int64_t i = 0; i < static_cast<int64_t>((1ULL << 32) / stride); ++i) {
        const uint32_t u = static_cast<uint32_t>(static_cast<uint64_t>(i) * stride);
        bad += differs(from_bits(u), b, rb);
        ++count;
    }
    if (stride > 1) {
        // every subnormal and small normal, and the top of the range, both signs
        for (uint32_t s = 0; s < 2; ++s) {
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad, count)
            for (int64_t u = 0; u < (1LL << 25); ++u) {
                bad += differs(from_bits((s << 31) | static_cast<uint32_t>(u)), b, rb);
                ++count;
            }
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad, count)
            for (int64_t u = 0x7e000000LL; u <= 0x7fffffffLL; ++u) {
                bad += differs(from_bits((s << 31) | static_cast<uint32_t>(u)), b, rb);
                ++count;
            }
        }
    }
    *checked += count;
    if (bad) std::printf("b = %.9g (0x%08x): %ld quotients differ\n", b, to_bits(b), bad);
    return bad;
}

int main()
{
    long bad = 0;
    uint64_t checked = 0;
    // every x: the first bias corrections of the usual betas and the ends
    // of the range
    for (float b : {bias_correction(0.9f, 1), bias_correction(0.999f, 1), bias_correction(0.9f, 2),
                    from_bits(0x33800000u) /* 2^-24 */, 1.0f, from_bits(0x3f7fffffu)})
        bad += check(b, 1, &checked);
    // sampled x: more steps and betas, and divisors spread over [2^-24, 1]
    std::vector<float> more;
    for (float beta : {0.5f, 0.9f, 0.95f, 0.99f, 0.999f, 0.9999f, 0.99999994f})
        for (int t : {2, 3, 7, 10, 100, 1000, 100000})
            more.push_back(bias_correction(beta, t));
    for (uint32_t u = 0x33800000u; u < 0x3f800000u; u += 0x00b3c5d1u) more.push_back(from_bits(u));
    for (float b : more)
        if (b >= from_bits(0x33800000u) && b <= 1.0f) bad += check(b, 61, &checked);
    if (bad) return 1;
    std::printf("ok %llu\n", static_cast<unsigned long long>(checked));
    return 0;
}
