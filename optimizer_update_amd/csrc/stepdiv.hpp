// stepdiv.hpp -- division by a per-step constant, correctly rounded
// (host and device; no HIP headers, so host-side checks compile it too).
#pragma once

namespace ou {

// The binary64 nearest to 1/b, formed on the host once per step.
constexpr double step_reciprocal(float b) { return 1.0 / static_cast<double>(b); }

// x / b, correctly rounded to binary32, for a per-step constant b in
// [2^-24, 1] (a bias correction), given rb = step_reciprocal(b).
// The binary64 product x * rb lies within 2^-52 (relative) of x / b.  A
// quotient of two binary32 numbers is never exactly halfway between two
// binary32 numbers (that would need an odd 25-bit significand times b's
// significand to fit in 24 bits), and when it is not, it lies at least
// 2^-49 (relative) from every halfway point -- in the subnormal range at
// least 2^-174 away, against an error below 2^-178 there; the overflow
// threshold is such a halfway point too.  So rounding the product to
// binary32 gives the correctly rounded quotient for every x, including
// +-0, subnormals, infinities and NaN: two conversions and a binary64
// multiply in place of the division sequence.
constexpr float div_step_constant(float x, double rb)
{
    return static_cast<float>(static_cast<double>(x) * rb);
}

}  // namespace ou
