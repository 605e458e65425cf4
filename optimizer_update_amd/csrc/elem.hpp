// elem.hpp -- per-element arithmetic of the 32-bit two-state update (device).
//
// Every launch variant (single-tensor dwordx4 and per-lane paths, every
// block width and unroll, the multi-tensor walk, graph replay) calls the
// functions in this file, so the arithmetic cannot depend on how the work is
// mapped to lanes -- the rule of the page "Investigate a 256-thread SM103
// path for small 32-bit optimizer tensors" (section "Correctness oracle"):
// changing the launch width must not change the optimizer arithmetic.
//
// Operations are plain binary32 with contraction off (the file pragma below
// and -ffp-contract=off), correctly rounded division and square root (HIP's
// default lowering for gfx950) and denormals preserved, so each line is one
// IEEE operation rounded to nearest even.  The two divisions by the bias
// corrections take a cheaper route to the same correctly rounded quotient
// (div_step_constant, stepdiv.hpp); the 8-bit kernels take the square root
// by a shorter form of the same correctly rounded sequence (sqrt_rn).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stepdiv.hpp"

#pragma clang fp contract(off)

namespace ou {

enum Kind : int { kAdam = 0, kAdemamix = 1, kMomentum = 2, kRmsprop = 3, kAdagrad = 4, kLion = 5 };

// Adam and AdEMAMix keep two fp32 states (state1, state2); the one-state
// kinds keep state1 only.
template <int KIND>
inline constexpr bool kTwoState = KIND <= kAdemamix;

// Per-step scalars, formed on the host once per step (see host.hip).
struct StepScalars {
    float beta1, beta2, beta3;
    float omb1, omb2, omb3;   // 1 - beta, binary32
    float alpha, eps, lr;
    float bc1, bc2;           // bias corrections fl32(1 - fl64(beta^step))
    float decay;              // fl32(1 - fl64(lr * weight_decay))
    float weight_decay;       // L2 coefficient of the momentum/RMSprop/Adagrad kinds
    int32_t skip_zeros;
    int32_t first_step;       // step == 1 (momentum starts its buffer from the gradient)
    int32_t decay_after;      // decoupled decay of the updated parameter: (p - lr*u)*d
    int32_t pad;
    double rbc1, rbc2;        // binary64 nearest to 1/bc1 and 1/bc2
};


// The moments of one element.  m: fast first moment, v: second moment,
// m2: slow EMA (AdEMAMix only).  Kingma & Ba (Algorithm 1) for m and v,
// Pagliardini et al. (Algorithm 1) for the slow EMA.
template <int KIND>
__device__ __forceinline__ void update_moments(float g, float& m, float& v, float& m2,
                                               const StepScalars& s)
{
    m = s.beta1 * m + s.omb1 * g;
    v = s.beta2 * v + s.omb2 * (g * g);
    if constexpr (KIND == kAdemamix) m2 = s.beta3 * m2 + s.omb3 * g;
}

// Square root, correctly rounded.  The hardware root is within one ulp; of
// it and its two neighbours, the signs of the exact residuals x - r'*r
// (fused multiply-adds) pick the rounded root.  For x >= 2^-96 (or +inf)
// this is the compiler's own correctly rounded sequence without the two
// steps that only other inputs need: rescaling a tiny x by 2^32 (and the
// root by 2^-16), and passing +-0 and +inf through unchanged (the
// residuals leave +inf in place).  A wave takes that short form when all
// its active lanes qualify, otherwise the full sequence; the results are
// the same bits either way.  The branch splits straight-line code, which
// costs the memory-bound 32-bit kernels more than the instructions it
// saves; the 8-bit kernels, bound by instruction issue, use it.
//
// sqrt_short is the short form alone, for x >= 2^-96 or +inf; sqrt_rn4 takes
// four roots with one decision for the wave.
__device__ __forceinline__ float sqrt_short(float x)
{
    const float r = __builtin_amdgcn_sqrtf(x);
    const uint32_t b = __builtin_bit_cast(uint32_t, r);
    const float down = __builtin_bit_cast(float, b - 1u);
    const float up = __builtin_bit_cast(float, b + 1u);
    float s = r;
    if (__builtin_fmaf(-down, r, x) <= 0.0f) s = down;
    if (__builtin_fmaf(-up, r, x) > 0.0f) s = up;
    return s;
}

__device__ __forceinline__ float sqrt_rn(float x)
{
    if (__builtin_amdgcn_ballot_w64(!(x >= 0x1p-96f)) != 0) return __builtin_sqrtf(x);
    return sqrt_short(x);
}

__device__ __forceinline__ void sqrt_rn4(const float (&x)[4], float (&r)[4])
{
    bool tiny = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) tiny |= !(x[j] >= 0x1p-96f);
    if (__builtin_amdgcn_ballot_w64(tiny) != 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = __builtin_sqrtf(x[j]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = sqrt_short(x[j]);
    }
}

// The update direction from the (new) moments: the parameter moves by
// lr * direction.  Bias correction of m and v only; alpha mixes in the slow
// EMA (not bias-corrected).  SHORT_ROOT: the square root by sqrt_rn.
// The two halves (bias_corrected, direction_from) let a caller take
// several elements' square roots together.
__device__ __forceinline__ void bias_corrected(float m, float v, const StepScalars& s, float& mh, float& vh)
{
    mh = div_step_constant(m, s.rbc1);   // m / bc1
    vh = div_step_constant(v, s.rbc2);   // v / bc2
}

template <int KIND>
__device__ __forceinline__ float direction_from(float mh, float root_vh, float m2, const StepScalars& s)
{
    const float den = root_vh + s.eps;
    float num = mh;
    if constexpr (KIND == kAdemamix) num = mh + s.alpha * m2;
    return num / den;
}

template <int KIND, bool SHORT_ROOT = false>
__device__ __forceinline__ float direction(float m, float v, float m2, const StepScalars& s)
{
    float mh, vh;
    bias_corrected(m, v, s, mh, vh);
    return direction_from<KIND>(mh, SHORT_ROOT ? sqrt_rn(vh) : __builtin_sqrtf(vh), m2, s);
}

// Decoupled weight decay of the old parameter and the step (Loshchilov &
// Hutter, Algorithm 2), or, with `after`, the decay of the updated
// parameter (the other order the update family has used).  The flag is
// uniform over a launch; both forms are plain binary32 operations.
__device__ __forceinline__ float step_param(float p, float u, float decay, float lr, int32_t after)
{
    return after ? (p - lr * u) * decay : p * decay - lr * u;
}

// One element of a one-state kind; m is the element's state.  gd adds the
// L2 term wd*p to the gradient (only when wd != 0), as torch.optim does.
//   momentum (Sutskever et al. 2013; dampening 0): m = gd on the first
//            step, else beta1*m + gd; p - lr*m
//   RMSprop  (Tieleman & Hinton 2012): m = beta1*m + (1-beta1)*(gd*gd);
//            p - lr*(gd/(sqrt(m)+eps))
//   Adagrad  (Duchi et al. 2011): m = m + gd*gd; p - lr*(gd/(sqrt(m)+eps))
//   Lion     (Chen et al. 2023): c = beta1*m + (1-beta1)*g; p*d - lr*sign(c)
//            (sign(0) = 0, NaN stays NaN; decay order as for Adam); then
//            m = beta2*m + (1-beta2)*g
template <int KIND>
__device__ __forceinline__ float update_one_state(float p, float g, float& m, const StepScalars& s)
{
    if constexpr (KIND == kLion) {
        const float c = s.beta1 * m + s.omb1 * g;
        const float u = (c != c) ? c : static_cast<float>((c > 0.0f) - (c < 0.0f));
        const float pn = step_param(p, u, s.decay, s.lr, s.decay_after);
        m = s.beta2 * m + s.omb2 * g;
        return pn;
    } else {
        const float gd = (s.weight_decay != 0.0f) ? g + s.weight_decay * p : g;
        if constexpr (KIND == kMomentum) {
            m = s.first_step ? gd : s.beta1 * m + gd;
            return p - s.lr * m;
        } else {
            if constexpr (KIND == kRmsprop)
                m = s.beta1 * m + s.omb1 * (gd * gd);
            else
                m = m + gd * gd;
            return p - s.lr * (gd / (__builtin_sqrtf(m) + s.eps));
        }
    }
}

// One element: moments, direction, parameter (two-state kinds), or the
// one-state rule.  p is the widened parameter; returns the new parameter
// before rounding to storage.
template <int KIND, bool SHORT_ROOT = false>
__device__ __forceinline__ float update_element(float p, float g, float& m, float& v,
                                                float& m2, const StepScalars& s)
{
    if constexpr (kTwoState<KIND>) {
        update_moments<KIND>(g, m, v, m2, s);
        return step_param(p, direction<KIND, SHORT_ROOT>(m, v, m2, s), s.decay, s.lr, s.decay_after);
    } else {
        return update_one_state<KIND>(p, g, m, s);
    }
}

// ---- storage types ---------------------------------------------------------
// Storage<T> widens to binary32 exactly and narrows with round to nearest,
// ties to even (gfx950 conversion instructions: v_cvt_f16_f32 under the
// default round-to-nearest mode, v_cvt_pk_bf16_f32 for bfloat16).  The
// 16-bit types also narrow two values into one packed word (narrow2: the
// first in the low half), one v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32.
struct F32 {
    using raw = float;
    static constexpr int bytes = 4;
    __device__ __forceinline__ static float widen(raw x) { return x; }
    __device__ __forceinline__ static raw narrow(float x) { return x; }
};

using f32x2 = float __attribute__((ext_vector_type(2)));

struct F16 {
    using raw = uint16_t;
    static constexpr int bytes = 2;
    using pair = _Float16 __attribute__((ext_vector_type(2)));
    __device__ __forceinline__ static float widen(raw x)
    {
        return static_cast<float>(__builtin_bit_cast(_Float16, x));
    }
    __device__ __forceinline__ static raw narrow(float x)
    {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    }
    __device__ __forceinline__ static uint32_t narrow2(float a, float b)
    {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, pair));
    }
};

struct BF16 {
    using raw = uint16_t;
    static constexpr int bytes = 2;
    using pair = __bf16 __attribute__((ext_vector_type(2)));
    __device__ __forceinline__ static float widen(raw x)
    {
        return __builtin_bit_cast(float, static_cast<uint32_t>(x) << 16);
    }
    __device__ __forceinline__ static raw narrow(float x)
    {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
    }
    __device__ __forceinline__ static uint32_t narrow2(float a, float b)
    {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, pair));
    }
};

// One element through widen -> update -> narrow.  With skip_zeros and a
// zero gradient (+0 or -0) nothing of the element is written.
template <int KIND, typename S>
__device__ __forceinline__ void update_scalar(typename S::raw* __restrict__ p,
                                              const typename S::raw* __restrict__ g,
                                              float* __restrict__ s1, float* __restrict__ s2,
                                              int64_t n, int64_t i, const StepScalars& s)
{
    const float gi = S::widen(g[i]);
    if (s.skip_zeros && gi == 0.0f) return;
    float m = s1[i], v = 0.0f, m2 = 0.0f;
    if constexpr (kTwoState<KIND>) v = s2[i];
    if constexpr (KIND == kAdemamix) m2 = s1[n + i];
    const float pn = update_element<KIND>(S::widen(p[i]), gi, m, v, m2, s);
    p[i] = S::narrow(pn);
    s1[i] = m;
    if constexpr (kTwoState<KIND>) s2[i] = v;
    if constexpr (KIND == kAdemamix) s1[n + i] = m2;
}

}  // namespace ou
