// kernels8.hip -- the update with 8-bit block-wise states (device).
//
// The page "Investigate a 256-thread SM103 path for small 32-bit optimizer
// tensors" times AdamW8bit collections whose tensors below min_8bit_size
// (4,096 elements) take the 32-bit path (sections "Problem" and "B300
// benchmark and acceptance").  This file is the other leg: Adam/AdamW and
// AdEMAMix with each moment stored as 8-bit codes of the dynamic type of
// qmap.hpp plus one fp32 absmax per block of 256 elements.
//
// One wave owns one block: lane l holds elements 4l .. 4l+3 (one dwordx4 of
// an fp32 stream, dwordx2 of a 16-bit one, one dword of codes per state).
// Per block: dequantize (code value x absmax), the 32-bit rule of elem.hpp
// on the fp32 values, the block's new absmax of every state by one wave
// reduction (exact, so the order does not matter: the states are paired
// across the wave's halves and rows by lane swaps, then DPP rotations
// finish each 16-lane row), then each state is requantized to the
// magnitude nearest to |value| / absmax: a key table indexed by the top
// bits of the binary64 estimate |value| * (1 / absmax) + 2^-27 names the
// one midpoint that can lie near the ratio, and one exact binary64 comparison
// of that midpoint times absmax with |value| decides (qmap.hpp).  The
// tables (12.5 KiB) are copied to LDS once per workgroup.  The parameter
// moves with the moments before quantization.  A partial last block, or a
// tensor whose streams are not aligned for the wide accesses, runs the same
// steps one element per slot.
//
// Each block is one dependent chain (loads, table reads, the cross-lane
// maximum, a reciprocal, the quantizer), so a wave keeps the next block's
// loads in flight while it computes one (run_wide8), and runs of blocks
// are long enough to amortize the table copy.  Per block the chain costs
// 270-380 VALU instructions against 2.5-4 KiB of HBM traffic: with 16-bit
// storage the kernel issues VALU work near the chip's peak rate, with fp32
// storage it sits between the two rooflines.
#include <type_traits>

#include "internal.h"
#include "qmap.hpp"

#pragma clang fp contract(off)

namespace ou {
namespace {

// The tables as built, copied into LDS per workgroup.
struct QSrc {
    QTables t;
    QKeys k;
};
static_assert(sizeof(QTables) % 4 == 0 && sizeof(QKeys) % 4 == 0, "tables are copied in dwords");

__constant__ QSrc kQ = {make_qtables(), make_qkeys(make_qtables())};

// LDS layout: the key tables follow the other tables, so the entry of key k
// (k >= kQKeyFirst) sits at byte k + kKeyAt, a constant offset of the LDS
// read, plus kQKeys for the unsigned type.
struct QLds {
    QTables t;
    uint8_t ks[kQKeys];   // signed type: entry of bucket t = key - kQKeyFirst
    uint8_t ku[kQKeys];   // unsigned type
};
constexpr int kKeyAt = static_cast<int>(sizeof(QTables)) - kQKeyFirst;
static_assert(kKeyAt >= 0 && offsetof(QLds, ks) == sizeof(QTables) &&
                  offsetof(QLds, ku) == sizeof(QTables) + kQKeys,
              "QLds layout");

using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
using u32x2 = uint32_t __attribute__((ext_vector_type(2)));

// Copies the tables into LDS; every thread of the block must call it.
__device__ __forceinline__ void load_qtables(QLds* T)
{
    constexpr int kTableWords = static_cast<int>(sizeof(QTables) / 4);
    constexpr int kKeyWords = static_cast<int>(sizeof(QKeys) / 4);
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&kQ);
    uint32_t* dst = reinterpret_cast<uint32_t*>(T);
    for (int i = static_cast<int>(threadIdx.x); i < kTableWords + kKeyWords; i += static_cast<int>(blockDim.x))
        dst[i] = src[i];
    __syncthreads();
}

__device__ __forceinline__ float deq_signed(const QLds& T, uint32_t code)
{
    return T.t.svalue[code];
}

// Code of a state v in a block with absmax A and reciprocal r (qmap.hpp):
// the key of the estimate |v| * r + 2^-27, plus a constant, is the LDS
// address of its entry.
__device__ __forceinline__ uint32_t quant_signed(const QLds& T, float v, double r, double A)
{
    const uint32_t est = reinterpret_cast<const uint8_t*>(&T)[qkey(qestimate(v, r)) + kKeyAt];
    return qsigned(v, qindex(est, T.t.sbound, A, v));
}

__device__ __forceinline__ uint32_t quant_unsigned(const QLds& T, float v, double r, double A)
{
    const uint32_t est =
        reinterpret_cast<const uint8_t*>(&T)[qkey(qestimate(v, r)) + kKeyAt + kQKeys];
    return qindex(est, T.t.ubound, A, v);
}

// Value of lane (l + N) mod 16 of the same 16-lane row (DPP row_ror:N).
template <int N>
__device__ __forceinline__ uint32_t row_ror(uint32_t x)
{
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x120 + N, 0xf, 0xf, false));
}

__device__ __forceinline__ uint32_t lane_value(uint32_t x, int lane)
{
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), lane));
}

__device__ __forceinline__ float lane_float(float x, int lane)
{
    return __builtin_bit_cast(float, lane_value(__builtin_bit_cast(uint32_t, x), lane));
}

__device__ __forceinline__ double lane_double(double x, int lane)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint64_t lo = lane_value(static_cast<uint32_t>(u), lane);
    const uint64_t hi = lane_value(static_cast<uint32_t>(u >> 32), lane);
    return __builtin_bit_cast(double, (hi << 32) | lo);
}

// Maxima over the wave of two or three lane values, each a non-negative
// binary32 that is not a NaN (so that the order of the bit patterns as
// integers is the order of the values); every lane must be active.
// v_permlane32_swap exchanges rows 2-3 of its first operand with rows 0-1
// of its second, v_permlane16_swap the odd rows of the first with the even
// rows of the second (rows of 16 lanes), so the maximum of each swapped
// pair folds two halves, or two rows, of different states into one
// register; rotations by 1, 2, 4, 8 then finish every row.
__device__ __forceinline__ uint32_t max_swap32(uint32_t a, uint32_t b)
{
    const auto s = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    return max(static_cast<uint32_t>(s[0]), static_cast<uint32_t>(s[1]));
}

__device__ __forceinline__ uint32_t max_swap16(uint32_t a, uint32_t b)
{
    const auto s = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    return max(static_cast<uint32_t>(s[0]), static_cast<uint32_t>(s[1]));
}

__device__ __forceinline__ uint32_t row_max(uint32_t b)
{
    b = max(b, row_ror<1>(b));
    b = max(b, row_ror<2>(b));
    b = max(b, row_ror<4>(b));
    return max(b, row_ror<8>(b));
}

// Two states: lanes 0-31 get the maximum of x, lanes 32-63 that of y.
__device__ __forceinline__ float wave_max2(float x, float y)
{
    uint32_t z = max_swap32(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y));
    z = max_swap16(z, z);   // rows 0-1: x over all lanes, rows 2-3: y
    return __builtin_bit_cast(float, row_max(z));
}

// Three states: lanes 0-15 get the maximum of x, 16-31 and 48-63 that of w,
// 32-47 that of y.
__device__ __forceinline__ float wave_max3(float x, float y, float w)
{
    const uint32_t z = max_swap32(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y));
    const uint32_t ww = __builtin_bit_cast(uint32_t, w);
    const uint32_t h = max_swap32(ww, ww);   // every row: w over two rows
    return __builtin_bit_cast(float, row_max(max_swap16(z, h)));
}

// 1 / l in binary64 for a block maximum l (non-negative, not a NaN), and 0
// for l = 0 or +inf: the binary64 reciprocal estimate refined by two Newton
// steps (a probe over every positive binary32 measured 2^-53 relative).
// The quantizer needs it within 2^-22 (qmap.hpp), which recip_max's test
// shows: rounded to binary32 it is the correctly rounded 1/l for every
// binary32 l >= 0, so it lies within one binary32 ulp of 1/l, 2^-23
// relative while 1/l is a normal binary32 and at most 2^-22 for the
// subnormal 1/l of l > 2^126 (1/l >= 2^-128).  With l = +inf the estimate
// is a NaN, so the select covers it.
__device__ __forceinline__ double recip_max64(float l)
{
    const double d = static_cast<double>(l);
    double y = __builtin_amdgcn_rcp(d);
    y = __builtin_fma(__builtin_fma(-d, y, 1.0), y, y);
    y = __builtin_fma(__builtin_fma(-d, y, 1.0), y, y);
    return (l > 0.0f && l < __builtin_huge_valf()) ? y : 0.0;
}

// recip_max64 rounded to binary32 (the test hook): a quotient of two
// binary32 numbers is never a binary32 rounding midpoint and lies far
// enough from every one that rounding a value this close gives the
// correctly rounded quotient; the test suite compares it with 1/l for every
// binary32 l >= 0.
__device__ __forceinline__ float recip_max(float l)
{
    return static_cast<float>(recip_max64(l));
}

// Buffer resources over the arrays of one run of whole blocks, based at the
// run's first block b0.  Inside the run an access is the lane's 32-bit byte
// offset (a vector register that never changes) plus the block's byte
// offset from b0 (a scalar register), so a block takes no vector address
// arithmetic; the accesses are non-temporal like the per-pointer ones.  The
// record count is the largest the descriptor holds, as every offset stays
// within the run's few kilobytes.
struct Run8 {
    __amdgpu_buffer_rsrc_t p, g, c1, c2, c3;
    int64_t b0;
};

constexpr int kBufRsrcWord3 = 0x00020000;   // raw 32-bit records (CDNA descriptor format)
constexpr int kBufNonTemporal = 2;          // cache-policy operand: nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t run_rsrc(const void* base)
{
    // the address is the same on every lane: read it from the first, so the
    // descriptor is known to sit in scalar registers
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)));
    void* const u = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, 0, 0x7fffffff, kBufRsrcWord3);
}

template <int KIND, typename S>
__device__ __forceinline__ Run8 make_run8(const Seg8& d, int64_t b0)
{
    using raw = typename S::raw;
    Run8 r;
    const int64_t e = b0 * kQBlock;
    r.p = run_rsrc(static_cast<const raw*>(d.p) + e);
    r.g = run_rsrc(static_cast<const raw*>(d.g) + e);
    r.c1 = run_rsrc(d.c1 + e);
    r.c2 = run_rsrc(d.c2 + e);
    r.c3 = run_rsrc(KIND == kAdemamix ? d.c1 + d.n + e : d.c1 + e);
    r.b0 = b0;
    return r;
}

// Byte offset of block b from the run's start in an array of T.
template <typename T>
__device__ __forceinline__ int32_t run_off(const Run8& r, int64_t b)
{
    return static_cast<int32_t>((b - r.b0) * kQBlock * static_cast<int64_t>(sizeof(T)));
}

// The inputs of one quantization block, as loaded by one wave: lane l
// holds elements 4l .. 4l+3.  WIDE: the block is known to be whole and on
// the wide path (no per-element checks).
template <typename S>
struct Block8 {
    typename S::raw praw[4], graw[4];
    uint32_t w1, w2, w3;   // four codes of each state
    float A1, A2, A3;      // the block's absmax of each state
    bool live[4];          // element inside the tensor
    bool full;             // whole block on the wide path
};

template <int KIND, typename S, bool WIDE>
__device__ __forceinline__ Block8<S> load_block8(const Seg8& d, int64_t b, int lane, const Run8& run)
{
    using raw = typename S::raw;
    constexpr bool kMix = KIND == kAdemamix;
    const raw* __restrict__ p = static_cast<const raw*>(d.p);
    const raw* __restrict__ g = static_cast<const raw*>(d.g);
    const uint8_t* __restrict__ c1 = d.c1;
    const uint8_t* __restrict__ c2 = d.c2;
    const int64_t n = d.n;
    const int64_t e0 = b * kQBlock + 4 * lane;
    Block8<S> in;
    in.full = WIDE || (d.vec_ok && (b + 1) * kQBlock <= n);
    in.A1 = d.a1[b];
    in.A2 = d.a2[b];
    in.A3 = 0.0f;
    if constexpr (kMix) in.A3 = d.a1[d.nb + b];
    raw* praw = in.praw;
    raw* graw = in.graw;
    bool* live = in.live;
    uint32_t w1 = 0, w2 = 0, w3 = 0;
    if (in.full) {
        // lane l's four elements: 4l .. 4l+3 of the block
        using Vec = typename std::conditional<S::bytes == 4, u32x4, u32x2>::type;
        Vec xp, xg;
        if constexpr (WIDE) {
            const uint32_t lo = static_cast<uint32_t>(lane) * 4u;   // byte offset of the lane's codes
            const int32_t so = run_off<raw>(run, b), sc = run_off<uint8_t>(run, b);
            if constexpr (S::bytes == 4) {
                xp = __builtin_amdgcn_raw_buffer_load_b128(run.p, lo * 4u, so, kBufNonTemporal);
                xg = __builtin_amdgcn_raw_buffer_load_b128(run.g, lo * 4u, so, kBufNonTemporal);
            } else {
                xp = __builtin_amdgcn_raw_buffer_load_b64(run.p, lo * 2u, so, kBufNonTemporal);
                xg = __builtin_amdgcn_raw_buffer_load_b64(run.g, lo * 2u, so, kBufNonTemporal);
            }
            w1 = __builtin_amdgcn_raw_buffer_load_b32(run.c1, lo, sc, kBufNonTemporal);
            w2 = __builtin_amdgcn_raw_buffer_load_b32(run.c2, lo, sc, kBufNonTemporal);
            if constexpr (kMix) w3 = __builtin_amdgcn_raw_buffer_load_b32(run.c3, lo, sc, kBufNonTemporal);
        } else {
            xp = __builtin_nontemporal_load(reinterpret_cast<const Vec*>(p + e0));
            xg = __builtin_nontemporal_load(reinterpret_cast<const Vec*>(g + e0));
            w1 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(c1 + e0));
            w2 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(c2 + e0));
            if constexpr (kMix) w3 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(c1 + n + e0));
        }
        if constexpr (S::bytes == 4) {
            // Elements are copied to scalars before the bit cast: this
            // compiler reads element 0 for a bit cast of a vector element.
            const uint32_t p0 = xp.x, p1 = xp.y, p2 = xp.z, p3 = xp.w;
            const uint32_t g0 = xg.x, g1 = xg.y, g2 = xg.z, g3 = xg.w;
            praw[0] = __builtin_bit_cast(float, p0); praw[1] = __builtin_bit_cast(float, p1);
            praw[2] = __builtin_bit_cast(float, p2); praw[3] = __builtin_bit_cast(float, p3);
            graw[0] = __builtin_bit_cast(float, g0); graw[1] = __builtin_bit_cast(float, g1);
            graw[2] = __builtin_bit_cast(float, g2); graw[3] = __builtin_bit_cast(float, g3);
        } else {
            praw[0] = static_cast<raw>(xp.x & 0xffffu); praw[1] = static_cast<raw>(xp.x >> 16);
            praw[2] = static_cast<raw>(xp.y & 0xffffu); praw[3] = static_cast<raw>(xp.y >> 16);
            graw[0] = static_cast<raw>(xg.x & 0xffffu); graw[1] = static_cast<raw>(xg.x >> 16);
            graw[2] = static_cast<raw>(xg.y & 0xffffu); graw[3] = static_cast<raw>(xg.y >> 16);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) live[j] = true;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t e = e0 + j;
            live[j] = e < n;
            praw[j] = 0;
            graw[j] = 0;
            if (live[j]) {
                praw[j] = p[e];
                graw[j] = g[e];
                w1 |= static_cast<uint32_t>(c1[e]) << (8 * j);
                w2 |= static_cast<uint32_t>(c2[e]) << (8 * j);
                if constexpr (kMix) w3 |= static_cast<uint32_t>(c1[n + e]) << (8 * j);
            }
        }
    }
    in.w1 = w1;
    in.w2 = w2;
    in.w3 = w3;
    return in;
}

// The bias corrections of a dense run.  Once beta^t is below half an ulp
// of 1 (for beta1 = 0.9 from step 165, for beta2 = 0.999 from step 17,318),
// fl32(1 - beta^t) is exactly 1, its binary64 reciprocal is 1 and the
// division returns its operand unchanged (every value; the moments are
// results of arithmetic, never signalling NaNs), so the run leaves it out:
// BC bit 0 for m / bc1, bit 1 for v / bc2.
template <int BC>
__device__ __forceinline__ void bias_corrected_bc(float m, float v, const StepScalars& s, float& mh,
                                                  float& vh)
{
    mh = (BC & 1) ? m : div_step_constant(m, s.rbc1);
    vh = (BC & 2) ? v : div_step_constant(v, s.rbc2);
}

// Dequantize, update, requantize and store one block loaded by load_block8.
// DENSE (with WIDE): skip_zeros is off, so every block is dense; BC (dense
// runs): the bias corrections that are exactly 1 (bias_corrected_bc).
template <int KIND, typename S, bool WIDE, bool DENSE = false, int BC = 0>
__device__ __forceinline__ void finish_block8(const Seg8& d, int64_t b, const QLds& T,
                                              const StepScalars& sc, int lane, Block8<S>& in,
                                              const Run8& run)
{
    using raw = typename S::raw;
    constexpr bool kMix = KIND == kAdemamix;
    raw* __restrict__ p = static_cast<raw*>(d.p);
    uint8_t* __restrict__ c1 = d.c1;
    uint8_t* __restrict__ c2 = d.c2;
    const int64_t n = d.n;
    const int64_t e0 = b * kQBlock + 4 * lane;
    const bool full = WIDE || in.full;
    const float A1 = in.A1, A2 = in.A2, A3 = in.A3;
    const uint32_t w1 = in.w1, w2 = in.w2, w3 = in.w3;
    raw* praw = in.praw;
    const raw* graw = in.graw;
    const bool* live = in.live;

    // dequantize and update.  A dense block (whole, no skipped elements:
    // wave-uniform) updates every element with no per-element branch, and
    // with 16-bit storage narrows its new parameters in pairs at the store.
    // On the wide path the choice is made once per run (DENSE).
    const bool dense = WIDE ? DENSE : (full && !sc.skip_zeros);
    float m[4], v[4], m2[4], pn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        m[j] = deq_signed(T, (w1 >> (8 * j)) & 0xffu) * A1;
        v[j] = T.t.umag[(w2 >> (8 * j)) & 0xffu] * A2;
        m2[j] = 0.0f;
        if constexpr (kMix) m2[j] = deq_signed(T, (w3 >> (8 * j)) & 0xffu) * A3;
    }
    if (dense) {
        // update_element's steps, the four square roots together
        float mh[4], vh[4], root[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            update_moments<KIND>(S::widen(graw[j]), m[j], v[j], m2[j], sc);
            bias_corrected_bc<BC>(m[j], v[j], sc, mh[j], vh[j]);
        }
        sqrt_rn4(vh, root);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pn[j] = step_param(S::widen(praw[j]), direction_from<KIND>(mh[j], root[j], m2[j], sc), sc.decay,
                               sc.lr, sc.decay_after);
            if constexpr (S::bytes == 4) praw[j] = pn[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (!WIDE && !live[j]) {
                m[j] = 0.0f;
                v[j] = 0.0f;
                m2[j] = 0.0f;
                continue;
            }
            const float gj = S::widen(graw[j]);
            if (sc.skip_zeros && gj == 0.0f) continue;   // moments keep their values, p is not written
            praw[j] = S::narrow(update_element<KIND, true>(S::widen(praw[j]), gj, m[j], v[j], m2[j], sc));
        }
    }

    // new absmax of each state (maxNum from 0: a NaN is passed over, so
    // each lane's value is a non-negative number)
    float l1 = 0.0f, l2 = 0.0f, l3 = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        l1 = __builtin_fmaxf(l1, __builtin_fabsf(m[j]));
        l2 = __builtin_fmaxf(l2, __builtin_fabsf(v[j]));
        if constexpr (kMix) l3 = __builtin_fmaxf(l3, __builtin_fabsf(m2[j]));
    }
    // lane of each state's maximum in l
    constexpr int kLane2 = 32, kLane3 = 16;
    const float l = kMix ? wave_max3(l1, l2, l3) : wave_max2(l1, l2);
    l1 = lane_float(l, 0);
    l2 = lane_float(l, kLane2);
    if constexpr (kMix) l3 = lane_float(l, kLane3);

    // requantize to the magnitude nearest to |value| / absmax.  With
    // absmax 0 (every value +-0 or NaN) or +inf the reciprocal is 0 and the
    // estimate 0 or NaN, which the key takes to the first bucket, and the
    // exact comparison gives index 0 as the definition does.  One
    // reciprocal instruction sequence serves all states.
    const double r = recip_max64(l);
    const double r1 = lane_double(r, 0);
    const double r2 = lane_double(r, kLane2);
    double r3 = 0.0;
    if constexpr (kMix) r3 = lane_double(r, kLane3);
    const double A1d = l1, A2d = l2, A3d = l3;
    uint32_t o1 = 0, o2 = 0, o3 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o1 |= quant_signed(T, m[j], r1, A1d) << (8 * j);
        o2 |= quant_unsigned(T, v[j], r2, A2d) << (8 * j);
        if constexpr (kMix) o3 |= quant_signed(T, m2[j], r3, A3d) << (8 * j);
    }

    // store
    if (full) {
        const uint32_t lo = static_cast<uint32_t>(lane) * 4u;
        if constexpr (S::bytes == 4) {
            // A 16-byte store stays a global store, also on the wide path:
            // after a buffer store of more than 8 bytes with a scalar
            // offset the compiler inserts no wait state before an
            // instruction that overwrites the data registers, and on gfx950
            // that write can reach the store (seen as a wrong first word in
            // some lanes when the next instruction reused the register).
            // Global stores get the wait state; stores of 4 and 8 bytes
            // need none.
            const u32x4 xp = {__builtin_bit_cast(uint32_t, praw[0]), __builtin_bit_cast(uint32_t, praw[1]),
                              __builtin_bit_cast(uint32_t, praw[2]), __builtin_bit_cast(uint32_t, praw[3])};
            __builtin_nontemporal_store(xp, reinterpret_cast<u32x4*>(p + e0));
        } else {
            const u32x2 xp =
                dense ? u32x2{S::narrow2(pn[0], pn[1]), S::narrow2(pn[2], pn[3])}
                      : u32x2{static_cast<uint32_t>(praw[0]) | (static_cast<uint32_t>(praw[1]) << 16),
                              static_cast<uint32_t>(praw[2]) | (static_cast<uint32_t>(praw[3]) << 16)};
            if constexpr (WIDE)
                __builtin_amdgcn_raw_buffer_store_b64(xp, run.p, lo * 2u, run_off<raw>(run, b), kBufNonTemporal);
            else
                __builtin_nontemporal_store(xp, reinterpret_cast<u32x2*>(p + e0));
        }
        if constexpr (WIDE) {
            const int32_t so = run_off<uint8_t>(run, b);
            __builtin_amdgcn_raw_buffer_store_b32(o1, run.c1, lo, so, kBufNonTemporal);
            __builtin_amdgcn_raw_buffer_store_b32(o2, run.c2, lo, so, kBufNonTemporal);
            if constexpr (kMix) __builtin_amdgcn_raw_buffer_store_b32(o3, run.c3, lo, so, kBufNonTemporal);
        } else {
            __builtin_nontemporal_store(o1, reinterpret_cast<uint32_t*>(c1 + e0));
            __builtin_nontemporal_store(o2, reinterpret_cast<uint32_t*>(c2 + e0));
            if constexpr (kMix) __builtin_nontemporal_store(o3, reinterpret_cast<uint32_t*>(c1 + n + e0));
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t e = e0 + j;
            if (!live[j]) continue;
            p[e] = praw[j];
            c1[e] = static_cast<uint8_t>(o1 >> (8 * j));
            c2[e] = static_cast<uint8_t>(o2 >> (8 * j));
            if constexpr (kMix) c1[n + e] = static_cast<uint8_t>(o3 >> (8 * j));
        }
    }
    // every lane holds the block maxima: all store them (one address each),
    // which keeps the store out of a branch
    d.a1[b] = l1;
    d.a2[b] = l2;
    if constexpr (kMix) d.a1[d.nb + b] = l3;
}

// Blocks b0, b0 + stride, ... (count of them, stopping at the tensor's
// end) by one wave, the next block's loads issued before the current block
// is computed.  Any block: partial, or on the element-by-element path.
template <int KIND, typename S>
__device__ __forceinline__ void run_blocks8(const Seg8& d, int64_t b0, int64_t stride, int count,
                                            const QLds& T, const StepScalars& sc, int lane)
{
    if (count <= 0 || b0 >= d.nb) return;
    const Run8 none{};   // per-pointer accesses only
    Block8<S> cur = load_block8<KIND, S, false>(d, b0, lane, none);
    for (int r = 0; r < count; ++r) {
        const int64_t b = b0 + static_cast<int64_t>(r) * stride;
        const int64_t bn = b + stride;
        const bool more = (r + 1 < count) && bn < d.nb;
        Block8<S> nxt;
        if (more) nxt = load_block8<KIND, S, false>(d, bn, lane, none);
        finish_block8<KIND, S, false>(d, b, T, sc, lane, cur, none);
        if (!more) break;
        cur = nxt;
    }
}

// Whether blocks b0 + r * stride (r < count) can all take run_wide8: an
// even count, every block whole, the tensor on the wide path.
__device__ __forceinline__ bool wide_run8(const Seg8& d, int64_t b0, int64_t stride, int count)
{
    return d.vec_ok && count >= 2 && count % 2 == 0 &&
           (b0 + static_cast<int64_t>(count - 1) * stride + 1) * kQBlock <= d.n;
}

// The same blocks when wide_run8 holds, with `a` holding block b0's
// inputs and `run` based at b0.  Two block buffers alternate and every load
// is unconditional, so the loads of one block stay in flight while the
// other is computed (no register copies between iterations, whose waits
// would drain them).  DENSE: skip_zeros is off (straight-line blocks); BC:
// as for finish_block8.
template <int KIND, typename S, bool DENSE, int BC>
__device__ __forceinline__ void run_wide8(const Seg8& d, int64_t b0, int64_t stride, int count,
                                          const QLds& T, const StepScalars& sc, int lane, Block8<S> a,
                                          const Run8& run)
{
    int64_t b = b0;
    for (int r = 2; r < count; r += 2) {
        Block8<S> c = load_block8<KIND, S, true>(d, b + stride, lane, run);
        finish_block8<KIND, S, true, DENSE, BC>(d, b, T, sc, lane, a, run);
        a = load_block8<KIND, S, true>(d, b + 2 * stride, lane, run);
        finish_block8<KIND, S, true, DENSE, BC>(d, b + stride, T, sc, lane, c, run);
        b += 2 * stride;
    }
    Block8<S> c = load_block8<KIND, S, true>(d, b + stride, lane, run);
    finish_block8<KIND, S, true, DENSE, BC>(d, b, T, sc, lane, a, run);
    finish_block8<KIND, S, true, DENSE, BC>(d, b + stride, T, sc, lane, c, run);
}

template <int KIND, typename S>
__device__ __forceinline__ void run_wide8_any(const Seg8& d, int64_t b0, int64_t stride, int count,
                                              const QLds& T, const StepScalars& sc, int lane,
                                              const Block8<S>& a, const Run8& run)
{
    if (sc.skip_zeros)
        run_wide8<KIND, S, false, 0>(d, b0, stride, count, T, sc, lane, a, run);
    else if (sc.rbc1 == 1.0 && sc.rbc2 == 1.0)
        run_wide8<KIND, S, true, 3>(d, b0, stride, count, T, sc, lane, a, run);
    else if (sc.rbc1 == 1.0)   // beta1 < beta2: m's correction reaches 1 first
        run_wide8<KIND, S, true, 1>(d, b0, stride, count, T, sc, lane, a, run);
    else
        run_wide8<KIND, S, true, 0>(d, b0, stride, count, T, sc, lane, a, run);
}

// Single tensor: workgroup w (in XCD runs, xcd_tile) takes blocks
// [w*W*R, (w+1)*W*R) with W waves of R blocks each, interleaved so that the
// W waves work on W neighbouring blocks at a time.
template <int KIND, typename S>
__device__ __forceinline__ void single8(Seg8 d, StepScalars sc, int32_t blocks_per_wave, int32_t xcd_log2)
{
    __shared__ QLds T;
    const int waves = static_cast<int>(blockDim.x) / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int lane = static_cast<int>(threadIdx.x) % kWave;
    const int64_t wg = xcd_tile(blockIdx.x, gridDim.x, xcd_log2);
    const int64_t first = wg * waves * blocks_per_wave + wave;
    // the first block's loads overlap the table copy
    const bool wide = wide_run8(d, first, waves, blocks_per_wave);
    const Run8 run = make_run8<KIND, S>(d, first);   // scalar work only; used when wide
    Block8<S> a;
    if (wide) a = load_block8<KIND, S, true>(d, first, lane, run);
    load_qtables(&T);
    if (wide)
        run_wide8_any<KIND, S>(d, first, waves, blocks_per_wave, T, sc, lane, a, run);
    else
        run_blocks8<KIND, S>(d, first, waves, blocks_per_wave, T, sc, lane);
}

template <int KIND, typename S>
__global__ void __launch_bounds__(1024)
k8_single(Seg8 d, StepScalars sc, int32_t blocks_per_wave, int32_t xcd_log2)
{
    single8<KIND, S>(d, sc, blocks_per_wave, xcd_log2);
}

// The same with at least 6 waves resident per SIMD (at most 80 VGPRs, 3 of
// them spilled), for Adam with fp32 storage: that kernel reaches neither
// the VALU issue rate nor HBM's, and at 83 VGPRs only 5 waves per SIMD
// hide its latencies.  Measured on MI355X at 2^28 elements, interleaved
// with the 5-wave build: -0.6% and -1.7% of the time on two boxes.  The
// 16-bit kernels are issue-bound and lost 1-9% under the same bound (the
// AdEMAMix ones spill), AdEMAMix with fp32 storage lost 0.6% at 5 waves.
template <int KIND, typename S>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(6)))
k8_single_w6(Seg8 d, StepScalars sc, int32_t blocks_per_wave, int32_t xcd_log2)
{
    single8<KIND, S>(d, sc, blocks_per_wave, xcd_log2);
}

// Collection: one wave per work item (segment, run of `chunk_blocks`
// blocks starting at chunk * chunk_blocks).
template <int KIND, typename S>
__global__ void __launch_bounds__(1024)
k8_multi(const Seg8* __restrict__ segs, const WorkItem* __restrict__ items, int64_t n_items,
         int32_t chunk_blocks, StepScalars sc)
{
    __shared__ QLds T;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int lane = static_cast<int>(threadIdx.x) % kWave;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + wave;
    const bool active = w < n_items;
    Seg8 d{};
    int64_t b0 = 0;
    bool wide = false;
    Block8<S> a;
    if (active) {
        const WorkItem it = items[w];
        d = segs[__builtin_amdgcn_readfirstlane(it.seg)];
        b0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(it.chunk)) * chunk_blocks;
        // the first block's loads overlap the table copy
        wide = wide_run8(d, b0, 1, chunk_blocks);
    }
    const Run8 run = make_run8<KIND, S>(d, b0);   // scalar work only; used when wide
    if (wide) a = load_block8<KIND, S, true>(d, b0, lane, run);
    load_qtables(&T);   // every thread reaches the barrier
    if (!active) return;
    if (wide)
        run_wide8_any<KIND, S>(d, b0, 1, chunk_blocks, T, sc, lane, a, run);
    else
        run_blocks8<KIND, S>(d, b0, 1, chunk_blocks, T, sc, lane);
}

// recip_max on n values (test hook).
__global__ void __launch_bounds__(256)
k8_recip(const float* __restrict__ in, float* __restrict__ out, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = recip_max(in[i]);
}

// The quantizer alone on n (value, absmax) pairs (test hook): the signed
// code of value and the unsigned code of |value|, with the reciprocal of
// absmax taken as the update kernels take that of a block maximum.  absmax
// must be >= 0 and not a NaN, and |value| <= absmax (or a NaN value, or an
// infinite absmax), as in a block.
__global__ void __launch_bounds__(256)
k8_quant(const float* __restrict__ v, const float* __restrict__ absmax, uint8_t* __restrict__ cs,
         uint8_t* __restrict__ cu, int64_t n)
{
    __shared__ QLds T;
    load_qtables(&T);   // every thread reaches the barrier
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = v[i];
        const float a = absmax[i];
        const double r = recip_max64(a);
        cs[i] = static_cast<uint8_t>(quant_signed(T, x, r, a));
        cu[i] = static_cast<uint8_t>(quant_unsigned(T, __builtin_fabsf(x), r, a));
    }
}

template <int KIND, typename S>
const void* pick8(bool multi)
{
    if (multi) return reinterpret_cast<const void*>(&k8_multi<KIND, S>);
    return reinterpret_cast<const void*>(&k8_single<KIND, S>);
}

template <>
const void* pick8<kAdam, F32>(bool multi)
{
    if (multi) return reinterpret_cast<const void*>(&k8_multi<kAdam, F32>);
    return reinterpret_cast<const void*>(&k8_single_w6<kAdam, F32>);
}

template <int KIND>
const void* pick8_dtype(bool multi, int dtype)
{
    switch (dtype) {
    case 0: return pick8<KIND, F32>(multi);
    case 1: return pick8<KIND, F16>(multi);
    case 2: return pick8<KIND, BF16>(multi);
    default: return nullptr;
    }
}

}  // namespace

const void* recip_kernel8() { return reinterpret_cast<const void*>(&k8_recip); }
const void* quant_kernel8() { return reinterpret_cast<const void*>(&k8_quant); }

const void* kernel8(bool multi, int kind, int dtype)
{
    if (kind == kAdam) return pick8_dtype<kAdam>(multi, dtype);
    if (kind == kAdemamix) return pick8_dtype<kAdemamix>(multi, dtype);
    return nullptr;
}

}  // namespace ou
