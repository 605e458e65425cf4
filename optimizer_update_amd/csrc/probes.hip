// probes.hip -- test-hook kernels (device): the bandwidth and VALU-issue
// probes that measure what the device reaches beside the update, and the
// update's storage rounding and square root on their own, for exhaustive
// checks against IEEE references.  None of them is on the update's path.
#include "internal.h"
#include "stream.hpp"

#pragma clang fp contract(off)

namespace ou {

namespace {

// ---- bandwidth probes (test hook) -----------------------------------------------

// The plain fp32 Adam update's traffic with no arithmetic, in k_single's
// tiles, groups, non-temporal accesses and XCD runs, and its two halves:
//   MODE 0: four fp32 streams read (p, g, m, v), three written back (p, m,
//           v).  Each stored value is the loaded one xor (g & mask), mask = 0
//           from the host: the gradient is really read, no store can be
//           dropped as rewriting the loaded value, and every value written
//           equals the one read.
//   MODE 1: the four reads alone.  The xor of everything read is stored only
//           if it matches a pattern under the runtime mask (never, with
//           mask = 0), so no load can be dropped and nothing is written.
//   MODE 2: the three writes alone: p, m, v receive a value formed from the
//           runtime mask and the index (their contents are destroyed).
// They measure what this read/write mix, its reads and its writes reach on
// the device.
template <int MODE, int U>
__global__ void __launch_bounds__(1024)
k_stream_probe(float* __restrict__ p, const float* __restrict__ g, float* __restrict__ s1,
               float* __restrict__ s2, int64_t nvec, uint32_t mask, int32_t xcd_log2)
{
    const int64_t bdim = blockDim.x;
    const int64_t nthreads = static_cast<int64_t>(gridDim.x) * bdim;
    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x, xcd_log2);
    uint32_t acc = 0;
    for (int64_t base = bid * bdim * U + threadIdx.x; base < nvec; base += nthreads * U) {
        Words<4> wp[U], wg[U], wm[U], wv[U];
        if constexpr (MODE != 2) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t vi = base + u * bdim;
                if (vi >= nvec) continue;
                wp[u] = load_words<4>(p + 4 * vi);
                wg[u] = load_words<4>(g + 4 * vi);
                wm[u] = load_words<4>(s1 + 4 * vi);
                wv[u] = load_words<4>(s2 + 4 * vi);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t vi = base + u * bdim;
            if (vi >= nvec) continue;
            if constexpr (MODE == 1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) acc ^= wp[u].w[j] ^ wg[u].w[j] ^ wm[u].w[j] ^ wv[u].w[j];
            } else {
                if constexpr (MODE == 2) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t x = mask ^ static_cast<uint32_t>(4 * vi + j);
                        wp[u].w[j] = x;
                        wm[u].w[j] = x;
                        wv[u].w[j] = x;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {   // every stored value depends on the mask
                        const uint32_t x = wg[u].w[j] & mask;
                        wp[u].w[j] ^= x;
                        wm[u].w[j] ^= x;
                        wv[u].w[j] ^= x;
                    }
                }
                store_words<4>(p + 4 * vi, wp[u]);
                store_words<4>(s1 + 4 * vi, wm[u]);
                store_words<4>(s2 + 4 * vi, wv[u]);
            }
        }
    }
    if constexpr (MODE == 1) {
        if (mask != 0 && (acc & mask) == 0x9e3779b9u) p[0] = static_cast<float>(acc);
    }
}

// VALU issue probe (test hook): every lane runs `iters` rounds of 64
// independent full-rate binary32 operations (8 chains, 8 deep per round)
// on registers, with no memory traffic; the result is stored only if it
// matches a pattern under the runtime mask (never, with mask = 0).  OP 0:
// fused multiply-adds (v_fmac_f32); OP 1: additions (v_add_f32), which
// draw less power, so the clock can stay higher.  Run with enough waves to
// fill every SIMD, it measures the rate at which the device issues
// full-rate VALU instructions (one quad-cycle each) under that load.
template <int OP>
__global__ void __launch_bounds__(256)
k_valu_probe(float* __restrict__ out, int32_t iters, uint32_t mask)
{
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = static_cast<float>(threadIdx.x + k);
    // runtime operands (mask = 0), so that no operation folds away
    const float a = __builtin_bit_cast(float, 0x3a800000u ^ mask);
    const float b = __builtin_bit_cast(float, 0x3f7fbe77u ^ mask) * static_cast<float>(threadIdx.x & 1);
    for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = OP == 0 ? __builtin_fmaf(a, b, x[k]) : x[k] + a;
    }
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += x[k];
    if (mask != 0 && (__builtin_bit_cast(uint32_t, acc) & mask) == 0x9e3779b9u) out[0] = acc;
}

// The storage rounding of the update kernels (S::narrow of elem.hpp) on n
// binary32 values, for testing it on every bit pattern (test hook).
template <typename S>
__global__ void __launch_bounds__(256)
k_narrow(const float* __restrict__ in, typename S::raw* __restrict__ out, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = S::narrow(in[i]);
}

// The same by pairs (S::narrow2, the 8-bit kernels' packed form): n even,
// out 4-byte aligned.
template <typename S>
__global__ void __launch_bounds__(256)
k_narrow2(const float* __restrict__ in, uint32_t* __restrict__ out, int64_t npairs)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < npairs; i += stride)
        out[i] = S::narrow2(in[2 * i], in[2 * i + 1]);
}

// The 8-bit kernels' square root (sqrt_rn of elem.hpp) on n binary32
// values, for testing it on every bit pattern (test hook).  Consecutive
// values go to consecutive lanes, so a wave whose inputs are all >= 2^-96
// takes sqrt_rn's short form.
__global__ void __launch_bounds__(256)
k_sqrt(const float* __restrict__ in, float* __restrict__ out, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = sqrt_rn(in[i]);
}

}  // namespace

const void* sqrt_kernel() { return reinterpret_cast<const void*>(&k_sqrt); }

const void* valu_probe_kernel(int op)
{
    switch (op) {
    case 0: return reinterpret_cast<const void*>(&k_valu_probe<0>);
    case 1: return reinterpret_cast<const void*>(&k_valu_probe<1>);
    default: return nullptr;
    }
}

const void* narrow_kernel(int dtype, bool pairs)
{
    if (dtype == 1) return pairs ? reinterpret_cast<const void*>(&k_narrow2<F16>)
                                 : reinterpret_cast<const void*>(&k_narrow<F16>);
    if (dtype == 2) return pairs ? reinterpret_cast<const void*>(&k_narrow2<BF16>)
                                 : reinterpret_cast<const void*>(&k_narrow<BF16>);
    return nullptr;
}

template <int MODE>
const void* pick_probe(int unroll)
{
    switch (unroll) {
    case 1: return reinterpret_cast<const void*>(&k_stream_probe<MODE, 1>);
    case 2: return reinterpret_cast<const void*>(&k_stream_probe<MODE, 2>);
    case 4: return reinterpret_cast<const void*>(&k_stream_probe<MODE, 4>);
    default: return nullptr;
    }
}

const void* stream_probe_kernel(int mode, int unroll)
{
    switch (mode) {
    case 0: return pick_probe<0>(unroll);
    case 1: return pick_probe<1>(unroll);
    case 2: return pick_probe<2>(unroll);
    default: return nullptr;
    }
}

}  // namespace ou
