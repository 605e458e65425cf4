// stream.hpp -- the update kernels' raw 16-byte / 8-byte moves of a lane's
// words (device).  Shared by the update kernels and by the bandwidth probe
// that moves the same traffic with no arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ou {
namespace {

template <int DW>
struct Words {
    uint32_t w[DW];
};

// Every byte is touched once per step, so loads and stores carry the
// non-temporal hint (streamed past the caches): on gfx950 this lifts the
// 4-read/3-write stream of the update by ~5-8% over plain accesses.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int DW>
__device__ __forceinline__ Words<DW> load_words(const void* ptr)
{
    Words<DW> r;
    if constexpr (DW == 2) {
        const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(ptr));
        r.w[0] = x.x;
        r.w[1] = x.y;
    } else {
        static_assert(DW % 4 == 0, "dwordx4 granularity");
#pragma unroll
        for (int k = 0; k < DW / 4; ++k) {
            const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr) + k);
            r.w[4 * k + 0] = x.x;
            r.w[4 * k + 1] = x.y;
            r.w[4 * k + 2] = x.z;
            r.w[4 * k + 3] = x.w;
        }
    }
    return r;
}

template <int DW>
__device__ __forceinline__ void store_words(void* ptr, const Words<DW>& r)
{
    if constexpr (DW == 2) {
        const u32x2 x = {r.w[0], r.w[1]};
        __builtin_nontemporal_store(x, reinterpret_cast<u32x2*>(ptr));
    } else {
#pragma unroll
        for (int k = 0; k < DW / 4; ++k) {
            const u32x4 x = {r.w[4 * k + 0], r.w[4 * k + 1], r.w[4 * k + 2], r.w[4 * k + 3]};
            __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(ptr) + k);
        }
    }
}

}  // namespace
}  // namespace ou
