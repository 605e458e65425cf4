// kernels.hip -- HIP kernels of the 32-bit two-state update for gfx950.
//
// The update is elementwise and bound by HBM traffic (28 B per element for
// fp32 Adam), so the kernels are plain streams: no LDS, no barriers, no
// cross-lane work.  Lanes own EPL consecutive elements ("vector group") and
// move every stream with 16-byte global loads/stores (dwordx4), so one wave
// instruction covers 1 KiB of contiguous memory; UNROLL vector groups per
// lane are loaded before any is computed, to keep enough bytes in flight.
//
//   k_single: one tensor; one tile of blockDim * UNROLL vector groups per
//             block (a grid-stride loop takes over only if the grid had to be
//             capped), then the ragged tail (and any tensor whose streams are
//             not all 16-byte aligned) one element per lane.
//   k_multi:  a collection; each wave takes one work item (segment, chunk)
//             from a device-side list and streams that chunk.  Item and
//             segment descriptor are wave-uniform (scalar loads), so a small
//             tensor costs one wave instead of one block.
//
// Both call update_element from elem.hpp, so launch shape never changes
// the arithmetic.
//
// Measured on MI355X (2^28 elements): one tile per block (grid covering the
// tensor, no grid-stride) with 512 threads and two groups of 4 elements per
// lane runs fp32 Adam at ~5.9 TB/s, the same as a trivial kernel with the
// same 4-read/3-write pattern; a capped grid-stride grid loses 10-20%, and 8
// elements per lane (two dwordx4 per lane per stream) loses up to 40% with
// non-temporal accesses.
#include "internal.h"

#pragma clang fp contract(off)

namespace ou {
namespace {

// ---- raw 16-byte / 8-byte moves ---------------------------------------------

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

// Element j of a word array holding storage values.
template <typename S, int DW>
__device__ __forceinline__ typename S::raw get_raw(const Words<DW>& x, int j)
{
    if constexpr (S::bytes == 4) {
        return __builtin_bit_cast(float, x.w[j]);
    } else {
        const uint32_t w = x.w[j >> 1];
        return static_cast<uint16_t>((j & 1) ? (w >> 16) : (w & 0xffffu));
    }
}

template <typename S, int DW>
__device__ __forceinline__ void set_raw(Words<DW>& x, int j, typename S::raw v)
{
    if constexpr (S::bytes == 4) {
        x.w[j] = __builtin_bit_cast(uint32_t, v);
    } else {
        const uint32_t b = static_cast<uint32_t>(v);
        if (j & 1)
            x.w[j >> 1] = (x.w[j >> 1] & 0xffffu) | (b << 16);
        else
            x.w[j >> 1] = (x.w[j >> 1] & 0xffff0000u) | b;
    }
}

// ---- one vector group: EPL consecutive elements of every stream -------------

template <int KIND, typename S, int EPL>
struct Group {
    static constexpr int SDW = EPL * S::bytes / 4;  // storage dwords
    static constexpr int FDW = EPL;                 // fp32 state dwords
    Words<SDW> p, g;
    Words<FDW> m, v, m2;

    // vi: index of the vector group (element offset vi * EPL).
    __device__ __forceinline__ void load(const typename S::raw* pp, const typename S::raw* gp,
                                         const float* s1, const float* s2, int64_t n, int64_t vi)
    {
        const int64_t e = vi * EPL;
        p = load_words<SDW>(pp + e);
        g = load_words<SDW>(gp + e);
        m = load_words<FDW>(s1 + e);
        v = load_words<FDW>(s2 + e);
        if constexpr (KIND == kAdemamix) m2 = load_words<FDW>(s1 + n + e);
    }

    __device__ __forceinline__ void compute(const StepScalars& sc)
    {
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const float gj = S::widen(get_raw<S>(g, j));
            const typename S::raw praw = get_raw<S>(p, j);
            float mj = __builtin_bit_cast(float, m.w[j]);
            float vj = __builtin_bit_cast(float, v.w[j]);
            float m2j = 0.0f;
            if constexpr (KIND == kAdemamix) m2j = __builtin_bit_cast(float, m2.w[j]);
            const float pn = update_element<KIND>(S::widen(praw), gj, mj, vj, m2j, sc);
            const bool keep = sc.skip_zeros && gj == 0.0f;   // skipped: old bits stay
            set_raw<S>(p, j, keep ? praw : S::narrow(pn));
            if (!keep) {
                m.w[j] = __builtin_bit_cast(uint32_t, mj);
                v.w[j] = __builtin_bit_cast(uint32_t, vj);
                if constexpr (KIND == kAdemamix) m2.w[j] = __builtin_bit_cast(uint32_t, m2j);
            }
        }
    }

    __device__ __forceinline__ void store(typename S::raw* pp, float* s1, float* s2, int64_t n,
                                          int64_t vi) const
    {
        const int64_t e = vi * EPL;
        store_words<SDW>(pp + e, p);
        store_words<FDW>(s1 + e, m);
        store_words<FDW>(s2 + e, v);
        if constexpr (KIND == kAdemamix) store_words<FDW>(s1 + n + e, m2);
    }
};

// ---- single tensor ------------------------------------------------------------

template <int KIND, typename S, int EPL, int U>
__global__ void __launch_bounds__(1024)
k_single(typename S::raw* __restrict__ p, const typename S::raw* __restrict__ g,
         float* __restrict__ s1, float* __restrict__ s2, int64_t n, StepScalars sc,
         int32_t vec_ok)
{
    const int64_t nvec = vec_ok ? n / EPL : 0;
    const int64_t bdim = blockDim.x;
    const int64_t nthreads = static_cast<int64_t>(gridDim.x) * bdim;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * bdim * U + threadIdx.x; base < nvec;
         base += nthreads * U) {
        Group<KIND, S, EPL> grp[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t vi = base + u * bdim;
            if (vi < nvec) grp[u].load(p, g, s1, s2, n, vi);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t vi = base + u * bdim;
            if (vi < nvec) {
                grp[u].compute(sc);
                grp[u].store(p, s1, s2, n, vi);
            }
        }
    }
    for (int64_t i = nvec * EPL + static_cast<int64_t>(blockIdx.x) * bdim + threadIdx.x; i < n;
         i += nthreads)
        update_scalar<KIND, S>(p, g, s1, s2, n, i, sc);
}

// ---- multi tensor ---------------------------------------------------------------

template <int KIND, typename S, int EPL, int U>
__global__ void __launch_bounds__(512)
k_multi(const SegDesc* __restrict__ segs, const WorkItem* __restrict__ items, int64_t n_items,
        int32_t chunk, StepScalars sc)
{
    using raw = typename S::raw;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int lane = static_cast<int>(threadIdx.x) % kWave;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + wave;
    if (w >= n_items) return;
    const WorkItem it = items[w];
    const SegDesc d = segs[__builtin_amdgcn_readfirstlane(it.seg)];
    raw* __restrict__ p = static_cast<raw*>(d.p);
    const raw* __restrict__ g = static_cast<const raw*>(d.g);
    float* __restrict__ s1 = d.s1;
    float* __restrict__ s2 = d.s2;
    const int64_t n = d.n;
    const int64_t start = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(it.chunk)) * chunk;
    const int64_t len = (n - start < chunk) ? (n - start) : chunk;

    int64_t done = 0;
    if (d.vec_ok) {
        const int64_t nv = len / EPL;
        const int64_t v0 = start / EPL;   // chunk is a multiple of EPL
        for (int64_t base = lane; base < nv; base += kWave * U) {
            Group<KIND, S, EPL> grp[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = base + u * kWave;
                if (j < nv) grp[u].load(p, g, s1, s2, n, v0 + j);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = base + u * kWave;
                if (j < nv) {
                    grp[u].compute(sc);
                    grp[u].store(p, s1, s2, n, v0 + j);
                }
            }
        }
        done = nv * EPL;
    }
    for (int64_t i = start + done + lane; i < start + len; i += kWave)
        update_scalar<KIND, S>(p, g, s1, s2, n, i, sc);
}

// ---- instantiation tables ---------------------------------------------------------

template <int KIND, typename S, int EPL>
const void* pick_single(int unroll)
{
    switch (unroll) {
    case 1: return reinterpret_cast<const void*>(&k_single<KIND, S, EPL, 1>);
    case 2: return reinterpret_cast<const void*>(&k_single<KIND, S, EPL, 2>);
    case 4: return reinterpret_cast<const void*>(&k_single<KIND, S, EPL, 4>);
    default: return nullptr;
    }
}

template <int KIND, typename S, int EPL>
const void* pick_multi(int unroll)
{
    switch (unroll) {
    case 1: return reinterpret_cast<const void*>(&k_multi<KIND, S, EPL, 1>);
    case 2: return reinterpret_cast<const void*>(&k_multi<KIND, S, EPL, 2>);
    case 4: return reinterpret_cast<const void*>(&k_multi<KIND, S, EPL, 4>);
    default: return nullptr;
    }
}

template <int KIND, typename S>
const void* pick(bool multi, int epl, int unroll)
{
    if (epl == 4) return multi ? pick_multi<KIND, S, 4>(unroll) : pick_single<KIND, S, 4>(unroll);
    if (epl == 8) return multi ? pick_multi<KIND, S, 8>(unroll) : pick_single<KIND, S, 8>(unroll);
    return nullptr;
}

template <int KIND>
const void* pick_dtype(bool multi, int dtype, int epl, int unroll)
{
    switch (dtype) {
    case 0: return pick<KIND, F32>(multi, epl, unroll);
    case 1: return pick<KIND, F16>(multi, epl, unroll);
    case 2: return pick<KIND, BF16>(multi, epl, unroll);
    default: return nullptr;
    }
}

const void* pick_all(bool multi, int kind, int dtype, int epl, int unroll)
{
    if (kind == kAdam) return pick_dtype<kAdam>(multi, dtype, epl, unroll);
    if (kind == kAdemamix) return pick_dtype<kAdemamix>(multi, dtype, epl, unroll);
    return nullptr;
}

}  // namespace

const void* single_kernel(int kind, int dtype, int epl, int unroll)
{
    return pick_all(false, kind, dtype, epl, unroll);
}

const void* multi_kernel(int kind, int dtype, int epl, int unroll)
{
    return pick_all(true, kind, dtype, epl, unroll);
}

}  // namespace ou
