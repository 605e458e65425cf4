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
#include "stream.hpp"

#pragma clang fp contract(off)

namespace ou {
namespace {

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
        if constexpr (kTwoState<KIND>) v = load_words<FDW>(s2 + e);
        if constexpr (KIND == kAdemamix) m2 = load_words<FDW>(s1 + n + e);
    }

    __device__ __forceinline__ void compute(const StepScalars& sc)
    {
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const float gj = S::widen(get_raw<S>(g, j));
            const typename S::raw praw = get_raw<S>(p, j);
            float mj = __builtin_bit_cast(float, m.w[j]);
            float vj = 0.0f;
            if constexpr (kTwoState<KIND>) vj = __builtin_bit_cast(float, v.w[j]);
            float m2j = 0.0f;
            if constexpr (KIND == kAdemamix) m2j = __builtin_bit_cast(float, m2.w[j]);
            const float pn = update_element<KIND>(S::widen(praw), gj, mj, vj, m2j, sc);
            const bool keep = sc.skip_zeros && gj == 0.0f;   // skipped: old bits stay
            set_raw<S>(p, j, keep ? praw : S::narrow(pn));
            if (!keep) {
                m.w[j] = __builtin_bit_cast(uint32_t, mj);
                if constexpr (kTwoState<KIND>) v.w[j] = __builtin_bit_cast(uint32_t, vj);
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
        if constexpr (kTwoState<KIND>) store_words<FDW>(s2 + e, v);
        if constexpr (KIND == kAdemamix) store_words<FDW>(s1 + n + e, m2);
    }
};

// ---- single tensor ------------------------------------------------------------


// MAXT is the largest block the instantiation accepts.  With four groups
// per lane in flight AdEMAMix's five fp32 streams need more than the 128
// VGPRs a lane may hold under a 1024-thread bound (it spills), so the
// four-group shapes of at most 256 threads have a 256-thread instantiation
// of their own; larger blocks take the 1024-thread one.  The arithmetic is
// the same inline update_element in both.
template <int KIND, typename S, int EPL, int U, int MAXT>
__global__ void __launch_bounds__(MAXT)
k_single(typename S::raw* __restrict__ p, const typename S::raw* __restrict__ g,
         float* __restrict__ s1, float* __restrict__ s2, int64_t n, StepScalars sc,
         int32_t vec_ok, int32_t xcd_log2)
{
    const int64_t nvec = vec_ok ? n / EPL : 0;
    const int64_t bdim = blockDim.x;
    const int64_t nthreads = static_cast<int64_t>(gridDim.x) * bdim;
    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x, xcd_log2);
    for (int64_t base = bid * bdim * U + threadIdx.x; base < nvec;
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
    for (int64_t i = nvec * EPL + bid * bdim + threadIdx.x; i < n; i += nthreads)
        update_scalar<KIND, S>(p, g, s1, s2, n, i, sc);
}

// ---- multi tensor ---------------------------------------------------------------

template <int KIND, typename S, int EPL, int U>
__global__ void __launch_bounds__(kMultiMaxThreads)
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

// ---- update-norm clipping ------------------------------------------------------
//
// Three launches: (1) k_clip_moments updates the moments and writes, for each
// fixed chunk of kClipChunk elements, the binary64 partial sums of u^2 and
// p^2; (2) k_clip_finalize sums the partials and forms the clip factor s and
// fl32(lr * s); (3) k_clip_apply recomputes u from the stored moments (the
// same operations on the same values, so the same u) and moves p.  The chunk
// partition, each thread's elements within a chunk and every summation
// order are fixed, so the result does not depend on the launch shape of
// pass 3 or on the vector/per-element choice.

constexpr int kClipThreads = 256;
constexpr int kClipChunk = 2048;   // = kClipThreads * 2 groups * 4 elements

// Sum of (a, b) over a block of NW waves in a fixed order: an xor
// butterfly inside each wave (partners add the same two values, so every
// lane ends with the same sum), then the wave sums as a balanced pairwise
// tree (w0 + w1) + (w2 + w3) ...  lds holds NW entries.
template <int NW>
__device__ __forceinline__ double2 block_sum2(double a, double b, double2* lds)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        a += __shfl_xor(a, off);
        b += __shfl_xor(b, off);
    }
    const int wave = static_cast<int>(threadIdx.x) / kWave;
    if (threadIdx.x % kWave == 0) lds[wave] = make_double2(a, b);
    __syncthreads();
    double2 v[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) v[w] = lds[w];
#pragma unroll
    for (int width = 1; width < NW; width *= 2)
#pragma unroll
        for (int w = 0; w + width < NW; w += 2 * width) {
            v[w].x += v[w + width].x;
            v[w].y += v[w + width].y;
        }
    return v[0];
}

// Pass 1 body for one chunk: thread t owns the elements
// chunk*2048 + h*1024 + 4t + j (h = 0, 1; j = 0..3) and adds their u^2 and
// p^2 in that order; returns the block's sums (same value in every thread).
// A chunk that lies wholly inside a 16-byte-aligned tensor is moved with
// 16-byte accesses, all loads issued before any arithmetic; the last,
// partial chunk (and unaligned tensors) go element by element.  Both paths
// add in the same order.
template <int KIND, typename S>
__device__ __forceinline__ double2 clip_chunk(const typename S::raw* __restrict__ p,
                                              const typename S::raw* __restrict__ g,
                                              float* __restrict__ s1, float* __restrict__ s2,
                                              int64_t n, const StepScalars& sc, bool vec_ok,
                                              int64_t chunk, double2* lds)
{
    constexpr int SDW = 4 * S::bytes / 4;
    const int64_t first = chunk * kClipChunk + 4 * static_cast<int64_t>(threadIdx.x);
    const bool full = vec_ok && (chunk + 1) * kClipChunk <= n;
    float pv[2][4], gv[2][4], mv[2][4], vv[2][4], m2v[2][4];
    if (full) {
        Words<SDW> wp[2], wg[2];
        Words<4> wm[2], wv[2], wm2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t e0 = first + h * (kClipChunk / 2);
            wp[h] = load_words<SDW>(p + e0);
            wg[h] = load_words<SDW>(g + e0);
            wm[h] = load_words<4>(s1 + e0);
            wv[h] = load_words<4>(s2 + e0);
            if constexpr (KIND == kAdemamix) wm2[h] = load_words<4>(s1 + n + e0);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pv[h][j] = S::widen(get_raw<S>(wp[h], j));
                gv[h][j] = S::widen(get_raw<S>(wg[h], j));
                mv[h][j] = __builtin_bit_cast(float, wm[h].w[j]);
                vv[h][j] = __builtin_bit_cast(float, wv[h].w[j]);
                m2v[h][j] = (KIND == kAdemamix) ? __builtin_bit_cast(float, wm2[h].w[j]) : 0.0f;
            }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t e = first + h * (kClipChunk / 2) + j;
                const bool in = e < n;
                pv[h][j] = in ? S::widen(p[e]) : 0.0f;
                gv[h][j] = in ? S::widen(g[e]) : 0.0f;
                mv[h][j] = in ? s1[e] : 0.0f;
                vv[h][j] = in ? s2[e] : 0.0f;
                m2v[h][j] = (KIND == kAdemamix && in) ? s1[n + e] : 0.0f;
            }
    }
    double usq = 0.0, psq = 0.0;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (first + h * (kClipChunk / 2) + j >= n) continue;
            psq += static_cast<double>(pv[h][j]) * static_cast<double>(pv[h][j]);
            if (sc.skip_zeros && gv[h][j] == 0.0f) continue;
            update_moments<KIND>(gv[h][j], mv[h][j], vv[h][j], m2v[h][j], sc);
            const float u = direction<KIND>(mv[h][j], vv[h][j], m2v[h][j], sc);
            usq += static_cast<double>(u) * static_cast<double>(u);
        }
    if (full) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t e0 = first + h * (kClipChunk / 2);
            Words<4> wm, wv, wm2;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wm.w[j] = __builtin_bit_cast(uint32_t, mv[h][j]);
                wv.w[j] = __builtin_bit_cast(uint32_t, vv[h][j]);
                wm2.w[j] = __builtin_bit_cast(uint32_t, m2v[h][j]);
            }
            store_words<4>(s1 + e0, wm);
            store_words<4>(s2 + e0, wv);
            if constexpr (KIND == kAdemamix) store_words<4>(s1 + n + e0, wm2);
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t e = first + h * (kClipChunk / 2) + j;
                if (e >= n) continue;
                s1[e] = mv[h][j];
                s2[e] = vv[h][j];
                if constexpr (KIND == kAdemamix) s1[n + e] = m2v[h][j];
            }
    }
    return block_sum2<kClipThreads / kWave>(usq, psq, lds);
}

// Pass 1, one tensor: one block per chunk (grid = number of chunks), the
// chunk of a block in XCD runs (xcd_tile); each chunk's sums go to its own
// slot, so the order does not reach the result.
template <int KIND, typename S>
__global__ void __launch_bounds__(kClipThreads)
k_clip_moments(const typename S::raw* __restrict__ p, const typename S::raw* __restrict__ g,
               float* __restrict__ s1, float* __restrict__ s2, int64_t n, StepScalars sc,
               int32_t vec_ok, double2* __restrict__ partials, int32_t xcd_log2)
{
    __shared__ double2 lds[kClipThreads / kWave];
    const int64_t chunk = xcd_tile(blockIdx.x, gridDim.x, xcd_log2);
    const double2 tot = clip_chunk<KIND, S>(p, g, s1, s2, n, sc, vec_ok != 0, chunk, lds);
    if (threadIdx.x == 0) partials[chunk] = tot;
}

// Pass 1, collection: one block per (segment, chunk) item; the chunk's sums
// go to the segment's slice of the partials.
template <int KIND, typename S>
__global__ void __launch_bounds__(kClipThreads)
k_clip_moments_multi(const SegDesc* __restrict__ segs, const WorkItem* __restrict__ items,
                     StepScalars sc, double2* __restrict__ partials)
{
    using raw = typename S::raw;
    __shared__ double2 lds[kClipThreads / kWave];
    const WorkItem it = items[blockIdx.x];
    const SegDesc d = segs[__builtin_amdgcn_readfirstlane(it.seg)];
    const int64_t chunk = __builtin_amdgcn_readfirstlane(it.chunk);
    const double2 tot = clip_chunk<KIND, S>(static_cast<const raw*>(d.p), static_cast<const raw*>(d.g),
                                            d.s1, d.s2, d.n, sc, d.vec_ok != 0, chunk, lds);
    if (threadIdx.x == 0) partials[d.clip_base + chunk] = tot;
}

// Pass 2 body (kFinalThreads threads): thread t adds the partials of
// chunks t, t + kFinalThreads, ... in order (kAhead loads in flight), then
// the block sum.  out[0] = fl32(lr * s), out[1] = s with
// s = min(1, max_unorm * ||p|| / ||u||) (1 when ||u|| = 0).
constexpr int kFinalThreads = 1024;

__device__ __forceinline__ void clip_finalize(const double2* __restrict__ partials, int64_t nchunks,
                                              float max_unorm, float lr, float* __restrict__ out,
                                              double2* lds)
{
    double usq = 0.0, psq = 0.0;
    constexpr int kAhead = 16;
    int64_t c = threadIdx.x;
    for (; c + (kAhead - 1) * kFinalThreads < nchunks; c += kAhead * kFinalThreads) {
        double2 v[kAhead];
#pragma unroll
        for (int k = 0; k < kAhead; ++k) v[k] = partials[c + k * kFinalThreads];
#pragma unroll
        for (int k = 0; k < kAhead; ++k) {
            usq += v[k].x;
            psq += v[k].y;
        }
    }
    for (; c < nchunks; c += kFinalThreads) {
        usq += partials[c].x;
        psq += partials[c].y;
    }
    const double2 tot = block_sum2<kFinalThreads / kWave>(usq, psq, lds);
    if (threadIdx.x == 0) {
        float s = 1.0f;
        if (max_unorm > 0.0f && tot.x > 0.0) {
            const double r = static_cast<double>(max_unorm) * __builtin_sqrt(tot.y) / __builtin_sqrt(tot.x);
            if (r < 1.0) s = static_cast<float>(r);
        }
        out[0] = lr * s;
        out[1] = s;
    }
}

// Pass 2, one tensor: a single block.
__global__ void __launch_bounds__(kFinalThreads)
k_clip_finalize(const double2* __restrict__ partials, int64_t nchunks, float max_unorm, float lr,
                float* __restrict__ out)
{
    __shared__ double2 lds[kFinalThreads / kWave];
    clip_finalize(partials, nchunks, max_unorm, lr, out, lds);
}

// Pass 2, collection: one block per segment; out holds two floats per segment.
__global__ void __launch_bounds__(kFinalThreads)
k_clip_finalize_multi(const SegDesc* __restrict__ segs, const double2* __restrict__ partials,
                      float max_unorm, float lr, float* __restrict__ out)
{
    __shared__ double2 lds[kFinalThreads / kWave];
    const SegDesc d = segs[blockIdx.x];
    const int64_t nchunks = (d.n + kClipChunk - 1) / kClipChunk;
    clip_finalize(partials + d.clip_base, nchunks, max_unorm, lr, out + 2 * static_cast<int64_t>(blockIdx.x),
                  lds);
}

// The parameter step of pass 3 for 4 elements already in registers.
template <int KIND, typename S>
__device__ __forceinline__ void clip_step4(float pv[4], const float gv[4], const float mv[4],
                                           const float vv[4], const float m2v[4],
                                           const StepScalars& sc, float lr)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float dir = direction<KIND>(mv[j], vv[j], m2v[j], sc);
        const float pn = step_param(pv[j], dir, sc.decay, lr, sc.decay_after);
        if (!(sc.skip_zeros && gv[j] == 0.0f)) pv[j] = pn;
    }
}

// One element of pass 3 (tails and unaligned tensors).
template <int KIND, typename S>
__device__ __forceinline__ void clip_step1(typename S::raw* __restrict__ p,
                                           const typename S::raw* __restrict__ g,
                                           const float* __restrict__ s1, const float* __restrict__ s2,
                                           int64_t n, int64_t i, const StepScalars& sc, float lr)
{
    if (sc.skip_zeros && S::widen(g[i]) == 0.0f) return;
    const float m2 = (KIND == kAdemamix) ? s1[n + i] : 0.0f;
    const float dir = direction<KIND>(s1[i], s2[i], m2, sc);
    p[i] = S::narrow(step_param(S::widen(p[i]), dir, sc.decay, lr, sc.decay_after));
}

// Pass 3: the parameter step with the clipped learning rate *lr_eff, any
// launch shape: U dwordx4 groups per lane (tiles, grid-stride if the grid
// is capped), then the ragged tail one element per lane.  The gradient is
// read only to find skipped elements.
template <int KIND, typename S, int U>
__global__ void __launch_bounds__(1024)
k_clip_apply(typename S::raw* __restrict__ p, const typename S::raw* __restrict__ g,
             const float* __restrict__ s1, const float* __restrict__ s2, int64_t n, StepScalars sc,
             int32_t vec_ok, const float* __restrict__ lr_eff, int32_t xcd_log2)
{
    constexpr int SDW = 4 * S::bytes / 4;
    const float lr = lr_eff[0];
    const int64_t nvec = vec_ok ? n / 4 : 0;
    const int64_t bdim = blockDim.x;
    const int64_t nthreads = static_cast<int64_t>(gridDim.x) * bdim;
    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x, xcd_log2);
    for (int64_t base = bid * bdim * U + threadIdx.x; base < nvec;
         base += nthreads * U) {
        Words<SDW> wp[U], wg[U];
        Words<4> wm[U], wv[U], wm2[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t vi = base + u * bdim;
            if (vi >= nvec) continue;
            wp[u] = load_words<SDW>(p + 4 * vi);
            if (sc.skip_zeros) wg[u] = load_words<SDW>(g + 4 * vi);
            wm[u] = load_words<4>(s1 + 4 * vi);
            wv[u] = load_words<4>(s2 + 4 * vi);
            if constexpr (KIND == kAdemamix) wm2[u] = load_words<4>(s1 + n + 4 * vi);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t vi = base + u * bdim;
            if (vi >= nvec) continue;
            float pv[4], gv[4], mv[4], vv[4], m2v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pv[j] = S::widen(get_raw<S>(wp[u], j));
                gv[j] = sc.skip_zeros ? S::widen(get_raw<S>(wg[u], j)) : 1.0f;
                mv[j] = __builtin_bit_cast(float, wm[u].w[j]);
                vv[j] = __builtin_bit_cast(float, wv[u].w[j]);
                m2v[j] = (KIND == kAdemamix) ? __builtin_bit_cast(float, wm2[u].w[j]) : 0.0f;
            }
            clip_step4<KIND, S>(pv, gv, mv, vv, m2v, sc, lr);
#pragma unroll
            for (int j = 0; j < 4; ++j) set_raw<S>(wp[u], j, S::narrow(pv[j]));
            store_words<SDW>(p + 4 * vi, wp[u]);
        }
    }
    for (int64_t i = 4 * nvec + bid * bdim + threadIdx.x; i < n; i += nthreads)
        clip_step1<KIND, S>(p, g, s1, s2, n, i, sc, lr);
}

// Pass 3, collection: one wave per item of the plan's regular work list,
// with the segment's clipped learning rate.  item_threads (a multiple of
// the wave, dividing the block) work on one item together, so an item's
// 4-element groups are spread over item_threads / 64 waves.
template <int KIND, typename S>
__global__ void __launch_bounds__(kMultiMaxThreads)
k_clip_apply_multi(const SegDesc* __restrict__ segs, const WorkItem* __restrict__ items,
                   int64_t n_items, int32_t chunk, StepScalars sc, const float* __restrict__ seg_out,
                   int32_t item_threads)
{
    using raw = typename S::raw;
    const int per_block = static_cast<int>(blockDim.x) / item_threads;   // items per block
    const int slot = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / item_threads);
    const int lane = static_cast<int>(threadIdx.x) % item_threads;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * per_block + slot;
    if (w >= n_items) return;
    const WorkItem it = items[w];
    const int seg = __builtin_amdgcn_readfirstlane(it.seg);
    const SegDesc d = segs[seg];
    const float lr = seg_out[2 * static_cast<int64_t>(seg)];
    raw* __restrict__ p = static_cast<raw*>(d.p);
    const raw* __restrict__ g = static_cast<const raw*>(d.g);
    const int64_t n = d.n;
    const int64_t start = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(it.chunk)) * chunk;
    const int64_t len = (n - start < chunk) ? (n - start) : chunk;
    constexpr int SDW = 4 * S::bytes / 4;
    const float* __restrict__ s1 = d.s1;
    const float* __restrict__ s2 = d.s2;
    const int64_t nv = d.vec_ok ? len / 4 : 0;   // chunk starts are multiples of 4
    for (int64_t j4 = lane; j4 < nv; j4 += item_threads) {
        const int64_t e0 = start + 4 * j4;
        Words<SDW> wp = load_words<SDW>(p + e0), wg;
        if (sc.skip_zeros) wg = load_words<SDW>(g + e0);
        const Words<4> wm = load_words<4>(s1 + e0), wv = load_words<4>(s2 + e0);
        Words<4> wm2;
        if constexpr (KIND == kAdemamix) wm2 = load_words<4>(s1 + n + e0);
        float pv[4], gv[4], mv[4], vv[4], m2v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pv[j] = S::widen(get_raw<S>(wp, j));
            gv[j] = sc.skip_zeros ? S::widen(get_raw<S>(wg, j)) : 1.0f;
            mv[j] = __builtin_bit_cast(float, wm.w[j]);
            vv[j] = __builtin_bit_cast(float, wv.w[j]);
            m2v[j] = (KIND == kAdemamix) ? __builtin_bit_cast(float, wm2.w[j]) : 0.0f;
        }
        clip_step4<KIND, S>(pv, gv, mv, vv, m2v, sc, lr);
#pragma unroll
        for (int j = 0; j < 4; ++j) set_raw<S>(wp, j, S::narrow(pv[j]));
        store_words<SDW>(p + e0, wp);
    }
    for (int64_t i = start + 4 * nv + lane; i < start + len; i += item_threads)
        clip_step1<KIND, S>(p, g, s1, s2, n, i, sc, lr);
}

// ---- instantiation tables ---------------------------------------------------------

template <int KIND, typename S, int EPL>
const void* pick_single(int unroll, int block)
{
    switch (unroll) {
    case 1: return reinterpret_cast<const void*>(&k_single<KIND, S, EPL, 1, 1024>);
    case 2: return reinterpret_cast<const void*>(&k_single<KIND, S, EPL, 2, 1024>);
    case 4:
        return block <= 256 ? reinterpret_cast<const void*>(&k_single<KIND, S, EPL, 4, 256>)
                            : reinterpret_cast<const void*>(&k_single<KIND, S, EPL, 4, 1024>);
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
const void* pick(bool multi, int epl, int unroll, int block)
{
    if (epl == 4) return multi ? pick_multi<KIND, S, 4>(unroll) : pick_single<KIND, S, 4>(unroll, block);
    if constexpr (kTwoState<KIND>) {   // 8 elements per lane only for the two-state kinds
        if (epl == 8) return multi ? pick_multi<KIND, S, 8>(unroll) : pick_single<KIND, S, 8>(unroll, block);
    }
    return nullptr;
}

template <int KIND>
const void* pick_dtype(bool multi, int dtype, int epl, int unroll, int block)
{
    switch (dtype) {
    case 0: return pick<KIND, F32>(multi, epl, unroll, block);
    case 1: return pick<KIND, F16>(multi, epl, unroll, block);
    case 2: return pick<KIND, BF16>(multi, epl, unroll, block);
    default: return nullptr;
    }
}

const void* pick_all(bool multi, int kind, int dtype, int epl, int unroll, int block)
{
    switch (kind) {
    case kAdam: return pick_dtype<kAdam>(multi, dtype, epl, unroll, block);
    case kAdemamix: return pick_dtype<kAdemamix>(multi, dtype, epl, unroll, block);
    case kMomentum: return pick_dtype<kMomentum>(multi, dtype, epl, unroll, block);
    case kRmsprop: return pick_dtype<kRmsprop>(multi, dtype, epl, unroll, block);
    case kAdagrad: return pick_dtype<kAdagrad>(multi, dtype, epl, unroll, block);
    case kLion: return pick_dtype<kLion>(multi, dtype, epl, unroll, block);
    default: return nullptr;
    }
}

template <int KIND, typename S>
const void* pick_clip(int pass, int unroll)
{
    if (pass == 1) return reinterpret_cast<const void*>(&k_clip_moments<KIND, S>);
    if (pass == 11) return reinterpret_cast<const void*>(&k_clip_moments_multi<KIND, S>);
    if (pass == 13) return reinterpret_cast<const void*>(&k_clip_apply_multi<KIND, S>);
    switch (unroll) {
    case 1: return reinterpret_cast<const void*>(&k_clip_apply<KIND, S, 1>);
    case 2: return reinterpret_cast<const void*>(&k_clip_apply<KIND, S, 2>);
    case 4: return reinterpret_cast<const void*>(&k_clip_apply<KIND, S, 4>);
    default: return nullptr;
    }
}

template <int KIND>
const void* pick_clip_dtype(int pass, int dtype, int unroll)
{
    switch (dtype) {
    case 0: return pick_clip<KIND, F32>(pass, unroll);
    case 1: return pick_clip<KIND, F16>(pass, unroll);
    case 2: return pick_clip<KIND, BF16>(pass, unroll);
    default: return nullptr;
    }
}

}  // namespace

const void* clip_kernel(int pass, int kind, int dtype, int unroll)
{
    if (pass == 2) return reinterpret_cast<const void*>(&k_clip_finalize);
    if (pass == 12) return reinterpret_cast<const void*>(&k_clip_finalize_multi);
    if (kind == kAdam) return pick_clip_dtype<kAdam>(pass, dtype, unroll);
    if (kind == kAdemamix) return pick_clip_dtype<kAdemamix>(pass, dtype, unroll);
    return nullptr;
}

const void* single_kernel(int kind, int dtype, int epl, int unroll, int block)
{
    return pick_all(false, kind, dtype, epl, unroll, block);
}

const void* multi_kernel(int kind, int dtype, int epl, int unroll)
{
    return pick_all(true, kind, dtype, epl, unroll, 0);
}

}  // namespace ou
