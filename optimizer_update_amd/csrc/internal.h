// internal.h -- declarations shared by the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "elem.hpp"

namespace ou {

// Segment descriptor of the multi-tensor walk (device-resident table).
struct SegDesc {
    void* p;
    const void* g;
    float* s1;
    float* s2;
    int64_t n;
    int32_t vec_ok;  // every stream 16-byte aligned (dwordx4 path)
    int32_t pad;
    int64_t clip_base;  // first partial-norm slot of this segment (clipped steps)
};
static_assert(sizeof(SegDesc) == 56, "SegDesc layout");

// Work item: one wave updates elements [chunk*chunk_elems, min(n, +chunk_elems))
// of segment seg.
struct WorkItem {
    int32_t seg;
    int32_t chunk;
};
static_assert(sizeof(WorkItem) == 8, "WorkItem layout");

// Launch shape of the single-tensor kernel.
struct SingleLaunch {
    int block;    // threads per block: 64, 128, 256, 512 or 1024
    int epl;      // elements per lane per vector group: 4 or 8
    int unroll;   // vector groups in flight per lane: 1, 2 or 4
    int64_t grid; // blocks
    int lds;      // dynamic LDS bytes reserved (not used by the kernel) to cap blocks per CU
    int xcd_log2; // XCD tile runs of 2^xcd_log2 tiles (k_single's xcd_tile), -1: block order
};

// Launch bound of the multi-tensor kernels (k_multi, k_clip_apply_multi):
// at most 8 waves per block.
constexpr int kMultiMaxThreads = 512;

// Launch shape of the multi-tensor kernel.
struct MultiLaunch {
    int waves;    // waves per block: 1, 2, 4 or 8
    int epl;      // 4 or 8
    int unroll;   // 1, 2 or 4
    int lds;      // dynamic LDS bytes reserved to cap blocks per CU (0 = no cap)
    int xcd_run;  // blocks per XCD run of the work list's order (xcd_tile)
};

// Device facts the launch selection depends on (cached per device id).
struct DeviceProps {
    int cu_count = 0;
    int lds_per_cu = 0;      // bytes of LDS per compute unit
    int lds_per_block = 0;   // largest LDS allocation of one block
    bool gfx950 = false;
    char arch[64] = {0};
};

// Dynamic LDS that limits a kernel with no LDS of its own to at most
// `blocks` resident blocks per CU (0 when the device does not say).
int lds_cap(const DeviceProps& d, int blocks);

// Kernel entry for the single-tensor streaming kernel launched with `block`
// threads (nullptr if the combination is not instantiated).
const void* single_kernel(int kind, int dtype, int epl, int unroll, int block);
// Kernel entry for the multi-tensor kernel.
const void* multi_kernel(int kind, int dtype, int epl, int unroll);
// Kernels of update-norm clipping: pass 1 (moments and chunk partial
// norms), 2 (finalize: clip factor), 3 (parameter step, unroll 1/2/4);
// 11, 12, 13: the same passes over a plan's collection.
const void* clip_kernel(int pass, int kind, int dtype, int unroll);

// Bandwidth probes (test hook): mode 0 the plain fp32 Adam update's
// traffic (4 fp32 streams read, 3 written), mode 1 its reads alone, mode 2
// its writes alone.
const void* stream_probe_kernel(int mode, int unroll);

// The update kernels' storage rounding alone, dtype OU_F16 or OU_BF16, one
// value at a time or by packed pairs (test hook).
const void* narrow_kernel(int dtype, bool pairs);

// The update kernels' square root alone (test hook).
const void* sqrt_kernel();

// VALU issue probe: 32 binary32 FMAs per round per lane, no memory (test hook).
const void* valu_probe_kernel(int op);   // 0: FMA chains, 1: add chains; nullptr otherwise
constexpr int kClipChunkElems = 2048;   // elements per partial-norm chunk
constexpr int kClipThreadsHost = 256;   // threads of pass 1
constexpr int kClipFinalThreadsHost = 1024;   // threads of pass 2

constexpr int kWave = 64;

// Tile (or work-item group) of block b of a grid of g blocks.  MI355X deals
// workgroups to its 8 XCDs round-robin (block b runs on XCD b mod 8).  With
// log2c >= 0, XCD x takes the runs of c = 2^log2c consecutive tiles at x*c of
// every 8c: each XCD streams contiguous memory while the eight stay within
// one window.  Blocks past the last whole 8c keep their order.  A
// permutation of [0, g): it changes only which block does which tile.
// Plans apply it on the host, to the order of their work lists.
__host__ __device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t g, int32_t log2c)
{
    if (log2c < 0) return b;
    const int64_t span = int64_t(8) << log2c;
    if (b >= (g & ~(span - 1))) return b;
    const int64_t r = b >> 3;
    return ((r >> log2c) << (log2c + 3)) + ((b & 7) << log2c) + (r & ((int64_t(1) << log2c) - 1));
}

// Segment descriptor of the 8-bit block-wise path: codes c1 ([K][n] signed,
// K = 1 Adam, 2 AdEMAMix), c2 ([n] unsigned), absmax a1 ([K][nb]) and a2
// ([nb]) with nb = ceil(n / 256).
struct Seg8 {
    void* p;
    const void* g;
    uint8_t* c1;
    uint8_t* c2;
    float* a1;
    float* a2;
    int64_t n;
    int64_t nb;
    int32_t vec_ok;   // p, g aligned for 4-element accesses, code planes 4-byte aligned
    int32_t pad;
};
static_assert(sizeof(Seg8) == 72, "Seg8 layout");

// Kernels of the 8-bit path: k8_single (Seg8 by value, StepScalars,
// int32 blocks per wave) or k8_multi (Seg8 table, work items, item count,
// int32 blocks per item, StepScalars).  nullptr for other kinds.
const void* kernel8(bool multi, int kind, int dtype);

// The 8-bit kernels' reciprocal of a block maximum alone (test hook).
const void* recip_kernel8();

// The 8-bit kernels' quantizer alone (test hook).
const void* quant_kernel8();

}  // namespace ou
