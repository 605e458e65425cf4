// host.hip -- C ABI of the 32-bit two-state optimizer update (host side).
//
// Validation, the per-step scalars, launch selection, the per-device
// property cache, plans (device-resident segment table + work list) and
// graph replay.  The arithmetic itself lives in elem.hpp and runs only on the
// GPU.
//
// The operation is the per-tensor direct op of the page "Investigate a
// 256-thread SM103 path for small 32-bit optimizer tensors" (bitsandbytes
// fork, issue 8), sections "Correctness oracle" and "B300 benchmark and
// acceptance"; the page's own notes on launch selection (section "Scope")
// ask for device detection cached per current device and safe under graph
// capture, which is what DeviceCache does.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/optimizer_update.h"
#include "host_internal.h"
#include "internal.h"
#include "ou_testing.h"

namespace ou {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char* what)
{
    return fail(OU_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- per-device properties, cached per device id (never per process) --------

constexpr int kMaxDevices = 64;

class DeviceCache {
public:
    // Properties of the current device; queried once per device id.
    int current(const DeviceProps** out)
    {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipErrorNoDevice) return fail(OU_EUNSUPPORTED, "no HIP device");
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        if (dev < 0 || dev >= kMaxDevices) return fail(OU_EUNSUPPORTED, "device id %d", dev);
        if (!ready_[dev].load(std::memory_order_acquire)) {
            std::lock_guard<std::mutex> lk(mu_);
            if (!ready_[dev].load(std::memory_order_relaxed)) {
                DeviceProps p;
                e = hipDeviceGetAttribute(&p.cu_count, hipDeviceAttributeMultiprocessorCount, dev);
                if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
                e = hipDeviceGetAttribute(&p.lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
                if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
                e = hipDeviceGetAttribute(&p.lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
                if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
                hipDeviceProp_t prop;
                e = hipGetDeviceProperties(&prop, dev);
                if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
                std::snprintf(p.arch, sizeof p.arch, "%s", prop.gcnArchName);
                p.gfx950 = std::strncmp(p.arch, "gfx950", 6) == 0;
                props_[dev] = p;
                ready_[dev].store(true, std::memory_order_release);
            }
        }
        if (!props_[dev].gfx950)
            return fail(OU_EUNSUPPORTED, "device %d is %s; this library is built for gfx950", dev,
                        props_[dev].arch);
        *out = &props_[dev];
        return OU_OK;
    }

private:
    std::mutex mu_;
    std::atomic<bool> ready_[kMaxDevices] = {};
    DeviceProps props_[kMaxDevices];
};

DeviceCache g_devices;

int current_device(const DeviceProps** out) { return g_devices.current(out); }

// test-only: entry points stop after their argument checks (ou__validate_only)
std::atomic<int> g_validate_only{0};
bool validate_only() { return g_validate_only.load(std::memory_order_relaxed) != 0; }

int lds_cap(const DeviceProps& d, int blocks)
{
    if (blocks < 1 || d.lds_per_cu <= 0 || d.lds_per_block <= 0) return 0;
    // blocks * x fits, (blocks + 1) * x does not; 1 KiB granules
    int x = (d.lds_per_cu / (blocks + 1) + 1024) & ~1023;
    if (x * blocks > d.lds_per_cu || x > d.lds_per_block) return 0;
    return x;
}

// ---- test-only forcing of launch shapes (not part of the public ABI) ---------

std::atomic<int> g_force_block{0}, g_force_epl{0}, g_force_unroll{0}, g_force_scalar{0};
std::atomic<int64_t> g_force_grid{0};
std::atomic<int> g_force_waves{0}, g_force_mepl{0}, g_force_munroll{0}, g_force_chunk{0};
std::atomic<int> g_force_lds{0}, g_force_mlds{0};   // -1 = no cap
std::atomic<int> g_force_xcd{0};                     // tile run length; -1 = block order

// ---- validation -------------------------------------------------------------

int storage_bytes(int dtype) { return dtype == OU_F32 ? 4 : 2; }

bool valid_beta(float b) { return std::isfinite(b) && b >= 0.0f && b < 1.0f; }

bool valid_kind(int kind) { return kind >= OU_ADAM && kind <= OU_LION; }

// Adam and AdEMAMix read and write state2; the one-state kinds ignore it.
bool two_state(int kind) { return kind == OU_ADAM || kind == OU_ADEMAMIX; }

// A kind argument is an ou_kind, optionally OR'ed with OU_DECAY_AFTER
// (kinds with decoupled decay only: ADAM, ADEMAMIX, LION).
int split_kind(int arg, int* kind, int* after)
{
    const int base = arg & ~OU_DECAY_AFTER;
    if (!valid_kind(base)) return fail(OU_EINVAL, "unknown kind %d", arg);
    *kind = base;
    *after = (arg & OU_DECAY_AFTER) ? 1 : 0;
    if (*after && !two_state(base) && base != OU_LION)
        return fail(OU_EINVAL, "OU_DECAY_AFTER applies to ADAM, ADEMAMIX and LION only (kind %d)", base);
    return OU_OK;
}

int check_hparams(int kind, const ou_hparams& h)
{
    if (!valid_kind(kind)) return fail(OU_EINVAL, "unknown kind %d", kind);
    if (!valid_beta(h.beta1) || !valid_beta(h.beta2))
        return fail(OU_EINVAL, "beta1/beta2 must lie in [0, 1) (got %g, %g)", h.beta1, h.beta2);
    if (kind == OU_ADEMAMIX && (!valid_beta(h.beta3) || !std::isfinite(h.alpha)))
        return fail(OU_EINVAL, "beta3 must lie in [0, 1) and alpha be finite (got %g, %g)",
                    h.beta3, h.alpha);
    if (!std::isfinite(h.eps) || h.eps < 0.0f) return fail(OU_EINVAL, "eps must be finite and >= 0");
    if (!std::isfinite(h.lr)) return fail(OU_EINVAL, "lr must be finite");
    if (!std::isfinite(h.weight_decay)) return fail(OU_EINVAL, "weight_decay must be finite");
    if (h.step < 1) return fail(OU_EINVAL, "step must be >= 1 (got %lld)", (long long)h.step);
    return OU_OK;
}

// Pointers, sizes and alignment of one segment; appends its byte ranges.
int check_segment(int kind, const ou_segment& s, int idx, std::vector<Range>* ranges)
{
    if (s.dtype != OU_F32 && s.dtype != OU_F16 && s.dtype != OU_BF16)
        return fail(OU_EINVAL, "segment %d: unknown dtype %d", idx, s.dtype);
    if (s.n < 0) return fail(OU_EINVAL, "segment %d: n < 0", idx);
    if (s.reserved != 0) return fail(OU_EINVAL, "segment %d: reserved field must be 0", idx);
    if (s.n == 0) return OU_OK;
    const bool two = two_state(kind);
    if (!s.param || !s.grad || !s.state1 || (two && !s.state2))
        return fail(OU_EINVAL, "segment %d: null pointer with n > 0", idx);
    const uintptr_t sb = static_cast<uintptr_t>(storage_bytes(s.dtype));
    const uintptr_t P = reinterpret_cast<uintptr_t>(s.param);
    const uintptr_t G = reinterpret_cast<uintptr_t>(s.grad);
    const uintptr_t S1 = reinterpret_cast<uintptr_t>(s.state1);
    const uintptr_t S2 = two ? reinterpret_cast<uintptr_t>(s.state2) : 0;
    if (P % sb || G % sb) return fail(OU_EALIGN, "segment %d: param/grad not %u-byte aligned", idx, (unsigned)sb);
    if (S1 % 4 || S2 % 4) return fail(OU_EALIGN, "segment %d: states not 4-byte aligned", idx);
    const uintptr_t n = static_cast<uintptr_t>(s.n);
    if (n > (uintptr_t(1) << 40)) return fail(OU_EINVAL, "segment %d: n too large", idx);
    const uintptr_t k = (kind == OU_ADEMAMIX) ? 2 : 1;
    ranges->push_back({P, P + n * sb, true, idx});
    ranges->push_back({G, G + n * sb, false, idx});
    ranges->push_back({S1, S1 + k * n * 4, true, idx});
    if (two) ranges->push_back({S2, S2 + n * 4, true, idx});
    return OU_OK;
}

// No range may run past the end of the address space, and no written range
// may overlap any other range (read-only ranges may share).
int check_overlap(std::vector<Range>& r)
{
    for (const Range& x : r)
        if (x.hi < x.lo) return fail(OU_EINVAL, "segment %d: a buffer runs past the end of the address space", x.seg);
    std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
    // Sweep: track the written range reaching furthest and any range reaching furthest.
    uintptr_t any_hi = 0, w_hi = 0;
    int any_seg = -1, w_seg = -1;
    for (const Range& x : r) {
        if (x.lo < w_hi)
            return fail(OU_EOVERLAP, "segment %d overlaps a written buffer of segment %d", x.seg, w_seg);
        if (x.written && x.lo < any_hi)
            return fail(OU_EOVERLAP, "a written buffer of segment %d overlaps segment %d", x.seg, any_seg);
        if (x.hi > any_hi) { any_hi = x.hi; any_seg = x.seg; }
        if (x.written && x.hi > w_hi) { w_hi = x.hi; w_seg = x.seg; }
    }
    return OU_OK;
}

bool streams_16b_aligned(int kind, const ou_segment& s)
{
    uintptr_t a = reinterpret_cast<uintptr_t>(s.param) | reinterpret_cast<uintptr_t>(s.grad) |
                  reinterpret_cast<uintptr_t>(s.state1);
    if (two_state(kind)) a |= reinterpret_cast<uintptr_t>(s.state2);
    uintptr_t slow = 0;
    if (kind == OU_ADEMAMIX) slow = reinterpret_cast<uintptr_t>(s.state1 + s.n);
    return ((a | slow) & 15u) == 0;
}

// ---- per-step scalars ---------------------------------------------------------

// bc = fl32(1 - fl64(beta^step)) and d = fl32(1 - fl64(lr * wd)) in binary64
// from the binary32 arguments; 1 - beta in binary32.
StepScalars make_scalars(const ou_hparams& h, int decay_after)
{
    StepScalars s;
    const double t = static_cast<double>(h.step);
    s.beta1 = h.beta1;
    s.beta2 = h.beta2;
    s.beta3 = h.beta3;
    s.omb1 = 1.0f - h.beta1;
    s.omb2 = 1.0f - h.beta2;
    s.omb3 = 1.0f - h.beta3;
    s.alpha = h.alpha;
    s.eps = h.eps;
    s.lr = h.lr;
    s.bc1 = static_cast<float>(1.0 - std::pow(static_cast<double>(h.beta1), t));
    s.bc2 = static_cast<float>(1.0 - std::pow(static_cast<double>(h.beta2), t));
    s.decay = static_cast<float>(1.0 - static_cast<double>(h.lr) * static_cast<double>(h.weight_decay));
    s.weight_decay = h.weight_decay;
    s.skip_zeros = h.skip_zeros ? 1 : 0;
    s.first_step = h.step == 1 ? 1 : 0;
    s.decay_after = decay_after;
    s.pad = 0;
    s.rbc1 = step_reciprocal(s.bc1);
    s.rbc2 = step_reciprocal(s.bc2);
    return s;
}

// ---- launch selection ---------------------------------------------------------

// Single tensor.  Every lane takes UNROLL groups of 4 elements (one
// dwordx4 of each fp32 stream, dwordx2 of a 16-bit one).  Small tensors (the
// launch-latency regime) get one block sized to the tensor.  Large ones get
// one-wave blocks of 2 groups per lane (a 512-element tile per block), a
// grid that covers the tensor, a cap on resident blocks per CU once the
// grid oversubscribes the CUs 4 times over (single_blocks_per_cu), and
// tiles in runs of 64 per XCD.
// Measured on MI355X in 21 interleaved rounds per case against the earlier
// shapes (256 x 2 at two blocks per CU and runs of 16; fp32 Adam 128 x 4 and
// runs of 32): Adam and AdEMAMix, fp32 and bf16 storage, 2^28 and 2^30
// elements, +2 to +4% in seven of the eight cases and even (-1 to 0%) for
// fp32 AdEMAMix at 2^30; runs of 128 were as good at 2^28 but 3-6% slower
// at 2^30.  Capping residency at all (8 waves per CU instead of up to 32)
// keeps fewer tiles in flight, and the seven streams' DRAM accesses more
// local: 6-10% over full occupancy.  Grid-stride and persistent grids,
// with or without register double-buffering, were slower.
//
// The clipped step's parameter pass (plain = false: p, m, v read, p
// written) takes the same one-wave blocks and runs of 64 with no residency
// cap, and its moments pass (256-thread blocks, one 2,048-element chunk
// each, a block barrier at the end) runs of 64 at full occupancy: measured
// per pass on MI355X at 2^28 (fp32 Adam), passes 1 and 3 take 1,036 and 689
// us against 1,142 and 698 us with 256-thread blocks at two per CU and runs
// of 16 (6.16 against 5.76 TB/s for the whole step, over 40 B per element).
constexpr int kXcdRun = 64;
constexpr int kXcdRunClip = 64;
constexpr int kXcdRunMulti = 16;
constexpr int kSingleBlocksPerCu = 8;

// Resident one-wave blocks per CU of a large single tensor or collection,
// from the bytes a tile reads per element (2 storage values and 1-3 fp32
// states): the more it reads, the fewer tiles in flight keep the streams'
// DRAM accesses local.  Measured on MI355X in 10-20 interleaved rounds per
// cap on four boxes: reading 20 B (fp32 AdEMAMix) 6 beat 8 by 0.1-4.7%,
// reading 16 B (fp32 Adam, 16-bit AdEMAMix) 7 beat 8 by 0.1-3.9%, reading
// 12 B or less (16-bit Adam, the one-state kinds) 8 was level with 10-12.
int single_blocks_per_cu(int kind, int dtype)
{
    const int states = kind == OU_ADEMAMIX ? 3 : two_state(kind) ? 2 : 1;
    const int reads = 2 * storage_bytes(dtype) + 4 * states;
    if (reads >= 20) return 6;
    if (reads >= 16) return 7;
    return kSingleBlocksPerCu;
}

// The clipped step's pass 1 (256-thread blocks of 2,048-element chunks,
// reading p, g, m, v and writing m, v and a partial sum) keeps at most 5
// blocks (20 waves) per CU once its grid oversubscribes the CUs 4 times
// over.  Measured on MI355X at 2^28 fp32 elements, per pass in one kernel
// trace: 1,007 us at 4 or 5 blocks per CU against 1,039 us at full
// occupancy (8 blocks), 1,022-1,035 us at 6-8 and 1,075-1,216 us at 2-3.
// Pass 3 ran best with no cap (693 us against 711 us at 8 one-wave
// blocks per CU) and keeps none.
constexpr int kClipMomentsBlocksPerCu = 5;

int clip_moments_lds(const DeviceProps& d, int64_t grid)
{
    if (d.cu_count <= 0 || grid < 4LL * kClipMomentsBlocksPerCu * d.cu_count) return 0;
    return lds_cap(d, kClipMomentsBlocksPerCu);
}

// Tile runs per XCD (xcd_tile): log2 of the run length for grids of at
// least 64 runs, else -1 (block order).
int xcd_log2_for(int64_t grid, int run)
{
    if (run <= 0 || (run & (run - 1)) != 0) return -1;
    const int lg = __builtin_ctz(static_cast<unsigned>(run));
    return grid >= 64 * int64_t(run) ? lg : -1;
}

// The run after test forcing (ou__force_xcd): -1 = block order.
int xcd_run_forced(int run)
{
    const int f = g_force_xcd.load();
    return f == 0 ? run : f;
}

SingleLaunch select_single(const DeviceProps& d, int kind, int dtype, int64_t n, bool vec, bool plain)
{
    SingleLaunch L;
    L.epl = 4;
    L.lds = 0;
    L.xcd_log2 = -1;
    const int64_t units = vec ? (n + L.epl - 1) / L.epl : n;   // lanes' work units
    if (units <= 1024) {
        L.unroll = 1;
        int64_t b = ((units + kWave - 1) / kWave) * kWave;
        L.block = static_cast<int>(std::max<int64_t>(kWave, std::min<int64_t>(b, 256)));
        L.grid = (units + L.block - 1) / L.block;
        if (L.grid < 1) L.grid = 1;
        return L;
    }
    L.block = kWave;
    L.unroll = 2;
    const int64_t per_block = static_cast<int64_t>(L.block) * L.unroll;
    L.grid = std::max<int64_t>(1, std::min<int64_t>((units + per_block - 1) / per_block, INT32_MAX));
    // cap only when the grid oversubscribes the CUs several times over
    if (plain && d.cu_count > 0 && L.grid >= 4LL * kSingleBlocksPerCu * d.cu_count)
        L.lds = lds_cap(d, single_blocks_per_cu(kind, dtype));
    L.xcd_log2 = xcd_log2_for(L.grid, plain ? kXcdRun : kXcdRunClip);
    return L;
}

// Multi tensor: waves per block, EPL and unroll; the chunk (elements per
// work item) is a multiple of 64 * EPL * unroll so chunk starts keep 16-byte
// alignment.  Large collections get the shape and the residency cap of
// large single tensors (single_blocks_per_cu): over the 505-tensor
// collection (287.9 M elements), 10-16 interleaved rounds per cap, fp32
// Adam ran 3.6-3.9% faster at 7 blocks per CU than at 8, fp32 AdEMAMix
// 3.8-4.7% faster at 6 and bf16 AdEMAMix 2.5% faster at 7; bf16 Adam was
// level from 8 to 10.
// Measured on MI355X in 15 interleaved rounds per shape with the 505-tensor
// bf16 collection (287.9 M elements) and its 408 tensors of <= 16,384
// elements (3.4 M): a large collection runs as the large single tensor
// does, one-wave blocks of 2 groups per lane with one 512-element chunk
// each, at most 8 per CU, in runs of 64 blocks per XCD (990.6 us, 1% ahead
// of 4-wave blocks of 1024-element chunks at 2 per CU, and of the 1-wave
// shape with 1024-element chunks or runs of 32); a collection of small
// tensors needs short chunks to put enough waves on the GPU: 256-element
// chunks, one group per lane, 4 waves per block, no cap (13.3 us, 6% ahead
// of 512-element chunks with 2 groups).  The collection of tensors of
// <= 4,096 elements takes 4.4-4.6 us in every shape (bound by the launch).
constexpr int64_t kLargeCollection = int64_t(1) << 24;

MultiLaunch select_multi(const DeviceProps& d, int kind, int dtype, int64_t total_elements)
{
    MultiLaunch L;
    L.epl = 4;
    if (total_elements >= kLargeCollection) {
        L.waves = 1;
        L.unroll = 2;
        L.lds = lds_cap(d, single_blocks_per_cu(kind, dtype));
        L.xcd_run = kXcdRun;
    } else {
        L.waves = 4;
        L.unroll = 1;
        L.lds = 0;
        L.xcd_run = kXcdRunMulti;
    }
    return L;
}

int64_t select_chunk(int64_t total_elements)
{
    return total_elements >= kLargeCollection ? 512 : 256;
}

void apply_single_forcing(SingleLaunch* L, bool* vec)
{
    if (g_force_scalar.load()) *vec = false;
    if (int b = g_force_block.load()) L->block = b;
    if (int e = g_force_epl.load()) L->epl = e;
    if (int u = g_force_unroll.load()) L->unroll = u;
    if (int64_t gsz = g_force_grid.load()) L->grid = gsz;
    if (int c = g_force_lds.load()) L->lds = c < 0 ? 0 : c;
    if (g_force_xcd.load()) L->xcd_log2 = xcd_log2_for(L->grid, xcd_run_forced(kXcdRun));
}

hipError_t launch(const void* fn, int64_t grid, int block, int lds, void** args, hipStream_t stream)
{
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(static_cast<unsigned>(block)),
                           args, static_cast<size_t>(lds), stream);
}

bool capturing(hipStream_t stream)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess) return false;
    return st != hipStreamCaptureStatusNone;
}

// ---- plans --------------------------------------------------------------------

// One dtype group of a plan: its tables, launch shape and argument storage.
struct Group {
    int dtype;
    MultiLaunch L;
    int64_t chunk;
    int64_t n_items;
    const SegDesc* d_segs;
    const WorkItem* d_items;
    const void* fn;
    int64_t grid;
    // graph replay: node of the plain step (0) and of the clipped step's
    // three passes (1-3)
    hipGraphNode_t node[4];
    // argument storage for launches and graph nodes
    StepScalars sc;
    int32_t chunk32;
    void* args[5];
    float clip_mu, clip_lr;
    const float* clip_seg_out;
    void* clip_args1[4];
    void* clip_args2[5];
    void* clip_args3[7];
    // pass 3's shape: threads per work item, block, grid
    int32_t clip_item_threads;
    int clip_block3;
    int64_t clip_grid3;
    // update-norm clipping: one item per (segment, 2048-element chunk),
    // binary64 partial sums per item, two floats (fl32(lr*s), s) per segment
    int64_t n_segs;
    int64_t n_clip_items;
    int clip_lds1;   // dynamic LDS of pass 1 (its residency cap, clip_moments_lds)
    const WorkItem* d_clip_items;
    double2* d_partials;
    float* d_seg_out;
};

}  // namespace ou

struct ou_plan_s {
    int kind = 0;
    int decay_after = 0;
    int64_t n_elements = 0;
    void* dmem = nullptr;
    std::vector<std::pair<int, int64_t>> seg_map;   // caller's index -> (group, slot), group -1 if n = 0
    std::vector<ou::Group> groups;
    hipGraph_t graph = nullptr;            // plain step
    hipGraphExec_t exec = nullptr;
    hipGraph_t clip_graph = nullptr;       // clipped step
    hipGraphExec_t clip_exec = nullptr;
    int device = -1;
};

namespace ou {
namespace {

int build_plan(int kind_arg, const ou_segment* segs, int32_t nseg, ou_plan_s** out)
{
    *out = nullptr;
    int kind = 0, after = 0;
    if (int st = split_kind(kind_arg, &kind, &after)) return st;
    if (nseg < 0 || (nseg > 0 && !segs)) return fail(OU_EINVAL, "bad segment array");
    std::vector<Range> ranges;
    ranges.reserve(static_cast<size_t>(nseg) * 4);
    for (int i = 0; i < nseg; ++i)
        if (int st = check_segment(kind, segs[i], i, &ranges)) return st;
    if (int st = check_overlap(ranges)) return st;
    if (validate_only()) return OU_OK;
    const DeviceProps* dp = nullptr;
    if (int st = g_devices.current(&dp)) return st;

    ou_plan_s* plan = new (std::nothrow) ou_plan_s;
    if (!plan) return fail(OU_ENOMEM, "plan");
    plan->kind = kind;
    plan->decay_after = after;
    (void)hipGetDevice(&plan->device);

    // Host tables per dtype group: descriptors, then work items (largest
    // chunks first so the long items start early), then the clip items.
    struct HostGroup {
        std::vector<SegDesc> segs;
        std::vector<std::pair<int64_t, WorkItem>> items;   // (length, item)
        std::vector<WorkItem> clip_items;
        int64_t clip_slots = 0;
        MultiLaunch L;
        int64_t chunk;
    };
    HostGroup hg[3];
    int64_t group_elems[3] = {0, 0, 0};
    for (int i = 0; i < nseg; ++i) group_elems[segs[i].dtype] += segs[i].n;
    for (int dt = 0; dt < 3; ++dt) {
        hg[dt].L = select_multi(*dp, kind, dt, group_elems[dt]);
        if (int w = g_force_waves.load()) hg[dt].L.waves = w;
        if (int e = g_force_mepl.load()) hg[dt].L.epl = e;
        if (int u = g_force_munroll.load()) hg[dt].L.unroll = u;
        if (int c = g_force_mlds.load()) hg[dt].L.lds = c < 0 ? 0 : c;
        hg[dt].chunk = select_chunk(group_elems[dt]);
        if (int c = g_force_chunk.load()) hg[dt].chunk = c;
    }
    plan->seg_map.assign(static_cast<size_t>(nseg), {-1, 0});
    for (int i = 0; i < nseg; ++i) {
        const ou_segment& s = segs[i];
        if (s.n == 0) continue;
        HostGroup& G = hg[s.dtype];
        SegDesc d;
        d.p = s.param;
        d.g = s.grad;
        d.s1 = s.state1;
        d.s2 = two_state(kind) ? s.state2 : nullptr;
        d.n = s.n;
        d.vec_ok = streams_16b_aligned(kind, s) ? 1 : 0;
        d.pad = 0;
        d.clip_base = G.clip_slots;
        const int32_t seg_idx = static_cast<int32_t>(G.segs.size());
        plan->seg_map[static_cast<size_t>(i)] = {s.dtype, seg_idx};
        G.segs.push_back(d);
        const int64_t nchunks = (s.n + G.chunk - 1) / G.chunk;
        const int64_t nclip = (s.n + kClipChunkElems - 1) / kClipChunkElems;
        if (nchunks > INT32_MAX || nclip > INT32_MAX) { delete plan; return fail(OU_EINVAL, "segment %d: too many chunks", i); }
        for (int64_t c = 0; c < nchunks; ++c) {
            const int64_t len = std::min<int64_t>(G.chunk, s.n - c * G.chunk);
            G.items.push_back({len, WorkItem{seg_idx, static_cast<int32_t>(c)}});
        }
        for (int64_t c = 0; c < nclip; ++c) G.clip_items.push_back(WorkItem{seg_idx, static_cast<int32_t>(c)});
        G.clip_slots += nclip;
        plan->n_elements += s.n;
    }
    auto align16 = [](size_t x) { return (x + 15) & ~size_t(15); };
    size_t bytes = 0;
    for (auto& G : hg) {
        std::stable_sort(G.items.begin(), G.items.end(),
                         [](const auto& a, const auto& b) { return a.first > b.first; });
        const int64_t nblk = static_cast<int64_t>(G.items.size()) / G.L.waves;
        xcd_order(G.items, G.L.waves, xcd_log2_for(nblk, xcd_run_forced(G.L.xcd_run)));
        // clip pass 1 runs one block per clip item
        const int64_t nclip = static_cast<int64_t>(G.clip_items.size());
        xcd_order(G.clip_items, 1, xcd_log2_for(nclip, xcd_run_forced(kXcdRunClip)));
        if (G.segs.empty()) continue;
        bytes = align16(bytes + G.segs.size() * sizeof(SegDesc));
        bytes = align16(bytes + G.items.size() * sizeof(WorkItem));
        bytes = align16(bytes + G.clip_items.size() * sizeof(WorkItem));
        bytes = align16(bytes + static_cast<size_t>(G.clip_slots) * sizeof(double2));
        bytes = align16(bytes + G.segs.size() * 2 * sizeof(float));
    }
    if (bytes > 0) {
        hipError_t e = hipMalloc(&plan->dmem, bytes);
        if (e != hipSuccess) { delete plan; return fail(OU_ENOMEM, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e)); }
        std::vector<unsigned char> host(bytes, 0);
        unsigned char* base = static_cast<unsigned char*>(plan->dmem);
        size_t off = 0;
        for (int dt = 0; dt < 3; ++dt) {
            HostGroup& G = hg[dt];
            if (G.segs.empty()) continue;
            Group grp{};
            grp.dtype = dt;
            grp.L = G.L;
            grp.chunk = G.chunk;
            grp.n_items = static_cast<int64_t>(G.items.size());
            grp.n_segs = static_cast<int64_t>(G.segs.size());
            grp.n_clip_items = static_cast<int64_t>(G.clip_items.size());
            grp.clip_lds1 = clip_moments_lds(*dp, grp.n_clip_items);
            grp.d_segs = reinterpret_cast<const SegDesc*>(base + off);
            std::memcpy(host.data() + off, G.segs.data(), G.segs.size() * sizeof(SegDesc));
            off = align16(off + G.segs.size() * sizeof(SegDesc));
            grp.d_items = reinterpret_cast<const WorkItem*>(base + off);
            for (size_t k = 0; k < G.items.size(); ++k)
                std::memcpy(host.data() + off + k * sizeof(WorkItem), &G.items[k].second, sizeof(WorkItem));
            off = align16(off + G.items.size() * sizeof(WorkItem));
            grp.d_clip_items = reinterpret_cast<const WorkItem*>(base + off);
            std::memcpy(host.data() + off, G.clip_items.data(), G.clip_items.size() * sizeof(WorkItem));
            off = align16(off + G.clip_items.size() * sizeof(WorkItem));
            grp.d_partials = reinterpret_cast<double2*>(base + off);
            off = align16(off + static_cast<size_t>(G.clip_slots) * sizeof(double2));
            grp.d_seg_out = reinterpret_cast<float*>(base + off);
            for (size_t k = 0; k < G.segs.size(); ++k) {   // (lr_eff, s) = (0, 1) until a clipped step
                const float init[2] = {0.0f, 1.0f};
                std::memcpy(host.data() + off + k * sizeof(init), init, sizeof(init));
            }
            off = align16(off + G.segs.size() * 2 * sizeof(float));
            grp.fn = multi_kernel(kind, dt, grp.L.epl, grp.L.unroll);
            if (!grp.fn || grp.chunk % (kWave * grp.L.epl) != 0 || grp.chunk > INT32_MAX ||
                grp.chunk % 4 != 0 || grp.L.waves < 1 || grp.L.waves * kWave > kMultiMaxThreads) {
                (void)hipFree(plan->dmem);
                delete plan;
                return fail(OU_EINVAL, "no multi-tensor kernel for waves=%d epl=%d unroll=%d chunk=%lld",
                            grp.L.waves, grp.L.epl, grp.L.unroll, (long long)grp.chunk);
            }
            grp.grid = (grp.n_items + grp.L.waves - 1) / grp.L.waves;
            grp.chunk32 = static_cast<int32_t>(grp.chunk);
            // The clipped step's parameter pass (three streams read, one
            // written) gives a 512-element item of the large shape to a
            // two-wave block, one group per lane, as the single-tensor
            // parameter pass does; other shapes keep one wave per item.
            if (grp.L.waves == 1 && grp.L.unroll == 2) {
                grp.clip_item_threads = 2 * kWave;
                grp.clip_block3 = 2 * kWave;
                grp.clip_grid3 = grp.n_items;
            } else {
                grp.clip_item_threads = kWave;
                grp.clip_block3 = grp.L.waves * kWave;
                grp.clip_grid3 = grp.grid;
            }
            plan->groups.push_back(grp);
        }
        e = hipMemcpy(plan->dmem, host.data(), bytes, hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            (void)hipFree(plan->dmem);
            delete plan;
            return hip_fail(e, "hipMemcpy(plan tables)");
        }
    }
    *out = plan;
    return OU_OK;
}

void set_group_args(Group& g, const StepScalars& sc)
{
    g.sc = sc;
    g.args[0] = const_cast<SegDesc**>(&g.d_segs);
    g.args[1] = const_cast<WorkItem**>(&g.d_items);
    g.args[2] = &g.n_items;
    g.args[3] = &g.chunk32;
    g.args[4] = &g.sc;
}

// Arguments of the clipped step's three passes: (1) moments and partial
// norms per (segment, chunk); (2) one block per segment forms the clip
// factor s and fl32(lr * s); (3) the parameter step over the regular work
// list.
void set_clip_args(Group& g, const StepScalars& sc, float max_unorm)
{
    g.sc = sc;
    g.clip_mu = max_unorm;
    g.clip_lr = sc.lr;
    g.clip_seg_out = g.d_seg_out;
    g.clip_args1[0] = const_cast<SegDesc**>(&g.d_segs);
    g.clip_args1[1] = const_cast<WorkItem**>(&g.d_clip_items);
    g.clip_args1[2] = &g.sc;
    g.clip_args1[3] = &g.d_partials;
    g.clip_args2[0] = const_cast<SegDesc**>(&g.d_segs);
    g.clip_args2[1] = &g.d_partials;
    g.clip_args2[2] = &g.clip_mu;
    g.clip_args2[3] = &g.clip_lr;
    g.clip_args2[4] = &g.d_seg_out;
    g.clip_args3[0] = const_cast<SegDesc**>(&g.d_segs);
    g.clip_args3[1] = const_cast<WorkItem**>(&g.d_items);
    g.clip_args3[2] = &g.n_items;
    g.clip_args3[3] = &g.chunk32;
    g.clip_args3[4] = &g.sc;
    g.clip_args3[5] = const_cast<float**>(&g.clip_seg_out);
    g.clip_args3[6] = &g.clip_item_threads;
}

// Launch shape of one launch of a group's step (pass 0: the plain step;
// passes 1-3: the clipped step), with the arguments set above.
int group_launch(int kind, Group& g, int pass, hipKernelNodeParams* kp)
{
    *kp = hipKernelNodeParams{};
    int64_t grid = g.grid;
    int block = g.L.waves * kWave, lds = g.L.lds;
    const void* fn = g.fn;
    void** args = g.args;
    if (pass == 1) {
        fn = clip_kernel(11, kind, g.dtype, 0);
        grid = g.n_clip_items;
        block = kClipThreadsHost;
        lds = g.clip_lds1;
        args = g.clip_args1;
    } else if (pass == 2) {
        fn = clip_kernel(12, kind, g.dtype, 0);
        grid = g.n_segs;
        block = kClipFinalThreadsHost;
        lds = 0;
        args = g.clip_args2;
    } else if (pass == 3) {
        fn = clip_kernel(13, kind, g.dtype, 0);
        grid = g.clip_grid3;
        block = g.clip_block3;
        lds = 0;   // the parameter pass runs best with no residency cap (clip_moments_lds)
        args = g.clip_args3;
    }
    if (!fn) return fail(OU_EINVAL, "no kernel for pass %d, dtype %d", pass, g.dtype);
    kp->func = const_cast<void*>(fn);
    kp->gridDim = dim3(static_cast<unsigned>(grid));
    kp->blockDim = dim3(static_cast<unsigned>(block));
    kp->sharedMemBytes = static_cast<unsigned>(lds);
    kp->kernelParams = args;
    kp->extra = nullptr;
    return OU_OK;
}

int plan_launch(ou_plan_s* plan, const StepScalars& sc, hipStream_t stream)
{
    for (Group& g : plan->groups) {
        set_group_args(g, sc);
        hipError_t e = launch(g.fn, g.grid, g.L.waves * kWave, g.L.lds, g.args, stream);
        if (e != hipSuccess) return hip_fail(e, "launch multi-tensor kernel");
    }
    return OU_OK;
}

// The clipped step of a plan: three launches per dtype group.
int plan_launch_clip(ou_plan_s* plan, const StepScalars& sc, float max_unorm, hipStream_t stream)
{
    for (Group& g : plan->groups) {
        set_clip_args(g, sc, max_unorm);
        for (int pass = 1; pass <= 3; ++pass) {
            hipKernelNodeParams kp;
            if (int st = group_launch(plan->kind, g, pass, &kp)) return st;
            hipError_t e = hipLaunchKernel(kp.func, kp.gridDim, kp.blockDim, kp.kernelParams,
                                           kp.sharedMemBytes, stream);
            if (e != hipSuccess)
                return fail(OU_EHIP, "launch clip pass %d (collection): %s", pass, hipGetErrorString(e));
        }
    }
    return OU_OK;
}

// A step through a HIP graph: the plain step (one node per dtype group) or
// the clipped one (three nodes per group).  Built and instantiated on the
// first call of its form; later calls write the step's scalars into the
// nodes and replay.  All nodes form one chain: groups touch disjoint memory
// and could run side by side, but measured on MI355X a replay costs ~16 us
// of host time for a chain of 1-3 kernel nodes and 31-81 us for 2-3
// independent ones.
int plan_graph_launch(ou_plan_s* plan, const StepScalars& sc, float max_unorm, bool clipped,
                      hipStream_t s)
{
    for (Group& g : plan->groups) {
        if (clipped)
            set_clip_args(g, sc, max_unorm);
        else
            set_group_args(g, sc);
    }
    hipGraph_t& graph = clipped ? plan->clip_graph : plan->graph;
    hipGraphExec_t& exec = clipped ? plan->clip_exec : plan->exec;
    const int first = clipped ? 1 : 0, last = clipped ? 3 : 0;
    hipError_t e;
    if (!exec) {
        auto drop = [&graph]() {
            (void)hipGraphDestroy(graph);
            graph = nullptr;
        };
        e = hipGraphCreate(&graph, 0);
        if (e != hipSuccess) {
            graph = nullptr;
            return hip_fail(e, "hipGraphCreate");
        }
        hipGraphNode_t prev = nullptr;
        for (Group& g : plan->groups) {
            for (int pass = first; pass <= last; ++pass) {
                hipKernelNodeParams kp;
                if (int st = group_launch(plan->kind, g, pass, &kp)) {
                    drop();
                    return st;
                }
                e = hipGraphAddKernelNode(&g.node[pass], graph, prev ? &prev : nullptr, prev ? 1 : 0, &kp);
                if (e != hipSuccess) {
                    drop();
                    return hip_fail(e, "hipGraphAddKernelNode");
                }
                prev = g.node[pass];
            }
        }
        e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        if (e != hipSuccess) {
            exec = nullptr;
            drop();
            return hip_fail(e, "hipGraphInstantiate");
        }
    } else {
        for (Group& g : plan->groups)
            for (int pass = first; pass <= last; ++pass) {
                hipKernelNodeParams kp;
                if (int st = group_launch(plan->kind, g, pass, &kp)) return st;
                e = hipGraphExecKernelNodeSetParams(exec, g.node[pass], &kp);
                if (e != hipSuccess) return hip_fail(e, "hipGraphExecKernelNodeSetParams");
            }
    }
    e = hipGraphLaunch(exec, s);
    if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
    return OU_OK;
}

int check_plan_device(ou_plan_s* plan)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != plan->device) return fail(OU_EINVAL, "plan was created on device %d, current is %d", plan->device, dev);
    return OU_OK;
}

// Workspace of the clipped step: 256 bytes (the factor fl32(lr*s), s at
// bytes 0-7), then one binary64 pair of partial sums per 2,048-element chunk.
constexpr int64_t clip_workspace_bytes(int64_t n)
{
    return 256 + (n > 0 ? (n + kClipChunkElems - 1) / kClipChunkElems : 0) * 16;
}

// ---- the static device scratch of optimizer_update_32bit_clip_noalloc -------
//
// For callers that cannot allocate device memory: the clipped step's chunk
// partial norms (16 B per 2,048 elements) and its clip factor (256 B) live
// in this file-scope device array, 8 MiB + 256 B, enough for 2^30 elements.
// Every GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, never device memory:
// its device address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address is passed to kernels.  Calls
// on one GPU share the array, so calls that overlap in time on one GPU
// (different streams, or host threads) race.  Nothing in it has to start
// at zero: pass 1 writes every chunk's partial sums before pass 2 reads
// them, and pass 2 writes the factor that pass 3 reads.
constexpr int64_t kScratchMaxElems = int64_t(1) << 30;
constexpr int64_t kScratchBytes = clip_workspace_bytes(kScratchMaxElems);
static_assert(kScratchBytes == 256 + (int64_t(16) << 19), "8 MiB + 256 B");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

class ScratchCache {
public:
    // Device address of `scratch` on the current device.
    int current(void** out)
    {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        if (dev < 0 || dev >= kMaxDevices) return fail(OU_EUNSUPPORTED, "device id %d", dev);
        void* p = ptr_[dev].load(std::memory_order_acquire);
        if (!p) {
            std::lock_guard<std::mutex> lk(mu_);
            p = ptr_[dev].load(std::memory_order_relaxed);
            if (!p) {
                e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
                if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
                if (!p || reinterpret_cast<uintptr_t>(p) % 256)
                    return fail(OU_EHIP, "hipGetSymbolAddress(scratch) returned an unaligned address");
                ptr_[dev].store(p, std::memory_order_release);
            }
        }
        *out = p;
        return OU_OK;
    }

private:
    std::mutex mu_;
    std::atomic<void*> ptr_[kMaxDevices] = {};
};

ScratchCache g_scratch;

// The clipped step of one tensor.  With `static_scratch` the chunk partials
// and the clip factor live in this file's device array `scratch` (tensors
// of at most kScratchMaxElems elements), otherwise in the caller's
// workspace.  Nothing here allocates device memory.
int clip_step(int kind_arg, int dtype, void* param, const void* grad, float* state1, float* state2, int64_t n,
              float beta1, float beta2, float beta3, float alpha, float eps, float weight_decay, int64_t step,
              float lr, int skip_zeros, float max_unorm, void* workspace, int64_t workspace_bytes,
              bool static_scratch, void* stream)
{
    if (!std::isfinite(max_unorm) || max_unorm < 0.0f)
        return fail(OU_EINVAL, "max_unorm must be finite and >= 0 (got %g)", max_unorm);
    if (max_unorm == 0.0f)
        return optimizer_update_32bit(kind_arg, dtype, param, grad, state1, state2, n, beta1, beta2,
                                      beta3, alpha, eps, weight_decay, step, lr, skip_zeros, stream);
    int kind = 0, after = 0;
    if (int st = split_kind(kind_arg, &kind, &after)) return st;
    if (!two_state(kind))
        return fail(OU_EINVAL, "update-norm clipping is defined for ADAM and ADEMAMIX only");
    ou_hparams h;
    h.beta1 = beta1; h.beta2 = beta2; h.beta3 = beta3; h.alpha = alpha; h.eps = eps;
    h.weight_decay = weight_decay; h.lr = lr; h.skip_zeros = skip_zeros; h.step = step;
    if (int st = check_hparams(kind, h)) return st;
    ou_segment s{param, grad, state1, state2, n, dtype, 0};
    std::vector<Range> ranges;
    ranges.reserve(5);
    if (int st = check_segment(kind, s, 0, &ranges)) return st;
    if (n == 0) return OU_OK;
    const int64_t need = clip_workspace_bytes(n);
    if (static_scratch) {
        if (n > kScratchMaxElems)
            return fail(OU_EINVAL, "n = %lld exceeds the %lld elements the library's static scratch serves; "
                        "use optimizer_update_32bit_clip with a workspace", (long long)n,
                        (long long)kScratchMaxElems);
    } else {
        if (!workspace) return fail(OU_EINVAL, "null workspace with max_unorm > 0");
        if (reinterpret_cast<uintptr_t>(workspace) % 16) return fail(OU_EALIGN, "workspace not 16-byte aligned");
        if (workspace_bytes < need)
            return fail(OU_EINVAL, "workspace has %lld bytes, needs %lld", (long long)workspace_bytes, (long long)need);
        const uintptr_t W = reinterpret_cast<uintptr_t>(workspace);
        ranges.push_back({W, W + static_cast<uintptr_t>(need), true, 1});
    }
    if (int st = check_overlap(ranges)) return st;
    if (validate_only()) return OU_OK;
    const DeviceProps* dp = nullptr;
    if (int st = g_devices.current(&dp)) return st;
    if (static_scratch) {
        if (int st = g_scratch.current(&workspace)) return st;
    }

    bool vec = streams_16b_aligned(kind, s);
    SingleLaunch L = select_single(*dp, kind, dtype, n, vec, false);
    L.epl = 4;
    // The parameter pass (three streams read, one written) takes its
    // 512-element tiles as two-wave blocks of one group per lane: over
    // 2^28 fp32 elements, 2 x 8 interleaved rounds on one MI355X, 657.8 us
    // against 687.2 us for one-wave blocks of two groups (the plain update's
    // shape, which in turn beats this one by 13% on the 4-read, 3-write
    // update); 256 x 2 took 668.8 us, 512 x 1 676.3 us.
    if (L.block == kWave && L.unroll == 2) {
        L.block = 2 * kWave;
        L.unroll = 1;
    }
    apply_single_forcing(&L, &vec);
    L.epl = 4;
    const void* f1 = clip_kernel(1, kind, dtype, 0);
    const void* f2 = clip_kernel(2, kind, dtype, 0);
    const void* f3 = clip_kernel(3, kind, dtype, L.unroll);
    // pass 3 covers groups of 4 elements
    const int64_t groups = (n + 3) / 4;
    const int64_t per_block = static_cast<int64_t>(L.block) * L.unroll;
    int64_t grid3 = g_force_grid.load() ? L.grid : (groups + per_block - 1) / per_block;
    grid3 = std::max<int64_t>(1, std::min<int64_t>(grid3, INT32_MAX));
    if (!f1 || !f2 || !f3 || L.block < kWave || L.block > 1024 || L.block % kWave ||
        L.lds < 0 || L.lds > dp->lds_per_block)
        return fail(OU_EINVAL, "no clip kernel for block=%d unroll=%d", L.block, L.unroll);
    const int64_t chunks = (n + kClipChunkElems - 1) / kClipChunkElems;
    if (chunks > INT32_MAX) return fail(OU_EINVAL, "tensor too large");
    StepScalars sc = make_scalars(h, after);
    int32_t vec_ok = vec ? 1 : 0;
    float* out = static_cast<float*>(workspace);
    double2* partials = reinterpret_cast<double2*>(static_cast<unsigned char*>(workspace) + 256);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const void* cp = param;
    int32_t xcd1 = xcd_log2_for(chunks, xcd_run_forced(kXcdRunClip));
    int32_t xcd3 = xcd_log2_for(grid3, xcd_run_forced(kXcdRunClip));
    void* a1[] = {&cp, const_cast<void**>(&grad), &state1, &state2, &n, &sc, &vec_ok, &partials, &xcd1};
    int lds1 = clip_moments_lds(*dp, chunks);
    if (int c = g_force_lds.load()) lds1 = c < 0 ? 0 : c;
    hipError_t e = launch(f1, chunks, kClipThreadsHost, lds1, a1, hs);
    if (e != hipSuccess) return hip_fail(e, "launch clip pass 1");
    float lr_arg = lr;
    void* a2[] = {&partials, const_cast<int64_t*>(&chunks), &max_unorm, &lr_arg, &out};
    e = launch(f2, 1, kClipFinalThreadsHost, 0, a2, hs);
    if (e != hipSuccess) return hip_fail(e, "launch clip pass 2");
    const float* lr_eff = out;
    void* a3[] = {&param, const_cast<void**>(&grad), &state1, &state2, &n, &sc, &vec_ok, &lr_eff, &xcd3};
    e = launch(f3, grid3, L.block, L.lds, a3, hs);
    if (e != hipSuccess) return hip_fail(e, "launch clip pass 3");
    return OU_OK;
}

}  // namespace

// Kernel-node parameters of a plan's plain step, one per dtype group, for a
// graph that spans several plans (host_graph.hip).  The parameters point
// into the plan's own argument storage; they are valid until the plan's next
// step of any form.
int plan_node_params(ou_plan_s* plan, const ou_hparams& hp, std::vector<hipKernelNodeParams>* out)
{
    if (int st = check_hparams(plan->kind, hp)) return st;
    if (int st = check_plan_device(plan)) return st;
    const StepScalars sc = make_scalars(hp, plan->decay_after);
    for (Group& g : plan->groups) {
        set_group_args(g, sc);
        hipKernelNodeParams kp;
        if (int st = group_launch(plan->kind, g, 0, &kp)) return st;
        out->push_back(kp);
    }
    return OU_OK;
}

int plan_device(const ou_plan_s* plan) { return plan->device; }

}  // namespace ou

// =============================================================== C ABI

using namespace ou;

extern "C" {

__attribute__((visibility("default")))
int optimizer_update_32bit(int kind_arg, int dtype, void* param, const void* grad, float* state1,
                           float* state2, int64_t n, float beta1, float beta2, float beta3,
                           float alpha, float eps, float weight_decay, int64_t step, float lr,
                           int skip_zeros, void* stream)
{
    int kind = 0, after = 0;
    if (int st = split_kind(kind_arg, &kind, &after)) return st;
    ou_hparams h;
    h.beta1 = beta1; h.beta2 = beta2; h.beta3 = beta3; h.alpha = alpha; h.eps = eps;
    h.weight_decay = weight_decay; h.lr = lr; h.skip_zeros = skip_zeros; h.step = step;
    if (int st = check_hparams(kind, h)) return st;
    ou_segment s{param, grad, state1, state2, n, dtype, 0};
    std::vector<Range> ranges;
    ranges.reserve(4);
    if (int st = check_segment(kind, s, 0, &ranges)) return st;
    if (n == 0) return OU_OK;
    if (int st = check_overlap(ranges)) return st;
    if (validate_only()) return OU_OK;
    const DeviceProps* dp = nullptr;
    if (int st = g_devices.current(&dp)) return st;

    bool vec = streams_16b_aligned(kind, s);
    SingleLaunch L = select_single(*dp, kind, dtype, n, vec, true);
    apply_single_forcing(&L, &vec);
    const void* fn = single_kernel(kind, dtype, L.epl, L.unroll, L.block);
    if (!fn || L.block < kWave || L.block > 1024 || L.block % kWave || L.grid < 1 || L.grid > INT32_MAX ||
        L.lds < 0 || L.lds > dp->lds_per_block)
        return fail(OU_EINVAL, "no kernel for block=%d epl=%d unroll=%d grid=%lld", L.block, L.epl,
                    L.unroll, (long long)L.grid);
    StepScalars sc = make_scalars(h, after);
    int32_t vec_ok = vec ? 1 : 0;
    int32_t xcd = L.xcd_log2;
    void* args[] = {&param, const_cast<void**>(&grad), &state1, &state2, &n, &sc, &vec_ok, &xcd};
    hipError_t e = launch(fn, L.grid, L.block, L.lds, args, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "launch single-tensor kernel");
    return OU_OK;
}

__attribute__((visibility("default")))
int64_t ou_clip_workspace_bytes(int64_t n) { return clip_workspace_bytes(n); }

__attribute__((visibility("default")))
int optimizer_update_32bit_clip(int kind_arg, int dtype, void* param, const void* grad, float* state1,
                                float* state2, int64_t n, float beta1, float beta2, float beta3,
                                float alpha, float eps, float weight_decay, int64_t step, float lr,
                                int skip_zeros, float max_unorm, void* workspace,
                                int64_t workspace_bytes, void* stream)
{
    return clip_step(kind_arg, dtype, param, grad, state1, state2, n, beta1, beta2, beta3, alpha, eps,
                     weight_decay, step, lr, skip_zeros, max_unorm, workspace, workspace_bytes, false, stream);
}

__attribute__((visibility("default")))
int optimizer_update_32bit_clip_noalloc(int kind_arg, int dtype, void* param, const void* grad,
                                        float* state1, float* state2, int64_t n, float beta1, float beta2,
                                        float beta3, float alpha, float eps, float weight_decay,
                                        int64_t step, float lr, int skip_zeros, float max_unorm, void* stream)
{
    return clip_step(kind_arg, dtype, param, grad, state1, state2, n, beta1, beta2, beta3, alpha, eps,
                     weight_decay, step, lr, skip_zeros, max_unorm, nullptr, 0, true, stream);
}

__attribute__((visibility("default")))
int64_t ou_clip_noalloc_max_elements(void) { return kScratchMaxElems; }

__attribute__((visibility("default")))
int optimizer_update_32bit_multi(int kind_arg, const ou_segment* segs, int32_t nseg, const ou_hparams* hp,
                                 void* stream)
{
    if (!hp) return fail(OU_EINVAL, "null hparams");
    int kind = 0, after = 0;
    if (int st = split_kind(kind_arg, &kind, &after)) return st;
    if (int st = check_hparams(kind, *hp)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!validate_only() && capturing(s))
        return fail(OU_ECAPTURE, "optimizer_update_32bit_multi allocates; use a plan under capture");
    ou_plan_s* plan = nullptr;
    if (int st = build_plan(kind_arg, segs, nseg, &plan)) return st;
    if (!plan) return OU_OK;   // validate-only mode
    int st = plan_launch(plan, make_scalars(*hp, after), s);
    hipError_t e = hipStreamSynchronize(s);
    ou_plan_destroy(plan);
    if (st) return st;
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    return OU_OK;
}

__attribute__((visibility("default")))
int ou_plan_create(int kind, const ou_segment* segs, int32_t nseg, ou_plan* out)
{
    if (!out) return fail(OU_EINVAL, "null output handle");
    *out = nullptr;
    return build_plan(kind, segs, nseg, out);
}

__attribute__((visibility("default")))
int ou_plan_step(ou_plan plan, const ou_hparams* hp, void* stream)
{
    if (!plan || !hp) return fail(OU_EINVAL, "null plan or hparams");
    if (int st = check_hparams(plan->kind, *hp)) return st;
    if (int st = check_plan_device(plan)) return st;
    return plan_launch(plan, make_scalars(*hp, plan->decay_after), static_cast<hipStream_t>(stream));
}

__attribute__((visibility("default")))
int ou_plan_step_clip(ou_plan plan, const ou_hparams* hp, float max_unorm, void* stream)
{
    if (!plan || !hp) return fail(OU_EINVAL, "null plan or hparams");
    if (!std::isfinite(max_unorm) || max_unorm < 0.0f)
        return fail(OU_EINVAL, "max_unorm must be finite and >= 0 (got %g)", max_unorm);
    if (int st = check_hparams(plan->kind, *hp)) return st;
    if (int st = check_plan_device(plan)) return st;
    const StepScalars sc = make_scalars(*hp, plan->decay_after);
    if (max_unorm == 0.0f) return plan_launch(plan, sc, static_cast<hipStream_t>(stream));
    if (!two_state(plan->kind))
        return fail(OU_EINVAL, "update-norm clipping is defined for ADAM and ADEMAMIX only");
    return plan_launch_clip(plan, sc, max_unorm, static_cast<hipStream_t>(stream));
}

__attribute__((visibility("default")))
int ou_plan_clip_factors(ou_plan plan, float* out, int32_t nseg)
{
    if (!plan || (!out && nseg > 0)) return fail(OU_EINVAL, "null plan or output");
    if (nseg != static_cast<int32_t>(plan->seg_map.size()))
        return fail(OU_EINVAL, "plan has %zu segments, not %d", plan->seg_map.size(), nseg);
    if (int st = check_plan_device(plan)) return st;
    // one copy per dtype group of its (fl32(lr*s), s) pairs, then scatter
    std::vector<float> pairs[3];
    for (const Group& g : plan->groups) {
        std::vector<float>& h = pairs[g.dtype];
        h.resize(static_cast<size_t>(2 * g.n_segs));
        hipError_t e = hipMemcpy(h.data(), g.d_seg_out, h.size() * sizeof(float), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpy(clip factors)");
    }
    for (int32_t i = 0; i < nseg; ++i) {
        const auto [dt, slot] = plan->seg_map[static_cast<size_t>(i)];
        out[i] = dt < 0 ? 1.0f : pairs[dt][static_cast<size_t>(2 * slot + 1)];
    }
    return OU_OK;
}

__attribute__((visibility("default")))
int ou_plan_graph_step(ou_plan plan, const ou_hparams* hp, void* stream)
{
    if (!plan || !hp) return fail(OU_EINVAL, "null plan or hparams");
    if (int st = check_hparams(plan->kind, *hp)) return st;
    if (int st = check_plan_device(plan)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (capturing(s)) return fail(OU_ECAPTURE, "ou_plan_graph_step inside a stream capture");
    if (plan->groups.empty()) return OU_OK;
    return plan_graph_launch(plan, make_scalars(*hp, plan->decay_after), 0.0f, false, s);
}

__attribute__((visibility("default")))
int ou_plan_graph_step_clip(ou_plan plan, const ou_hparams* hp, float max_unorm, void* stream)
{
    if (!plan || !hp) return fail(OU_EINVAL, "null plan or hparams");
    if (!std::isfinite(max_unorm) || max_unorm < 0.0f)
        return fail(OU_EINVAL, "max_unorm must be finite and >= 0 (got %g)", max_unorm);
    if (int st = check_hparams(plan->kind, *hp)) return st;
    if (int st = check_plan_device(plan)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (capturing(s)) return fail(OU_ECAPTURE, "ou_plan_graph_step_clip inside a stream capture");
    if (max_unorm > 0.0f && !two_state(plan->kind))
        return fail(OU_EINVAL, "update-norm clipping is defined for ADAM and ADEMAMIX only");
    if (plan->groups.empty()) return OU_OK;
    return plan_graph_launch(plan, make_scalars(*hp, plan->decay_after), max_unorm, max_unorm > 0.0f, s);
}

__attribute__((visibility("default")))
int ou_plan_describe(ou_plan plan, int32_t* n_groups, int64_t* n_work_items, int64_t* n_elements)
{
    if (!plan) return fail(OU_EINVAL, "null plan");
    int64_t items = 0;
    for (const Group& g : plan->groups) items += g.n_items;
    if (n_groups) *n_groups = static_cast<int32_t>(plan->groups.size());
    if (n_work_items) *n_work_items = items;
    if (n_elements) *n_elements = plan->n_elements;
    return OU_OK;
}

__attribute__((visibility("default")))
void ou_plan_destroy(ou_plan plan)
{
    if (!plan) return;
    if (plan->exec) (void)hipGraphExecDestroy(plan->exec);
    if (plan->graph) (void)hipGraphDestroy(plan->graph);
    if (plan->clip_exec) (void)hipGraphExecDestroy(plan->clip_exec);
    if (plan->clip_graph) (void)hipGraphDestroy(plan->clip_graph);
    if (plan->dmem) (void)hipFree(plan->dmem);
    delete plan;
}

__attribute__((visibility("default")))
const char* ou_status_string(int status)
{
    switch (status) {
    case OU_OK: return "OU_OK";
    case OU_EINVAL: return "OU_EINVAL: invalid argument";
    case OU_EUNSUPPORTED: return "OU_EUNSUPPORTED: unsupported device";
    case OU_EALIGN: return "OU_EALIGN: misaligned pointer";
    case OU_EOVERLAP: return "OU_EOVERLAP: overlapping buffers";
    case OU_ENOMEM: return "OU_ENOMEM: allocation failed";
    case OU_EHIP: return "OU_EHIP: HIP runtime error";
    case OU_ECAPTURE: return "OU_ECAPTURE: not allowed during stream capture";
    default: return "unknown status";
    }
}

__attribute__((visibility("default")))
const char* ou_last_error(void) { return g_last_error.c_str(); }

// ---- test hooks (declared in ou_testing.h, not in the public header) -----------

__attribute__((visibility("default")))
int ou__select_single(int cu_count, int lds_per_cu, int lds_per_block, int kind, int dtype, int64_t n,
                      int aligned, int64_t out[5])
{
    if (!out) return OU_EINVAL;
    DeviceProps d;
    d.cu_count = cu_count;
    d.lds_per_cu = lds_per_cu;
    d.lds_per_block = lds_per_block;
    d.gfx950 = true;
    SingleLaunch L = select_single(d, kind, dtype, n, aligned != 0, true);
    out[0] = L.block;
    out[1] = L.epl;
    out[2] = L.unroll;
    out[3] = L.grid;
    out[4] = L.lds;
    return OU_OK;
}

__attribute__((visibility("default")))
void ou__force_single(int block, int epl, int unroll, int64_t grid, int scalar_only, int lds)
{
    g_force_lds = lds;
    g_force_block = block;
    g_force_epl = epl;
    g_force_unroll = unroll;
    g_force_grid = grid;
    g_force_scalar = scalar_only;
}

__attribute__((visibility("default")))
void ou__force_multi(int waves, int epl, int unroll, int chunk, int lds)
{
    g_force_mlds = lds;
    g_force_waves = waves;
    g_force_mepl = epl;
    g_force_munroll = unroll;
    g_force_chunk = chunk;
}

__attribute__((visibility("default")))
void ou__validate_only(int on) { g_validate_only = on ? 1 : 0; }

__attribute__((visibility("default")))
void ou__force_xcd(int run) { g_force_xcd = run; }

__attribute__((visibility("default")))
int ou__step_scalars(const ou_hparams* hp, float out[12])
{
    if (!hp || !out) return OU_EINVAL;
    StepScalars s = make_scalars(*hp, 0);
    const float v[12] = {s.beta1, s.beta2, s.beta3, s.omb1, s.omb2, s.omb3,
                         s.alpha, s.eps, s.lr, s.bc1, s.bc2, s.decay};
    std::memcpy(out, v, sizeof v);
    return OU_OK;
}

}  // extern "C"
