// host8.hip -- C ABI of the update with 8-bit block-wise states (host side).
//
// Validation, launch shapes and plans of the 8-bit leg of the page's
// AdamW8bit collections ("Investigate a 256-thread SM103 path for small
// 32-bit optimizer tensors", sections "Problem" and "B300 benchmark and
// acceptance"); the arithmetic is in kernels8.hip and elem.hpp.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/optimizer_update.h"
#include "host_internal.h"
#include "internal.h"
#include "ou_testing.h"
#include "qmap.hpp"

namespace ou {
namespace {

// Launch shape: 4 waves per workgroup (8 for a single tensor with fp32
// storage); a wave takes a run of blocks (single tensor, select_bpw8) or one
// work item of up to 16 blocks (collection; 16 measured best on the bf16
// AdamW8bit collection against 2, 4, 8 and 32, and 4 waves against 8), so a
// workgroup's table copy into LDS serves 4 (8) runs.  Measured on MI355X at
// 2^28 elements in interleaved rounds: fp32 storage 715 us with 8 waves of
// 4 blocks against 742 us with 4 waves of 8; 16-bit storage gains nothing
// from 8 waves.
constexpr int kWaves8 = 4;
constexpr int kWaves8F32 = 8;
constexpr int kChunkBlocks8 = 16;
// Workgroups per XCD run (xcd_tile), single tensors and the launch order of
// plan work items.
constexpr int kXcdRun8 = 16;

// test-only forcing (not part of the public ABI)
std::atomic<int> g8_waves{0}, g8_bpw{0}, g8_chunk{0}, g8_scalar{0};

int64_t nblocks(int64_t n) { return (n + kQBlock - 1) / kQBlock; }

// Blocks per wave of the single-tensor kernel: as many as still leave 4
// workgroups per CU (a longer run amortizes the table copy and keeps the
// two-block pipeline full), even (the wide path takes blocks in pairs), and
// at most 16 for 16-bit storage, 4 for fp32 (measured at 2^28 elements:
// longer runs stop paying there).
int32_t select_bpw8(const DeviceProps& dp, int dtype, int64_t nb, int waves)
{
    const int64_t cap = dtype == OU_F32 ? 4 : 16;
    const int64_t cus = dp.cu_count > 0 ? dp.cu_count : 1;
    const int64_t b = std::min(cap, std::max<int64_t>(2, nb / (cus * 4 * waves)));
    return static_cast<int32_t>(b & ~int64_t(1));
}

int split_kind8(int arg, int* kind, int* after)
{
    if (int st = split_kind(arg, kind, after)) return st;
    if (!two_state(*kind)) return fail(OU_EINVAL, "8-bit states are defined for ADAM and ADEMAMIX only");
    return OU_OK;
}

int check_segment8(int kind, const ou_segment8& s, int idx, std::vector<Range>* ranges)
{
    if (s.dtype != OU_F32 && s.dtype != OU_F16 && s.dtype != OU_BF16)
        return fail(OU_EINVAL, "segment %d: unknown dtype %d", idx, s.dtype);
    if (s.n < 0) return fail(OU_EINVAL, "segment %d: n < 0", idx);
    if (s.reserved != 0) return fail(OU_EINVAL, "segment %d: reserved field must be 0", idx);
    if (s.n == 0) return OU_OK;
    if (!s.param || !s.grad || !s.state1 || !s.state2 || !s.absmax1 || !s.absmax2)
        return fail(OU_EINVAL, "segment %d: null pointer with n > 0", idx);
    const uintptr_t sb = static_cast<uintptr_t>(storage_bytes(s.dtype));
    const uintptr_t P = reinterpret_cast<uintptr_t>(s.param);
    const uintptr_t G = reinterpret_cast<uintptr_t>(s.grad);
    const uintptr_t C1 = reinterpret_cast<uintptr_t>(s.state1);
    const uintptr_t C2 = reinterpret_cast<uintptr_t>(s.state2);
    const uintptr_t A1 = reinterpret_cast<uintptr_t>(s.absmax1);
    const uintptr_t A2 = reinterpret_cast<uintptr_t>(s.absmax2);
    if (P % sb || G % sb) return fail(OU_EALIGN, "segment %d: param/grad not %u-byte aligned", idx, (unsigned)sb);
    if (A1 % 4 || A2 % 4) return fail(OU_EALIGN, "segment %d: absmax not 4-byte aligned", idx);
    const uintptr_t n = static_cast<uintptr_t>(s.n);
    if (n > (uintptr_t(1) << 40)) return fail(OU_EINVAL, "segment %d: n too large", idx);
    const uintptr_t k = (kind == OU_ADEMAMIX) ? 2 : 1;
    const uintptr_t nb = static_cast<uintptr_t>(nblocks(s.n));
    ranges->push_back({P, P + n * sb, true, idx});
    ranges->push_back({G, G + n * sb, false, idx});
    ranges->push_back({C1, C1 + k * n, true, idx});
    ranges->push_back({C2, C2 + n, true, idx});
    ranges->push_back({A1, A1 + k * nb * 4, true, idx});
    ranges->push_back({A2, A2 + nb * 4, true, idx});
    return OU_OK;
}

Seg8 make_seg8(int kind, const ou_segment8& s)
{
    Seg8 d;
    d.p = s.param;
    d.g = s.grad;
    d.c1 = s.state1;
    d.c2 = s.state2;
    d.a1 = s.absmax1;
    d.a2 = s.absmax2;
    d.n = s.n;
    d.nb = nblocks(s.n);
    const uintptr_t wide = static_cast<uintptr_t>(4 * storage_bytes(s.dtype));
    const uintptr_t pg = reinterpret_cast<uintptr_t>(s.param) | reinterpret_cast<uintptr_t>(s.grad);
    uintptr_t codes = reinterpret_cast<uintptr_t>(s.state1) | reinterpret_cast<uintptr_t>(s.state2);
    if (kind == OU_ADEMAMIX) codes |= reinterpret_cast<uintptr_t>(s.state1 + s.n);
    d.vec_ok = (pg % wide == 0 && codes % 4 == 0 && !g8_scalar.load()) ? 1 : 0;
    d.pad = 0;
    return d;
}

}  // namespace
}  // namespace ou

struct ou_plan8_s {
    int kind = 0;
    int decay_after = 0;
    int device = -1;
    void* dmem = nullptr;
    struct Group {
        int dtype = 0;
        int64_t n_items = 0;
        const ou::Seg8* d_segs = nullptr;
        const ou::WorkItem* d_items = nullptr;
        const void* fn = nullptr;
        int waves = 0;
        int32_t chunk_blocks = 0;
        int64_t grid = 0;
        // argument storage of the launch and of the graph node
        ou::StepScalars sc{};
        void* args[5] = {};
        hipGraphNode_t node = nullptr;
    };
    std::vector<Group> groups;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

using namespace ou;

namespace {

// Points the group's argument array at its own storage, with this step's
// scalars (k8_multi: segs, items, n_items, chunk_blocks, scalars).
void set_args8(ou_plan8_s::Group& g, const StepScalars& sc)
{
    g.sc = sc;
    g.args[0] = &g.d_segs;
    g.args[1] = &g.d_items;
    g.args[2] = &g.n_items;
    g.args[3] = &g.chunk_blocks;
    g.args[4] = &g.sc;
}

hipKernelNodeParams node_params8(ou_plan8_s::Group& g)
{
    hipKernelNodeParams kp{};
    kp.func = const_cast<void*>(g.fn);
    kp.gridDim = dim3(static_cast<unsigned>(g.grid));
    kp.blockDim = dim3(static_cast<unsigned>(g.waves * kWave));
    kp.sharedMemBytes = 0;
    kp.kernelParams = g.args;
    kp.extra = nullptr;
    return kp;
}

int check_plan8(ou_plan8 plan, const ou_hparams* hp)
{
    if (!plan || !hp) return fail(OU_EINVAL, "null plan or hparams");
    if (int st = check_hparams(plan->kind, *hp)) return st;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != plan->device) return fail(OU_EINVAL, "plan was created on device %d, current is %d", plan->device, dev);
    return OU_OK;
}

}  // namespace

namespace ou {

// Kernel-node parameters of an 8-bit plan's step, one per dtype group, for a
// graph that spans several plans (host_graph.hip); valid until the plan's
// next step of any form.
int plan8_node_params(ou_plan8_s* plan, const ou_hparams& hp, std::vector<hipKernelNodeParams>* out)
{
    if (int st = check_plan8(plan, &hp)) return st;
    const StepScalars sc = make_scalars(hp, plan->decay_after);
    for (ou_plan8_s::Group& g : plan->groups) {
        set_args8(g, sc);
        out->push_back(node_params8(g));
    }
    return OU_OK;
}

int plan8_device(const ou_plan8_s* plan) { return plan->device; }

}  // namespace ou

extern "C" {

__attribute__((visibility("default")))
int ou_8bit_qmap(int is_signed, float* out, int32_t count)
{
    const int want = is_signed ? 128 : 256;
    if (!out || count != want) return fail(OU_EINVAL, "ou_8bit_qmap: need %d entries, got %d", want, count);
    std::memcpy(out, is_signed ? kQTablesHost.smag : kQTablesHost.umag, sizeof(float) * want);
    return OU_OK;
}

__attribute__((visibility("default")))
int optimizer_update_8bit_blockwise(int kind_arg, int dtype, void* param, const void* grad,
                                    uint8_t* state1, uint8_t* state2, float* absmax1,
                                    float* absmax2, int64_t n, float beta1, float beta2,
                                    float beta3, float alpha, float eps, float weight_decay,
                                    int64_t step, float lr, int skip_zeros, void* stream)
{
    int kind = 0, after = 0;
    if (int st = split_kind8(kind_arg, &kind, &after)) return st;
    ou_hparams h;
    h.beta1 = beta1; h.beta2 = beta2; h.beta3 = beta3; h.alpha = alpha; h.eps = eps;
    h.weight_decay = weight_decay; h.lr = lr; h.skip_zeros = skip_zeros; h.step = step;
    if (int st = check_hparams(kind, h)) return st;
    ou_segment8 s{param, grad, state1, state2, absmax1, absmax2, n, dtype, 0};
    std::vector<Range> ranges;
    ranges.reserve(6);
    if (int st = check_segment8(kind, s, 0, &ranges)) return st;
    if (n == 0) return OU_OK;
    if (int st = check_overlap(ranges)) return st;
    if (validate_only()) return OU_OK;
    const DeviceProps* dp = nullptr;
    if (int st = current_device(&dp)) return st;

    int waves = dtype == OU_F32 ? kWaves8F32 : kWaves8;
    if (int w = g8_waves.load()) waves = w;
    const void* fn = kernel8(false, kind, dtype);
    if (!fn || waves < 1 || waves > 16) return fail(OU_EINVAL, "no 8-bit kernel for waves=%d", waves);
    Seg8 d = make_seg8(kind, s);
    int32_t bpw = select_bpw8(*dp, dtype, d.nb, waves);
    if (int b = g8_bpw.load()) bpw = b;
    if (bpw < 1) return fail(OU_EINVAL, "blocks per wave must be >= 1");
    const int64_t per_group = static_cast<int64_t>(waves) * bpw;
    const int64_t grid = (d.nb + per_group - 1) / per_group;
    if (grid > INT32_MAX) return fail(OU_EINVAL, "tensor too large");
    StepScalars sc = make_scalars(h, after);
    int32_t xcd = xcd_log2_for(grid, xcd_run_forced(kXcdRun8));
    void* args[] = {&d, &sc, &bpw, &xcd};
    hipError_t e = launch(fn, grid, waves * kWave, 0, args, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "launch 8-bit kernel");
    return OU_OK;
}

__attribute__((visibility("default")))
int ou_plan8_create(int kind_arg, const ou_segment8* segs, int32_t nseg, ou_plan8* out)
{
    if (!out) return fail(OU_EINVAL, "null output handle");
    *out = nullptr;
    int kind = 0, after = 0;
    if (int st = split_kind8(kind_arg, &kind, &after)) return st;
    if (nseg < 0 || (nseg > 0 && !segs)) return fail(OU_EINVAL, "bad segment array");
    std::vector<Range> ranges;
    ranges.reserve(static_cast<size_t>(nseg) * 6);
    for (int i = 0; i < nseg; ++i)
        if (int st = check_segment8(kind, segs[i], i, &ranges)) return st;
    if (int st = check_overlap(ranges)) return st;
    if (validate_only()) return OU_OK;
    const DeviceProps* dp = nullptr;
    if (int st = current_device(&dp)) return st;

    int waves = kWaves8;
    int32_t chunk = kChunkBlocks8;
    if (int w = g8_waves.load()) waves = w;
    if (int c = g8_chunk.load()) chunk = c;
    if (waves < 1 || waves > 16 || chunk < 1) return fail(OU_EINVAL, "bad forced 8-bit plan shape");

    ou_plan8_s* plan = new (std::nothrow) ou_plan8_s;
    if (!plan) return fail(OU_ENOMEM, "plan");
    plan->kind = kind;
    plan->decay_after = after;
    (void)hipGetDevice(&plan->device);

    std::vector<Seg8> hs[3];
    std::vector<WorkItem> hi[3];
    for (int i = 0; i < nseg; ++i) {
        const ou_segment8& s = segs[i];
        if (s.n == 0) continue;
        const Seg8 d = make_seg8(kind, s);
        const int64_t items = (d.nb + chunk - 1) / chunk;
        if (items > INT32_MAX || hs[s.dtype].size() >= static_cast<size_t>(INT32_MAX)) {
            delete plan;
            return fail(OU_EINVAL, "segment %d: too many blocks", i);
        }
        const int32_t idx = static_cast<int32_t>(hs[s.dtype].size());
        hs[s.dtype].push_back(d);
        for (int64_t c = 0; c < items; ++c) hi[s.dtype].push_back(WorkItem{idx, static_cast<int32_t>(c)});
    }
    // launch order of the work items: runs of blocks per XCD (xcd_tile)
    for (int dt = 0; dt < 3; ++dt) {
        const int64_t nblk = static_cast<int64_t>(hi[dt].size()) / waves;
        xcd_order(hi[dt], waves, xcd_log2_for(nblk, xcd_run_forced(kXcdRun8)));
    }
    auto align16 = [](size_t x) { return (x + 15) & ~size_t(15); };
    size_t bytes = 0;
    for (int dt = 0; dt < 3; ++dt)
        bytes += align16(hs[dt].size() * sizeof(Seg8)) + align16(hi[dt].size() * sizeof(WorkItem));
    if (bytes > 0) {
        hipError_t e = hipMalloc(&plan->dmem, bytes);
        if (e != hipSuccess) {
            delete plan;
            return fail(OU_ENOMEM, "hipMalloc(%zu) for the plan: %s", bytes, hipGetErrorString(e));
        }
        std::vector<unsigned char> host(bytes, 0);
        size_t off = 0;
        for (int dt = 0; dt < 3; ++dt) {
            if (hs[dt].empty()) continue;
            ou_plan8_s::Group g;
            g.dtype = dt;
            g.waves = waves;
            g.chunk_blocks = chunk;
            g.n_items = static_cast<int64_t>(hi[dt].size());
            g.fn = kernel8(true, kind, dt);
            g.grid = (g.n_items + waves - 1) / waves;
            std::memcpy(host.data() + off, hs[dt].data(), hs[dt].size() * sizeof(Seg8));
            g.d_segs = reinterpret_cast<const Seg8*>(static_cast<unsigned char*>(plan->dmem) + off);
            off = align16(off + hs[dt].size() * sizeof(Seg8));
            std::memcpy(host.data() + off, hi[dt].data(), hi[dt].size() * sizeof(WorkItem));
            g.d_items = reinterpret_cast<const WorkItem*>(static_cast<unsigned char*>(plan->dmem) + off);
            off = align16(off + hi[dt].size() * sizeof(WorkItem));
            if (!g.fn || g.grid > INT32_MAX) {
                (void)hipFree(plan->dmem);
                delete plan;
                return fail(OU_EINVAL, "no 8-bit multi-tensor kernel");
            }
            plan->groups.push_back(g);
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

__attribute__((visibility("default")))
int ou_plan8_step(ou_plan8 plan, const ou_hparams* hp, void* stream)
{
    if (int st = check_plan8(plan, hp)) return st;
    const StepScalars sc = make_scalars(*hp, plan->decay_after);
    for (ou_plan8_s::Group& g : plan->groups) {
        set_args8(g, sc);
        hipError_t e = launch(g.fn, g.grid, g.waves * kWave, 0, g.args, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "launch 8-bit multi-tensor kernel");
    }
    return OU_OK;
}

__attribute__((visibility("default")))
int ou_plan8_graph_step(ou_plan8 plan, const ou_hparams* hp, void* stream)
{
    if (int st = check_plan8(plan, hp)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (capturing(s)) return fail(OU_ECAPTURE, "ou_plan8_graph_step inside a stream capture");
    if (plan->groups.empty()) return OU_OK;
    const StepScalars sc = make_scalars(*hp, plan->decay_after);
    hipError_t e;
    if (!plan->exec) {
        e = hipGraphCreate(&plan->graph, 0);
        if (e != hipSuccess) return hip_fail(e, "hipGraphCreate");
        hipGraphNode_t prev = nullptr;
        for (ou_plan8_s::Group& g : plan->groups) {
            set_args8(g, sc);
            const hipKernelNodeParams kp = node_params8(g);
            // one chain (a replay of independent nodes costs far more host time)
            e = hipGraphAddKernelNode(&g.node, plan->graph, prev ? &prev : nullptr, prev ? 1 : 0, &kp);
            if (e != hipSuccess) return hip_fail(e, "hipGraphAddKernelNode");
            prev = g.node;
        }
        e = hipGraphInstantiate(&plan->exec, plan->graph, nullptr, nullptr, 0);
        if (e != hipSuccess) {
            plan->exec = nullptr;
            return hip_fail(e, "hipGraphInstantiate");
        }
    } else {
        for (ou_plan8_s::Group& g : plan->groups) {
            set_args8(g, sc);
            const hipKernelNodeParams kp = node_params8(g);
            e = hipGraphExecKernelNodeSetParams(plan->exec, g.node, &kp);
            if (e != hipSuccess) return hip_fail(e, "hipGraphExecKernelNodeSetParams");
        }
    }
    e = hipGraphLaunch(plan->exec, s);
    if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
    return OU_OK;
}

__attribute__((visibility("default")))
void ou_plan8_destroy(ou_plan8 plan)
{
    if (!plan) return;
    if (plan->exec) (void)hipGraphExecDestroy(plan->exec);
    if (plan->graph) (void)hipGraphDestroy(plan->graph);
    if (plan->dmem) (void)hipFree(plan->dmem);
    delete plan;
}

// ---- test hooks (ou_testing.h) ------------------------------------------------

__attribute__((visibility("default")))
void ou__force_8bit(int waves, int blocks_per_wave, int chunk_blocks, int scalar_only)
{
    g8_waves = waves;
    g8_bpw = blocks_per_wave;
    g8_chunk = chunk_blocks;
    g8_scalar = scalar_only;
}

__attribute__((visibility("default")))
int ou__recip8(const float* in, float* out, int64_t n, void* stream)
{
    if (!in || !out || n <= 0) return fail(OU_EINVAL, "recip8: bad arguments");
    if (reinterpret_cast<uintptr_t>(in) % 4 || reinterpret_cast<uintptr_t>(out) % 4)
        return fail(OU_EALIGN, "recip8: misaligned buffers");
    if (validate_only()) return OU_OK;
    const DeviceProps* dp = nullptr;
    if (int st = current_device(&dp)) return st;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 1 << 20));
    const float* a0 = in;
    float* a1 = out;
    void* args[] = {const_cast<float**>(&a0), &a1, &n};
    hipError_t e = launch(recip_kernel8(), grid, 256, 0, args, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "launch recip8");
    return OU_OK;
}

__attribute__((visibility("default")))
int ou__quant8(const float* v, const float* absmax, uint8_t* cs, uint8_t* cu, int64_t n, void* stream)
{
    if (!v || !absmax || !cs || !cu || n <= 0) return fail(OU_EINVAL, "quant8: bad arguments");
    if (reinterpret_cast<uintptr_t>(v) % 4 || reinterpret_cast<uintptr_t>(absmax) % 4)
        return fail(OU_EALIGN, "quant8: misaligned buffers");
    if (validate_only()) return OU_OK;
    const DeviceProps* dp = nullptr;
    if (int st = current_device(&dp)) return st;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 1 << 16));
    const float* a0 = v;
    const float* a1 = absmax;
    uint8_t* a2 = cs;
    uint8_t* a3 = cu;
    void* args[] = {const_cast<float**>(&a0), const_cast<float**>(&a1), &a2, &a3, &n};
    hipError_t e = launch(quant_kernel8(), grid, 256, 0, args, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "launch quant8");
    return OU_OK;
}

}  // extern "C"
