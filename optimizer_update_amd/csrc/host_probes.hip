// host_probes.hip -- entry points of the test-hook kernels of probes.hip
// (not part of the public ABI; declared in ou_testing.h): the storage
// rounding and square root of the update on their own, the bandwidth probe
// in the launch shapes of the single-tensor update, and the VALU issue
// probe.
#include <algorithm>

#include "../../include/optimizer_update.h"
#include "host_internal.h"
#include "ou_testing.h"

using namespace ou;

extern "C" {

__attribute__((visibility("default")))
int ou__select_multi(int cu_count, int lds_per_cu, int lds_per_block, int kind, int dtype, int64_t total_elements,
                     int64_t out[7])
{
    if (!out || cu_count < 0 || lds_per_cu < 0 || lds_per_block < 0 || total_elements < 0) return OU_EINVAL;
    DeviceProps d;
    d.cu_count = cu_count;
    d.lds_per_cu = lds_per_cu;
    d.lds_per_block = lds_per_block;
    d.gfx950 = true;
    const MultiLaunch L = select_multi(d, kind, dtype, total_elements);
    out[0] = L.waves;
    out[1] = L.epl;
    out[2] = L.unroll;
    out[3] = L.lds;
    out[4] = L.xcd_run;
    out[5] = select_chunk(total_elements);
    // pass 1 of a clipped step over the same elements, one block per chunk
    out[6] = clip_moments_lds(d, (total_elements + kClipChunkElems - 1) / kClipChunkElems);
    return OU_OK;
}

__attribute__((visibility("default")))
int ou__narrow(int dtype, const float* in, uint16_t* out, int64_t n, void* stream)
{
    const bool pairs = dtype >= 16;
    const void* fn = narrow_kernel(pairs ? dtype - 16 : dtype, pairs);
    if (!fn || !in || !out || n <= 0 || (pairs && n % 2)) return fail(OU_EINVAL, "narrow: bad arguments");
    if (reinterpret_cast<uintptr_t>(in) % 4 || reinterpret_cast<uintptr_t>(out) % (pairs ? 4 : 2))
        return fail(OU_EALIGN, "narrow: misaligned buffers");
    if (validate_only()) return OU_OK;
    const DeviceProps* dp = nullptr;
    if (int st = current_device(&dp)) return st;
    int64_t count = pairs ? n / 2 : n;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((count + 255) / 256, 1 << 20));
    const float* a0 = in;
    uint16_t* a1 = out;
    void* args[] = {const_cast<float**>(&a0), &a1, &count};
    hipError_t e = launch(fn, grid, 256, 0, args, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "launch narrow");
    return OU_OK;
}

__attribute__((visibility("default")))
int ou__sqrt(const float* in, float* out, int64_t n, void* stream)
{
    if (!in || !out || n <= 0) return fail(OU_EINVAL, "sqrt: bad arguments");
    if (reinterpret_cast<uintptr_t>(in) % 4 || reinterpret_cast<uintptr_t>(out) % 4)
        return fail(OU_EALIGN, "sqrt: misaligned buffers");
    if (validate_only()) return OU_OK;
    const DeviceProps* dp = nullptr;
    if (int st = current_device(&dp)) return st;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 1 << 20));
    const float* a0 = in;
    float* a1 = out;
    void* args[] = {const_cast<float**>(&a0), &a1, &n};
    hipError_t e = launch(sqrt_kernel(), grid, 256, 0, args, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "launch sqrt");
    return OU_OK;
}

__attribute__((visibility("default")))
int ou__stream_probe(int mode, float* p, const float* g, float* s1, float* s2, int64_t n, void* stream)
{
    if (mode < 0 || mode > 2 || !p || !g || !s1 || !s2 || n <= 0 || n % 4)
        return fail(OU_EINVAL, "stream probe: bad arguments");
    const uintptr_t a = reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(g) |
                        reinterpret_cast<uintptr_t>(s1) | reinterpret_cast<uintptr_t>(s2);
    if (a % 16) return fail(OU_EALIGN, "stream probe: buffers must be 16-byte aligned");
    if (validate_only()) return OU_OK;
    const DeviceProps* dp = nullptr;
    if (int st = current_device(&dp)) return st;
    bool vec = true;
    SingleLaunch L = select_single(*dp, OU_ADAM, OU_F32, n, vec, true);
    apply_single_forcing(&L, &vec);
    const void* fn = stream_probe_kernel(mode, L.unroll);
    if (!fn || L.epl != 4 || !vec || L.block < kWave || L.block > 1024 || L.block % kWave ||
        L.grid < 1 || L.grid > INT32_MAX || L.lds < 0 || L.lds > dp->lds_per_block)
        return fail(OU_EINVAL, "stream probe: no kernel for this shape");
    int64_t nvec = n / 4;
    uint32_t mask = 0;
    int32_t xcd = L.xcd_log2;
    void* args[] = {&p, const_cast<float**>(&g), &s1, &s2, &nvec, &mask, &xcd};
    hipError_t e = launch(fn, L.grid, L.block, L.lds, args, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "launch stream probe");
    return OU_OK;
}

__attribute__((visibility("default")))
int ou__valu_probe(int op, int64_t blocks, int32_t iters, float* out, void* stream)
{
    const void* fn = valu_probe_kernel(op);
    if (!fn || blocks < 1 || blocks > INT32_MAX || iters < 1 || !out)
        return fail(OU_EINVAL, "valu probe: bad arguments");
    if (reinterpret_cast<uintptr_t>(out) % 4) return fail(OU_EALIGN, "valu probe: misaligned output");
    if (validate_only()) return OU_OK;
    const DeviceProps* dp = nullptr;
    if (int st = current_device(&dp)) return st;
    uint32_t mask = 0;
    void* args[] = {&out, &iters, &mask};
    hipError_t e = launch(fn, blocks, 256, 0, args, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "launch valu probe");
    return OU_OK;
}

}  // extern "C"
