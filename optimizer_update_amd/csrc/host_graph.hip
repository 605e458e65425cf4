// host_graph.hip -- one HIP graph over the plain steps of several plans.
//
// The page's AdamW8bit collections step two plans per optimizer step
// (tensors of at least min_8bit_size elements with 8-bit states, the others
// with fp32 states; "Investigate a 256-thread SM103 path for small 32-bit
// optimizer tensors", sections "Problem" and "B300 benchmark and
// acceptance").  An ou_graph replays all of their launches as one graph:
// built and instantiated on the first step, then every step writes the
// new per-step scalars into its kernel nodes and replays.  The nodes form
// one chain in the order of the plans given (32-bit plans first, then 8-bit
// ones), because on MI355X a replay of a chain of 1-3 kernel nodes costs
// ~16 us of host time and a replay of 2-3 independent nodes 31-81 us.
#include <new>
#include <vector>

#include "../../include/optimizer_update.h"
#include "host_internal.h"

struct ou_graph_s {
    std::vector<ou_plan> plans;
    std::vector<ou_plan8> plans8;
    int device = -1;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    std::vector<hipGraphNode_t> nodes;
};

using namespace ou;

extern "C" {

__attribute__((visibility("default")))
int ou_graph_create(const ou_plan* plans, int32_t nplans, const ou_plan8* plans8, int32_t nplans8,
                    ou_graph* out)
{
    if (!out) return fail(OU_EINVAL, "null output handle");
    *out = nullptr;
    if (nplans < 0 || nplans8 < 0 || (nplans > 0 && !plans) || (nplans8 > 0 && !plans8))
        return fail(OU_EINVAL, "bad plan arrays");
    int device = -1;
    for (int32_t i = 0; i < nplans; ++i) {
        if (!plans[i]) return fail(OU_EINVAL, "plan %d is null", i);
        if (device >= 0 && plan_device(plans[i]) != device) return fail(OU_EINVAL, "plans on different devices");
        device = plan_device(plans[i]);
    }
    for (int32_t i = 0; i < nplans8; ++i) {
        if (!plans8[i]) return fail(OU_EINVAL, "8-bit plan %d is null", i);
        if (device >= 0 && plan8_device(plans8[i]) != device) return fail(OU_EINVAL, "plans on different devices");
        device = plan8_device(plans8[i]);
    }
    ou_graph_s* g = new (std::nothrow) ou_graph_s;
    if (!g) return fail(OU_ENOMEM, "graph");
    g->plans.assign(plans, plans + nplans);
    g->plans8.assign(plans8, plans8 + nplans8);
    g->device = device;
    *out = g;
    return OU_OK;
}

__attribute__((visibility("default")))
int ou_graph_step(ou_graph g, const ou_hparams* hp, void* stream)
{
    if (!g || !hp) return fail(OU_EINVAL, "null graph or hparams");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (capturing(s)) return fail(OU_ECAPTURE, "ou_graph_step inside a stream capture");
    std::vector<hipKernelNodeParams> kps;
    for (ou_plan p : g->plans)
        if (int st = plan_node_params(p, *hp, &kps)) return st;
    for (ou_plan8 p : g->plans8)
        if (int st = plan8_node_params(p, *hp, &kps)) return st;
    if (kps.empty()) return OU_OK;
    hipError_t e;
    if (!g->exec) {
        e = hipGraphCreate(&g->graph, 0);
        if (e != hipSuccess) {
            g->graph = nullptr;
            return hip_fail(e, "hipGraphCreate");
        }
        g->nodes.assign(kps.size(), nullptr);
        for (size_t i = 0; i < kps.size(); ++i) {
            hipGraphNode_t* prev = i ? &g->nodes[i - 1] : nullptr;
            e = hipGraphAddKernelNode(&g->nodes[i], g->graph, prev, prev ? 1 : 0, &kps[i]);
            if (e == hipSuccess) continue;
            (void)hipGraphDestroy(g->graph);
            g->graph = nullptr;
            return hip_fail(e, "hipGraphAddKernelNode");
        }
        e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
        if (e != hipSuccess) {
            g->exec = nullptr;
            (void)hipGraphDestroy(g->graph);
            g->graph = nullptr;
            return hip_fail(e, "hipGraphInstantiate");
        }
    } else {
        if (kps.size() != g->nodes.size()) return fail(OU_EINVAL, "the plans' launch count changed");
        for (size_t i = 0; i < kps.size(); ++i) {
            e = hipGraphExecKernelNodeSetParams(g->exec, g->nodes[i], &kps[i]);
            if (e != hipSuccess) return hip_fail(e, "hipGraphExecKernelNodeSetParams");
        }
    }
    e = hipGraphLaunch(g->exec, s);
    if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
    return OU_OK;
}

__attribute__((visibility("default")))
void ou_graph_destroy(ou_graph g)
{
    if (!g) return;
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    if (g->graph) (void)hipGraphDestroy(g->graph);
    delete g;
}

}  // extern "C"
