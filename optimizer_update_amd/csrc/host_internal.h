// host_internal.h -- host-side helpers shared by the 32-bit and the 8-bit
// entry points (validation, errors, per-step scalars, launches).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/optimizer_update.h"
#include "internal.h"

namespace ou {

// Records a thread-local message for ou_last_error() and returns status.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int hip_fail(hipError_t e, const char* what);

// Properties of the current device (cached per device id); OU_EUNSUPPORTED
// unless it is a gfx950.
int current_device(const DeviceProps** out);
// Test-only switch (ou__validate_only): entry points return OU_OK after their
// argument checks, before they query or touch a device.
bool validate_only();

int storage_bytes(int dtype);
bool valid_kind(int kind);
bool two_state(int kind);
// Splits a kind argument into an ou_kind and the OU_DECAY_AFTER flag.
int split_kind(int arg, int* kind, int* after);
int check_hparams(int kind, const ou_hparams& h);

// A byte range of one buffer, for the overlap check.
struct Range {
    uintptr_t lo, hi;   // [lo, hi)
    bool written;
    int seg;
};
// OU_EINVAL if a range wraps past the end of the address space; OU_EOVERLAP
// if a written range overlaps any other range (read-only ranges may share).
int check_overlap(std::vector<Range>& r);

StepScalars make_scalars(const ou_hparams& h, int decay_after);

hipError_t launch(const void* fn, int64_t grid, int block, int lds, void** args, hipStream_t stream);

// log2 of the XCD tile run for a grid (xcd_tile), or -1, after forcing.
int xcd_log2_for(int64_t grid, int run);
// Launch shape of the single-tensor update (plain = false: the clipped
// step's parameter pass), and the test hooks' forcing of it.
SingleLaunch select_single(const DeviceProps& d, int kind, int dtype, int64_t n, bool vec, bool plain);
void apply_single_forcing(SingleLaunch* L, bool* vec);
// Launch shape and chunk (elements per work item) of a plan's dtype group
// holding `total_elements`, before any test forcing.
MultiLaunch select_multi(const DeviceProps& d, int kind, int dtype, int64_t total_elements);
int64_t select_chunk(int64_t total_elements);
// Dynamic LDS of the clipped step's pass 1 for a grid of `grid` chunks.
int clip_moments_lds(const DeviceProps& d, int64_t grid);
int xcd_run_forced(int run);

// A plan's work list in launch order: block b (items [b*per_block,
// (b+1)*per_block)) gets the items of tile xcd_tile(b); whole blocks only.
template <typename T>
void xcd_order(std::vector<T>& items, int per_block, int log2c)
{
    if (log2c < 0 || per_block < 1) return;
    const int64_t nfull = static_cast<int64_t>(items.size()) / per_block;
    const std::vector<T> in(items);
    for (int64_t b = 0; b < nfull; ++b) {
        const int64_t t = xcd_tile(b, nfull, log2c);
        for (int w = 0; w < per_block; ++w) items[b * per_block + w] = in[t * per_block + w];
    }
}
bool capturing(hipStream_t stream);

// Kernel-node parameters of one plain step of a plan (a node per dtype
// group; the hyperparameters checked for the plan's kind, the current device
// checked against the plan's), appended to `out` in launch order; they
// point into the plan's argument storage and stay valid until the plan's
// next step.  For graphs that span several plans.
int plan_node_params(ou_plan_s* plan, const ou_hparams& hp, std::vector<hipKernelNodeParams>* out);
int plan8_node_params(ou_plan8_s* plan, const ou_hparams& hp, std::vector<hipKernelNodeParams>* out);
int plan_device(const ou_plan_s* plan);
int plan8_device(const ou_plan8_s* plan);

}  // namespace ou
