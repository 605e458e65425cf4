/*
 * optimizer_update.h -- C ABI of the MI355X (gfx950) 32-bit two-state
 * optimizer update: Adam/AdamW with decoupled weight decay, and AdEMAMix
 * with its extra slow EMA.
 *
 * The operation is the one named on the page "Investigate a 256-thread SM103
 * path for small 32-bit optimizer tensors" (bitsandbytes fork, issue 8):
 * the per-tensor direct op `optimizer_update_32bit` with a parameter, its
 * gradient and two fp32 state buffers (sections "Correctness oracle" and
 * "B300 benchmark and acceptance"), kinds ADAM and ADEMAMIX, parameter and
 * gradient storage fp32/fp16/bf16, optional skip_zeros.  The page prints no
 * formula; every entry point computes, per element i (binary32, each
 * operation correctly rounded, no fused multiply-add):
 *
 *   if (skip_zeros && g == 0)  leave p, state1, state2 of i untouched
 *   m  = beta1*m  + (1-beta1)*g            state1[i]       (Kingma & Ba, Alg. 1)
 *   v  = beta2*v  + (1-beta2)*(g*g)        state2[i]
 *   m2 = beta3*m2 + (1-beta3)*g            state1[n+i]     (AdEMAMix only;
 *                                          Pagliardini et al., Alg. 1)
 *   u  = (m/bc1 [+ alpha*m2]) / (sqrt(v/bc2) + eps)
 *   p  = p*d - lr*u                        (decay of the old p; Loshchilov &
 *                                           Hutter, Alg. 2)
 *   param[i] = p rounded to the storage type (nearest, ties to even)
 *
 * with the per-step scalars bc1 = fl32(1 - fl64(beta1^step)),
 * bc2 = fl32(1 - fl64(beta2^step)), d = fl32(1 - fl64(lr*weight_decay)),
 * 1-beta formed in binary32.  step is 1-based (the update being applied).
 * The slow EMA is not bias-corrected; alpha and beta3 are constants.
 *
 * Layout:  param, grad: n elements of the storage dtype.  state1: n floats
 * (ADAM) or 2n floats (ADEMAMIX: fast EMA at [0,n), slow EMA at [n,2n)).
 * state2: n floats (two-state kinds only).  All pointers are device pointers on the current HIP
 * device and must be aligned to their element size.  16-byte alignment of
 * all streams selects the dwordx4 path; any other alignment runs the same
 * arithmetic one element per lane (results are bitwise identical).
 *
 * Ownership: the caller owns every buffer.  The library allocates only plan
 * memory (segment table, work list, graph) and frees it in ou_plan_destroy.
 * grad is never written.
 *
 * Errors: every function returns a status.  Arguments are validated before
 * anything is launched; on error nothing is launched and nothing is written
 * (all or nothing across the segments of a multi-tensor call).
 * ou_last_error() gives a thread-local message for the last failure.
 * Device faults surface, as usual in HIP, at the caller's next
 * synchronisation.
 *
 * Streams are hipStream_t passed as void* (NULL = the default stream).
 * Calls enqueue work and return without synchronising, except
 * optimizer_update_32bit_multi (see there).
 */
#ifndef OPTIMIZER_UPDATE_H
#define OPTIMIZER_UPDATE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { OU_F32 = 0, OU_F16 = 1, OU_BF16 = 2 } ou_dtype;
/* Kinds.  ADAM and ADEMAMIX are the two-state update above.  The
 * one-state kinds keep state1 only (n floats); state2 is ignored and may be
 * NULL.  They are the textbook rules of the optimizers that the 32-bit
 * update family of the same library also carries (per element, binary32,
 * g' = g + weight_decay*p when weight_decay != 0, else g' = g):
 *   OU_MOMENTUM  m = g' on step 1, else beta1*m + g';  p = p - lr*m
 *                (heavy ball, no dampening, no Nesterov)
 *   OU_RMSPROP   m = beta1*m + (1-beta1)*(g'*g');  p = p - lr*(g'/(sqrt(m)+eps))
 *                (beta1 is RMSprop's smoothing constant)
 *   OU_ADAGRAD   m = m + g'*g';  p = p - lr*(g'/(sqrt(m)+eps))
 *   OU_LION      c = beta1*m + (1-beta1)*g;  p = p*d - lr*sign(c), sign(0) = 0;
 *                then m = beta2*m + (1-beta2)*g  (decoupled decay d as above)
 * skip_zeros applies to them as to the two-state kinds.  beta1 and beta2
 * must lie in [0, 1) for every kind (pass 0 where a kind has no beta).
 * Update-norm clipping is defined for ADAM and ADEMAMIX only. */
typedef enum {
    OU_ADAM = 0,
    OU_ADEMAMIX = 1,
    OU_MOMENTUM = 2,
    OU_RMSPROP = 3,
    OU_ADAGRAD = 4,
    OU_LION = 5
} ou_kind;

/* Weight-decay order.  The page says (section "Scope") that the order of
 * the decoupled decay and the step differs between versions of the update
 * without saying which is right.  By default the decay applies to the old
 * parameter, p*d - lr*u (Loshchilov & Hutter, Alg. 2; torch.optim.AdamW).
 * Every `kind` argument below may be OR'ed with OU_DECAY_AFTER to decay the
 * updated parameter instead: (p - lr*u)*d, rounded once per operation as
 * written.  Valid with ADAM, ADEMAMIX and LION (the kinds with decoupled
 * decay); OU_EINVAL with the others.  With weight_decay = 0 (d = 1) both
 * orders give the same bits.  A plan keeps the order it was created with. */
#define OU_DECAY_AFTER 0x100

enum {
    OU_OK = 0,
    OU_EINVAL = -1,       /* bad pointer, size, kind, dtype, step or hyperparameter */
    OU_EUNSUPPORTED = -2, /* device is not gfx950, or no HIP device */
    OU_EALIGN = -3,       /* a pointer is not aligned to its element size */
    OU_EOVERLAP = -4,     /* two buffers overlap (a written buffer with anything) */
    OU_ENOMEM = -5,       /* plan allocation failed */
    OU_EHIP = -6,         /* a HIP runtime call failed */
    OU_ECAPTURE = -7      /* call not allowed while the stream is being captured */
};

/* Hyperparameters of one step (the arguments of optimizer_update_32bit).
 * beta1, beta2 in [0, 1); beta3 in [0, 1) and alpha finite (AdEMAMix only,
 * ignored for ADAM); eps >= 0; lr, weight_decay finite; step >= 1;
 * skip_zeros != 0 enables skipping of zero-gradient elements. */
typedef struct {
    float beta1, beta2, beta3, alpha, eps, weight_decay, lr;
    int32_t skip_zeros;
    int64_t step;
} ou_hparams;

/* One tensor of a collection.  dtype is an ou_dtype; layout as above. */
typedef struct {
    void* param;
    const void* grad;
    float* state1;
    float* state2;
    int64_t n;
    int32_t dtype;
    int32_t reserved; /* must be 0 */
} ou_segment;

/* One optimizer step over one tensor of n elements (n = 0: no-op).
 * The per-tensor direct op of section "B300 benchmark and acceptance" of
 * the page.  Asynchronous on `stream`; capture-safe (no allocation, no
 * synchronisation, device properties cached per device). */
int optimizer_update_32bit(int kind, int dtype, void* param, const void* grad,
                           float* state1, float* state2, int64_t n,
                           float beta1, float beta2, float beta3, float alpha,
                           float eps, float weight_decay, int64_t step, float lr,
                           int skip_zeros, void* stream);

/* Update-norm clipping (the page's "max_unorm" option, which it names as a
 * launch predicate and as a separate precondition/reduction kernel but does
 * not define).  With max_unorm > 0 the direction u of the whole tensor
 * (the per-element value that the plain update multiplies by lr, zero for
 * elements skipped by skip_zeros) is scaled by
 *     s = min(1, max_unorm * ||p||_2 / ||u||_2)      (s = 1 if ||u|| = 0),
 * p being the parameter before the step, both norms summed in binary64 in a
 * fixed order; each parameter becomes p*d - fl32(lr*s)*u.  The moments are
 * those of the plain step.  max_unorm = 0 is exactly optimizer_update_32bit
 * (workspace unused).
 *
 * `workspace` is caller-owned device memory of at least
 * ou_clip_workspace_bytes(n) bytes, 16-byte aligned, not overlapping any
 * other buffer; it holds per-chunk partial norms and the clip factor
 * (workspace bytes [4, 8) hold s as a float after the step).  Three
 * launches on `stream`; no allocation, capture-safe.  A one-state kind with
 * max_unorm > 0 is rejected (OU_EINVAL). */
int64_t ou_clip_workspace_bytes(int64_t n);

int optimizer_update_32bit_clip(int kind, int dtype, void* param, const void* grad,
                                float* state1, float* state2, int64_t n,
                                float beta1, float beta2, float beta3, float alpha,
                                float eps, float weight_decay, int64_t step, float lr,
                                int skip_zeros, float max_unorm, void* workspace,
                                int64_t workspace_bytes, void* stream);

/* The clipped step of optimizer_update_32bit_clip without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * partial norms and the clip factor live in a static device array of the
 * library, 8 MiB + 256 bytes per GPU, held from the first call on a device
 * until the process ends.  Same arguments and results (bitwise) as
 * optimizer_update_32bit_clip, minus workspace and workspace_bytes; n may
 * be at most ou_clip_noalloc_max_elements() = 2^30 (larger n: OU_EINVAL,
 * nothing launched).  The call allocates nothing: no hipMalloc, hipFree or
 * allocating library routine.  All calls on one GPU share the array, so
 * calls that overlap in time on one GPU (other streams, other host
 * threads) race; calls in one stream's order do not.  After a call the
 * clip factor s of its step is not readable by the caller (use the
 * workspace form for that). */
int optimizer_update_32bit_clip_noalloc(int kind, int dtype, void* param, const void* grad,
                                        float* state1, float* state2, int64_t n,
                                        float beta1, float beta2, float beta3, float alpha,
                                        float eps, float weight_decay, int64_t step, float lr,
                                        int skip_zeros, float max_unorm, void* stream);

/* Largest n optimizer_update_32bit_clip_noalloc accepts (2^30). */
int64_t ou_clip_noalloc_max_elements(void);

/* One optimizer step over a collection of nseg tensors (any mix of
 * dtypes), one launch per dtype group (the eager optimizer.step() of
 * section "B300 benchmark and acceptance").  Convenience form: builds and
 * uploads the segment table on every call and synchronises `stream` before
 * returning; not allowed during stream capture.  For repeated steps use a
 * plan. */
int optimizer_update_32bit_multi(int kind, const ou_segment* segs, int32_t nseg,
                                 const ou_hparams* hp, void* stream);

/* A plan: the device-resident segment table and work list of a fixed
 * collection.  Pointers and sizes are captured at creation and must stay
 * valid and unchanged until ou_plan_destroy.  Segments with n = 0 are
 * dropped.  A plan is not thread-safe. */
typedef struct ou_plan_s* ou_plan;

int ou_plan_create(int kind, const ou_segment* segs, int32_t nseg, ou_plan* out);

/* One step of the plan's collection: one launch per dtype group, on
 * `stream`.  Capture-safe. */
int ou_plan_step(ou_plan plan, const ou_hparams* hp, void* stream);

/* The same step through a HIP graph: built and instantiated on the first
 * call, then replayed with this step's scalars written into its kernel
 * nodes.  Bitwise identical to ou_plan_step.  Not allowed while `stream` is
 * being captured. */
int ou_plan_graph_step(ou_plan plan, const ou_hparams* hp, void* stream);

/* One step of the plan's collection with update-norm clipping, per tensor
 * (the rule of optimizer_update_32bit_clip applied to every segment with
 * its own norms): three launches per dtype group, on `stream`.  Bitwise
 * identical to optimizer_update_32bit_clip on each tensor.  max_unorm = 0 is
 * ou_plan_step.  The plan holds the partial norms; capture-safe. */
int ou_plan_step_clip(ou_plan plan, const ou_hparams* hp, float max_unorm, void* stream);

/* The clipped step through a HIP graph of its own (a chain of the three
 * launches per dtype group), built and instantiated on the first call, then
 * replayed with this step's scalars and max_unorm written into its kernel
 * nodes.  Bitwise identical to ou_plan_step_clip; max_unorm = 0 is
 * ou_plan_graph_step.  Not allowed while `stream` is being captured. */
int ou_plan_graph_step_clip(ou_plan plan, const ou_hparams* hp, float max_unorm, void* stream);

/* Clip factors s of the last clipped step, in the order of the segments
 * given to ou_plan_create (1 for segments with n = 0 or before any clipped
 * step has run).  Synchronous copy to host memory; nseg must equal the
 * plan's segment count. */
int ou_plan_clip_factors(ou_plan plan, float* out, int32_t nseg);

/* Shape of a plan: dtype groups (= launches per step), work items, elements. */
int ou_plan_describe(ou_plan plan, int32_t* n_groups, int64_t* n_work_items,
                     int64_t* n_elements);

/* Frees the plan (waits for nothing: the caller makes sure no step of it is
 * still running).  NULL is a no-op. */
void ou_plan_destroy(ou_plan plan);

/* ---- 8-bit block-wise states ------------------------------------------
 *
 * The page times AdamW8bit collections, in which tensors of fewer than
 * min_8bit_size = 4,096 elements take the 32-bit path above (sections
 * "Problem" and "B300 benchmark and acceptance").  These entry points are
 * the other leg: ADAM and ADEMAMIX (optionally | OU_DECAY_AFTER) with each
 * moment kept as 8-bit codes plus one fp32 absmax per block of
 * OU_8BIT_BLOCK elements (block-wise quantization, Dettmers et al. 2022).
 *
 * Codes.  First moments use the signed dynamic type (bit 7 = sign, bits 0-6
 * = magnitude index), the second moment the unsigned one (bits 0-7 =
 * magnitude index).  Magnitude index 0 is 0; the others are the centres of
 * 2^F equal bins of [0.1, 1] in the decades 10^-E (the dynamic tree type of
 * Dettmers 2016 with E + F = 6 signed, 7 unsigned), increasing with the
 * index, the largest set to 1.  ou_8bit_qmap returns them.
 *
 * Step, per block of elements [256 b, min(n, 256 (b+1))):
 *   1. each moment = magnitude(code) (signed as coded) * absmax[b];
 *   2. the 32-bit rule above updates the moments and the parameter
 *      (skip_zeros: the element's moments keep their values, its parameter
 *      is not written);
 *   3. the new absmax of each moment is its largest |value| in the block;
 *   4. each moment is stored as the code of the magnitude nearest to
 *      |value| / absmax in exact arithmetic: its index counts the exact
 *      midpoints mid of neighbouring magnitudes with mid * absmax < |value|,
 *      so a ratio exactly halfway goes to the smaller magnitude; bit 7 of a
 *      signed code is set for value < 0; a NaN value, and a finite value in
 *      a block whose absmax is +inf, take index 0.
 * All-zero codes with zero absmax are the zero state.
 *
 * Layout: state1 holds n codes (ADAM) or 2n (ADEMAMIX: fast EMA at [0, n),
 * slow EMA at [n, 2n)); state2 n codes; absmax1 nb floats (ADAM) or 2nb
 * (ADEMAMIX: [0, nb) fast, [nb, 2nb) slow); absmax2 nb floats, with
 * nb = ceil(n / 256).  Device pointers, aligned to their element size; the
 * wide path needs param and grad aligned to 4 elements and the code planes
 * to 4 bytes (otherwise the same steps run element by element).  Errors,
 * ownership and asynchrony as for optimizer_update_32bit. */
#define OU_8BIT_BLOCK 256

/* Copies the magnitudes of the signed (128) or unsigned (256) type to host
 * memory `out`; count must be 128 or 256 accordingly. */
int ou_8bit_qmap(int is_signed, float* out, int32_t count);

int optimizer_update_8bit_blockwise(int kind, int dtype, void* param, const void* grad,
                                    uint8_t* state1, uint8_t* state2, float* absmax1,
                                    float* absmax2, int64_t n, float beta1, float beta2,
                                    float beta3, float alpha, float eps, float weight_decay,
                                    int64_t step, float lr, int skip_zeros, void* stream);

/* One tensor of an 8-bit collection; layout as above. */
typedef struct {
    void* param;
    const void* grad;
    uint8_t* state1;
    uint8_t* state2;
    float* absmax1;
    float* absmax2;
    int64_t n;
    int32_t dtype;
    int32_t reserved; /* must be 0 */
} ou_segment8;

/* A plan over a fixed 8-bit collection: device-resident segment table and
 * work list, one launch per dtype group per step (capture-safe).  Pointers
 * must stay valid until ou_plan8_destroy.  Not thread-safe. */
typedef struct ou_plan8_s* ou_plan8;
int ou_plan8_create(int kind, const ou_segment8* segs, int32_t nseg, ou_plan8* out);
int ou_plan8_step(ou_plan8 plan, const ou_hparams* hp, void* stream);

/* The same step through a HIP graph built on the first call and replayed
 * with this step's scalars written into its kernel nodes (as
 * ou_plan_graph_step).  Bitwise identical to ou_plan8_step.  Not allowed
 * while `stream` is being captured. */
int ou_plan8_graph_step(ou_plan8 plan, const ou_hparams* hp, void* stream);

void ou_plan8_destroy(ou_plan8 plan);

/* ---- one graph over several plans ----------------------------------------
 *
 * The page's AdamW8bit collections (sections "Problem" and "B300 benchmark
 * and acceptance") step two plans per optimizer step: the tensors of at
 * least min_8bit_size elements through an 8-bit plan, the others through a
 * 32-bit plan.  An ou_graph replays the plain steps of any set of plans on
 * one device as a single HIP graph: built and instantiated on the first
 * ou_graph_step, later steps write the step's scalars (per plan, with its
 * own kind and decay order) into the kernel nodes and replay.  The launches
 * run in one chain, the 32-bit plans in the order given, then the 8-bit
 * ones; results are bitwise those of ou_plan_step / ou_plan8_step on each
 * plan.  The plans must outlive the graph (destroy the graph first) and are
 * not copied.  ou_graph_step is not allowed while `stream` is being
 * captured; hp must be valid for every plan's kind. */
typedef struct ou_graph_s* ou_graph;
int ou_graph_create(const ou_plan* plans, int32_t nplans, const ou_plan8* plans8, int32_t nplans8,
                    ou_graph* out);
int ou_graph_step(ou_graph graph, const ou_hparams* hp, void* stream);
void ou_graph_destroy(ou_graph graph);

const char* ou_status_string(int status);
const char* ou_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* OPTIMIZER_UPDATE_H */
