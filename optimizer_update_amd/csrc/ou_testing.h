// ou_testing.h -- test-only hooks of liboptimizer_update.so.
//
// Not part of the public ABI (include/optimizer_update.h): launch-shape
// forcing stays out of the public interface, as the page "Investigate a
// 256-thread SM103 path for small 32-bit optimizer tensors" asks for its own
// variant forcing (section "Scope").  The tests use these to run every
// launch variant and compare results bitwise, and to check launch selection
// on a CPU with fabricated device properties.
#pragma once

#include <stdint.h>

#include "../../include/optimizer_update.h"

#ifdef __cplusplus
extern "C" {
#endif

// Launch shape the single-tensor entry would pick for a device with the
// given CU count and LDS sizes: out = {block, epl, unroll, grid, lds}.
int ou__select_single(int cu_count, int lds_per_cu, int lds_per_block, int kind, int dtype, int64_t n,
                      int aligned, int64_t out[5]);

// Launch shape a plan would pick for a dtype group of `total_elements`
// on such a device: out = {waves, epl, unroll, lds, xcd_run, chunk, lds of
// the clipped step's pass 1 over as many elements}.
int ou__select_multi(int cu_count, int lds_per_cu, int lds_per_block, int kind, int dtype,
                     int64_t total_elements, int64_t out[7]);

// Force the single-tensor launch shape (0 = no forcing for that field;
// lds -1 = no occupancy cap); scalar_only != 0 forces the
// one-element-per-lane path.  Process-wide.
void ou__force_single(int block, int epl, int unroll, int64_t grid, int scalar_only, int lds);

// Force the multi-tensor shape used by plans created afterwards
// (0 = no forcing; lds -1 = no cap).  chunk must be a multiple of 64 * epl * unroll
// and waves at most 8 (the kernels' 512-thread launch bound); plan creation
// refuses other shapes with OU_EINVAL.
void ou__force_multi(int waves, int epl, int unroll, int chunk, int lds);

// Force the XCD tile runs (xcd_tile) of the single-tensor kernel and of
// plans created afterwards: run > 0 = runs of `run` tiles (a power of two;
// block order for grids under 64 runs), -1 = block order, 0 = no forcing.
// Process-wide.
void ou__force_xcd(int run);

// The update kernels' rounding of binary32 to the storage dtype (OU_F16 or
// OU_BF16) on n values: out[i] = narrow(in[i]).  dtype + 16 takes the packed
// form of the 8-bit kernels, two values per conversion (n even, out 4-byte
// aligned).  Asynchronous on `stream`.
int ou__narrow(int dtype, const float* in, uint16_t* out, int64_t n, void* stream);

// The 8-bit update kernels' square root on n values: out[i] = sqrt(in[i]),
// correctly rounded.  Asynchronous on `stream`.
int ou__sqrt(const float* in, float* out, int64_t n, void* stream);

// The 8-bit kernels' reciprocal of a block maximum on n values: out[i] =
// fl32(1 / in[i]) for in[i] > 0 finite, 0 for +0 and +inf (negative inputs
// and NaN are outside its domain and give 0).  Asynchronous on `stream`.
int ou__recip8(const float* in, float* out, int64_t n, void* stream);

// The 8-bit kernels' quantizer on n pairs: cs[i] = signed code of v[i],
// cu[i] = unsigned code of |v[i]|, each in a block whose absmax is
// absmax[i] (>= 0, not a NaN, with |v[i]| <= absmax[i] unless v[i] is a NaN
// or absmax[i] is +inf).  Asynchronous on `stream`.
int ou__quant8(const float* v, const float* absmax, uint8_t* cs, uint8_t* cu, int64_t n, void* stream);

// Bandwidth probes in the launch shape of the plain fp32 Adam update of n
// elements, with no arithmetic; n a multiple of 4, buffers 16-byte aligned.
// mode 0: its traffic (p, g, s1, s2 read; p, s1, s2 written back
// unchanged); mode 1: the four reads alone (nothing written); mode 2: the
// three writes alone (p, s1, s2 overwritten with a pattern).  Asynchronous
// on `stream`.  For measuring what the read/write mix, its reads and its
// writes reach.
int ou__stream_probe(int mode, float* p, const float* g, float* s1, float* s2, int64_t n, void* stream);

// VALU issue probe: `blocks` blocks of 256 threads, each lane running
// `iters` rounds of 64 independent full-rate binary32 operations on
// registers (64 * iters VALU instructions per wave, no memory traffic; `out`
// is never written): op 0 fused multiply-adds, op 1 additions (less power
// per instruction).  Asynchronous on `stream`.  For measuring the device's
// VALU issue rate; OU_EINVAL for another op.
int ou__valu_probe(int op, int64_t blocks, int32_t iters, float* out, void* stream);

// While on != 0, every entry point returns OU_OK right after its argument
// checks, before it queries or touches a device: no launch, no allocation
// (plan creation returns a NULL handle).  Lets the validation tests pass
// fabricated addresses on any machine.  Process-wide.
void ou__validate_only(int on);

// The per-step scalars: beta1..3, 1-beta1..3, alpha, eps, lr, bc1, bc2, decay.
int ou__step_scalars(const ou_hparams* hp, float out[12]);

// Force the 8-bit launch shape (0 = no forcing): waves per workgroup,
// blocks per wave of the single-tensor kernel, blocks per work item of
// plans created afterwards; scalar_only != 0 forces the element-by-element
// path.  Process-wide.
void ou__force_8bit(int waves, int blocks_per_wave, int chunk_blocks, int scalar_only);

#ifdef __cplusplus
}
#endif
