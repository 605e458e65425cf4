/*
 * CPU oracle for the 32-bit two-state optimizer update (Adam/AdamW and
 * AdEMAMix).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path loads, links or
 * calls this file.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it, and it shares no code, header, table or helper
 * with the HIP library.
 *
 * Subject page: "Investigate a 256-thread SM103 path for small 32-bit
 * optimizer tensors" (bitsandbytes fork, issue 8).  The page names the two
 * update kinds ADAM and ADEMAMIX, fp32/fp16/bf16 parameter and gradient
 * storage with fp32 states (section "Correctness oracle"), decoupled weight
 * decay (section "Scope") and an unchanged state layout (section
 * "Non-goals").  It prints no formula, so the formulas are the textbook ones:
 *   - moments and bias correction: Kingma & Ba 2015, Algorithm 1;
 *   - decoupled weight decay:     Loshchilov & Hutter 2019, Algorithm 2;
 *   - slow EMA mixed in with alpha: Pagliardini, Ablin & Grangier 2024,
 *     Algorithm 1 (the slow EMA is not bias-corrected; alpha and beta3 are
 *     held constant).
 *
 * Two instantiations:
 *   oracle_update_f32  every operation is one IEEE binary32 operation with
 *                      round-to-nearest-even (build with -ffp-contract=off,
 *                      no fast-math, no flush-to-zero).  This is the parity
 *                      oracle: the page fixes the states at 32 bits.
 *   oracle_update_f64  the same steps in binary64, used only to check the
 *                      formulas against closed forms.
 *
 * Storage conversions (binary16 and bfloat16) are written out from the IEEE
 * 754 / bfloat16 encodings: round to nearest, ties to even; overflow goes to
 * infinity; subnormals are kept; a NaN stays a quiet NaN (payload not kept).
 *
 * oracle_update1_f32 / oracle_update1_f64 cover the one-state kinds
 * (momentum SGD, RMSprop, Adagrad, Lion; the page implies a one-state sibling
 * of the two-state path without naming one).
 *
 * oracle_update_f32_clip / oracle_update_f64_clip add update-norm clipping
 * (the page's "max_unorm"; it names the option only, so the clip rule is
 * stated at the function).
 *
 * oracle_update_8bit_f32 keeps the moments in 8-bit block-wise states
 * (the page's AdamW8bit collections, whose tensors below min_8bit_size fall
 * back to the 32-bit path); the data type and the step are stated at the
 * functions.
 *
 * Weight-decay order.  The page (section "Scope") says the order of the
 * decoupled decay and the step is being changed upstream without saying
 * which order is right.  The default here decays the old parameter,
 * p*d - lr*u (Loshchilov & Hutter, Algorithm 2; torch.optim.AdamW).  A kind
 * OR'ed with ORACLE_DECAY_AFTER applies the decay to the updated parameter
 * instead, (p - lr*u)*d.  The flag is valid for the kinds with decoupled
 * decay (ADAM, ADEMAMIX, LION); the L2 kinds reject it.
 *
 * ORACLE_PLANT (compile-time, default 0) plants one known mistake so that
 * the test suite can show its pins catch it.  It is never set in a normal
 * build.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif

enum { ORACLE_ADAM = 0, ORACLE_ADEMAMIX = 1,
       ORACLE_MOMENTUM = 2, ORACLE_RMSPROP = 3, ORACLE_ADAGRAD = 4, ORACLE_LION = 5 };
enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };
#define ORACLE_DECAY_AFTER 0x100

/* Splits a kind argument into the kind and the decay-order flag; -1 for
 * unknown flag bits. */
static int split_kind(int kind_arg, int* kind, int* after)
{
    if (kind_arg & ~(0xff | ORACLE_DECAY_AFTER))
        return -1;
    *kind = kind_arg & 0xff;
    *after = (kind_arg & ORACLE_DECAY_AFTER) != 0;
#if ORACLE_PLANT == 22
    *after = 0;                                     /* planted: decay-order flag ignored */
#endif
    return 0;
}

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, sizeof f); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, sizeof u); return u; }

/* ---------------------------------------------------------------- storage */

/* bfloat16 is the upper half of a binary32: widening appends 16 zero bits. */
float oracle_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even.  The kept part is
 * the upper 16 bits; the dropped part decides the rounding. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u = bits_from_f32(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)          /* NaN -> quiet NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
#if ORACLE_PLANT == 11
    dropped = 0;                                    /* planted: truncation */
#endif
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1;                                  /* carries into the exponent; max finite -> inf */
    return (uint16_t)kept;
}

/* binary16 -> binary32 (exact).  value = (-1)^s * m * 2^-24 for subnormals,
 * (-1)^s * (1024 + m) * 2^(e-25) for normals. */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    float mag;
    if (e == 0x1f)
        mag = m ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexpf((float)m, -24);
    else
        mag = ldexpf((float)(m + 1024), e - 25);
    return sign ? -mag : mag;
}

/* binary32 -> binary16, round to nearest, ties to even.
 * Write |x| = M * 2^E exactly, pick the binary16 quantum 2^Q that applies to
 * |x| (2^(floor(log2|x|) - 10) in the normal range, 2^-24 below it), round
 * M * 2^(E-Q) to an integer R (ties to even) and encode R * 2^Q. */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t u = bits_from_f32(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t e = (u >> 23) & 0xffu, frac = u & 0x7fffffu;
    if (e == 0xffu)
        return (uint16_t)(sign | (frac ? 0x7e00u : 0x7c00u));
    if (e == 0 && frac == 0)
        return sign;
    uint32_t M;
    int E;
    if (e == 0) { M = frac; E = -149; }
    else        { M = frac | 0x800000u; E = (int)e - 150; }
    int lead = E;                                   /* exponent of M's top bit */
    for (uint32_t t = M >> 1; t; t >>= 1) lead++;
    int Q = (lead >= -14) ? lead - 10 : -24;
#if ORACLE_PLANT == 12
    Q = lead - 10;                                  /* planted: no subnormal range */
#endif
    int s = Q - E;                                  /* bits dropped, always > 0 here */
    uint32_t R, rem, half;
    if (s > 25) {                                   /* M < 2^24 < half: rounds to 0 */
        R = 0; rem = 0; half = 1;
    } else {
        R = M >> s;
        rem = M - (R << s);
        half = 1u << (s - 1);
    }
    if (rem > half || (rem == half && (R & 1u)))
        R += 1;
    if (Q == -24)                                   /* subnormal; R == 1024 is the smallest normal */
        return (uint16_t)(sign | R);
    int be = Q + 25;                                /* biased exponent for R in [1024, 2048) */
    if (R == 2048) { R = 1024; be += 1; }
    if (be >= 31)
        return (uint16_t)(sign | 0x7c00u);          /* overflow -> infinity */
    return (uint16_t)(sign | ((uint32_t)be << 10) | (R - 1024));
}

void oracle_f32_to_bf16_array(const float* x, uint16_t* y, int64_t n)
{ for (int64_t i = 0; i < n; i++) y[i] = oracle_f32_to_bf16(x[i]); }
void oracle_f32_to_f16_array(const float* x, uint16_t* y, int64_t n)
{ for (int64_t i = 0; i < n; i++) y[i] = oracle_f32_to_f16(x[i]); }
void oracle_f16_to_f32_array(const uint16_t* x, float* y, int64_t n)
{ for (int64_t i = 0; i < n; i++) y[i] = oracle_f16_to_f32(x[i]); }
void oracle_bf16_to_f32_array(const uint16_t* x, float* y, int64_t n)
{ for (int64_t i = 0; i < n; i++) y[i] = oracle_bf16_to_f32(x[i]); }

static float load_storage(const void* base, int dtype, int64_t i)
{
    if (dtype == ORACLE_F32) return ((const float*)base)[i];
    if (dtype == ORACLE_F16) return oracle_f16_to_f32(((const uint16_t*)base)[i]);
    return oracle_bf16_to_f32(((const uint16_t*)base)[i]);
}

static void store_storage(void* base, int dtype, int64_t i, float x)
{
    if (dtype == ORACLE_F32) ((float*)base)[i] = x;
    else if (dtype == ORACLE_F16) ((uint16_t*)base)[i] = oracle_f32_to_f16(x);
    else ((uint16_t*)base)[i] = oracle_f32_to_bf16(x);
}

/* --------------------------------------------------------- step scalars */

/* Per-step scalars of the fp32 instantiation.  The bias corrections
 * 1 - beta^t and the decay factor 1 - lr*wd are formed in binary64 from the
 * binary32 arguments and then rounded to binary32; 1 - beta is formed in
 * binary32 (exact for beta in [0.5, 1]). */
typedef struct {
    float bc1, bc2, decay, omb1, omb2, omb3;
} oracle_scalars32;

void oracle_step_scalars(float beta1, float beta2, float beta3, float lr,
                         float weight_decay, int64_t step, oracle_scalars32* out)
{
    double t = (double)step;
#if ORACLE_PLANT == 13
    t = (double)(step + 1);                         /* planted: step off by one */
#endif
    out->bc1 = (float)(1.0 - pow((double)beta1, t));
    out->bc2 = (float)(1.0 - pow((double)beta2, t));
#if ORACLE_PLANT == 4
    out->decay = (float)(1.0 + (double)lr * (double)weight_decay);  /* planted: decay sign */
#else
    out->decay = (float)(1.0 - (double)lr * (double)weight_decay);
#endif
    out->omb1 = 1.0f - beta1;
    out->omb2 = 1.0f - beta2;
    out->omb3 = 1.0f - beta3;
}

/* ------------------------------------------------------ fp32 instantiation */

/* The moments and the update direction of one element, binary32.  m, v:
 * first and second moment; m2: slow EMA (AdEMAMix only).  Updates the
 * moments and returns the direction u (the parameter moves by lr * u). */
static float direction_f32(int kind, float g, float* m, float* v, float* m2,
                           const oracle_scalars32* s, float beta1, float beta2, float beta3,
                           float alpha, float eps)
{
    /* first and second moment (Kingma & Ba, Algorithm 1) */
    float mn = beta1 * (*m) + s->omb1 * g;
#if ORACLE_PLANT == 9
    float vn = beta2 * (*v) + s->omb2 * fabsf(g);   /* planted: dropped square */
#else
    float vn = beta2 * (*v) + s->omb2 * (g * g);
#endif
    float m2n = 0.0f;
    if (kind == ORACLE_ADEMAMIX)                   /* slow EMA (Pagliardini et al., Algorithm 1) */
        m2n = beta3 * (*m2) + s->omb3 * g;

    /* bias-corrected moments and the direction */
    float mh = mn / s->bc1;
#if ORACLE_PLANT == 1
    float vh = vn;                                  /* planted: v not bias-corrected */
#else
    float vh = vn / s->bc2;
#endif
#if ORACLE_PLANT == 2
    float den = sqrtf(vh + eps);                    /* planted: eps inside the root */
#else
    float den = sqrtf(vh) + eps;
#endif
    float num = mh;
    if (kind == ORACLE_ADEMAMIX) {
#if ORACLE_PLANT == 5
        num = mh + alpha * (m2n / s->bc1);          /* planted: slow EMA bias-corrected */
#elif ORACLE_PLANT == 6
        num = alpha * mh + m2n;                     /* planted: alpha on the wrong EMA */
#else
        num = mh + alpha * m2n;
#endif
    }
    float upd = num / den;
    *m = mn;
    *v = vn;
    if (kind == ORACLE_ADEMAMIX) *m2 = m2n;
    return upd;
}

/* Decoupled weight decay of the old parameter and the step along u
 * (Loshchilov & Hutter, Algorithm 2); with `after`, the decay of the
 * updated parameter.  Returns the new parameter before rounding to the
 * storage type. */
static float param_f32(float p, float upd, float decay, float lr, int after)
{
    if (after)
        return (p - lr * upd) * decay;
#if ORACLE_PLANT == 3
    return (p - lr * upd) * decay;                  /* planted: decay after the update */
#else
    return p * decay - lr * upd;
#endif
}

/* One element, binary32: direction, then parameter. */
static float element_f32(int kind, float p, float g, float* m, float* v, float* m2,
                         const oracle_scalars32* s, float beta1, float beta2, float beta3,
                         float alpha, float eps, float lr, int after)
{
    float upd = direction_f32(kind, g, m, v, m2, s, beta1, beta2, beta3, alpha, eps);
    return param_f32(p, upd, s->decay, lr, after);
}

/* One optimizer step over n elements, in place.
 *   param, grad : n elements of the storage dtype (fp32, fp16 or bf16 bits)
 *   state1      : n floats (ADAM) or 2n floats (ADEMAMIX: fast EMA at [0, n),
 *                 slow EMA at [n, 2n))
 *   state2      : n floats
 *   step        : 1-based index of the update being applied
 * With skip_zeros set, an element whose gradient compares equal to zero
 * (+0 or -0) is left untouched: no moment update and no decay.
 * grad is only read.  kind may carry ORACLE_DECAY_AFTER.  Returns 0, or -1
 * on an invalid kind or dtype. */
int oracle_update_f32(int kind_arg, int dtype, void* param, const void* grad,
                      float* state1, float* state2, int64_t n,
                      float beta1, float beta2, float beta3, float alpha, float eps,
                      float weight_decay, int64_t step, float lr, int skip_zeros,
                      int nthreads)
{
    int kind, after;
    if (split_kind(kind_arg, &kind, &after) ||
        (kind != ORACLE_ADAM && kind != ORACLE_ADEMAMIX) ||
        (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16))
        return -1;
    oracle_scalars32 s;
#if ORACLE_PLANT == 7
    oracle_step_scalars(beta2, beta1, beta3, lr, weight_decay, step, &s);  /* planted: betas swapped */
    { float t = beta1; beta1 = beta2; beta2 = t; }
#else
    oracle_step_scalars(beta1, beta2, beta3, lr, weight_decay, step, &s);
#endif
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t i = 0; i < n; i++) {
        float g = load_storage(grad, dtype, i);
        if (skip_zeros && g == 0.0f) {
#if ORACLE_PLANT == 8
            store_storage(param, dtype, i, load_storage(param, dtype, i) * s.decay);  /* planted: decay on skip */
#endif
            continue;
        }
        float p = load_storage(param, dtype, i);
        float* m2 = (kind == ORACLE_ADEMAMIX) ? &state1[n + i] : NULL;
#if ORACLE_PLANT == 14
        if (kind == ORACLE_ADEMAMIX) m2 = &state1[2 * n - 1 - i];   /* planted: slow plane reversed */
#endif
        float pn = element_f32(kind, p, g, &state1[i], &state2[i], m2, &s,
                               beta1, beta2, beta3, alpha, eps, lr, after);
        store_storage(param, dtype, i, pn);
#if ORACLE_PLANT == 10
        if (dtype == ORACLE_F32) ((float*)grad)[i] = pn;           /* planted: grad written */
#endif
    }
    return 0;
}

/* ------------------------------------------------------ fp64 instantiation */

/* The same update with every operation in binary64 and the step scalars
 * unrounded.  fp64 arrays only; used to check the formulas against closed
 * forms.  Layout and arguments as oracle_update_f32. */
int oracle_update_f64(int kind_arg, double* param, const double* grad, double* state1,
                      double* state2, int64_t n, double beta1, double beta2, double beta3,
                      double alpha, double eps, double weight_decay, int64_t step,
                      double lr, int skip_zeros)
{
    int kind, after;
    if (split_kind(kind_arg, &kind, &after) || (kind != ORACLE_ADAM && kind != ORACLE_ADEMAMIX))
        return -1;
#if ORACLE_PLANT == 7
    { double t = beta1; beta1 = beta2; beta2 = t; }
#endif
    double t = (double)step;
#if ORACLE_PLANT == 13
    t = (double)(step + 1);
#endif
    double bc1 = 1.0 - pow(beta1, t);
    double bc2 = 1.0 - pow(beta2, t);
    (void)bc2;
#if ORACLE_PLANT == 4
    double decay = 1.0 + lr * weight_decay;
#else
    double decay = 1.0 - lr * weight_decay;
#endif
    for (int64_t i = 0; i < n; i++) {
        double g = grad[i];
        if (skip_zeros && g == 0.0) {
#if ORACLE_PLANT == 8
            param[i] = param[i] * decay;
#endif
            continue;
        }
        double m = beta1 * state1[i] + (1.0 - beta1) * g;
#if ORACLE_PLANT == 9
        double v = beta2 * state2[i] + (1.0 - beta2) * fabs(g);
#else
        double v = beta2 * state2[i] + (1.0 - beta2) * (g * g);
#endif
        int64_t slow = n + i;
#if ORACLE_PLANT == 14
        slow = 2 * n - 1 - i;
#endif
        double m2 = 0.0;
        if (kind == ORACLE_ADEMAMIX)
            m2 = beta3 * state1[slow] + (1.0 - beta3) * g;
        double mh = m / bc1;
#if ORACLE_PLANT == 1
        double vh = v;
#else
        double vh = v / bc2;
#endif
#if ORACLE_PLANT == 2
        double den = sqrt(vh + eps);
#else
        double den = sqrt(vh) + eps;
#endif
        double num = mh;
        if (kind == ORACLE_ADEMAMIX) {
#if ORACLE_PLANT == 5
            num = mh + alpha * (m2 / bc1);
#elif ORACLE_PLANT == 6
            num = alpha * mh + m2;
#else
            num = mh + alpha * m2;
#endif
        }
        double upd = num / den;
#if ORACLE_PLANT == 3
        param[i] = (param[i] - lr * upd) * decay;
#else
        param[i] = after ? (param[i] - lr * upd) * decay : param[i] * decay - lr * upd;
#endif
        state1[i] = m;
        state2[i] = v;
        if (kind == ORACLE_ADEMAMIX) state1[slow] = m2;
    }
    return 0;
}

/* ------------------------------------------------------ one-state kinds */

/* One element of a one-state update, binary32; m is the element's state.
 * Returns the new parameter before rounding to storage.
 *   MOMENTUM  (SGD with momentum, Sutskever et al. 2013 / torch.optim.SGD,
 *             dampening 0): gd = g + wd*p (L2 term, only when wd != 0);
 *             m = gd on the first step, else beta1*m + gd; p - lr*m
 *   RMSPROP   (Tieleman & Hinton 2012): gd as above;
 *             m = beta1*m + (1-beta1)*(gd*gd); p - lr*(gd/(sqrt(m)+eps))
 *   ADAGRAD   (Duchi et al. 2011): gd as above; m = m + gd*gd;
 *             p - lr*(gd/(sqrt(m)+eps))
 *   LION      (Chen et al. 2023): c = beta1*m + (1-beta1)*g; u = sign(c)
 *             (0 for c = 0, NaN stays NaN); p*d - lr*u with the decoupled
 *             decay d = fl32(1 - fl64(lr*wd)); then m = beta2*m + (1-beta2)*g */
static float one_state_f32(int kind, float p, float g, float* m, float beta1, float beta2,
                           float eps, float wd, float lr, float decay, int first, int after)
{
    if (kind == ORACLE_LION) {
#if ORACLE_PLANT == 18
        *m = beta2 * (*m) + (1.0f - beta2) * g;     /* planted: moment updated before the sign */
#endif
        float c = beta1 * (*m) + (1.0f - beta1) * g;
        float u = (c != c) ? c : (float)((c > 0.0f) - (c < 0.0f));
        float pn = after ? (p - lr * u) * decay : p * decay - lr * u;
#if ORACLE_PLANT != 18
        *m = beta2 * (*m) + (1.0f - beta2) * g;
#endif
        return pn;
    }
    float gd = (wd != 0.0f) ? g + wd * p : g;
    if (kind == ORACLE_MOMENTUM) {
#if ORACLE_PLANT == 21
        float mn = first ? gd : beta1 * (*m) + (1.0f - beta1) * gd;   /* planted: dampening */
#else
        float mn = first ? gd : beta1 * (*m) + gd;
#endif
        *m = mn;
        return p - lr * mn;
    }
#if ORACLE_PLANT == 20
    float vn = (kind == ORACLE_RMSPROP) ? beta1 * (*m) + (1.0f - beta1) * (gd * gd)
                                        : (*m) + fabsf(gd);                /* planted: no square */
#else
    float vn = (kind == ORACLE_RMSPROP) ? beta1 * (*m) + (1.0f - beta1) * (gd * gd)
                                        : (*m) + gd * gd;
#endif
    *m = vn;
#if ORACLE_PLANT == 19
    return p - lr * (gd / sqrtf(vn + eps));       /* planted: eps inside the root */
#else
    return p - lr * (gd / (sqrtf(vn) + eps));
#endif
}

/* One step of a one-state kind over n elements, in place.  state1: n
 * floats; skip_zeros as for the two-state kinds (an element with g == 0 is
 * left untouched).  step is 1-based (MOMENTUM starts its buffer at step 1).
 * ORACLE_DECAY_AFTER is accepted for LION only.  Returns 0, or -1 on an
 * invalid kind or dtype. */
int oracle_update1_f32(int kind_arg, int dtype, void* param, const void* grad, float* state1,
                       int64_t n, float beta1, float beta2, float eps, float weight_decay,
                       int64_t step, float lr, int skip_zeros, int nthreads)
{
    int kind, after;
    if (split_kind(kind_arg, &kind, &after) || kind < ORACLE_MOMENTUM || kind > ORACLE_LION ||
        (after && kind != ORACLE_LION) ||
        (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16))
        return -1;
    float decay = (float)(1.0 - (double)lr * (double)weight_decay);
    int first = step == 1;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t i = 0; i < n; i++) {
        float g = load_storage(grad, dtype, i);
        if (skip_zeros && g == 0.0f) continue;
        float p = load_storage(param, dtype, i);
        store_storage(param, dtype, i, one_state_f32(kind, p, g, &state1[i], beta1, beta2, eps,
                                                     weight_decay, lr, decay, first, after));
    }
    return 0;
}

/* The one-state kinds in binary64 (fp64 arrays), for closed forms. */
int oracle_update1_f64(int kind_arg, double* param, const double* grad, double* state1,
                       int64_t n, double beta1, double beta2, double eps, double weight_decay,
                       int64_t step, double lr, int skip_zeros)
{
    int kind, after;
    if (split_kind(kind_arg, &kind, &after) || kind < ORACLE_MOMENTUM || kind > ORACLE_LION ||
        (after && kind != ORACLE_LION))
        return -1;
    double decay = 1.0 - lr * weight_decay;
    for (int64_t i = 0; i < n; i++) {
        double g = grad[i], p = param[i], m = state1[i];
        if (skip_zeros && g == 0.0) continue;
        if (kind == ORACLE_LION) {
#if ORACLE_PLANT == 18
            m = beta2 * m + (1.0 - beta2) * g;
#endif
            double c = beta1 * m + (1.0 - beta1) * g;
            double u = (c != c) ? c : (double)((c > 0.0) - (c < 0.0));
            param[i] = after ? (p - lr * u) * decay : p * decay - lr * u;
#if ORACLE_PLANT == 18
            state1[i] = m;
#else
            state1[i] = beta2 * m + (1.0 - beta2) * g;
#endif
            continue;
        }
        double gd = (weight_decay != 0.0) ? g + weight_decay * p : g;
        if (kind == ORACLE_MOMENTUM) {
#if ORACLE_PLANT == 21
            double mn = (step == 1) ? gd : beta1 * m + (1.0 - beta1) * gd;
#else
            double mn = (step == 1) ? gd : beta1 * m + gd;
#endif
            state1[i] = mn;
            param[i] = p - lr * mn;
            continue;
        }
#if ORACLE_PLANT == 20
        double vn = (kind == ORACLE_RMSPROP) ? beta1 * m + (1.0 - beta1) * (gd * gd) : m + fabs(gd);
#else
        double vn = (kind == ORACLE_RMSPROP) ? beta1 * m + (1.0 - beta1) * (gd * gd) : m + gd * gd;
#endif
        state1[i] = vn;
#if ORACLE_PLANT == 19
        param[i] = p - lr * (gd / sqrt(vn + eps));
#else
        param[i] = p - lr * (gd / (sqrt(vn) + eps));
#endif
    }
    return 0;
}

/* ------------------------------------------------- update-norm clipping */

/* Clip factor of update-norm clipping: s = min(1, max_unorm * ||p|| / ||u||)
 * from the squared norms (binary64); 1 when max_unorm <= 0 or ||u|| = 0. */
static double clip_factor(double max_unorm, double p_sq, double u_sq)
{
    if (!(max_unorm > 0.0) || !(u_sq > 0.0))
        return 1.0;
#if ORACLE_PLANT == 16
    double r = max_unorm * sqrt(p_sq) / u_sq;       /* planted: ||u||^2 for ||u|| */
#else
    double r = max_unorm * sqrt(p_sq) / sqrt(u_sq);
#endif
#if ORACLE_PLANT == 17
    return r;                                       /* planted: clips when below the bound */
#else
    return r < 1.0 ? r : 1.0;
#endif
}

/* One step with update-norm clipping.  The update direction u of every
 * element (the value that oracle_update_f32 multiplies by lr) is scaled,
 * for the whole tensor, by s = min(1, max_unorm * ||p|| / ||u||): p is the
 * parameter before the step, both 2-norms run over all n elements, and an
 * element left alone by skip_zeros contributes u = 0.  The squared norms
 * are summed in binary64 in index order, s is rounded to binary32, and each
 * parameter becomes p*d - fl32(lr*s)*u.  The moments are those of the
 * unclipped step.  max_unorm = 0 gives oracle_update_f32 exactly.  With
 * ORACLE_DECAY_AFTER each parameter becomes (p - fl32(lr*s)*u)*d.
 * *scale_out (if not NULL) receives s.  Returns 0, -1 on an invalid kind or
 * dtype, -2 if out of memory. */
int oracle_update_f32_clip(int kind_arg, int dtype, void* param, const void* grad,
                           float* state1, float* state2, int64_t n,
                           float beta1, float beta2, float beta3, float alpha, float eps,
                           float weight_decay, int64_t step, float lr, int skip_zeros,
                           float max_unorm, float* scale_out)
{
    int kind, after;
    if (split_kind(kind_arg, &kind, &after) ||
        (kind != ORACLE_ADAM && kind != ORACLE_ADEMAMIX) ||
        (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16))
        return -1;
    oracle_scalars32 s;
    oracle_step_scalars(beta1, beta2, beta3, lr, weight_decay, step, &s);
    float* u = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    unsigned char* skip = (unsigned char*)malloc((size_t)(n > 0 ? n : 1));
    if (!u || !skip) { free(u); free(skip); return -2; }
    double p_sq = 0.0, u_sq = 0.0;
    for (int64_t i = 0; i < n; i++) {
        float p = load_storage(param, dtype, i);
        p_sq += (double)p * (double)p;
        float g = load_storage(grad, dtype, i);
        skip[i] = (unsigned char)(skip_zeros && g == 0.0f);
        u[i] = 0.0f;
        if (skip[i]) continue;
        float* m2 = (kind == ORACLE_ADEMAMIX) ? &state1[n + i] : NULL;
        u[i] = direction_f32(kind, g, &state1[i], &state2[i], m2, &s, beta1, beta2, beta3,
                             alpha, eps);
        u_sq += (double)u[i] * (double)u[i];
    }
#if ORACLE_PLANT == 15
    p_sq = 0.0;                                     /* planted: norm of the new parameter */
    for (int64_t i = 0; i < n; i++) {
        float pn = param_f32(load_storage(param, dtype, i), u[i], s.decay, lr, after);
        p_sq += (double)pn * (double)pn;
    }
#endif
    float scale = (float)clip_factor((double)max_unorm, p_sq, u_sq);
    float lr_eff = lr * scale;
    for (int64_t i = 0; i < n; i++) {
        if (skip[i]) continue;
        store_storage(param, dtype, i, param_f32(load_storage(param, dtype, i), u[i], s.decay, lr_eff, after));
    }
    if (scale_out) *scale_out = scale;
    free(u);
    free(skip);
    return 0;
}

/* The clipped step in binary64 (s unrounded); fp64 arrays only.  u is
 * taken from an unclipped step with lr = 1 and no decay (as p_old - p_new;
 * that difference rounds at the level of ulp(p), far below the tolerance of
 * the closed forms this instantiation is checked against). */
int oracle_update_f64_clip(int kind_arg, double* param, const double* grad, double* state1,
                           double* state2, int64_t n, double beta1, double beta2, double beta3,
                           double alpha, double eps, double weight_decay, int64_t step,
                           double lr, int skip_zeros, double max_unorm, double* scale_out)
{
    int kind, after;
    if (split_kind(kind_arg, &kind, &after) || (kind != ORACLE_ADAM && kind != ORACLE_ADEMAMIX))
        return -1;
    double* p_new = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double* p_old = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!p_new || !p_old) { free(p_new); free(p_old); return -2; }
    /* the unclipped step with lr = 1 and no decay gives -u in p_new - p_old */
    double p_sq = 0.0;
    for (int64_t i = 0; i < n; i++) {
        p_old[i] = param[i];
        p_new[i] = param[i];
        p_sq += param[i] * param[i];
    }
    int rc = oracle_update_f64(kind, p_new, grad, state1, state2, n, beta1, beta2, beta3,
                               alpha, eps, 0.0, step, 1.0, skip_zeros);
    if (rc) { free(p_new); free(p_old); return rc; }
    double u_sq = 0.0;
    for (int64_t i = 0; i < n; i++) {
        double u = p_old[i] - p_new[i];
        u_sq += u * u;
    }
#if ORACLE_PLANT == 15
    p_sq = 0.0;
    for (int64_t i = 0; i < n; i++) {
        double pn = p_old[i] * (1.0 - lr * weight_decay) - lr * (p_old[i] - p_new[i]);
        p_sq += pn * pn;
    }
#endif
    double scale = clip_factor(max_unorm, p_sq, u_sq);
    double decay = 1.0 - lr * weight_decay;
    for (int64_t i = 0; i < n; i++) {
        double u = p_old[i] - p_new[i];
        if (skip_zeros && grad[i] == 0.0) continue;
        param[i] = after ? (p_old[i] - (lr * scale) * u) * decay : p_old[i] * decay - (lr * scale) * u;
    }
    if (scale_out) *scale_out = scale;
    free(p_new);
    free(p_old);
    return 0;
}


/* ------------------------------------------------ 8-bit block-wise states */

/* The 8-bit dynamic data type of block-wise quantized optimizer states
 * (Dettmers, "8-bit approximations for parallelism in deep learning", 2016,
 * dynamic tree quantization; Dettmers, Lewis, Shleifer & Zettlemoyer,
 * "8-bit Optimizers via Block-wise Quantization", 2022, section 2).  The page
 * names the 8-bit optimizers only (section "B300 benchmark and
 * acceptance"), so the type is written from that description:
 *
 *   signed code (first moments):  bit 7 = sign; the 7 payload bits hold the
 *       magnitude index 0..127.
 *   unsigned code (second moment): the sign bit is given to the payload; 8
 *       payload bits, magnitude index 0..255.
 *
 * Magnitude index 0 is zero.  The others enumerate, for E = P-1 down to 0
 * (P = payload bits), the decade 10^-E: in the tree code, E leading zero
 * bits, a 1 ending the exponent, and F = P-1-E fraction bits that split
 * [0.1, 1] into 2^F equal bins; a value is its bin's centre
 *     fl32( (0.1 + ((j + 1/2) * 0.9) / 2^F) / 10^E )   (binary64, then rounded)
 * with j = 0 .. 2^F - 1 ascending.  The largest magnitude (E = 0, last bin)
 * is replaced by 1, so that a block's largest state, which normalises to
 * +-1, is kept exactly.  Magnitudes increase with the index. */
#define OQ_BLOCK 256

static int qmap_payload(int is_signed) { return is_signed ? 7 : 8; }

/* Writes the 2^P magnitudes (128 signed, 256 unsigned); returns the count. */
int oracle_qmap(int is_signed, float* mags)
{
    int P = qmap_payload(is_signed);
    int k = 0;
    mags[k++] = 0.0f;
    for (int E = P - 1; E >= 0; E--) {
        int F = P - 1 - E;
        double bins = (double)(1 << F);
        double decade = 1.0;
        for (int e = 0; e < E; e++) decade *= 10.0;
        for (int j = 0; j < (1 << F); j++) {
            double centre = 0.1 + (((double)j + 0.5) * 0.9) / bins;
            mags[k++] = (float)(centre / decade);
        }
    }
#if ORACLE_PLANT != 28
    mags[k - 1] = 1.0f;
#endif
    return k;
}

/* Magnitude index of |value| / absmax: the index of the magnitude nearest to
 * that ratio in exact arithmetic, a ratio exactly halfway between two
 * magnitudes going to the smaller one.  That is the number of exact
 * midpoints (mag[k] + mag[k+1]) / 2 lying strictly below the ratio, counted
 * here as mid * absmax < |value|.  Both sides are exact in binary64: a
 * midpoint of two neighbouring binary32 magnitudes has at most 26
 * significant bits and absmax 24, so their product needs at most 50, and no
 * product comes near binary64's subnormal range.  The ratio is 0 for finite
 * values in a block whose absmax is infinite, and every value is +-0 or NaN
 * when the absmax is 0; a NaN compares false and gets index 0. */
static int qmap_index(const float* mags, int count, float value, float absmax)
{
    const double av = fabs((double)value);
    const double A = (double)absmax;
#if ORACLE_PLANT == 30
    /* planted: the ratio taken as value * fl32(1 / absmax) against binary32
     * midpoints (a rounded normalisation) */
    const float x = absmax > 0.0f ? fabsf(value) * (1.0f / absmax) : 0.0f;
#endif
    int idx = 0;
    for (int k = 0; k + 1 < count; k++) {
        double mid = ((double)mags[k] + (double)mags[k + 1]) * 0.5;
#if ORACLE_PLANT == 23
        mid = (double)mags[k + 1];                  /* planted: truncation, not nearest */
#endif
#if ORACLE_PLANT == 30
        if ((float)mid < x) idx++;
        continue;
#endif
        if (mid * A < av) idx++;
    }
    return idx;
}

/* Code of a state value in a block with the given absmax (|value| <= absmax):
 * the magnitude index of qmap_index, and for the signed type bit 7 for
 * value < 0 (not for -0 or NaN). */
int oracle_qcode(int is_signed, float value, float absmax)
{
    float mags[256];
    int count = oracle_qmap(is_signed, mags);
    int idx = qmap_index(mags, count, value, absmax);
    if (is_signed && value < 0.0f) idx |= 0x80;
    return idx;
}

/* Normalised value of a code: the magnitude its index selects, negated
 * when the signed type's bit 7 is set. */
float oracle_qvalue(int is_signed, int code)
{
    float mags[256];
    oracle_qmap(is_signed, mags);
    if (!is_signed) return mags[code & 0xff];
    float v = mags[code & 0x7f];
#if ORACLE_PLANT == 29
    return v;                                       /* planted: sign bit ignored */
#endif
    return (code & 0x80) ? -v : v;
}

/* One step with 8-bit block-wise states (kinds ADAM, ADEMAMIX; the kind may
 * carry ORACLE_DECAY_AFTER), in place.
 *   state1  : n signed codes (ADAM) or 2n (ADEMAMIX: fast EMA, then slow EMA)
 *   state2  : n unsigned codes
 *   absmax1 : one float per block of 256 elements (ADAM) or two planes
 *             (ADEMAMIX: [0, nb) fast, [nb, 2nb) slow), nb = ceil(n / 256)
 *   absmax2 : nb floats
 * Block b covers elements [256 b, min(n, 256 (b + 1))).  Per block:
 *   1. each state is its code's value times the block's absmax;
 *   2. the 32-bit rule of oracle_update_f32 updates the moments and the
 *      parameter from these values (skip_zeros: the element's moments keep
 *      their values and its parameter is not written);
 *   3. the new absmax of each state is the largest |value| in the block
 *      (maxNum: a NaN is passed over);
 *   4. each state is stored as the code of the magnitude nearest to
 *      |value| / absmax in exact arithmetic (qmap_index: a ratio exactly
 *      halfway goes to the smaller magnitude, a NaN to index 0), with the
 *      signed type's bit 7 set for value < 0.
 * The parameter moves with the moments before they are quantized.  Zero
 * codes with zero absmax are the zero state.  Returns 0, -1 on an invalid
 * kind or dtype, -2 if out of memory. */
int oracle_update_8bit_f32(int kind_arg, int dtype, void* param, const void* grad,
                           uint8_t* state1, uint8_t* state2, float* absmax1, float* absmax2,
                           int64_t n, float beta1, float beta2, float beta3, float alpha,
                           float eps, float weight_decay, int64_t step, float lr,
                           int skip_zeros, int nthreads)
{
    int kind, after;
    if (split_kind(kind_arg, &kind, &after) ||
        (kind != ORACLE_ADAM && kind != ORACLE_ADEMAMIX) ||
        (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16))
        return -1;
    int block = OQ_BLOCK;
#if ORACLE_PLANT == 27
    block = 2 * OQ_BLOCK;                           /* planted: wrong block size */
#endif
    float smag[128], umag[256];
    oracle_qmap(1, smag);
    oracle_qmap(0, umag);
    oracle_scalars32 s;
    oracle_step_scalars(beta1, beta2, beta3, lr, weight_decay, step, &s);
    const int64_t nb = (n + block - 1) / block;
    const int two = kind == ORACLE_ADEMAMIX;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t b = 0; b < nb; b++) {
        float m[2 * OQ_BLOCK], v[2 * OQ_BLOCK], m2[2 * OQ_BLOCK];
        const int64_t i0 = b * block;
        const int len = (int)((n - i0) < block ? (n - i0) : block);
        /* 1. dequantize */
        for (int k = 0; k < len; k++) {
            int64_t i = i0 + k;
            uint8_t c1 = state1[i], c2 = state2[i];
            float q1 = (c1 & 0x80) ? -smag[c1 & 0x7f] : smag[c1 & 0x7f];
#if ORACLE_PLANT == 26
            q1 = umag[c1];                          /* planted: sign of the first moment lost */
#endif
            m[k] = q1 * absmax1[b];
            v[k] = umag[c2] * absmax2[b];
            m2[k] = 0.0f;
            if (two) {
                uint8_t c3 = state1[n + i];
                m2[k] = ((c3 & 0x80) ? -smag[c3 & 0x7f] : smag[c3 & 0x7f]) * absmax1[nb + b];
            }
        }
#if ORACLE_PLANT == 24
        float old_a1 = 0.0f, old_a2 = 0.0f;         /* planted: absmax of the old states */
        for (int k = 0; k < len; k++) { old_a1 = fmaxf(old_a1, fabsf(m[k])); old_a2 = fmaxf(old_a2, v[k]); }
#endif
        /* 2. the 32-bit update */
        for (int k = 0; k < len; k++) {
            int64_t i = i0 + k;
            float g = load_storage(grad, dtype, i);
            if (skip_zeros && g == 0.0f) continue;
            float p = load_storage(param, dtype, i);
            float pn = element_f32(kind, p, g, &m[k], &v[k], two ? &m2[k] : NULL, &s,
                                   beta1, beta2, beta3, alpha, eps, lr, after);
#if ORACLE_PLANT != 25
            store_storage(param, dtype, i, pn);
#else
            (void)pn;
#endif
        }
        /* 3. new absmax */
        float a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
        for (int k = 0; k < len; k++) {
            a1 = fmaxf(a1, fabsf(m[k]));
            a2 = fmaxf(a2, v[k]);
            if (two) a3 = fmaxf(a3, fabsf(m2[k]));
        }
#if ORACLE_PLANT == 24
        a1 = old_a1 > 0.0f ? old_a1 : a1;
        a2 = old_a2 > 0.0f ? old_a2 : a2;
#endif
        /* 4. quantize */
        for (int k = 0; k < len; k++) {
            int64_t i = i0 + k;
            int c1 = qmap_index(smag, 128, m[k], a1);
            if (m[k] < 0.0f) c1 |= 0x80;
            state1[i] = (uint8_t)c1;
            state2[i] = (uint8_t)qmap_index(umag, 256, v[k], a2);
            if (two) {
                int c3 = qmap_index(smag, 128, m2[k], a3);
                if (m2[k] < 0.0f) c3 |= 0x80;
                state1[n + i] = (uint8_t)c3;
            }
        }
        absmax1[b] = a1;
        absmax2[b] = a2;
        if (two) absmax1[nb + b] = a3;
#if ORACLE_PLANT == 25
        /* planted: the parameter moves with the quantized new moments */
        for (int k = 0; k < len; k++) {
            int64_t i = i0 + k;
            float g = load_storage(grad, dtype, i);
            if (skip_zeros && g == 0.0f) continue;
            uint8_t c1 = state1[i];
            float mq = ((c1 & 0x80) ? -smag[c1 & 0x7f] : smag[c1 & 0x7f]) * a1;
            float vq = umag[state2[i]] * a2;
            float den = sqrtf(vq / s.bc2) + eps;
            float u = (mq / s.bc1) / den;
            store_storage(param, dtype, i, param_f32(load_storage(param, dtype, i), u, s.decay, lr, after));
        }
#endif
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int oracle_planted(void) { return ORACLE_PLANT; }
