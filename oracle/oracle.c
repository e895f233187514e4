/*
 * Oracle for the shard-local mixed-precision AdamW step of ZeRO-DP.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously-correct CPU code that the
 * tests, the smoke check and the CPU-baseline leg of the benchmark compare the
 * HIP library against.  The product path never loads, links or calls it, and
 * it shares no code, header or constant with the HIP library.
 *
 * Arithmetic is IEEE fp64 (no FMA contraction, no fast-math); results are
 * rounded once to their storage type (fp32 master/m/v, 16-bit params).
 * OpenMP only splits independent elements or independent partial sums; the
 * partial sums are combined in thread order with compensated summation.
 *
 * Sources (web pages on ZeRO):
 *  [P2] "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models"
 *       (paper summary page), sections "メモリ消費の定量化" (memory
 *       accounting of mixed-precision Adam), "ZeRO-DP" (Stage 1 P_os,
 *       Stage 2 P_os+g, Stage 3 P_os+g+p and the 7.5B-model memory table),
 *       "ZeRO-R" (CB: constant-size fused buffers).
 *  [P4] "ZeRO" (AI-library tutorial page), sections "显存背景" (16 bytes per
 *       parameter with AdamW), "ZeRO-1/2/3" (per-stage memory equations).
 * Where the pages are silent (remainder of the split, clip formula, bias
 * correction, rounding) the textbook reading is taken; each is named where
 * it is used.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------
 * Partition: [P2] ZeRO-DP, Stage 1 - the optimizer state is cut into Nd equal
 * parts and each data-parallel process keeps and updates only its own part.
 * Reading for Nd not dividing psi: contiguous parts whose sizes differ by at
 * most one, the first (psi mod Nd) ranks holding the larger size, no padding.
 * ---------------------------------------------------------------------- */
int orc_partition(uint64_t psi, uint32_t nd, uint32_t rank, uint64_t *begin, uint64_t *end)
{
    if (nd == 0 || rank >= nd)
        return 1;
    uint64_t small = psi / nd;          /* size of every part before the remainder */
    uint64_t extra = psi % nd;          /* this many leading ranks get one more */
    uint64_t start = 0;
    for (uint32_t r = 0; r < rank; ++r)  /* walk over the parts that precede rank */
        start += small + (r < extra ? 1 : 0);
    *begin = start;
    *end = start + small + (rank < extra ? 1 : 0);
    return 0;
}

/* ------------------------------------------------------------------------
 * Model-state bytes per rank.  [P2] memory accounting: 2 bytes fp16 params,
 * 2 bytes fp16 grads and K bytes of optimizer state per parameter (K = 12 for
 * mixed-precision Adam: fp32 copy, momentum, variance).  [P2] ZeRO-DP:
 * P_os keeps K*psi/Nd of optimizer state per rank, P_os+g also 2*psi/Nd of
 * grads, P_os+g+p also 2*psi/Nd of params.  [P4] ZeRO-1/2/3 give the same
 * three equations with b_p = b_g = 2, b_o = K.
 * stage 0 = plain data parallelism, 1 = P_os, 2 = P_os+g, 3 = P_os+g+p.
 * The sharded terms are counted for the largest part, ceil(psi/Nd) elements.
 * ---------------------------------------------------------------------- */
int orc_mem_bytes(uint32_t stage, uint64_t psi, uint32_t nd, uint32_t k, uint64_t *bytes)
{
    if (nd == 0 || stage > 3)
        return 1;
    uint64_t largest = psi / nd + (psi % nd ? 1 : 0);
    uint64_t params = 2 * psi, grads = 2 * psi, optim = (uint64_t)k * psi;
    if (stage >= 1) optim = (uint64_t)k * largest;
    if (stage >= 2) grads = 2 * largest;
    if (stage >= 3) params = 2 * largest;
    *bytes = params + grads + optim;
    return 0;
}

/* ------------------------------------------------------------------------
 * 16-bit storage formats (IEEE binary16 and bfloat16), decoded from the bit
 * fields and encoded by rounding to the nearest representable value, ties to
 * even.  Both are definitions, independent of any hardware conversion.
 * ---------------------------------------------------------------------- */
double orc_f16_value(uint16_t h)
{
    int neg = h >> 15, e = (h >> 10) & 0x1f, f = h & 0x3ff;
    double mag;
    if (e == 0x1f)
        mag = f ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)f, -24);               /* subnormal: f * 2^-24 */
    else
        mag = ldexp((double)(1024 + f), e - 25);   /* (1 + f/2^10) * 2^(e-15) */
    return neg ? -mag : mag;
}

double orc_bf16_value(uint16_t b)
{
    int neg = b >> 15, e = (b >> 7) & 0xff, f = b & 0x7f;
    double mag;
    if (e == 0xff)
        mag = f ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)f, -133);              /* subnormal: f * 2^-133 */
    else
        mag = ldexp((double)(128 + f), e - 134);   /* (1 + f/2^7) * 2^(e-127) */
    return neg ? -mag : mag;
}

/* Round |x| to a multiple of the spacing of the target format at |x|:
 * spacing = 2^(floor(log2|x|) - mant_bits) in the normal range and the
 * subnormal spacing below it; nearbyint() rounds half to even. */
static double round_to_format(double a, int mant_bits, int emin, int sub_exp)
{
    if (a < ldexp(1.0, emin))
        return nearbyint(a / ldexp(1.0, sub_exp)) * ldexp(1.0, sub_exp);
    int e;
    frexp(a, &e);                                   /* a = fr * 2^e, fr in [0.5, 1) */
    double q = ldexp(1.0, (e - 1) - mant_bits);
    return nearbyint(a / q) * q;
}

uint16_t orc_f16_bits(float xf)
{
    double x = xf;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return sign | 0x7e00;
    double r = round_to_format(fabs(x), 10, -14, -24);
    if (r > 65504.0)                                /* beyond the largest finite half */
        return sign | 0x7c00;
    if (r < ldexp(1.0, -14))
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    int e;
    double fr = frexp(r, &e);                       /* r = (2 fr) * 2^(e-1) */
    uint16_t exp_field = (uint16_t)(e - 1 + 15);
    uint16_t frac = (uint16_t)((2.0 * fr - 1.0) * 1024.0);
    return sign | (uint16_t)(exp_field << 10) | frac;
}

uint16_t orc_bf16_bits(float xf)
{
    double x = xf;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return sign | 0x7fc0;
    double r = round_to_format(fabs(x), 7, -126, -133);
    if (r > ldexp(255.0, 120))                      /* largest finite bf16 = (2 - 2^-7) 2^127 */
        return sign | 0x7f80;
    if (r < ldexp(1.0, -126))
        return sign | (uint16_t)(r / ldexp(1.0, -133));
    int e;
    double fr = frexp(r, &e);
    uint16_t exp_field = (uint16_t)(e - 1 + 127);
    uint16_t frac = (uint16_t)((2.0 * fr - 1.0) * 128.0);
    return sign | (uint16_t)(exp_field << 7) | frac;
}

static double value16(uint16_t bits, int is_bf16)
{
    return is_bf16 ? orc_bf16_value(bits) : orc_f16_value(bits);
}

void orc_value16_array(const uint16_t *bits, int is_bf16, double *out, uint64_t n)
{
    for (uint64_t i = 0; i < n; ++i)
        out[i] = value16(bits[i], is_bf16);
}

void orc_bits16_array(const float *x, int is_bf16, uint16_t *out, uint64_t n)
{
    for (uint64_t i = 0; i < n; ++i)
        out[i] = is_bf16 ? orc_bf16_bits(x[i]) : orc_f16_bits(x[i]);
}

/* ------------------------------------------------------------------------
 * Gradient statistics of one rank's shard: overflow flag (any non-finite
 * stored gradient) and the squared L2 norm of the gradients after division
 * by the loss scale.  The pages fix only that training is mixed precision
 * ([P2] memory accounting); unscale / overflow / norm follow the usual
 * mixed-precision recipe.  Sum: Neumaier-compensated fp64.
 * ---------------------------------------------------------------------- */
static void neumaier_add(double *s, double *c, double y)
{
    double t = *s + y;
    if (fabs(*s) >= fabs(y))
        *c += (*s - t) + y;
    else
        *c += (y - t) + *s;
    *s = t;
}

void orc_grad_stats(const uint16_t *g, int is_bf16, uint64_t n, double inv_scale,
                    double *sq_norm, uint32_t *overflow)
{
    int nt = omp_get_max_threads();
    double *ps = calloc((size_t)nt, sizeof(double));
    double *pc = calloc((size_t)nt, sizeof(double));
    uint32_t *pf = calloc((size_t)nt, sizeof(uint32_t));
#pragma omp parallel num_threads(nt)
    {
        int t = omp_get_thread_num(), T = omp_get_num_threads();
        uint64_t lo = (uint64_t)(((unsigned __int128)n * (unsigned)t) / (unsigned)T);
        uint64_t hi = (uint64_t)(((unsigned __int128)n * (unsigned)(t + 1)) / (unsigned)T);
        double s = 0.0, c = 0.0;
        uint32_t f = 0;
        for (uint64_t i = lo; i < hi; ++i) {
            double x = value16(g[i], is_bf16);
            if (!isfinite(x))
                f = 1;
            double u = x * inv_scale;
            neumaier_add(&s, &c, u * u);
        }
        ps[t] = s;
        pc[t] = c;
        pf[t] = f;
    }
    double s = 0.0, c = 0.0;
    uint32_t f = 0;
    for (int t = 0; t < nt; ++t) {
        neumaier_add(&s, &c, ps[t]);
        neumaier_add(&s, &c, pc[t]);
        f |= pf[t];
    }
    *sq_norm = s + c;
    *overflow = f;
    free(ps);
    free(pc);
    free(pf);
}

/* ------------------------------------------------------------------------
 * Per-step scalars.  Readings where the pages are silent:
 *  - a step whose gradients overflowed is skipped: nothing is written and
 *    the step counter does not advance;
 *  - gradient clipping by global norm c: coef = min(1, c / ||g||), off when
 *    c <= 0 or ||g|| = 0;
 *  - Adam bias corrections 1 - beta^t (Kingma & Ba).
 * ---------------------------------------------------------------------- */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay, max_grad_norm, inv_loss_scale;
} orc_hp;

typedef struct {
    uint64_t t;        /* step counter after this step */
    uint32_t skip;     /* 1: this step is skipped */
    uint32_t pad;
    double coef;       /* clip coefficient */
    double inv_scale;  /* 1 / loss scale */
    double bc1, bc2;   /* bias corrections 1 - beta1^t, 1 - beta2^t */
    double lr, beta1, beta2, eps, weight_decay;
} orc_scalars;

void orc_step_scalars(const orc_hp *hp, int have_stats, double sq_norm, uint32_t overflow,
                      uint64_t t_prev, orc_scalars *s)
{
    memset(s, 0, sizeof(*s));
    s->skip = (have_stats && overflow) ? 1u : 0u;
    s->t = s->skip ? t_prev : t_prev + 1;
    s->coef = 1.0;
    if (have_stats && !s->skip && hp->max_grad_norm > 0.0 && sq_norm > 0.0) {
        double norm = sqrt(sq_norm);
        if (hp->max_grad_norm < norm)
            s->coef = hp->max_grad_norm / norm;
    }
    s->inv_scale = hp->inv_loss_scale;
    s->bc1 = 1.0 - pow(hp->beta1, (double)s->t);
    s->bc2 = 1.0 - pow(hp->beta2, (double)s->t);
    s->lr = hp->lr;
    s->beta1 = hp->beta1;
    s->beta2 = hp->beta2;
    s->eps = hp->eps;
    s->weight_decay = hp->weight_decay;
}

/* ------------------------------------------------------------------------
 * AdamW on one element of the shard.  [P2] memory accounting names the five
 * arrays (fp16 param, fp16 grad, fp32 param copy, fp32 momentum, fp32
 * variance); [P2] ZeRO-DP Stage 1 has each rank update only its own part;
 * [P4] "显存背景" names AdamW with an fp32 master copy.  The update itself is
 * Adam (Kingma & Ba 2015) with decoupled weight decay (Loshchilov & Hutter
 * 2019), decay applied to the previous parameter value:
 *   g  = stored grad / loss scale * clip coef
 *   m' = b1 m + (1 - b1) g
 *   v' = b2 v + (1 - b2) g^2
 *   p' = p - lr wd p - lr (m'/bc1) / (sqrt(v'/bc2) + eps)
 * ---------------------------------------------------------------------- */
static void adamw_element(const orc_scalars *s, double graw, double p, double m, double v,
                          double *p_new, double *m_new, double *v_new)
{
    double g = graw * s->inv_scale * s->coef;
    double m1 = s->beta1 * m + (1.0 - s->beta1) * g;
    double v1 = s->beta2 * v + (1.0 - s->beta2) * g * g;
    double m_hat = m1 / s->bc1;
    double v_hat = v1 / s->bc2;
    *p_new = p - s->lr * s->weight_decay * p - s->lr * m_hat / (sqrt(v_hat) + s->eps);
    *m_new = m1;
    *v_new = v1;
}

/* In place on fp32 master/m/v; writes the 16-bit parameter rounded from the
 * new fp32 master.  Does nothing when the step is skipped. */
void orc_adamw(const orc_scalars *s, const uint16_t *g, int g_bf16, float *master, float *m,
               float *v, uint16_t *p16, int p_bf16, uint64_t n)
{
    if (s->skip)
        return;
#pragma omp parallel for schedule(static)
    for (uint64_t i = 0; i < n; ++i) {
        double pn, mn, vn;
        adamw_element(s, value16(g[i], g_bf16), master[i], m[i], v[i], &pn, &mn, &vn);
        master[i] = (float)pn;
        m[i] = (float)mn;
        v[i] = (float)vn;
        p16[i] = p_bf16 ? orc_bf16_bits(master[i]) : orc_f16_bits(master[i]);
    }
}

/* Same update with the fp64 results returned unrounded (for pin tests). */
void orc_adamw_f64(const orc_scalars *s, const uint16_t *g, int g_bf16, const float *master,
                   const float *m, const float *v, double *p_out, double *m_out, double *v_out,
                   uint64_t n)
{
    for (uint64_t i = 0; i < n; ++i)
        adamw_element(s, value16(g[i], g_bf16), master[i], m[i], v[i], &p_out[i], &m_out[i],
                      &v_out[i]);
}

/* ------------------------------------------------------------------------
 * Dynamic loss scaling.  [P2] "メモリ消費の定量化" trains in mixed precision
 * (fp16 params and grads, fp32 optimizer state) but says nothing about the loss
 * scale.  The rule taken is dynamic loss scaling as published in Micikevicius
 * et al., "Mixed Precision Training" (ICLR 2018), section on loss scaling: a
 * step whose scaled gradients overflow is skipped and the scale is reduced;
 * after a run of steps without overflow the scale is increased.  With the
 * usual parameters:
 *   overflow:  scale <- max(scale * backoff, min_scale); good <- 0
 *   otherwise: good <- good + 1; when good reaches the growth interval,
 *              scale <- min(scale * growth, max_scale) if that product is
 *              finite, and good <- 0.
 * The parameters are validated by the caller.
 * ---------------------------------------------------------------------- */
typedef struct {
    double init_scale, growth_factor, backoff_factor;
    uint64_t growth_interval;
    double min_scale, max_scale;
} orc_scaler;

typedef struct {
    double scale;
    double inv_scale;     /* 1 / scale */
    uint64_t good_steps;  /* steps without overflow since the last change */
    uint64_t overflows;   /* skipped steps so far */
} orc_scale_state;

void orc_loss_scale_init(const orc_scaler *c, orc_scale_state *s)
{
    s->scale = c->init_scale;
    s->inv_scale = 1.0 / c->init_scale;
    s->good_steps = 0;
    s->overflows = 0;
}

void orc_loss_scale_update(const orc_scaler *c, uint32_t overflow, orc_scale_state *s)
{
    if (overflow) {
        double reduced = s->scale * c->backoff_factor;
        s->scale = reduced > c->min_scale ? reduced : c->min_scale;
        s->good_steps = 0;
        s->overflows += 1;
    } else {
        s->good_steps += 1;
        if (s->good_steps == c->growth_interval) {
            double grown = s->scale * c->growth_factor;
            if (isfinite(grown))
                s->scale = grown < c->max_scale ? grown : c->max_scale;
            s->good_steps = 0;
        }
    }
    s->inv_scale = 1.0 / s->scale;
}

int orc_num_threads(void)
{
    return omp_get_max_threads();
}
