// AdamW step with the optimizer state offloaded to host memory ("ZeRO"
// AI-library tutorial page, section "ZeRO-Offload 与 ZeRO-Infinity": optimizer
// state moved to CPU memory to lift the GPU memory limit, at the price of
// PCIe transfers; "ZeRO optimization" glossary page, section "Как работает":
// offloading to CPU memory).
//
// The fp32 master, momentum and variance live in host memory; the 16-bit
// gradients and parameters stay on the device.  One step:
//   1. the device scalar kernel advances the step state from the gradient
//      statistics (skip, clip coefficient, bias corrections), as on the GPU
//      path, and the state is copied to the host;
//   2. the shard is processed in chunks through two pinned staging slots:
//      the gradients of chunk k+1 are copied device -> host while the host
//      cores update chunk k, whose 16-bit parameters are then copied
//      host -> device.
// The host loop performs the same correctly rounded fp64 operations in the
// same order as the device kernel (multiply, add, divide, sqrt, none fused),
// with the same fp64 scalars, and the same roundings to fp32 and to 16 bits.
#include <hip/hip_runtime_api.h>
#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "zero_internal.h"

using zero::fail;

namespace {

constexpr uint64_t kMinChunk = 4096;  // elements per staging slot, at least

// Hyper-parameters (beta1, beta2, eps, lr as given; 1 - beta1, 1 - beta2 and
// lr * wd formed in fp64) and the step's scalars from the device state.
struct Coeffs {
    double b1, omb1, b2, omb2, eps, lr, lrwd, inv, coef, bc1, bc2, inv_bc1, inv_bc2;
};

// a / b from rb = RN(1 / b) and one fused correction, as the device does it
// (the correctly rounded quotient, by Markstein's theorem); a zero dividend
// as is where it may be -0.
template <bool SIGNED_ZERO>
inline double div_by(double a, double b, double rb)
{
    const double q0 = a * rb;
    const double q = std::fma(std::fma(-b, q0, a), rb, q0);
    return SIGNED_ZERO && a == 0.0 ? a : q;
}

inline float f16_to_f32(uint16_t h)
{
    _Float16 x;
    std::memcpy(&x, &h, 2);
    return (float)x;
}

inline uint16_t f32_to_f16(float f)
{
    const _Float16 x = (_Float16)f;  // IEEE conversion: round to nearest, ties to even
    uint16_t h;
    std::memcpy(&h, &x, 2);
    return h;
}

inline float bf16_to_f32(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

inline uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u)  // NaN stays a (quiet) NaN
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One thread's contiguous part of a chunk.
template <bool GBF16, bool PBF16>
__attribute__((always_inline)) inline void
adamw_body(const Coeffs k, const uint16_t *__restrict g16, float *__restrict th,
           float *__restrict m, float *__restrict v, uint16_t *__restrict p, uint64_t cnt)
{
    for (uint64_t i = 0; i < cnt; ++i) {
        const double g = ((double)(GBF16 ? bf16_to_f32(g16[i]) : f16_to_f32(g16[i])) * k.inv) *
                         k.coef;
        const double m1 = k.b1 * (double)m[i] + k.omb1 * g;
        const double v1 = k.b2 * (double)v[i] + (k.omb2 * g) * g;
        const double m_hat = div_by<true>(m1, k.bc1, k.inv_bc1);
        const double v_hat = div_by<false>(v1, k.bc2, k.inv_bc2);
        const double p0 = (double)th[i];
        const double p1 = (p0 - k.lrwd * p0) - (k.lr * m_hat) / (std::sqrt(v_hat) + k.eps);
        const float t = (float)p1;
        th[i] = t;
        m[i] = (float)m1;
        v[i] = (float)v1;
        p[i] = PBF16 ? f32_to_bf16(t) : f32_to_f16(t);
    }
}

// The body compiled for several x86 levels, picked at run time (AVX-512,
// AVX2 + FMA + F16C, baseline), once per gradient/param dtype pair.
#define ZERO_HOST_RANGE(NAME, GB, PB)                                                       \
    __attribute__((target_clones("arch=x86-64-v4", "arch=x86-64-v3", "default"))) void      \
    NAME(const Coeffs k, const uint16_t *g, float *th, float *m, float *v, uint16_t *p,     \
         uint64_t cnt)                                                                      \
    {                                                                                       \
        adamw_body<GB, PB>(k, g, th, m, v, p, cnt);                                         \
    }
ZERO_HOST_RANGE(adamw_range_hh, false, false)
ZERO_HOST_RANGE(adamw_range_hb, false, true)
ZERO_HOST_RANGE(adamw_range_bh, true, false)
ZERO_HOST_RANGE(adamw_range_bb, true, true)
#undef ZERO_HOST_RANGE

using RangeFn = void (*)(const Coeffs, const uint16_t *, float *, float *, float *, uint16_t *,
                         uint64_t);

void adamw_chunk(RangeFn fn, const Coeffs &k, const uint16_t *g, float *th, float *m, float *v,
                 uint16_t *p, uint64_t cnt)
{
#pragma omp parallel
    {
        const uint64_t T = (uint64_t)omp_get_num_threads(), t = (uint64_t)omp_get_thread_num();
        const uint64_t lo = cnt * t / T, hi = cnt * (t + 1) / T;
        if (hi > lo)
            fn(k, g + lo, th + lo, m + lo, v + lo, p + lo, hi - lo);
    }
}

zero_status hip_ok(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(ZERO_EDEVICE, "zero_offload_adam_step: %s: %s", what, hipGetErrorString(e));
    return ZERO_OK;
}

struct Events {
    hipEvent_t e[4] = {nullptr, nullptr, nullptr, nullptr};
    ~Events()
    {
        for (hipEvent_t x : e)
            if (x)
                (void)hipEventDestroy(x);
    }
};

}  // namespace

extern "C" zero_status zero_offload_staging_bytes(uint64_t chunk_elems, size_t *bytes)
{
    if (!bytes)
        return fail(ZERO_EINVAL, "zero_offload_staging_bytes: NULL output");
    if (chunk_elems < kMinChunk || chunk_elems > (UINT64_MAX >> 4))
        return fail(ZERO_EINVAL, "zero_offload_staging_bytes: chunk_elems must be >= %llu",
                    (unsigned long long)kMinChunk);
    *bytes = (size_t)(2 * chunk_elems * 4);  // two slots of 2-byte grads + 2-byte params
    return ZERO_OK;
}

extern "C" zero_status zero_offload_adam_step(const zero_adamw *hp, const void *grad,
                                              zero_dtype gdt, float *master_host,
                                              float *exp_avg_host, float *exp_avg_sq_host,
                                              void *param_out, zero_dtype pdt, uint64_t n,
                                              const zero_grad_stats_t *d_stats,
                                              const zero_loss_scale_t *d_scale,
                                              zero_adam_state_t *d_state, void *staging,
                                              size_t staging_bytes, void *stream)
{
    const char *what = "zero_offload_adam_step";
    if (!hp || !d_state)
        return fail(ZERO_EINVAL, "%s: NULL hyper-parameters or d_state", what);
    if ((gdt != ZERO_F16 && gdt != ZERO_BF16) || (pdt != ZERO_F16 && pdt != ZERO_BF16))
        return fail(ZERO_EINVAL, "%s: grad and param dtypes must be F16 or BF16", what);
    if (zero_status hs = zero::check_adamw(*hp, d_scale == nullptr, what); hs != ZERO_OK)
        return hs;
    if (n > 0 && (!grad || !master_host || !exp_avg_host || !exp_avg_sq_host || !param_out ||
                  !staging))
        return fail(ZERO_EINVAL, "%s: NULL array with n > 0", what);
    if (n > (UINT64_MAX >> 4))
        return fail(ZERO_EINVAL, "%s: n too large", what);
    const uint64_t chunk = staging_bytes / 8;  // elements per slot
    if (n > 0 && chunk < kMinChunk)
        return fail(ZERO_ENOSPC, "%s: staging of %zu bytes holds fewer than %llu elements per "
                    "slot", what, staging_bytes, (unsigned long long)kMinChunk);
    if (((uintptr_t)grad | (uintptr_t)param_out | (uintptr_t)staging) & 1u ||
        ((uintptr_t)master_host | (uintptr_t)exp_avg_host | (uintptr_t)exp_avg_sq_host) & 3u ||
        ((uintptr_t)d_state & 7u) || ((uintptr_t)d_stats & 7u) || ((uintptr_t)d_scale & 7u))
        return fail(ZERO_EALIGN, "%s: misaligned pointer", what);
    {
        const uintptr_t host[4] = {(uintptr_t)master_host, (uintptr_t)exp_avg_host,
                                   (uintptr_t)exp_avg_sq_host, (uintptr_t)staging};
        const uint64_t len[4] = {4 * n, 4 * n, 4 * n, staging_bytes};
        for (int i = 0; i < 4; ++i)
            for (int j = i + 1; j < 4; ++j)
                if (len[i] && len[j] && host[i] < host[j] + len[j] && host[j] < host[i] + len[i])
                    return fail(ZERO_EINVAL, "%s: host buffers %d and %d overlap", what, i, j);
        const uintptr_t dev[5] = {(uintptr_t)grad, (uintptr_t)param_out, (uintptr_t)d_state,
                                  (uintptr_t)d_stats, (uintptr_t)d_scale};
        const uint64_t dlen[5] = {2 * n, 2 * n, sizeof(zero_adam_state_t),
                                  d_stats ? sizeof(zero_grad_stats_t) : 0,
                                  d_scale ? sizeof(zero_loss_scale_t) : 0};
        for (int i = 0; i < 5; ++i)
            for (int j = i + 1; j < 5; ++j)
                if (dlen[i] && dlen[j] && dev[i] < dev[j] + dlen[j] && dev[j] < dev[i] + dlen[i])
                    return fail(ZERO_EINVAL, "%s: device buffers %d and %d overlap", what, i, j);
    }
    hipStream_t s = (hipStream_t)stream;

    // 1. scalars on the device, as on the GPU path, then to the host
    zero_status st = zero::launch_adam_scalars(*hp, d_stats, d_scale, d_state, stream);
    if (st != ZERO_OK)
        return st;
    zero_adam_state_t hs;
    if ((st = hip_ok(hipMemcpyAsync(&hs, d_state, sizeof hs, hipMemcpyDeviceToHost, s),
                     "reading the step state")) != ZERO_OK ||
        (st = hip_ok(hipStreamSynchronize(s), "stream")) != ZERO_OK)
        return st;
    if (hs.skip || n == 0)
        return ZERO_OK;
    const Coeffs k{hp->beta1, 1.0 - hp->beta1, hp->beta2, 1.0 - hp->beta2, hp->eps, hp->lr,
                   hp->lr * hp->weight_decay, hs.inv_scale, hs.coef, hs.bc1, hs.bc2,
                   hs.inv_bc1, hs.inv_bc2};
    const bool gb = gdt == ZERO_BF16, pb = pdt == ZERO_BF16;
    const RangeFn fn = gb ? (pb ? adamw_range_bb : adamw_range_bh)
                          : (pb ? adamw_range_hb : adamw_range_hh);

    // 2. chunks through two staging slots: slot i holds chunk grads then params.
    // Once a copy is queued, an error still drains the stream before returning,
    // so no transfer into or out of `staging` outlives the call.
    auto drain = [s](zero_status r) {
        (void)hipStreamSynchronize(s);
        return r;
    };
    uint16_t *slot_g[2] = {(uint16_t *)staging, (uint16_t *)staging + chunk};
    uint16_t *slot_p[2] = {(uint16_t *)staging + 2 * chunk, (uint16_t *)staging + 3 * chunk};
    Events ev;  // e[0..1]: grads of a slot arrived; e[2..3]: params of a slot sent
    for (int i = 0; i < 4; ++i)
        if ((st = hip_ok(hipEventCreateWithFlags(&ev.e[i], hipEventDisableTiming),
                         "event")) != ZERO_OK)
            return st;
    const uint16_t *gd = (const uint16_t *)grad;
    uint16_t *pd = (uint16_t *)param_out;
    const uint64_t n_chunks = (n + chunk - 1) / chunk;
    auto fetch = [&](uint64_t c) -> zero_status {
        const uint64_t lo = c * chunk, cnt = std::min(chunk, n - lo);
        zero_status r = hip_ok(hipMemcpyAsync(slot_g[c % 2], gd + lo, 2 * cnt,
                                              hipMemcpyDeviceToHost, s), "grad copy");
        return r != ZERO_OK ? r : hip_ok(hipEventRecord(ev.e[c % 2], s), "event");
    };
    if ((st = fetch(0)) != ZERO_OK)
        return drain(st);
    for (uint64_t c = 0; c < n_chunks; ++c) {
        if (c + 1 < n_chunks && (st = fetch(c + 1)) != ZERO_OK)
            return drain(st);
        const int slot = (int)(c % 2);
        if ((st = hip_ok(hipEventSynchronize(ev.e[slot]), "grad copy")) != ZERO_OK)
            return drain(st);
        if (c >= 2 && (st = hip_ok(hipEventSynchronize(ev.e[2 + slot]), "param copy")) != ZERO_OK)
            return drain(st);
        const uint64_t lo = c * chunk, cnt = std::min(chunk, n - lo);
        adamw_chunk(fn, k, slot_g[slot], master_host + lo, exp_avg_host + lo,
                    exp_avg_sq_host + lo, slot_p[slot], cnt);
        if ((st = hip_ok(hipMemcpyAsync(pd + lo, slot_p[slot], 2 * cnt, hipMemcpyHostToDevice, s),
                         "param copy")) != ZERO_OK ||
            (st = hip_ok(hipEventRecord(ev.e[2 + slot], s), "event")) != ZERO_OK)
            return drain(st);
    }
    return hip_ok(hipStreamSynchronize(s), "stream");
}
