// Host-side planner of libzero_mi355x: status strings, thread-local error
// detail, shard partition, model-state accounting and the fused-bucket plan.
// Pure functions, no device access.
//
// Sources: "ZeRO: Memory Optimizations Toward Training Trillion Parameter
// Models" (paper summary page), sections ZeRO-DP (Stage 1/2/3 and the memory
// table), メモリ消費の定量化 (16 bytes per parameter) and ZeRO-R > CB; "ZeRO"
// (AI-library tutorial page), sections ZeRO-1/2/3.
#include "zero_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>

namespace zero {

static thread_local char g_last_error[512] = "";

zero_status fail(zero_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    int k = std::snprintf(g_last_error, sizeof g_last_error, "%s: ", zero_status_str(s));
    if (k < 0 || k >= (int)sizeof g_last_error)
        k = 0;
    std::vsnprintf(g_last_error + k, sizeof g_last_error - k, fmt, ap);
    va_end(ap);
    return s;
}

zero_status check_adamw(const zero_adamw &hp, bool host_inv_scale, const char *what)
{
    if (!(hp.lr >= 0.0 && std::isfinite(hp.lr)))
        return fail(ZERO_EINVAL, "%s: lr must be finite and >= 0", what);
    if (!(hp.beta1 >= 0.0 && hp.beta1 < 1.0) || !(hp.beta2 >= 0.0 && hp.beta2 < 1.0))
        return fail(ZERO_EINVAL, "%s: betas must be in [0, 1)", what);
    if (!(hp.eps > 0.0 && std::isfinite(hp.eps)))
        return fail(ZERO_EINVAL, "%s: eps must be finite and > 0", what);
    if (!(hp.weight_decay >= 0.0 && std::isfinite(hp.weight_decay)))
        return fail(ZERO_EINVAL, "%s: weight_decay must be finite and >= 0", what);
    if (host_inv_scale && !(std::isfinite(hp.inv_loss_scale) && hp.inv_loss_scale > 0.0))
        return fail(ZERO_EINVAL, "%s: inv_loss_scale must be finite and > 0", what);
    if (std::isnan(hp.max_grad_norm))
        return fail(ZERO_EINVAL, "%s: max_grad_norm is NaN", what);
    return ZERO_OK;
}

zero_status check_scaler(const zero_loss_scaler &c, const char *what)
{
    if (!(c.min_scale > 0.0 && std::isfinite(c.min_scale)))
        return fail(ZERO_EINVAL, "%s: min_scale must be finite and > 0", what);
    if (!(c.max_scale >= c.min_scale))  // +inf allowed, NaN rejected
        return fail(ZERO_EINVAL, "%s: max_scale must be >= min_scale", what);
    if (!(c.init_scale >= c.min_scale && c.init_scale <= c.max_scale &&
          std::isfinite(c.init_scale)))
        return fail(ZERO_EINVAL, "%s: init_scale must be finite and in [min_scale, max_scale]",
                    what);
    if (!(c.growth_factor >= 1.0 && std::isfinite(c.growth_factor)))
        return fail(ZERO_EINVAL, "%s: growth_factor must be finite and >= 1", what);
    if (!(c.backoff_factor > 0.0 && c.backoff_factor <= 1.0))
        return fail(ZERO_EINVAL, "%s: backoff_factor must be in (0, 1]", what);
    if (c.growth_interval == 0)
        return fail(ZERO_EINVAL, "%s: growth_interval must be >= 1", what);
    return ZERO_OK;
}

}  // namespace zero

using zero::fail;

extern "C" const char *zero_status_str(zero_status s)
{
    switch (s) {
    case ZERO_OK: return "ZERO_OK";
    case ZERO_EINVAL: return "ZERO_EINVAL";
    case ZERO_ENOSPC: return "ZERO_ENOSPC";
    case ZERO_EALIGN: return "ZERO_EALIGN";
    case ZERO_EDEVICE: return "ZERO_EDEVICE";
    case ZERO_EIO: return "ZERO_EIO";
    }
    return "ZERO_UNKNOWN";
}

extern "C" const char *zero_last_error(void) { return zero::g_last_error; }

// Balanced contiguous split: ranks below (psi mod nd) get one extra element,
// so rank r starts after r full-size parts plus min(r, psi mod nd) extras.
extern "C" zero_status zero_partition(uint64_t psi, uint32_t nd, uint32_t rank, uint64_t *begin,
                                      uint64_t *end)
{
    if (!begin || !end)
        return fail(ZERO_EINVAL, "zero_partition: NULL output pointer");
    if (nd == 0)
        return fail(ZERO_EINVAL, "zero_partition: nd must be >= 1");
    if (rank >= nd)
        return fail(ZERO_EINVAL, "zero_partition: rank %u >= nd %u", rank, nd);
    const uint64_t q = psi / nd, rem = psi % nd;
    const uint64_t lead = rank < rem ? rank : rem;
    *begin = q * rank + lead;  // <= psi, cannot overflow
    *end = *begin + q + (rank < rem ? 1 : 0);
    return ZERO_OK;
}

extern "C" zero_status zero_mem_bytes(uint32_t stage, uint64_t psi, uint32_t nd, uint32_t k,
                                      uint64_t *bytes)
{
    if (!bytes)
        return fail(ZERO_EINVAL, "zero_mem_bytes: NULL output pointer");
    if (stage > 3)
        return fail(ZERO_EINVAL, "zero_mem_bytes: stage %u > 3", stage);
    if (nd == 0)
        return fail(ZERO_EINVAL, "zero_mem_bytes: nd must be >= 1");
    const uint64_t shard = psi / nd + (psi % nd != 0);
    // Per-parameter byte counts of the three model-state kinds and whether
    // the stage shards them: params (2 B, stage 3), grads (2 B, stage >= 2),
    // optimizer state (k B, stage >= 1).
    const struct { uint64_t bpp; bool sharded; } kinds[3] = {
        {2, stage >= 3}, {2, stage >= 2}, {k, stage >= 1}};
    uint64_t total = 0;
    for (const auto &kd : kinds) {
        uint64_t term;
        if (__builtin_mul_overflow(kd.bpp, kd.sharded ? shard : psi, &term) ||
            __builtin_add_overflow(total, term, &total))
            return fail(ZERO_EINVAL, "zero_mem_bytes: result does not fit in 64 bits");
    }
    *bytes = total;
    return ZERO_OK;
}

extern "C" zero_status zero_bucket_plan(const uint64_t *numel, uint32_t n_tensors,
                                        uint64_t bucket_elems, uint64_t range_begin,
                                        uint64_t range_end, zero_segment *segs, uint64_t cap,
                                        uint64_t *n_segs)
{
    if (!n_segs)
        return fail(ZERO_EINVAL, "zero_bucket_plan: NULL n_segs");
    if (n_tensors > 0 && !numel)
        return fail(ZERO_EINVAL, "zero_bucket_plan: NULL numel");
    if (cap > 0 && !segs)
        return fail(ZERO_EINVAL, "zero_bucket_plan: NULL segs with cap > 0");
    if (bucket_elems == 0)
        return fail(ZERO_EINVAL, "zero_bucket_plan: bucket_elems must be >= 1");
    if (range_begin > range_end)
        return fail(ZERO_EINVAL, "zero_bucket_plan: range_begin > range_end");
    uint64_t psi = 0;
    for (uint32_t i = 0; i < n_tensors; ++i)
        if (__builtin_add_overflow(psi, numel[i], &psi))
            return fail(ZERO_EINVAL, "zero_bucket_plan: total size overflows 64 bits");
    if (range_end > psi)
        return fail(ZERO_EINVAL, "zero_bucket_plan: range_end %llu > psi %llu",
                    (unsigned long long)range_end, (unsigned long long)psi);

    // Walk the range once: at each position the piece ends at the nearest of
    // the current tensor's end, the current window's end and the range end.
    uint64_t count = 0, pos = range_begin, t_start = 0;
    uint32_t t = 0;
    while (pos < range_end) {
        while (t_start + numel[t] <= pos)  // skip tensors that end before pos
            t_start += numel[t++];
        const uint64_t bucket = pos / bucket_elems;
        uint64_t stop = t_start + numel[t];
        const uint64_t win_end = (bucket + 1 > UINT64_MAX / bucket_elems)
                                     ? UINT64_MAX : (bucket + 1) * bucket_elems;
        if (win_end < stop) stop = win_end;
        if (range_end < stop) stop = range_end;
        if (count < cap)
            segs[count] = zero_segment{bucket, t, pos - t_start, pos - range_begin, stop - pos};
        ++count;
        pos = stop;
    }
    *n_segs = count;
    if (count > cap)
        return fail(ZERO_ENOSPC, "zero_bucket_plan: %llu segments, capacity %llu",
                    (unsigned long long)count, (unsigned long long)cap);
    return ZERO_OK;
}

extern "C" zero_status zero_state_layout(uint64_t n, uint64_t pool_bytes, uint64_t offsets[5])
{
    if (!offsets)
        return fail(ZERO_EINVAL, "zero_state_layout: NULL offsets");
    if (n > (UINT64_MAX >> 5))
        return fail(ZERO_EINVAL, "zero_state_layout: n too large");
    constexpr uint64_t kAlign = 2ull << 20;  // 2 MiB
    const uint64_t need_tail = 2 * n + 16;   // the param array, plus room for its phase
    const uint64_t min_step = 4 * n + 16;    // the largest of the first four, plus phase
    uint64_t step = pool_bytes > need_tail ? (pool_bytes - need_tail) / 4 / kAlign * kAlign : 0;
    if (step < min_step)
        return fail(ZERO_ENOSPC, "zero_state_layout: a pool of %llu bytes cannot hold five "
                    "non-overlapping arrays of %llu elements (needs at least %llu)",
                    (unsigned long long)pool_bytes, (unsigned long long)n,
                    (unsigned long long)(4 * ((min_step + kAlign - 1) / kAlign * kAlign) +
                                         need_tail));
    for (int i = 0; i < 5; ++i)
        offsets[i] = (uint64_t)i * step;
    return ZERO_OK;
}
