/*
 * zero.h - C ABI of libzero_mi355x: one data-parallel rank's shard-local
 * mixed-precision AdamW step of ZeRO-DP (P_os / P_os+g), for AMD MI355X
 * (gfx950).
 *
 * Sources (web pages on ZeRO):
 *  [P2] "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models"
 *       (paper summary page): section 問題設定 > メモリ消費の定量化 (the five
 *       model-state arrays of mixed-precision Adam, 16 bytes per parameter),
 *       section 提案手法 > ZeRO-DP (Stage 1 P_os, Stage 2 P_os+g, Stage 3
 *       P_os+g+p, and the memory table), section ZeRO-R > CB (constant-size
 *       fused buffers), section 考察 (optimizer state is needed only at the
 *       end of the step).
 *  [P4] "ZeRO" (AI-library tutorial page): section 显存背景 (bf16/fp16 +
 *       AdamW + fp32 master = 16 bytes per parameter) and sections
 *       ZeRO-1 / ZeRO-2 / ZeRO-3 (per-stage memory equations).
 *
 * Conventions shared by every call:
 *  - Every call returns a zero_status; ZERO_OK is 0.  Nothing is thrown
 *    across the ABI.  After a failure, zero_last_error() returns a
 *    thread-local, NUL-terminated description of it.
 *  - The caller owns all memory.  The library never allocates device memory;
 *    the workspace size of zero_grad_stats comes from a query call.
 *  - Device calls are asynchronous and ordered on the caller's HIP stream,
 *    passed as `void *stream` (a hipStream_t; NULL is the null stream).  They
 *    never synchronise and never read device data on the host, except the
 *    calls that move data between device and host by design and say so:
 *    zero_offload_adam_step, zero_ckpt_save and zero_ckpt_load.  Argument
 *    checks happen on the host before any launch; a launch failure reported
 *    by the runtime returns ZERO_EDEVICE.
 *  - Device pointers are plain device addresses (e.g. a torch tensor's
 *    data_ptr()).  Counts and offsets are 64-bit element counts.
 *  - 16-bit buffers need 2-byte alignment and fp32 buffers 4-byte alignment;
 *    any other offset ("phase") inside a 16-byte line is legal and handled.
 *  - Output buffers must not overlap input buffers (ZERO_EINVAL), except for
 *    the documented in-place arrays.
 */
#ifndef ZERO_MI355X_H
#define ZERO_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ZERO_OK = 0,
    ZERO_EINVAL = 1, /* an argument is out of its domain */
    ZERO_ENOSPC = 2, /* a caller-provided capacity (segments, workspace) is too small */
    ZERO_EALIGN = 3, /* a pointer is not aligned to its element size */
    ZERO_EDEVICE = 4, /* the HIP runtime reported an error for a launch or copy */
    ZERO_EIO = 5      /* a checkpoint file could not be created, read or written */
} zero_status;

typedef enum { ZERO_F32 = 0, ZERO_F16 = 1, ZERO_BF16 = 2 } zero_dtype;

/* Static name of a status code. */
const char *zero_status_str(zero_status s);

/* Thread-local detail of the last failing call made by this thread ("" if
 * none).  The string stays valid until the next failing call on the thread. */
const char *zero_last_error(void);

/* ---------------------------------------------------------------- planner
 * Host-only, pure functions: no device access. */

/* [P2] ZeRO-DP, Stage 1: the flat vector of psi parameters is cut into nd
 * parts and each data-parallel rank keeps and updates only its own part.
 * Rank `rank` owns the contiguous range [*begin, *end).  When nd does not
 * divide psi, the parts differ in size by at most one element and the first
 * (psi mod nd) ranks hold the larger size; the ranges tile [0, psi) with no
 * padding.  Errors: ZERO_EINVAL if nd == 0, rank >= nd or an output pointer
 * is NULL. */
zero_status zero_partition(uint64_t psi, uint32_t nd, uint32_t rank, uint64_t *begin,
                           uint64_t *end);

/* [P2] memory accounting and the ZeRO-DP table; [P4] ZeRO-1/2/3 equations.
 * Model-state bytes held by the busiest rank: 2 bytes of 16-bit params,
 * 2 bytes of 16-bit grads and k bytes of optimizer state per parameter
 * (k = 12 for mixed-precision Adam: fp32 master, momentum, variance).
 *   stage 0 (plain DP):  (4 + k) psi
 *   stage 1 (P_os):      4 psi + k S
 *   stage 2 (P_os+g):    2 psi + (2 + k) S
 *   stage 3 (P_os+g+p):  (4 + k) S
 * with S = ceil(psi / nd), the largest part.  Activations, communication
 * buffers and allocator overhead are not model states and are not counted.
 * Errors: ZERO_EINVAL if stage > 3, nd == 0, bytes is NULL or the result
 * does not fit in 64 bits. */
zero_status zero_mem_bytes(uint32_t stage, uint64_t psi, uint32_t nd, uint32_t k,
                           uint64_t *bytes);

/* One piece of the bucket layout: elements [src_off, src_off + len) of
 * tensor `tensor` land at [dst_off, dst_off + len) of a buffer that holds
 * the planned range; the piece lies inside bucket window `bucket`. */
typedef struct {
    uint64_t bucket, tensor, src_off, dst_off, len;
} zero_segment;

/* [P2] ZeRO-R, CB: gradients are gathered into fused buffers of a constant
 * size instead of model-sized temporaries.  The n_tensors tensors (element
 * counts numel[]) are laid end to end in list order, without padding, into a
 * flat stream of psi = sum(numel) elements, and the stream is cut into
 * windows of bucket_elems elements (bucket b = [b*bucket_elems,
 * min((b+1)*bucket_elems, psi)); a tensor may straddle two windows).  The
 * plan lists, in flat order, every non-empty intersection of a tensor with a
 * window and with [range_begin, range_end); dst_off counts from range_begin.
 * Writes at most `cap` segments to segs (segs may be NULL when cap == 0) and
 * always stores the full count in *n_segs.  Errors: ZERO_EINVAL for
 * bucket_elems == 0, range_begin > range_end, range_end > psi, a NULL numel
 * with n_tensors > 0, or a NULL n_segs; ZERO_ENOSPC if cap < *n_segs (the
 * first cap segments are still written). */
zero_status zero_bucket_plan(const uint64_t *numel, uint32_t n_tensors, uint64_t bucket_elems,
                             uint64_t range_begin, uint64_t range_end, zero_segment *segs,
                             uint64_t cap, uint64_t *n_segs);

/* Where to put one rank's five state arrays inside one caller-allocated
 * device pool of pool_bytes bytes, for bandwidth.  The arrays are, in this
 * order: grad (n 16-bit values), master, exp_avg, exp_avg_sq (n fp32 each),
 * param (n 16-bit values).  ([P2] ZeRO-R, MD: model states go to
 * pre-allocated contiguous regions.  The pages say nothing about where in
 * HBM; the layout is this library's.)  On MI355X, AdamW streams the five
 * arrays at once and runs faster when they lie far apart in HBM: measured on
 * the 1.5B shard, 5.5-6.1 TB/s with separate allocations (depending on where
 * the allocator's pages fall) against 6.2 TB/s spread over a 200 GiB pool.
 * The arrays are therefore spread evenly: offsets[i] = i * step, with step a
 * multiple of 2 MiB and 4 * step + 2n + 16 <= pool_bytes, so every array may
 * also be shifted by up to 16 bytes (a 16-bit shard's phase in its flat
 * buffer).
 * The rest of the pool stays the caller's: other buffers placed in the gaps
 * (per-tensor gradients, say) leave the step's speed unchanged.
 * Errors: ZERO_EINVAL (NULL offsets, n too large), ZERO_ENOSPC (the pool is
 * too small for non-overlapping arrays: step < 4n + 16). */
zero_status zero_state_layout(uint64_t n, uint64_t pool_bytes, uint64_t offsets[5]);

/* ------------------------------------------------------------ device calls */

/* [P2] ZeRO-R, CB and MD: copies elements [range_begin, range_begin + count)
 * of the list-order flat stream of the tensors into the contiguous device
 * buffer dst (count elements of type dt), bit for bit.  With bucket size B,
 * bucket b is range_begin = b*B, count = min(B, psi - b*B); a rank's part of
 * the stream is range_begin = begin, count = end - begin.
 * tensor_ptrs (host array of n_tensors device pointers) and numel (host
 * array) describe the tensors; a pointer may be NULL only for a tensor that
 * does not intersect the range.  dst bytes beyond count are not written.
 * Errors: ZERO_EINVAL (dt not F32/F16/BF16, range beyond the stream, NULL
 * pointers, dst overlapping an intersecting source), ZERO_EALIGN (a pointer
 * not aligned to the element size), ZERO_EDEVICE.  count == 0 is a no-op. */
zero_status zero_bucket_flatten(const void *const *tensor_ptrs, const uint64_t *numel,
                                uint32_t n_tensors, zero_dtype dt, uint64_t range_begin,
                                uint64_t count, void *dst, void *stream);

/* Device-resident result of zero_grad_stats (16 bytes, 8-byte aligned). */
typedef struct {
    double sq_norm;    /* sum over the shard of (g / loss_scale)^2 */
    uint32_t overflow; /* 1 if any stored gradient is inf or NaN, else 0 */
    uint32_t pad;
} zero_grad_stats_t;

/* Dynamic loss scaling.  [P2] memory accounting trains in mixed fp16/fp32
 * precision; the pages do not describe the loss scale.  The rule is dynamic
 * loss scaling as published with mixed-precision training (Micikevicius et
 * al., "Mixed Precision Training", ICLR 2018): a step whose scaled gradients
 * overflow is skipped and the scale backs off; after growth_interval steps in
 * a row without overflow it grows.
 * Host-side parameters (fp64): */
typedef struct {
    double init_scale;       /* starting scale, in [min_scale, max_scale] */
    double growth_factor;    /* >= 1, finite */
    double backoff_factor;   /* in (0, 1] */
    uint64_t growth_interval; /* >= 1 */
    double min_scale;        /* > 0, finite: floor of the backoff */
    double max_scale;        /* >= min_scale, may be +inf: cap of the growth */
} zero_loss_scaler;

/* Device-resident loss-scale state (32 bytes, 8-byte aligned), written by
 * zero_loss_scale_init and zero_loss_scale_update.  The calls that unscale
 * gradients accept it in place of a host inv_loss_scale, so that the scale
 * never has to be read on the host. */
typedef struct {
    double scale;        /* the loss scale the next backward multiplies by */
    double inv_scale;    /* 1 / scale, in fp64 */
    uint64_t good_steps; /* steps without overflow since the scale last changed */
    uint64_t overflows;  /* steps skipped so far */
} zero_loss_scale_t;

/* Bytes of device workspace that zero_grad_stats needs for n gradients. */
zero_status zero_grad_stats_workspace(uint64_t n, size_t *bytes);

/* Mixed-precision gradient statistics of one rank's gradient shard ([P2]
 * memory accounting: fp16 gradients of mixed-precision training; [P2]
 * ZeRO-DP Stage 2: each rank holds only its part of the gradients).  Reads
 * n 16-bit gradients (gdt F16 or BF16, stored multiplied by the loss
 * scale), and writes *d_stats (device memory) with the overflow flag (any
 * non-finite element) and the squared L2 norm of g * inv, where inv is
 * d_scale->inv_scale read on the device when d_scale is not NULL, else the
 * host value inv_loss_scale (then ignored when d_scale is given); the norm is
 * accumulated in fp64 in a fixed order (bit-reproducible for a given n and
 * 16-byte phase of grad, and equal for the two ways of giving the same inv).
 * sq_norm is unspecified when overflow is set.
 * n == 0 writes {0, 0}.
 * Multi-rank callers sum sq_norm and take the max of overflow across ranks
 * on the same stream before zero_adam_step.
 * workspace: device memory of at least zero_grad_stats_workspace(n) bytes,
 * 16-byte aligned; its contents are scratch.  Errors: ZERO_EINVAL (NULL
 * grad with n > 0, NULL d_stats, bad dtype, no d_scale and inv_loss_scale
 * not finite and positive, overlapping buffers), ZERO_ENOSPC (workspace too
 * small), ZERO_EALIGN, ZERO_EDEVICE. */
zero_status zero_grad_stats(const void *grad, zero_dtype gdt, uint64_t n, double inv_loss_scale,
                            const zero_loss_scale_t *d_scale, void *workspace, size_t ws_bytes,
                            zero_grad_stats_t *d_stats, void *stream);

/* zero_grad_stats without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * checks, errors and results as zero_grad_stats (overflow bit-exact; sq_norm
 * in fp64, summed in a fixed order that depends only on n and grad's 16-byte
 * phase, equal to zero_grad_stats's up to that order), except that the
 * per-block partial sums live in the library's own device scratch: a static
 * 64 KiB array (8192 fp64 partials) that every GPU the library runs on holds
 * until the process ends.  The first pass folds the tiles of any n into at
 * most 8192 partials, so no n is too large for the scratch (n is limited as
 * for zero_grad_stats).  Each partial is written before it is read, so the
 * scratch needs no clearing; but every call on one GPU shares that GPU's
 * scratch, so calls that overlap in time on one GPU (on different streams,
 * or from different threads without ordering) race and may return wrong
 * statistics.  The first call on a device looks the scratch up with
 * hipGetSymbolAddress (no allocation).  `stream` must belong to the current
 * device, whose scratch the call uses.  Errors: as zero_grad_stats
 * (ZERO_EINVAL, ZERO_EALIGN); ZERO_EINVAL also for a stream of another device;
 * ZERO_EDEVICE when there is no current device or the lookup fails. */
zero_status zero_grad_stats_noalloc(const void *grad, zero_dtype gdt, uint64_t n,
                                    double inv_loss_scale, const zero_loss_scale_t *d_scale,
                                    zero_grad_stats_t *d_stats, void *stream);

/* Bytes of device workspace that zero_bucket_flatten_stats needs for the
 * elements [range_begin, range_begin + count) of the tensors numel[]. */
zero_status zero_bucket_flatten_stats_workspace(const uint64_t *numel, uint32_t n_tensors,
                                                uint64_t range_begin, uint64_t count,
                                                size_t *bytes);

/* zero_bucket_flatten fused with zero_grad_stats: gathers the elements
 * [range_begin, range_begin + count) of the list-order flat stream of 16-bit
 * gradient tensors into dst ([P2] ZeRO-R, CB) and, in the same pass, writes
 * *d_stats for the gathered values exactly as zero_grad_stats would for dst
 * (overflow flag; squared L2 norm of g * inv in fp64, with inv taken from
 * d_scale or inv_loss_scale as for zero_grad_stats, summed in a
 * fixed order that depends only on the tensor sizes, the range and dst's
 * 16-byte phase).  Each gradient is read from HBM once instead of twice.  For
 * callers whose gathered range is the rank's final gradient shard: a single
 * data-parallel rank, or gradients already reduced into the per-tensor
 * buffers.  gdt: F16 or BF16.  workspace: device memory of at least
 * zero_bucket_flatten_stats_workspace(...) bytes, 16-byte aligned.
 * count == 0 writes {0, 0}.  Errors: as zero_bucket_flatten and
 * zero_grad_stats (ZERO_EINVAL, ZERO_ENOSPC, ZERO_EALIGN, ZERO_EDEVICE). */
zero_status zero_bucket_flatten_stats(const void *const *tensor_ptrs, const uint64_t *numel,
                                      uint32_t n_tensors, zero_dtype gdt, uint64_t range_begin,
                                      uint64_t count, void *dst, double inv_loss_scale,
                                      const zero_loss_scale_t *d_scale, void *workspace,
                                      size_t ws_bytes, zero_grad_stats_t *d_stats, void *stream);

/* AdamW hyper-parameters (host memory, fp64). */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    double max_grad_norm;  /* clip by global norm; <= 0 disables clipping */
    double inv_loss_scale; /* 1 / loss scale applied to the stored gradients
                            * (ignored when a device loss-scale state is given) */
} zero_adamw;

/* Device-resident step state (64 bytes, 8-byte aligned).  The caller
 * zero-initialises it once; zero_adam_step then advances `step` and fills the
 * per-step fp64 scalars that its element kernel reads. */
typedef struct {
    uint64_t step;     /* number of steps taken (not advanced by skipped steps) */
    uint32_t skip;     /* 1 if the last call skipped (overflow) */
    uint32_t pad0;
    double coef;       /* clip coefficient of the last step */
    double inv_scale;  /* inverse loss scale the last step unscaled its gradients by */
    double bc1;        /* 1 - beta1^t of the last step */
    double bc2;        /* 1 - beta2^t of the last step */
    double inv_bc1;    /* 1 / bc1, correctly rounded */
    double inv_bc2;    /* 1 / bc2, correctly rounded */
} zero_adam_state_t;

/* [P2] ZeRO-DP Stage 1/2: each rank updates only its own part of the
 * optimizer state, once, at the end of the step ([P2] 考察); [P2] memory
 * accounting fixes the arrays: 16-bit params and grads, fp32 master,
 * momentum and variance; [P4] 显存背景 names the optimizer AdamW.
 * For every element i < n of the shard, in fp64 arithmetic on the stored
 * values, in this order:
 *   g  = (grad[i] * inv) * coef
 *   m  = beta1 m + (1 - beta1) g;   v = beta2 v + ((1 - beta2) g) g
 *   master = (master - (lr wd) master) -
 *            (lr (m / bc1)) / (sqrt(v / bc2) + eps)
 * with bc1 = 1 - beta1^t and bc2 = 1 - beta2^t (the two quotients by them
 * are formed from their correctly rounded reciprocals with one fused
 * correction, which gives the correctly rounded quotient: Markstein's
 * theorem); m, v and master are then stored rounded once to fp32 (nearest,
 * ties to even), and
 *   param_out[i] = the stored fp32 master rounded to pdt (nearest, ties to even)
 * with t the advanced step count, coef = min(1, max_grad_norm / ||g||)
 * (1 when clipping is off or d_stats is NULL), computed in fp64 on the
 * device from *d_stats, and inv = d_scale->inv_scale (read on the device)
 * when d_scale is not NULL, else hp->inv_loss_scale.  Every operation is
 * an IEEE fp64 operation, correctly rounded, none fused, so the results are
 * those of evaluating the lines above in fp64 as written.  With dynamic loss
 * scaling, call zero_loss_scale_update after this call, on the same stream,
 * so that the step uses the scale its gradients were computed with.  If
 * d_stats reports overflow, the step is skipped: nothing is written to the
 * arrays and `step` does not advance.
 * grad: n 16-bit gradients (gdt); master, exp_avg, exp_avg_sq: n fp32 each,
 * updated in place; param_out: n 16-bit params (pdt), written.  Any 16-bit
 * or fp32 position within 16 bytes is handled; when master, exp_avg and
 * exp_avg_sq do not share their position the update runs element by element,
 * about 15% slower (8.27 against 7.05 ms on 1.56e9 parameters).  d_stats:
 * device result of zero_grad_stats (or NULL: no clipping, never skip);
 * d_state: device step state.  n == 0 still advances d_state.
 * Occupancy: every block of the update reserves 48 KiB of LDS that it does
 * not use, so that at most three blocks run per CU (of gfx950's 160 KiB);
 * kernels that run beside it on other streams share the remaining LDS.
 * Errors: ZERO_EINVAL (NULL hp or d_state, NULL arrays with n > 0, bad
 * dtypes, lr < 0, beta outside [0, 1), eps <= 0, weight_decay < 0, no
 * d_scale and inv_loss_scale not finite and positive, NaN max_grad_norm,
 * overlapping arrays), ZERO_EALIGN, ZERO_EDEVICE. */
zero_status zero_adam_step(const zero_adamw *hp, const void *grad, zero_dtype gdt, float *master,
                           float *exp_avg, float *exp_avg_sq, void *param_out, zero_dtype pdt,
                           uint64_t n, const zero_grad_stats_t *d_stats,
                           const zero_loss_scale_t *d_scale, zero_adam_state_t *d_state,
                           void *stream);

/* ---------------------------------------- the step read from tensor lists
 * For a rank whose per-tensor gradient buffers already hold its final
 * gradients (one data-parallel rank, or gradients reduced in place), the
 * gathered flat gradient shard is written only to be read back.  [P2] ZeRO-R,
 * CB: the fused buffers bound temporary memory; these two calls need none,
 * and the step moves 30 bytes per parameter (statistics 2 + AdamW 28)
 * instead of 32 (gather with statistics 4 + AdamW 28). */

/* zero_grad_stats over elements [range_begin, range_begin + count) of the
 * list-order flat stream of the 16-bit gradient tensors (described as for
 * zero_bucket_flatten), read in place: nothing is written but *d_stats.  The
 * result equals, bit for bit, what zero_bucket_flatten_stats writes for the
 * same range into a 16-byte aligned dst.  workspace: at least
 * zero_bucket_flatten_stats_workspace(numel, n_tensors, range_begin, count)
 * bytes, 16-byte aligned.  count == 0 writes {0, 0}.  Errors: as
 * zero_bucket_flatten_stats (ZERO_EINVAL, ZERO_ENOSPC, ZERO_EALIGN,
 * ZERO_EDEVICE); the tensors must not overlap workspace, d_stats or d_scale. */
zero_status zero_grad_stats_tensors(const void *const *tensor_ptrs, const uint64_t *numel,
                                    uint32_t n_tensors, zero_dtype gdt, uint64_t range_begin,
                                    uint64_t count, double inv_loss_scale,
                                    const zero_loss_scale_t *d_scale, void *workspace,
                                    size_t ws_bytes, zero_grad_stats_t *d_stats, void *stream);

/* zero_adam_step with its gradients read in place from the tensors: element i
 * (i < count) of master, exp_avg, exp_avg_sq and param_out is updated with
 * the gradient at position range_begin + i of the tensors' list-order flat
 * stream (tensors described as for zero_bucket_flatten, gdt F16 or BF16).
 * The arithmetic, the step state, clipping, skipping and every result are
 * those of zero_adam_step on the gathered gradients, bit for bit.  master,
 * exp_avg and exp_avg_sq must lie at the same position within 16 bytes
 * (ZERO_EALIGN otherwise); param_out may lie anywhere 2-byte aligned.
 * count == 0 still advances d_state.  The tensors must not overlap any
 * output.  Errors: as zero_adam_step and zero_bucket_flatten (ZERO_EINVAL,
 * ZERO_EALIGN, ZERO_EDEVICE); arguments are checked before anything runs. */
zero_status zero_adam_step_tensors(const zero_adamw *hp, const void *const *tensor_ptrs,
                                   const uint64_t *numel, uint32_t n_tensors, zero_dtype gdt,
                                   uint64_t range_begin, uint64_t count, float *master,
                                   float *exp_avg, float *exp_avg_sq, void *param_out,
                                   zero_dtype pdt, const zero_grad_stats_t *d_stats,
                                   const zero_loss_scale_t *d_scale, zero_adam_state_t *d_state,
                                   void *stream);

/* Sets *d_scale (device) to {cfg->init_scale, 1 / init_scale, 0, 0} with a
 * one-thread kernel, ordered on `stream`.  Errors: ZERO_EINVAL (NULL
 * arguments, parameters outside the domains above), ZERO_EALIGN,
 * ZERO_EDEVICE. */
zero_status zero_loss_scale_init(const zero_loss_scaler *cfg, zero_loss_scale_t *d_scale,
                                 void *stream);

/* Advances *d_scale after a step from that step's *d_stats, on the device:
 *   overflow:  scale = max(scale * backoff_factor, min_scale), good_steps = 0,
 *              overflows += 1 (the step itself was skipped);
 *   otherwise: good_steps += 1; when it reaches growth_interval,
 *              scale = min(scale * growth_factor, max_scale) if that product
 *              is finite, and good_steps = 0;
 * then inv_scale = 1 / scale (fp64).  Errors: ZERO_EINVAL (NULL arguments,
 * parameters outside their domains, overlapping d_stats and d_scale),
 * ZERO_EALIGN, ZERO_EDEVICE. */
zero_status zero_loss_scale_update(const zero_loss_scaler *cfg, const zero_grad_stats_t *d_stats,
                                   zero_loss_scale_t *d_scale, void *stream);

/* --------------------------------------------- optimizer state in host memory */

/* Bytes of pinned host staging that zero_offload_adam_step needs to move
 * chunk_elems gradients and parameters per chunk (two slots; chunk_elems >=
 * 4096). */
zero_status zero_offload_staging_bytes(uint64_t chunk_elems, size_t *bytes);

/* ("ZeRO" AI-library tutorial page, section "ZeRO-Offload 与 ZeRO-Infinity":
 * optimizer state moved to CPU memory to lift the GPU memory limit, at the
 * cost of PCIe transfers; "ZeRO optimization" glossary page, section
 * "Как работает": offloading to CPU memory.)  The same update as
 * zero_adam_step, with the fp32 master, exp_avg and exp_avg_sq in HOST memory
 * (n elements each, updated in place by host threads) while the 16-bit grad
 * and param_out stay on the device.  The step state d_state and the optional
 * statistics d_stats and loss-scale state d_scale are device-resident, as
 * for zero_adam_step, and the skip, clip and bias corrections are computed
 * the same way.  The gradients
 * travel device -> host and the new 16-bit params host -> device in chunks
 * of staging_bytes / 8 elements through `staging`, caller-owned pinned host
 * memory (e.g. from hipHostMalloc), two slots deep so that transfers overlap
 * the host update.  The host loop evaluates the update with the device
 * kernel's fp64 operations in the same order, so its results equal the
 * device's bit for bit.  Synchronous: returns after the params have
 * reached the device (or at once when the step is skipped).
 * Errors: as zero_adam_step; ZERO_ENOSPC if staging holds fewer than 4096
 * elements per slot. */
zero_status zero_offload_adam_step(const zero_adamw *hp, const void *grad, zero_dtype gdt,
                                   float *master_host, float *exp_avg_host,
                                   float *exp_avg_sq_host, void *param_out, zero_dtype pdt,
                                   uint64_t n, const zero_grad_stats_t *d_stats,
                                   const zero_loss_scale_t *d_scale, zero_adam_state_t *d_state,
                                   void *staging, size_t staging_bytes, void *stream);

/* ------------------------------------------------------ sharded checkpoints */

/* Header of one rank's checkpoint file (64 bytes, little-endian). */
typedef struct {
    char magic[8];     /* "ZEROCKPT" */
    uint32_t version;  /* 1 */
    uint32_t nd;       /* ranks of the saved run */
    uint32_t rank;     /* this file's rank */
    uint32_t pad;
    uint64_t psi;      /* flat parameter count of the model */
    uint64_t begin;    /* this rank's range [begin, end) of the flat vector */
    uint64_t end;
    uint64_t step;     /* device step counter when saved */
    uint64_t flags;    /* bit 0: a 32-byte zero_loss_scale_t follows the arrays */
} zero_ckpt_header;

/* ("ZeRO" AI-library tutorial page, section "Checkpoint 与恢复": with sharded
 * checkpoints each rank writes only the state it is responsible for, and the
 * files carry the metadata a resume needs.)  Writes rank `rank`'s optimizer
 * state of a psi-parameter model split over nd ranks to `path`: the header,
 * then the n = end - begin fp32 master, exp_avg and exp_avg_sq values
 * (device arrays of the rank's shard, in that order), then, when d_scale is
 * not NULL, the 32-byte device loss-scale state (flags bit 0), so that a run
 * with dynamic loss scaling resumes exactly.  The 16-bit params are not
 * stored: they are the rounding of the master.  Synchronises `stream` first,
 * so pending updates are included; the file appears under `path` only once
 * complete (written to "<path>.tmp", flushed, renamed, directory flushed).
 * Errors: ZERO_EINVAL (bad partition, NULL path/arrays/d_state), ZERO_EIO,
 * ZERO_EDEVICE. */
zero_status zero_ckpt_save(const char *path, uint64_t psi, uint32_t nd, uint32_t rank,
                           const float *master, const float *exp_avg, const float *exp_avg_sq,
                           const zero_adam_state_t *d_state, const zero_loss_scale_t *d_scale,
                           void *stream);

/* Reads and checks the header of a checkpoint file: magic and version, a range
 * equal to zero_partition(psi, nd, rank), no unknown flag bits, and a file
 * size that matches them.
 * Errors: ZERO_EINVAL (not a shard, inconsistent range), ZERO_EIO. */
zero_status zero_ckpt_read_header(const char *path, zero_ckpt_header *out);

/* Restores rank `rank` of nd ranks from the n_paths shard files of one saved
 * run, which may have used any number of ranks (re-sharding: the saved run's
 * ranks and the new ranks partition the same flat vector differently).  The
 * files, in any order, must be every shard of one save: the same psi and
 * step, ranges that tile [0, psi) exactly.  Fills the device arrays master,
 * exp_avg, exp_avg_sq (this rank's n = end - begin elements) from the files
 * that intersect its range and sets *d_state to the saved step with the
 * per-step scalars cleared (the next zero_adam_step recomputes them).  When
 * d_scale is not NULL it is set to the saved loss-scale state, which every
 * file must carry, identically.  Synchronises `stream`.  Errors: ZERO_EINVAL
 * (wrong psi, files from different saves, gaps or overlaps, bad partition, a
 * loss-scale state asked for but missing or differing between files),
 * ZERO_EIO, ZERO_EDEVICE. */
zero_status zero_ckpt_load(const char *const *paths, uint32_t n_paths, uint64_t psi, uint32_t nd,
                           uint32_t rank, float *master, float *exp_avg, float *exp_avg_sq,
                           zero_adam_state_t *d_state, zero_loss_scale_t *d_scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_MI355X_H */
