// Gather, gradient statistics and loss-scale kernels of libzero_mi355x for
// AMD MI355X (gfx950, CDNA4, wave64), with their C entry points:
//   flatten_segments  - list-order gather of tensors into a contiguous buffer
//                       ("ZeRO: Memory Optimizations Toward Training Trillion
//                       Parameter Models", paper summary page, section ZeRO-R
//                       > CB: constant-size fused buffers); in its statistics
//                       modes it also sums the squares of what it writes
//   stats_segments    - the same statistics over the tensors, without the copy
//   stats_pass1, stats_reduce, stats_final
//                     - overflow flag and fp64 squared norm of a 16-bit
//                       gradient shard, fixed-order reduction of per-tile sums
//   loss_scale_init, loss_scale_update
//                     - the device-resident dynamic loss scale (Micikevicius
//                       et al., "Mixed Precision Training")
// The AdamW kernels are in zero_adam.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "zero_device.h"

namespace {

template <bool BF16>
__device__ __forceinline__ void accum2(uint32_t w, double &acc)
{
    const double a = (double)to_f32<BF16>(w & 0xffffu);
    const double b = (double)hi_to_f32<BF16>(w);
    acc = fma(a, a, acc);  // squares of 16-bit values are exact in fp64
    acc = fma(b, b, acc);
}

// Sum over the block in a fixed order (butterfly within waves, then waves in
// order); the result is valid in thread 0.  Safe to call once per loop trip.
__device__ __forceinline__ double block_sum(double x)
{
    __shared__ double s_part[kBlock / 64];
    x = wave_sum(x);
    if (threadIdx.x % 64 == 0)
        s_part[threadIdx.x / 64] = x;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0)
        for (int i = 0; i < kBlock / 64; ++i)
            t += s_part[i];
    __syncthreads();  // s_part is free again for the next call
    return t;
}

// Segment s's entries of the gather's table.  A block reads them right after
// the search, before any branch, so that they arrive in one round of scalar
// loads: the search and this read are then the only dependent loads before
// the block's first vector load (reading each entry where it is used cost
// three more rounds, and the in-place statistics pass 6% on the 13B list).
struct SegEntry {
    uint64_t e_lo, e_hi;  // destination elements [e_lo, e_hi)
    uint32_t t_lo, t_hi;  // the segment's tiles [t_lo, t_hi)
    const char *src;      // source address of element e_lo
};

__device__ __forceinline__ SegEntry seg_entry(const FlatArgs &a, uint32_t s)
{
    return SegEntry{a.seg_lo[s], a.seg_lo[s + 1], a.tile_lo[s], a.tile_lo[s + 1], a.src[s]};
}

// Tile of block b in a grid of `grid` blocks (a multiple of 8).  Block b runs
// on XCD b mod 8, and each XCD has its own L2: renumbering the tiles as
// (b mod 8) * grid/8 + b/8 gives every XCD a contiguous eighth of them, so
// that a 64-byte sector shared by two neighbouring tiles (tiles are 16-byte
// aligned, not 64-byte aligned, when the data sits at a 16-bit phase other
// than 0) is fetched or written back by one L2 instead of two.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t b, uint32_t grid)
{
    return (b % 8) * (grid / 8) + b / 8;
}

template <int ES, int SB, int MODE>
__device__ __forceinline__ void flatten_full_chunks(const char *src_line0, char *dst_line0,
                                                    uint64_t c_beg, uint64_t c_end, double &acc)
{
    // chunk c (relative to the segment's first full chunk) reads the aligned
    // source lines c and c+1 (shifted by SB bytes) and writes destination line c
    uint4 lo[kFlatChunksPerThread], hi[kFlatChunksPerThread];
#pragma unroll
    for (int j = 0; j < kFlatChunksPerThread; ++j) {
        const uint64_t c = c_beg + (uint64_t)j * kBlock + threadIdx.x;
        if (c < c_end) {
            const uint4 *s = reinterpret_cast<const uint4 *>(src_line0) + c;
            lo[j] = ld_global(s);
            if constexpr (SB != 0)
                hi[j] = ld_global(s + 1);
        }
    }
#pragma unroll
    for (int j = 0; j < kFlatChunksPerThread; ++j) {
        const uint64_t c = c_beg + (uint64_t)j * kBlock + threadIdx.x;
        if (c < c_end) {
            uint4 o;
            if constexpr (SB == 0)
                o = lo[j];
            else
                o = shift_lines<SB>(lo[j], hi[j]);
            reinterpret_cast<uint4 *>(dst_line0)[c] = o;
            if constexpr (MODE != kCopy) {
                constexpr bool bf = MODE == kStatsBF16;
                accum2<bf>(o.x, acc);
                accum2<bf>(o.y, acc);
                accum2<bf>(o.z, acc);
                accum2<bf>(o.w, acc);
            }
        }
    }
}

template <int ES, int MODE>
__global__ void __launch_bounds__(kBlock) flatten_segments(FlatArgs a)
{
    constexpr uint64_t V = 16 / ES;  // elements per 16-byte line
    const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);  // one tile per block
    if (tile >= a.n_tiles)  // the grid is the tile count rounded up to a multiple of 8
        return;
    const uint64_t ph = a.dst_phase;
    char *const dst = a.dst;
    const SegEntry g = seg_entry(a, find_segment(a, tile));
    const uint64_t e_lo = g.e_lo, e_hi = g.e_hi;
    // full destination lines inside the segment: [c0, c1) in line units
    const uint64_t c0 = (e_lo + ph + V - 1) / V, c1 = (e_hi + ph) / V;
    const bool has_full = c1 > c0;
    const uint64_t k = tile - g.t_lo;  // tile within the segment
    const char *src = g.src;
    double acc = 0.0;
    if (k == 0) {
        // partial lines at both ends, element by element
        const uint64_t head_end = has_full ? c0 * V - ph : e_hi;
        const uint64_t tail_beg = has_full ? c1 * V - ph : e_hi;
        const uint64_t n_head = head_end - e_lo, n_tail = e_hi - tail_beg;
        const uint64_t i = threadIdx.x;
        if (i < n_head + n_tail) {
            const uint64_t e = i < n_head ? e_lo + i : tail_beg + (i - n_head);
            if constexpr (ES == 2) {
                const uint16_t v = ld_global(reinterpret_cast<const uint16_t *>(src) + (e - e_lo));
                reinterpret_cast<uint16_t *>(dst)[e] = v;
                if constexpr (MODE != kCopy) {
                    const double x = (double)to_f32<MODE == kStatsBF16>(v);
                    acc = fma(x, x, acc);
                }
            } else {
                reinterpret_cast<uint32_t *>(dst)[e] =
                    ld_global(reinterpret_cast<const uint32_t *>(src) + (e - e_lo));
            }
        }
    }
    if (has_full) {
        const uint64_t t_beg = k * kFlatTileChunks;
        const uint64_t t_end =
            (t_beg + kFlatTileChunks < c1 - c0) ? t_beg + kFlatTileChunks : c1 - c0;
        // first full line's source bytes and their 16-byte phase (uniform)
        const uintptr_t s0 = (uintptr_t)(src + (c0 * V - ph - e_lo) * ES);
        const uint32_t sb = (uint32_t)(s0 & 15u);
        const char *sl = (const char *)(s0 - sb);
        char *dl = dst + (c0 * V - ph) * ES;
        switch (sb) {
        case 0: flatten_full_chunks<ES, 0, MODE>(sl, dl, t_beg, t_end, acc); break;
        case 4: flatten_full_chunks<ES, 4, MODE>(sl, dl, t_beg, t_end, acc); break;
        case 8: flatten_full_chunks<ES, 8, MODE>(sl, dl, t_beg, t_end, acc); break;
        case 12: flatten_full_chunks<ES, 12, MODE>(sl, dl, t_beg, t_end, acc); break;
        default:
            if constexpr (ES == 2) {
                switch (sb) {
                case 2: flatten_full_chunks<ES, 2, MODE>(sl, dl, t_beg, t_end, acc); break;
                case 6: flatten_full_chunks<ES, 6, MODE>(sl, dl, t_beg, t_end, acc); break;
                case 10: flatten_full_chunks<ES, 10, MODE>(sl, dl, t_beg, t_end, acc); break;
                default: flatten_full_chunks<ES, 14, MODE>(sl, dl, t_beg, t_end, acc); break;
                }
            }
            break;
        }
    }
    if constexpr (MODE != kCopy) {
        const double t = block_sum(acc);
        if (threadIdx.x == 0)
            a.part[a.tile_base + tile] = t;
    }
}

// Statistics of the gather's tiles without the copy: every block takes
// kStatsTilesPerBlock consecutive tiles and, for each, sums exactly the
// squares that flatten_segments<2, stats> sums for it, in the same order
// (the tile's edge elements first, then its thread's line), and leaves the
// same per-tile partial.  Consecutive tiles mostly lie in one segment, so the
// table is searched again only when a tile starts a new one; the loads of all
// the block's tiles are issued before any is summed, and the per-tile sums
// share one pass over LDS.  Six tiles (24 KiB) per block measured best on the
// 13B list: 3.95-3.96 ms against 4.01-4.02 (four), 4.07-4.08 (eight) and 4.81
// (two), all in one process.
#ifndef ZERO_STATS_TILES
#define ZERO_STATS_TILES 6
#endif
constexpr int kStatsTilesPerBlock = ZERO_STATS_TILES;

// Per-tile block sums of x[0..T) in a fixed order (within each wave by DPP,
// then the wave totals in wave order, as block_sum does); thread q < T ends
// with the sum of x[q].
template <int T>
__device__ __forceinline__ double block_sums(double (&x)[T])
{
    __shared__ double s_part[T][kBlock / 64];
#pragma unroll
    for (int q = 0; q < T; ++q)
        x[q] = wave_sum(x[q]);
    if (threadIdx.x % 64 == 0)
#pragma unroll
        for (int q = 0; q < T; ++q)
            s_part[q][threadIdx.x / 64] = x[q];
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x < T)
        for (int i = 0; i < kBlock / 64; ++i)
            t += s_part[threadIdx.x][i];
    return t;
}

template <bool BF16>
__global__ void __launch_bounds__(kBlock) stats_segments(FlatArgs a)
{
    constexpr int T = kStatsTilesPerBlock;
    uint4 lo[T], hi[T];
    uint32_t sb[T];
    bool line[T];
    uint16_t edge[T];
    bool has_edge[T];
    const uint32_t n_tiles = a.n_tiles;
    // groups of T tiles, renumbered per XCD; the grid is the group count
    // rounded up to a multiple of 8
    const uint32_t tile0 = xcd_tile(blockIdx.x, gridDim.x) * T;
    if (tile0 >= n_tiles)
        return;
    const uint64_t ph = a.dst_phase;
    SegEntry g = seg_entry(a, find_segment(a, tile0));
    // the lines of every tile first, then the edge elements, then the sums
#pragma unroll
    for (int q = 0; q < T; ++q) {
        line[q] = has_edge[q] = false;
        sb[q] = 0;
        hi[q] = make_uint4(0, 0, 0, 0);
        const uint32_t tile = tile0 + q;
        if (tile >= n_tiles)
            continue;
        if (q > 0 && tile >= g.t_hi)  // the tile starts a later segment
            g = seg_entry(a, find_segment(a, tile));
        const uint64_t e_lo = g.e_lo, e_hi = g.e_hi;
        const uint64_t c0 = (e_lo + ph + 7) / 8, c1 = (e_hi + ph) / 8;
        const bool has_full = c1 > c0;
        const uint64_t k = tile - g.t_lo;
        const uint16_t *src = reinterpret_cast<const uint16_t *>(g.src);
        if (has_full) {
            const uint64_t c = k * kFlatTileChunks + threadIdx.x;
            if (c < c1 - c0) {
                const uintptr_t s0 = (uintptr_t)(src + (c0 * 8 - ph - e_lo));
                sb[q] = (uint32_t)(s0 & 15u);
                const uint4 *sl = reinterpret_cast<const uint4 *>(s0 - sb[q]) + c;
                lo[q] = ld_global(sl);
                if (sb[q])
                    hi[q] = ld_global(sl + 1);
                line[q] = true;
            }
        }
        if (k == 0) {
            const uint64_t head_end = has_full ? c0 * 8 - ph : e_hi;
            const uint64_t tail_beg = has_full ? c1 * 8 - ph : e_hi;
            const uint64_t n_head = head_end - e_lo, n_tail = e_hi - tail_beg;
            const uint64_t i = threadIdx.x;
            if (i < n_head + n_tail) {
                const uint64_t e = i < n_head ? e_lo + i : tail_beg + (i - n_head);
                edge[q] = ld_global(src + (e - e_lo));
                has_edge[q] = true;
            }
        }
    }
    double acc[T];
#pragma unroll
    for (int q = 0; q < T; ++q) {
        acc[q] = 0.0;
        if (has_edge[q]) {
            const double x = (double)to_f32<BF16>(edge[q]);
            acc[q] = fma(x, x, acc[q]);
        }
        if (line[q]) {
            const uint4 o = sb[q] ? shift_lines_rt(lo[q], hi[q], sb[q]) : lo[q];
            accum2<BF16>(o.x, acc[q]);
            accum2<BF16>(o.y, acc[q]);
            accum2<BF16>(o.z, acc[q]);
            accum2<BF16>(o.w, acc[q]);
        }
    }
    const double t = block_sums<T>(acc);
    if (threadIdx.x < T && tile0 + threadIdx.x < n_tiles)
        a.part[a.tile_base + tile0 + threadIdx.x] = t;
}

// ============================================================ grad stats
// One tile of kStatsTileLines 16-byte lines (8 gradients each) per block; each
// tile leaves one fp64 partial sum of squares, and the partials are reduced in
// a fixed order (groups of kReduceGroup, then one block), so the result is
// bit-reproducible for a given n and 16-byte phase of the gradient buffer.
// Overflow needs no separate flag: the square of any finite 16-bit value is
// finite in fp64 (at most about 1.2e77), while an inf or NaN gradient makes its
// square and hence every sum that contains it non-finite.  So the shard holds a
// non-finite gradient exactly when the fp64 sum of squares is not finite.
#ifndef ZERO_STATS_LINES
#define ZERO_STATS_LINES 2   // 16-byte lines per thread in a stats tile
#endif
constexpr uint64_t kStatsTileLines = (uint64_t)kBlock * ZERO_STATS_LINES;
constexpr uint64_t kReduceGroup = (uint64_t)kBlock * 16;  // partials per level-2 block
constexpr uint64_t kFinalMax = (uint64_t)kBlock * 64;     // partials one block finishes

// Upper bound of the pass-1 tiles for n gradients at any 16-byte phase.
uint64_t stats_tiles_max(uint64_t n)
{
    const uint64_t lines = n / 8 + 1;
    const uint64_t t = (lines + kStatsTileLines - 1) / kStatsTileLines;
    return t ? t : 1;
}

// Workspace for `tiles` partials plus the second reduction level.
size_t partials_bytes(uint64_t tiles)
{
    const uint64_t words = tiles + (tiles + kReduceGroup - 1) / kReduceGroup;
    return (size_t)((words * sizeof(double) + 15) / 16 * 16);
}

size_t stats_workspace_bytes(uint64_t n) { return partials_bytes(stats_tiles_max(n)); }

// Adds the squares of tile `tile`'s gradients that this thread holds to acc:
// ZERO_STATS_LINES aligned 16-byte lines per thread, and, in tile 0, the
// elements outside the aligned lines ([0, head) and [tail_beg, n)).
template <bool BF16>
__device__ __forceinline__ void stats_tile(const uint16_t *g, uint64_t head, uint64_t nchunks,
                                           uint64_t tail_beg, uint64_t n, uint64_t tile,
                                           double &acc)
{
    const uint4 *lines = reinterpret_cast<const uint4 *>(g + head);
    const uint64_t base = tile * kStatsTileLines + threadIdx.x;
    uint4 w[ZERO_STATS_LINES];
#pragma unroll
    for (int j = 0; j < ZERO_STATS_LINES; ++j) {
        const uint64_t c = base + (uint64_t)j * kBlock;
        w[j] = c < nchunks ? lines[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < ZERO_STATS_LINES; ++j) {
        accum2<BF16>(w[j].x, acc);
        accum2<BF16>(w[j].y, acc);
        accum2<BF16>(w[j].z, acc);
        accum2<BF16>(w[j].w, acc);
    }
    if (tile == 0) {
        const uint64_t n_edge = head + (n - tail_beg);
        if (threadIdx.x < n_edge) {
            const uint64_t e = threadIdx.x < head ? threadIdx.x : tail_beg + (threadIdx.x - head);
            const double x = (double)to_f32<BF16>(g[e]);
            acc = fma(x, x, acc);
        }
    }
}

// One tile per block: the launch takes tiles [tile0, tile0 + tiles), block b
// the tile tile0 + xcd_tile(b, grid) (the grid is `tiles` rounded up to a
// multiple of 8), and leaves its partial.
template <bool BF16>
__global__ void __launch_bounds__(kBlock)
    stats_pass1(const uint16_t *g, uint64_t head, uint64_t nchunks, uint64_t tail_beg, uint64_t n,
                uint64_t tile0, uint32_t tiles, double *part)
{
    const uint32_t k = xcd_tile(blockIdx.x, gridDim.x);
    if (k >= tiles)
        return;
    double acc = 0.0;
    const uint64_t tile = tile0 + k;
    stats_tile<BF16>(g, head, nchunks, tail_beg, n, tile, acc);
    const double t = block_sum(acc);
    if (threadIdx.x == 0)
        part[tile] = t;
}

// A fixed number of partials for any n: partial j (j < slots) sums tiles
// j, j + slots, j + 2 slots, ... and is left in part[j].  The grid is slots
// rounded up to a multiple of 8, and block b computes partial xcd_tile(b), so
// that neighbouring tiles of one round are read through one XCD's L2; which
// block computes a partial does not change its value.
template <bool BF16>
__global__ void __launch_bounds__(kBlock)
    stats_pass1_strided(const uint16_t *g, uint64_t head, uint64_t nchunks, uint64_t tail_beg,
                        uint64_t n, uint64_t tiles, uint32_t slots, double *part)
{
    const uint32_t j = xcd_tile(blockIdx.x, gridDim.x);
    if (j >= slots)
        return;
    double acc = 0.0;
    for (uint64_t tile = j; tile < tiles; tile += slots)
        stats_tile<BF16>(g, head, nchunks, tail_beg, n, tile, acc);
    const double t = block_sum(acc);
    if (threadIdx.x == 0)
        part[j] = t;
}

// Block b sums partials [b*kReduceGroup, (b+1)*kReduceGroup) in a fixed order.
__global__ void __launch_bounds__(kBlock)
    stats_reduce(const double *in, uint64_t n_in, double *out)
{
    const uint64_t lo = (uint64_t)blockIdx.x * kReduceGroup;
    double s = 0.0;
    for (uint64_t k = threadIdx.x; k < kReduceGroup; k += kBlock)
        if (lo + k < n_in)
            s += in[lo + k];
    const double t = block_sum(s);
    if (threadIdx.x == 0)
        out[blockIdx.x] = t;
}

__global__ void __launch_bounds__(kBlock)
    stats_final(const double *in, uint64_t n_in, double inv_scale_sq,
                const zero_loss_scale_t *scale, zero_grad_stats_t *out)
{
    if (scale) {  // the device loss-scale state replaces the host value
        const double inv = scale->inv_scale;
        inv_scale_sq = inv * inv;
    }
    double s = 0.0;
    for (uint64_t k = threadIdx.x; k < n_in; k += kBlock)
        s += in[k];
    const double t = block_sum(s);
    if (threadIdx.x == 0) {
        const bool finite = __builtin_isfinite(t);
        out->sq_norm = t * inv_scale_sq;
        out->overflow = finite ? 0u : 1u;
        out->pad = 0;
    }
}

// Dynamic loss scaling (Micikevicius et al., "Mixed Precision Training"): one
// thread sets or advances the device-resident scale state.
__global__ void loss_scale_init(zero_loss_scaler c, zero_loss_scale_t *d)
{
    if (threadIdx.x != 0 || blockIdx.x != 0)
        return;
    d->scale = c.init_scale;
    d->inv_scale = 1.0 / c.init_scale;
    d->good_steps = 0;
    d->overflows = 0;
}

__global__ void loss_scale_update(zero_loss_scaler c, const zero_grad_stats_t *stats,
                                  zero_loss_scale_t *d)
{
    if (threadIdx.x != 0 || blockIdx.x != 0)
        return;
    double scale = d->scale;
    uint64_t good = d->good_steps, overflows = d->overflows;
    if (stats->overflow) {  // the step was skipped: back off
        const double reduced = scale * c.backoff_factor;
        scale = reduced > c.min_scale ? reduced : c.min_scale;
        good = 0;
        ++overflows;
    } else if (++good == c.growth_interval) {  // a full run without overflow: grow
        const double grown = scale * c.growth_factor;
        if (__builtin_isfinite(grown))
            scale = grown < c.max_scale ? grown : c.max_scale;
        good = 0;
    }
    d->scale = scale;
    d->inv_scale = 1.0 / scale;
    d->good_steps = good;
    d->overflows = overflows;
}

template <int ES, int MODE>
zero_status flatten_launch(FlatArgs &a, hipStream_t stream)
{
    // one tile per block, the grid rounded up to whole rounds of the 8 XCDs
    hipLaunchKernelGGL((flatten_segments<ES, MODE>), dim3((a.n_tiles + 7) / 8 * 8), dim3(kBlock),
                       0, stream, a);
    return launch_status("zero_bucket_flatten");
}

// Upper bound of the tiles that a gather of elements [range_begin, range_end)
// uses, over every 16-byte phase of the destination.
uint64_t flatten_tiles_max(const uint64_t *numel, uint32_t n_tensors, uint64_t range_begin,
                           uint64_t range_end)
{
    uint64_t tiles = 0, start = 0;
    for (uint32_t i = 0; i < n_tensors; ++i) {
        const uint64_t lo = start > range_begin ? start : range_begin;
        const uint64_t hi = start + numel[i] < range_end ? start + numel[i] : range_end;
        start += numel[i];
        if (lo >= hi)
            continue;
        const uint64_t full = (hi - lo) / 8;  // at most this many full 16-byte lines
        tiles += full ? (full + kFlatTileChunks - 1) / kFlatTileChunks : 1;
    }
    return tiles ? tiles : 1;
}

// Shared body of the gather entry points.  mode: kCopy or a stats mode; part:
// per-tile partials (stats modes), part_bytes long, which the sources must
// not overlap either.  *n_tiles: tiles used.
zero_status flatten_impl(const char *what, const void *const *tensor_ptrs, const uint64_t *numel,
                         uint32_t n_tensors, zero_dtype dt, uint64_t range_begin, uint64_t count,
                         void *dst, int mode, double *part, size_t part_bytes, hipStream_t stream,
                         uint64_t *n_tiles)
{
    *n_tiles = 0;
    uint64_t range_end;
    if (zero_status st = check_range(what, tensor_ptrs, numel, n_tensors, range_begin, count,
                                     &range_end);
        st != ZERO_OK)
        return st;
    if (count == 0)
        return ZERO_OK;
    const uint64_t es = dt == ZERO_F32 ? 4 : 2;
    if (!dst)
        return fail(ZERO_EINVAL, "%s: NULL dst", what);
    if (!aligned(dst, es))
        return fail(ZERO_EALIGN, "%s: dst not %llu-byte aligned", what, (unsigned long long)es);
    const Guard guards[2] = {{dst, count * es, "dst"}, {part, part_bytes, "workspace"}};
    FlatArgs a{};
    a.dst = (char *)dst;
    a.part = part;
    auto launch = [&](FlatArgs &t) -> zero_status {
        if (es == 4)
            return flatten_launch<4, kCopy>(t, stream);
        switch (mode) {
        case kStatsF16: return flatten_launch<2, kStatsF16>(t, stream);
        case kStatsBF16: return flatten_launch<2, kStatsBF16>(t, stream);
        default: return flatten_launch<2, kCopy>(t, stream);
        }
    };
    const uint64_t ph = ((uintptr_t)dst & 15u) / es;
    return segment_launches(what, tensor_ptrs, numel, n_tensors, es, range_begin, range_end, ph,
                            guards, 2, a, launch, n_tiles);
}

}  // namespace

namespace {
// Fixed-order reduction of `tiles` per-tile partials (at part) into *out:
// groups of kReduceGroup when there are many, then one block.
zero_status reduce_partials(double *part, uint64_t tiles, double inv_scale,
                            const zero_loss_scale_t *scale, zero_grad_stats_t *out, hipStream_t s)
{
    const double *last = part;
    uint64_t n_last = tiles;
    if (tiles > kFinalMax) {
        double *part2 = part + tiles;
        const uint64_t groups = (tiles + kReduceGroup - 1) / kReduceGroup;
        hipLaunchKernelGGL(stats_reduce, dim3((uint32_t)groups), dim3(kBlock), 0, s,
                           (const double *)part, tiles, part2);
        const zero_status st = launch_status("gradient statistics: reduce");
        if (st != ZERO_OK)
            return st;
        last = part2;
        n_last = groups;
    }
    hipLaunchKernelGGL(stats_final, dim3(1), dim3(kBlock), 0, s, last, n_last,
                       inv_scale * inv_scale, scale, out);
    return launch_status("gradient statistics: final");
}
}  // namespace

// ============================================================== C entry points
extern "C" zero_status zero_bucket_flatten(const void *const *tensor_ptrs, const uint64_t *numel,
                                           uint32_t n_tensors, zero_dtype dt, uint64_t range_begin,
                                           uint64_t count, void *dst, void *stream)
{
    if (dt != ZERO_F32 && dt != ZERO_F16 && dt != ZERO_BF16)
        return fail(ZERO_EINVAL, "zero_bucket_flatten: bad dtype %d", (int)dt);
    uint64_t tiles;
    return flatten_impl("zero_bucket_flatten", tensor_ptrs, numel, n_tensors, dt, range_begin,
                        count, dst, kCopy, nullptr, 0, (hipStream_t)stream, &tiles);
}

extern "C" zero_status zero_grad_stats_workspace(uint64_t n, size_t *bytes)
{
    if (!bytes)
        return fail(ZERO_EINVAL, "zero_grad_stats_workspace: NULL output");
    *bytes = stats_workspace_bytes(n);
    return ZERO_OK;
}

namespace {
// Checks shared by the two statistics entry points (everything but the
// workspace).  Returns the inverse loss scale to pass to the kernels.
zero_status check_stats_args(const char *what, const void *grad, zero_dtype gdt, uint64_t n,
                             double *inv_loss_scale, const zero_loss_scale_t *d_scale,
                             const zero_grad_stats_t *d_stats)
{
    if (gdt != ZERO_F16 && gdt != ZERO_BF16)
        return fail(ZERO_EINVAL, "%s: gradient dtype must be F16 or BF16", what);
    if (!d_stats)
        return fail(ZERO_EINVAL, "%s: NULL d_stats", what);
    if (!d_scale && !(std::isfinite(*inv_loss_scale) && *inv_loss_scale > 0.0))
        return fail(ZERO_EINVAL, "%s: inv_loss_scale must be finite and > 0", what);
    if (d_scale)
        *inv_loss_scale = 1.0;  // unused: the kernel reads the device state
    if (n > 0 && !grad)
        return fail(ZERO_EINVAL, "%s: NULL grad", what);
    if (n > UINT64_MAX / 4)
        return fail(ZERO_EINVAL, "%s: n too large", what);
    if (!aligned(grad, 2) || !aligned(d_stats, 8) || !aligned(d_scale, 8))
        return fail(ZERO_EALIGN, "%s: misaligned pointer", what);
    if (overlap(d_stats, sizeof *d_stats, grad, 2 * n) ||
        (d_scale && overlap(d_scale, sizeof *d_scale, d_stats, sizeof *d_stats)))
        return fail(ZERO_EINVAL, "%s: overlapping buffers", what);
    return ZERO_OK;
}

// The aligned body of n gradients at `grad`: elements [0, head) precede the
// first 16-byte line, nchunks whole lines follow, then [tail_beg, n).
struct StatsLayout {
    uint64_t head, nchunks, tail_beg, tiles;
};

StatsLayout stats_layout(const void *grad, uint64_t n)
{
    StatsLayout l;
    const uint64_t ph = ((uintptr_t)grad & 15u) / 2;
    l.head = (8 - ph) % 8;
    if (l.head > n) l.head = n;
    l.nchunks = (n - l.head) / 8;
    l.tail_beg = l.head + 8 * l.nchunks;
    l.tiles = (l.nchunks + kStatsTileLines - 1) / kStatsTileLines;
    if (l.tiles == 0) l.tiles = 1;  // tile 0 also takes the elements outside the lines
    return l;
}
}  // namespace

extern "C" zero_status zero_grad_stats(const void *grad, zero_dtype gdt, uint64_t n,
                                       double inv_loss_scale, const zero_loss_scale_t *d_scale,
                                       void *workspace, size_t ws_bytes,
                                       zero_grad_stats_t *d_stats, void *stream)
{
    const char *what = "zero_grad_stats";
    if (zero_status st = check_stats_args(what, grad, gdt, n, &inv_loss_scale, d_scale, d_stats);
        st != ZERO_OK)
        return st;
    if (!workspace)
        return fail(ZERO_EINVAL, "%s: NULL workspace", what);
    const size_t need = stats_workspace_bytes(n);
    if (ws_bytes < need)
        return fail(ZERO_ENOSPC, "%s: workspace %zu bytes < %zu", what, ws_bytes, need);
    if (!aligned(workspace, 16))
        return fail(ZERO_EALIGN, "%s: misaligned workspace", what);
    if (overlap(workspace, ws_bytes, d_stats, sizeof *d_stats) ||
        overlap(workspace, ws_bytes, grad, 2 * n) ||
        (d_scale && overlap(d_scale, sizeof *d_scale, workspace, ws_bytes)))
        return fail(ZERO_EINVAL, "%s: overlapping buffers", what);
    hipStream_t s = (hipStream_t)stream;
    const StatsLayout l = stats_layout(grad, n);
    double *part = (double *)workspace;
    const uint16_t *g = (const uint16_t *)grad;
    // one tile per block, in launches of at most kMaxLaunchBlocks tiles (a
    // multiple of 8, so the rounded-up grid stays within it)
    for (uint64_t t0 = 0; t0 < l.tiles; t0 += kMaxLaunchBlocks) {
        const uint32_t tiles = (uint32_t)(l.tiles - t0 < kMaxLaunchBlocks ? l.tiles - t0
                                                                          : kMaxLaunchBlocks);
        const uint32_t grid = (tiles + 7) / 8 * 8;
        if (gdt == ZERO_BF16)
            hipLaunchKernelGGL(stats_pass1<true>, dim3(grid), dim3(kBlock), 0, s, g, l.head,
                               l.nchunks, l.tail_beg, n, t0, tiles, part);
        else
            hipLaunchKernelGGL(stats_pass1<false>, dim3(grid), dim3(kBlock), 0, s, g, l.head,
                               l.nchunks, l.tail_beg, n, t0, tiles, part);
        const zero_status st = launch_status("zero_grad_stats pass 1");
        if (st != ZERO_OK)
            return st;
    }
    return reduce_partials(part, l.tiles, inv_loss_scale, d_scale, d_stats, s);
}

// ------------------------------------------- statistics without allocation
// Device memory of zero_grad_stats_noalloc: the fp64 partials of its first
// pass, one per block of a grid of at most kScratchPartials blocks (64 KiB).
// Every GPU the library runs on holds its own copy until the process ends.
// Host code reaches it only through the address that hipGetSymbolAddress
// returns for the current device (the array's name is a host-side stand-in).
constexpr uint64_t kScratchPartials = 8192;
static_assert(kScratchPartials <= kFinalMax && kScratchPartials % 8 == 0,
              "one block must finish the scratch partials, a whole number of XCD rounds");
static __device__ __align__(256) double scratch[kScratchPartials];

namespace {
// Device address of `scratch` on the current device, looked up once per device.
// The kernels run on `stream`'s device, so that must be the current one (whose
// copy of the array the address names).
zero_status scratch_address(const char *what, hipStream_t stream, double **out)
{
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static double *addr[kMaxDev];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
        return fail(ZERO_EDEVICE, "%s: no current HIP device (or device index %d >= %d)", what,
                    dev, kMaxDev);
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess)
        return fail(ZERO_EINVAL, "%s: not a valid stream", what);
    if (sdev != dev)
        return fail(ZERO_EINVAL, "%s: the stream belongs to device %d, but device %d is current",
                    what, (int)sdev, dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(ZERO_EDEVICE, "%s: hipGetSymbolAddress(scratch) on device %d: %s", what,
                        dev, hipGetErrorString(e));
        addr[dev] = (double *)p;
    }
    *out = addr[dev];
    return ZERO_OK;
}
}  // namespace

extern "C" zero_status zero_grad_stats_noalloc(const void *grad, zero_dtype gdt, uint64_t n,
                                               double inv_loss_scale,
                                               const zero_loss_scale_t *d_scale,
                                               zero_grad_stats_t *d_stats, void *stream)
{
    const char *what = "zero_grad_stats_noalloc";
    if (zero_status st = check_stats_args(what, grad, gdt, n, &inv_loss_scale, d_scale, d_stats);
        st != ZERO_OK)
        return st;
    double *part = nullptr;
    if (zero_status st = scratch_address(what, (hipStream_t)stream, &part); st != ZERO_OK)
        return st;
    const StatsLayout l = stats_layout(grad, n);
    // every tile is folded into one of at most kScratchPartials block partials,
    // so the scratch holds the partials of any n
    const uint64_t blocks = l.tiles < kScratchPartials ? l.tiles : kScratchPartials;
    if (overlap(part, kScratchPartials * sizeof(double), grad, 2 * n) ||
        overlap(part, kScratchPartials * sizeof(double), d_stats, sizeof *d_stats) ||
        (d_scale && overlap(part, kScratchPartials * sizeof(double), d_scale, sizeof *d_scale)))
        return fail(ZERO_EINVAL, "%s: a buffer overlaps the library's scratch", what);
    hipStream_t s = (hipStream_t)stream;
    const uint16_t *g = (const uint16_t *)grad;
    const uint32_t grid = ((uint32_t)blocks + 7) / 8 * 8;  // kScratchPartials is a multiple of 8
    if (gdt == ZERO_BF16)
        hipLaunchKernelGGL(stats_pass1_strided<true>, dim3(grid), dim3(kBlock), 0, s, g, l.head,
                           l.nchunks, l.tail_beg, n, l.tiles, (uint32_t)blocks, part);
    else
        hipLaunchKernelGGL(stats_pass1_strided<false>, dim3(grid), dim3(kBlock), 0, s, g, l.head,
                           l.nchunks, l.tail_beg, n, l.tiles, (uint32_t)blocks, part);
    if (zero_status st = launch_status("zero_grad_stats_noalloc pass 1"); st != ZERO_OK)
        return st;
    return reduce_partials(part, blocks, inv_loss_scale, d_scale, d_stats, s);
}

extern "C" zero_status zero_bucket_flatten_stats_workspace(const uint64_t *numel, uint32_t n_tensors,
                                                          uint64_t range_begin, uint64_t count,
                                                          size_t *bytes)
{
    if (!bytes)
        return fail(ZERO_EINVAL, "zero_bucket_flatten_stats_workspace: NULL output");
    if (n_tensors > 0 && !numel)
        return fail(ZERO_EINVAL, "zero_bucket_flatten_stats_workspace: NULL numel");
    uint64_t range_end;
    if (__builtin_add_overflow(range_begin, count, &range_end))
        return fail(ZERO_EINVAL, "zero_bucket_flatten_stats_workspace: range overflows");
    *bytes = partials_bytes(flatten_tiles_max(numel, n_tensors, range_begin, range_end));
    return ZERO_OK;
}

extern "C" zero_status zero_bucket_flatten_stats(const void *const *tensor_ptrs,
                                                 const uint64_t *numel, uint32_t n_tensors,
                                                 zero_dtype gdt, uint64_t range_begin,
                                                 uint64_t count, void *dst, double inv_loss_scale,
                                                 const zero_loss_scale_t *d_scale,
                                                 void *workspace, size_t ws_bytes,
                                                 zero_grad_stats_t *d_stats, void *stream)
{
    const char *what = "zero_bucket_flatten_stats";
    if (gdt != ZERO_F16 && gdt != ZERO_BF16)
        return fail(ZERO_EINVAL, "%s: gradient dtype must be F16 or BF16", what);
    if (!d_stats)
        return fail(ZERO_EINVAL, "%s: NULL d_stats", what);
    if (!d_scale && !(std::isfinite(inv_loss_scale) && inv_loss_scale > 0.0))
        return fail(ZERO_EINVAL, "%s: inv_loss_scale must be finite and > 0", what);
    if (d_scale)
        inv_loss_scale = 1.0;  // unused: the kernel reads the device state
    if (!workspace)
        return fail(ZERO_EINVAL, "%s: NULL workspace", what);
    if (n_tensors > 0 && !numel)
        return fail(ZERO_EINVAL, "%s: NULL numel", what);
    uint64_t range_end;
    if (__builtin_add_overflow(range_begin, count, &range_end))
        return fail(ZERO_EINVAL, "%s: range overflows", what);
    const size_t need = partials_bytes(flatten_tiles_max(numel, n_tensors, range_begin, range_end));
    if (ws_bytes < need)
        return fail(ZERO_ENOSPC, "%s: workspace %zu bytes < %zu", what, ws_bytes, need);
    if (!aligned(workspace, 16) || !aligned(d_stats, 8) || !aligned(d_scale, 8))
        return fail(ZERO_EALIGN, "%s: misaligned workspace, d_stats or d_scale", what);
    if (overlap(workspace, ws_bytes, d_stats, sizeof *d_stats) ||
        overlap(workspace, ws_bytes, dst, 2 * count) ||
        overlap(d_stats, sizeof *d_stats, dst, 2 * count) ||
        (d_scale && (overlap(d_scale, sizeof *d_scale, workspace, ws_bytes) ||
                     overlap(d_scale, sizeof *d_scale, d_stats, sizeof *d_stats) ||
                     overlap(d_scale, sizeof *d_scale, dst, 2 * count))))
        return fail(ZERO_EINVAL, "%s: overlapping buffers", what);
    hipStream_t s = (hipStream_t)stream;
    uint64_t tiles = 0;
    const zero_status st =
        flatten_impl(what, tensor_ptrs, numel, n_tensors, gdt, range_begin, count, dst,
                     gdt == ZERO_BF16 ? kStatsBF16 : kStatsF16, (double *)workspace, ws_bytes,
                     s, &tiles);
    if (st != ZERO_OK)
        return st;
    return reduce_partials((double *)workspace, tiles, inv_loss_scale, d_scale, d_stats, s);
}

// ------------------------------------------------ steps from tensor lists
extern "C" zero_status zero_grad_stats_tensors(const void *const *tensor_ptrs,
                                               const uint64_t *numel, uint32_t n_tensors,
                                               zero_dtype gdt, uint64_t range_begin,
                                               uint64_t count, double inv_loss_scale,
                                               const zero_loss_scale_t *d_scale,
                                               void *workspace, size_t ws_bytes,
                                               zero_grad_stats_t *d_stats, void *stream)
{
    const char *what = "zero_grad_stats_tensors";
    if (gdt != ZERO_F16 && gdt != ZERO_BF16)
        return fail(ZERO_EINVAL, "%s: gradient dtype must be F16 or BF16", what);
    if (!d_stats)
        return fail(ZERO_EINVAL, "%s: NULL d_stats", what);
    if (!d_scale && !(std::isfinite(inv_loss_scale) && inv_loss_scale > 0.0))
        return fail(ZERO_EINVAL, "%s: inv_loss_scale must be finite and > 0", what);
    if (d_scale)
        inv_loss_scale = 1.0;  // unused: the kernel reads the device state
    if (!workspace)
        return fail(ZERO_EINVAL, "%s: NULL workspace", what);
    uint64_t range_end;
    if (zero_status st = check_range(what, tensor_ptrs, numel, n_tensors, range_begin, count,
                                     &range_end);
        st != ZERO_OK)
        return st;
    const size_t need = partials_bytes(flatten_tiles_max(numel, n_tensors, range_begin, range_end));
    if (ws_bytes < need)
        return fail(ZERO_ENOSPC, "%s: workspace %zu bytes < %zu", what, ws_bytes, need);
    if (!aligned(workspace, 16) || !aligned(d_stats, 8) || !aligned(d_scale, 8))
        return fail(ZERO_EALIGN, "%s: misaligned workspace, d_stats or d_scale", what);
    if (overlap(workspace, ws_bytes, d_stats, sizeof *d_stats) ||
        (d_scale && (overlap(d_scale, sizeof *d_scale, workspace, ws_bytes) ||
                     overlap(d_scale, sizeof *d_scale, d_stats, sizeof *d_stats))))
        return fail(ZERO_EINVAL, "%s: overlapping buffers", what);
    hipStream_t s = (hipStream_t)stream;
    const Guard guards[3] = {{workspace, ws_bytes, "workspace"},
                             {d_stats, sizeof *d_stats, "d_stats"},
                             {d_scale, d_scale ? sizeof *d_scale : 0, "d_scale"}};
    FlatArgs a{};
    a.part = (double *)workspace;
    auto launch = [&](FlatArgs &t) -> zero_status {
        const uint32_t groups = (t.n_tiles + kStatsTilesPerBlock - 1) / kStatsTilesPerBlock;
        const uint32_t grid = (groups + 7) / 8 * 8;  // whole rounds of the 8 XCDs
        if (gdt == ZERO_BF16)
            hipLaunchKernelGGL(stats_segments<true>, dim3(grid), dim3(kBlock), 0, s, t);
        else
            hipLaunchKernelGGL(stats_segments<false>, dim3(grid), dim3(kBlock), 0, s, t);
        return launch_status(what);
    };
    uint64_t tiles = 0;
    if (count > 0)
        if (zero_status st = segment_launches(what, tensor_ptrs, numel, n_tensors, 2, range_begin,
                                              range_end, 0, guards, 3, a, launch, &tiles);
            st != ZERO_OK)
            return st;
    return reduce_partials((double *)workspace, tiles, inv_loss_scale, d_scale, d_stats, s);
}

extern "C" zero_status zero_loss_scale_init(const zero_loss_scaler *cfg, zero_loss_scale_t *d_scale,
                                            void *stream)
{
    const char *what = "zero_loss_scale_init";
    if (!cfg || !d_scale)
        return fail(ZERO_EINVAL, "%s: NULL argument", what);
    if (zero_status st = zero::check_scaler(*cfg, what); st != ZERO_OK)
        return st;
    if (!aligned(d_scale, 8))
        return fail(ZERO_EALIGN, "%s: misaligned d_scale", what);
    hipLaunchKernelGGL(loss_scale_init, dim3(1), dim3(64), 0, (hipStream_t)stream, *cfg, d_scale);
    return launch_status(what);
}

extern "C" zero_status zero_loss_scale_update(const zero_loss_scaler *cfg,
                                              const zero_grad_stats_t *d_stats,
                                              zero_loss_scale_t *d_scale, void *stream)
{
    const char *what = "zero_loss_scale_update";
    if (!cfg || !d_stats || !d_scale)
        return fail(ZERO_EINVAL, "%s: NULL argument", what);
    if (zero_status st = zero::check_scaler(*cfg, what); st != ZERO_OK)
        return st;
    if (!aligned(d_scale, 8) || !aligned(d_stats, 8))
        return fail(ZERO_EALIGN, "%s: misaligned d_stats or d_scale", what);
    if (overlap(d_scale, sizeof *d_scale, d_stats, sizeof *d_stats))
        return fail(ZERO_EINVAL, "%s: d_stats and d_scale overlap", what);
    hipLaunchKernelGGL(loss_scale_update, dim3(1), dim3(64), 0, (hipStream_t)stream, *cfg,
                       d_stats, d_scale);
    return launch_status(what);
}
