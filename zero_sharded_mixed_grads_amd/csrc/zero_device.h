// Device and launch helpers shared by the kernels of libzero_mi355x (AMD
// MI355X, gfx950, CDNA4, wave64): 16-bit conversions, realignment of 16-bit
// streams, wave reductions, the gather's segment table and its host-side
// construction, launch limits and argument checks.
//
// Memory access rules used throughout: every global load and store is
// naturally aligned (16-byte vectors on 16-byte boundaries, dwords on 4,
// shorts on 2).  A 16-bit stream whose 16-byte phase differs from the fp32
// streams is realigned in registers: the 8 wanted elements are funnel-shifted
// out of two aligned 16-byte lines (v_alignbyte), and stores are assembled
// into whole aligned lines with the neighbouring lane's values, or split into
// naturally aligned pieces at the edges.  An aligned line that holds at least
// one byte of a live buffer lies inside a mapped page, so the over-read of
// such a line never faults; over-read bytes are discarded.  Reductions run in
// a fixed order and there are no atomics: results are bit-reproducible.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "zero_internal.h"

namespace {

using zero::fail;

#ifndef ZERO_BLOCK
#define ZERO_BLOCK 256
#endif
constexpr int kBlock = ZERO_BLOCK;  // threads per block (waves of 64 lanes)

// 16-byte lines per thread in a gather tile (compile-time; the measured best).
#ifndef ZERO_FLAT_CPT
#define ZERO_FLAT_CPT 1
#endif

// Plain global accesses of the streaming kernels (non-temporal hints were
// measured slower on this part).
template <typename T>
__device__ __forceinline__ T ld_stream(const T *p)
{
    return *p;
}

template <typename T>
__device__ __forceinline__ void st_stream(T *p, const T &v)
{
    *p = v;
}

// A load through a pointer that the compiler cannot prove global (a tensor
// address read from a table), issued as a global load: a flat load would
// also count against the scalar-memory counter, so every later scalar load
// (the next tile's table lookup) would wait for it.
template <typename T>
__device__ __forceinline__ T ld_global(const T *p)
{
    return *(const __attribute__((address_space(1))) T *)p;
}

// (uint4's copy constructor would take a generic reference: load a native
// vector instead.)
__device__ __forceinline__ uint4 ld_global(const uint4 *p)
{
    typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
    const v4u32 x = *(const __attribute__((address_space(1))) v4u32 *)p;
    return make_uint4(x.x, x.y, x.z, x.w);
}

// ------------------------------------------------------------ 16-bit helpers
template <bool BF16>
__device__ __forceinline__ float to_f32(uint32_t h)  // h: bits in the low half
{
    if constexpr (BF16) {
        return __uint_as_float(h << 16);
    } else {
        _Float16 x;
        uint16_t b = (uint16_t)h;
        __builtin_memcpy(&x, &b, 2);
        return (float)x;  // exact widening
    }
}

template <bool BF16>
__device__ __forceinline__ float hi_to_f32(uint32_t w)  // the upper half of a dword
{
    if constexpr (BF16)
        return __uint_as_float(w & 0xffff0000u);
    else
        return to_f32<false>(w >> 16);
}

// Round to nearest, ties to even.
template <bool BF16>
__device__ __forceinline__ uint32_t from_f32(float x)
{
    if constexpr (BF16) {
        uint32_t u = __float_as_uint(x);
        if ((u & 0x7fffffffu) > 0x7f800000u)  // NaN: keep it a (quiet) NaN
            return (u >> 16) | 0x40u;
        u += 0x7fffu + ((u >> 16) & 1u);
        return u >> 16;
    } else {
        // The barrier makes x an opaque, already rounded fp32 value: without it
        // the backend folds "fma then convert" into v_fma_mixlo_f16, which
        // rounds the exact fma result to f16 once instead of rounding the
        // stored fp32 master, and differs from it at fp32 ties.
        asm volatile("" : "+v"(x));
        _Float16 h = (_Float16)x;  // v_cvt_f16_f32, round-to-nearest-even mode
        uint16_t b;
        __builtin_memcpy(&b, &h, 2);
        return b;
    }
}

// Bytes [SB, SB + 16) of the 32-byte concatenation lo:hi (SB even).
template <int SB>
__device__ __forceinline__ uint4 shift_lines(const uint4 &lo, const uint4 &hi)
{
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    constexpr int q = SB / 4, r = SB % 4;
    uint4 o;
    if constexpr (r == 0) {
        o.x = w[q]; o.y = w[q + 1]; o.z = w[q + 2]; o.w = w[q + 3];
    } else {
        o.x = __builtin_amdgcn_alignbyte(w[q + 1], w[q], r);
        o.y = __builtin_amdgcn_alignbyte(w[q + 2], w[q + 1], r);
        o.z = __builtin_amdgcn_alignbyte(w[q + 3], w[q + 2], r);
        o.w = __builtin_amdgcn_alignbyte(w[q + 4], w[q + 3], r);
    }
    return o;
}

// Runtime-uniform byte shift (0..14, even) dispatched to the templates.
__device__ __forceinline__ uint4 shift_lines_rt(const uint4 &lo, const uint4 &hi, uint32_t sb)
{
    switch (sb) {
    case 0: return lo;
    case 2: return shift_lines<2>(lo, hi);
    case 4: return shift_lines<4>(lo, hi);
    case 6: return shift_lines<6>(lo, hi);
    case 8: return shift_lines<8>(lo, hi);
    case 10: return shift_lines<10>(lo, hi);
    case 12: return shift_lines<12>(lo, hi);
    default: return shift_lines<14>(lo, hi);
    }
}

// Stores halves h[0..COUNT) into slots [SLOT, SLOT + COUNT) of the aligned
// 16-byte line at `line`, as naturally aligned short/dword/dwordx2/dwordx4.
template <int SLOT, int COUNT>
__device__ __forceinline__ void store_run(uint16_t *line, const uint32_t *h)
{
    if constexpr (COUNT <= 0) {
        return;
    } else if constexpr ((SLOT & 1) || COUNT == 1) {
        st_stream(line + SLOT, (uint16_t)h[0]);
        store_run<SLOT + 1, COUNT - 1>(line, h + 1);
    } else if constexpr (SLOT % 8 == 0 && COUNT >= 8) {
        st_stream(reinterpret_cast<uint4 *>(line + SLOT),
                  make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16,
                             h[6] | h[7] << 16));
        store_run<SLOT + 8, COUNT - 8>(line, h + 8);
    } else if constexpr (SLOT % 4 == 0 && COUNT >= 4) {
        st_stream(reinterpret_cast<uint2 *>(line + SLOT),
                  make_uint2(h[0] | h[1] << 16, h[2] | h[3] << 16));
        store_run<SLOT + 4, COUNT - 4>(line, h + 4);
    } else {
        st_stream(reinterpret_cast<uint32_t *>(line + SLOT), h[0] | h[1] << 16);
        store_run<SLOT + 2, COUNT - 2>(line, h + 2);
    }
}

// Eight halves whose first element sits at slot PH of the aligned line
// `line` span two lines: slots PH..7 of this line (the head) and slots
// 0..PH-1 of the next one (the tail).  Each part is written on its own, as
// naturally aligned pieces, by the lanes that cannot form a whole line.
template <int PH>
__device__ __forceinline__ void store_head(uint16_t *line, const uint32_t *h)
{
    store_run<PH, 8 - PH>(line, h);
}

template <int PH>
__device__ __forceinline__ void store_tail(uint16_t *next_line, const uint32_t *h)
{
    store_run<0, PH>(next_line, h + 8 - PH);
}

__device__ __forceinline__ void store_head_rt(uint16_t *line, const uint32_t *h, uint32_t ph)
{
    switch (ph) {
    case 1: store_head<1>(line, h); break;
    case 2: store_head<2>(line, h); break;
    case 3: store_head<3>(line, h); break;
    case 4: store_head<4>(line, h); break;
    case 5: store_head<5>(line, h); break;
    case 6: store_head<6>(line, h); break;
    default: store_head<7>(line, h); break;
    }
}

__device__ __forceinline__ void store_tail_rt(uint16_t *next_line, const uint32_t *h, uint32_t ph)
{
    switch (ph) {
    case 1: store_tail<1>(next_line, h); break;
    case 2: store_tail<2>(next_line, h); break;
    case 3: store_tail<3>(next_line, h); break;
    case 4: store_tail<4>(next_line, h); break;
    case 5: store_tail<5>(next_line, h); break;
    case 6: store_tail<6>(next_line, h); break;
    default: store_tail<7>(next_line, h); break;
    }
}

// A dword moved one lane along the whole wave by DPP: wave_shl:1 (CTRL 0x130)
// gives lane i the value of lane i + 1, wave_shr:1 (0x138) that of lane i - 1;
// the lane with no source (the last, the first) gets 0.  On the VALU, unlike
// a ds_bpermute shuffle, which goes through the LDS unit.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_wave_shift(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// The 16 bytes of lane + 1 (down) or lane - 1 (up) within the wave.  Callers
// use only values that come from active lanes.
__device__ __forceinline__ uint4 shfl_line_down(const uint4 &x)
{
    return make_uint4(dpp_wave_shift<0x130>(x.x), dpp_wave_shift<0x130>(x.y),
                      dpp_wave_shift<0x130>(x.z), dpp_wave_shift<0x130>(x.w));
}

__device__ __forceinline__ uint4 shfl_line_up(const uint4 &x)
{
    return make_uint4(dpp_wave_shift<0x138>(x.x), dpp_wave_shift<0x138>(x.y),
                      dpp_wave_shift<0x138>(x.z), dpp_wave_shift<0x138>(x.w));
}

// x moved across lanes by one DPP pattern (both 32-bit halves).  Only the
// rows in ROW_MASK receive a defined value.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_moved(double x)
{
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK,
                                                              0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL,
                                                              ROW_MASK, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// fp64 sum over the 64 lanes of a wave in a fixed order, returned to every
// lane; every lane must be active.  DPP within each 16-lane row (two quad
// permutes, then the half-row and row mirrors leave the row's sum in all its
// lanes); then row 1 adds row 0 and row 3 adds row 2 (row_bcast:15, rows 1
// and 3 only), and row 3 adds row 1 (row_bcast:31, rows 2 and 3), so lane 63
// holds the total, which is read out.  Rows 0 and 2 end undefined and are
// never read.  No LDS.
__device__ __forceinline__ double wave_sum(double x)
{
    x += dpp_moved<0xB1>(x);       // quad_perm [1, 0, 3, 2]
    x += dpp_moved<0x4E>(x);       // quad_perm [2, 3, 0, 1]
    x += dpp_moved<0x141>(x);      // row_half_mirror
    x += dpp_moved<0x140>(x);      // row_mirror
    x += dpp_moved<0x142, 0xA>(x); // row_bcast:15 into rows 1 and 3
    x += dpp_moved<0x143, 0xC>(x); // row_bcast:31 into rows 2 and 3
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// ================================================================ flatten
// Segments per launch (kernel-argument table), found by a two-level search:
// 16 coarse entries, then 8 fine ones, each level one scalar load.
constexpr int kSegFan = 8;
constexpr int kSegCoarse = 16;
constexpr int kMaxSegs = kSegCoarse * kSegFan;
constexpr int kFlatChunksPerThread = ZERO_FLAT_CPT;
constexpr uint64_t kFlatTileChunks = (uint64_t)kBlock * kFlatChunksPerThread;

// Gather modes: a plain copy, or a copy that also sums the squares of the
// 16-bit values each tile writes (fp16 or bf16), one fp64 partial per tile.
enum { kCopy = 0, kStatsF16 = 1, kStatsBF16 = 2 };

constexpr uint32_t kTilePad = 0x7fffffffu;  // table entries past the last segment

struct FlatArgs {
    uint32_t coarse[kSegCoarse];   // coarse[j] = tile_lo[kSegFan * j] (one 64-byte load)
    char *dst;                     // element 0 of the destination range
    double *part;                  // per-tile partial sums (stats modes)
    uint64_t tile_base;            // global index of this launch's first tile
    uint32_t n_segs;
    uint32_t dst_phase;            // (dst address mod 16) / element size
    uint32_t n_tiles;              // tiles of this launch
    uint32_t tile_lo[kMaxSegs + kSegFan];  // first tile of each segment, then
                                           // n_tiles, then kTilePad
    uint64_t seg_lo[kMaxSegs + 1]; // destination element offset of each segment
    const char *src[kMaxSegs];     // address of each segment's first source element
};

// Entries c of a table that are <= t, for values below 2^31: t - c is then
// negative exactly when c > t.
template <int N>
__device__ __forceinline__ uint32_t count_le(const uint32_t *c, uint32_t t)
{
    uint32_t above = 0;
#pragma unroll
    for (int i = 0; i < N; ++i)
        above += (t - c[i]) >> 31;
    return N - above;
}

// Segment of tile `tile`: the largest s with tile_lo[s] <= tile (uniform).
// tile_lo rises strictly from tile_lo[0] = 0 and then reads values above
// every tile, so s + 1 is the count of entries <= tile: found as a count
// among the coarse entries, then among the chosen slot's fine entries.
__device__ __forceinline__ uint32_t find_segment(const FlatArgs &a, uint32_t tile)
{
    const uint32_t j = count_le<kSegCoarse>(a.coarse, tile) - 1;
    return j * kSegFan + count_le<kSegFan>(a.tile_lo + j * kSegFan, tile) - 1;
}

// ------------------------------------------------------------ host helpers
inline bool aligned(const void *p, uintptr_t k) { return ((uintptr_t)p & (k - 1)) == 0; }

inline bool overlap(const void *a, uint64_t an, const void *b, uint64_t bn)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return an && bn && x < y + bn && y < x + an;
}

inline zero_status launch_status(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ZERO_EDEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ZERO_OK;
}

// Blocks of `kernel` that the current device keeps resident at once (CUs x
// blocks per CU from the occupancy calculator), cached per device.
template <typename K>
uint32_t resident_blocks(K kernel, size_t dyn_lds = 0)
{
    constexpr int kMaxDev = 64;
    static std::atomic<uint32_t> cache[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
        return 1024;
    uint32_t v = cache[dev].load(std::memory_order_relaxed);
    if (v)
        return v;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, dyn_lds) !=
            hipSuccess ||
        per_cu <= 0)
        per_cu = 4;
    v = (uint32_t)(cus * per_cu);
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

// Blocks of one launch.  A dispatch is kept below 2^31 work-items, inside
// both the dispatch packet's 32-bit grid size and the runtime's int-typed grid
// limits; a multiple of 8, so that a capped grid spans whole rounds of XCDs.
// A smaller cap (a multiple of 8) can be set at build time to exercise the
// multi-launch and multi-round paths on small inputs.
#ifndef ZERO_MAX_LAUNCH_BLOCKS
#define ZERO_MAX_LAUNCH_BLOCKS (0x7fffffffu / kBlock / 8 * 8)
#endif
constexpr uint64_t kMaxLaunchBlocks = ZERO_MAX_LAUNCH_BLOCKS;
static_assert(kMaxLaunchBlocks >= 8 && kMaxLaunchBlocks % 8 == 0 &&
                  kMaxLaunchBlocks <= 0x7fffffffu / kBlock,
              "launch cap: a positive multiple of 8 below 2^31 work-items");

inline uint32_t grid_for(uint64_t work_items, uint64_t per_block, uint32_t max_blocks)
{
    uint64_t b = (work_items + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > max_blocks) b = max_blocks;
    return (uint32_t)b;
}

// Tiles of one gather launch: one block each (and fewer than kTilePad).
constexpr uint64_t kMaxLaunchTiles = kMaxLaunchBlocks;
static_assert(kMaxLaunchTiles < kTilePad, "tile indices must stay below the table padding");

// Checks the tensor table and the range [range_begin, range_begin + count)
// of the flat stream; *range_end receives its end.
inline zero_status check_range(const char *what, const void *const *tensor_ptrs, const uint64_t *numel,
                               uint32_t n_tensors, uint64_t range_begin, uint64_t count,
                               uint64_t *range_end)
{
    if (n_tensors > 0 && (!tensor_ptrs || !numel))
        return fail(ZERO_EINVAL, "%s: NULL tensor table", what);
    uint64_t psi = 0;
    for (uint32_t i = 0; i < n_tensors; ++i)
        if (__builtin_add_overflow(psi, numel[i], &psi))
            return fail(ZERO_EINVAL, "%s: total size overflows", what);
    if (__builtin_add_overflow(range_begin, count, range_end) || *range_end > psi)
        return fail(ZERO_EINVAL, "%s: range [%llu, +%llu) beyond %llu elements", what,
                    (unsigned long long)range_begin, (unsigned long long)count,
                    (unsigned long long)psi);
    if (count > UINT64_MAX / 4)
        return fail(ZERO_EINVAL, "%s: count too large", what);
    return ZERO_OK;
}

// A device buffer that the tensors read by a segment launch must not overlap.
struct Guard {
    const void *p;
    uint64_t bytes;
    const char *name;
};

// Cuts the range [range_begin, range_end) of the tensors' flat stream into
// segment tables and launches each one with launch(a): every intersecting
// tensor is one segment, or several when a launch has room for fewer tiles.
// Tiles follow the 16-byte lines of a notional destination whose element 0
// sits at element phase ph (es-byte elements): a segment's full lines go in
// tiles of kFlatTileChunks lines, and a segment without a full line takes one
// tile.  a.tile_base counts the tiles of earlier launches.  Every
// intersecting tensor must be non-NULL, aligned to es and overlap none of
// the guards.  *n_tiles: tiles used in all.
template <typename Launch>
zero_status segment_launches(const char *what, const void *const *tensor_ptrs,
                             const uint64_t *numel, uint32_t n_tensors, uint64_t es,
                             uint64_t range_begin, uint64_t range_end, uint64_t ph,
                             const Guard *guards, int n_guards, FlatArgs &a, Launch launch,
                             uint64_t *n_tiles)
{
    *n_tiles = 0;
    const uint64_t V = 16 / es;
    auto seg_tiles = [&](uint64_t d_lo, uint64_t d_hi) {
        const uint64_t c0 = (d_lo + ph + V - 1) / V, c1 = (d_hi + ph) / V;
        const uint64_t full = c1 > c0 ? c1 - c0 : 0;
        return full ? (full + kFlatTileChunks - 1) / kFlatTileChunks : (uint64_t)1;
    };

    // check every intersecting tensor before launching anything
    uint64_t start = 0;
    for (uint32_t i = 0; i < n_tensors; ++i) {
        const uint64_t t_lo = start, t_hi = start + numel[i];
        start = t_hi;
        const uint64_t lo = t_lo > range_begin ? t_lo : range_begin;
        const uint64_t hi = t_hi < range_end ? t_hi : range_end;
        if (lo >= hi)
            continue;
        const char *src = (const char *)tensor_ptrs[i];
        if (!src)
            return fail(ZERO_EINVAL, "%s: NULL pointer for tensor %u", what, i);
        if (!aligned(src, es))
            return fail(ZERO_EALIGN, "%s: tensor %u not %llu-byte aligned", what, i,
                        (unsigned long long)es);
        for (int k = 0; k < n_guards; ++k)
            if (overlap(src + (lo - t_lo) * es, (hi - lo) * es, guards[k].p, guards[k].bytes))
                return fail(ZERO_EINVAL, "%s: %s overlaps tensor %u", what, guards[k].name, i);
    }

    a.n_segs = 0;
    a.tile_base = 0;
    a.dst_phase = (uint32_t)ph;
    uint64_t launch_tiles = 0;  // tiles of the segments in the table
    // launches the segments in the table, after completing the search tables
    auto flush = [&]() -> zero_status {
        a.n_tiles = (uint32_t)launch_tiles;
        a.tile_lo[a.n_segs] = a.n_tiles;
        for (uint32_t i = a.n_segs + 1; i < (uint32_t)(kMaxSegs + kSegFan); ++i)
            a.tile_lo[i] = kTilePad;
        for (int j = 0; j < kSegCoarse; ++j)
            a.coarse[j] = a.tile_lo[kSegFan * j];
        const zero_status st = launch(a);
        a.tile_base += launch_tiles;
        a.n_segs = 0;
        launch_tiles = 0;
        return st;
    };
    start = 0;
    for (uint32_t i = 0; i < n_tensors; ++i) {
        const uint64_t t_lo = start, t_hi = start + numel[i];
        start = t_hi;
        const uint64_t lo = t_lo > range_begin ? t_lo : range_begin;
        const uint64_t hi = t_hi < range_end ? t_hi : range_end;
        if (lo >= hi)
            continue;
        // destination elements [d_lo, d_hi), as one segment, or as several if the
        // launch has room for fewer tiles: a piece then ends after `room` tiles
        // of whole lines, so the pieces have the tiles of the whole
        uint64_t d_lo = lo - range_begin;
        const uint64_t d_hi = hi - range_begin;
        const char *src = (const char *)tensor_ptrs[i] + (lo - t_lo) * es;
        while (d_lo < d_hi) {
            const uint64_t room = kMaxLaunchTiles - launch_tiles;  // > 0
            uint64_t tiles = seg_tiles(d_lo, d_hi), d_end = d_hi;
            if (tiles > room) {
                d_end = ((d_lo + ph + V - 1) / V + room * kFlatTileChunks) * V - ph;
                tiles = room;
            }
            const uint32_t s = a.n_segs;
            a.seg_lo[s] = d_lo;
            a.seg_lo[s + 1] = d_end;
            a.src[s] = src;
            a.tile_lo[s] = (uint32_t)launch_tiles;
            launch_tiles += tiles;
            a.n_segs = s + 1;
            src += (d_end - d_lo) * es;
            d_lo = d_end;
            if (a.n_segs == kMaxSegs || launch_tiles == kMaxLaunchTiles ||
                (d_lo == d_hi && hi == range_end))
                if (zero_status st = flush(); st != ZERO_OK)
                    return st;
        }
    }
    *n_tiles = a.tile_base;
    return ZERO_OK;
}

}  // namespace
