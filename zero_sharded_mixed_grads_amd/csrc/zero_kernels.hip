// Device path of libzero_mi355x for AMD MI355X (gfx950, CDNA4, wave64).
//
// Three HBM-bound streaming kernels and one-thread / one-block epilogues:
//   flatten_segments  - list-order gather of tensors into a contiguous buffer
//                       ("ZeRO: Memory Optimizations Toward Training Trillion
//                       Parameter Models", paper summary page, section ZeRO-R
//                       > CB: constant-size fused buffers); in its statistics
//                       modes it also sums the squares of what it writes
//   stats_pass1, stats_reduce, stats_final
//                     - overflow flag and fp64 squared norm of a 16-bit
//                       gradient shard, fixed-order reduction of per-tile sums
//   adam_scalars      - per-step scalars in fp64 (skip, clip, bias corrections)
//   adamw_stream      - the fused AdamW update of one rank's shard (same page,
//                       section ZeRO-DP, Stage 1: each rank updates only its
//                       1/Nd of the optimizer state; section メモリ消費の定量化:
//                       16-bit params and grads, fp32 master, momentum and
//                       variance), 28 bytes of HBM traffic per element
//   loss_scale_init, loss_scale_update
//                     - the device-resident dynamic loss scale (Micikevicius
//                       et al., "Mixed Precision Training")
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
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "zero_internal.h"

using zero::fail;

namespace {

#ifndef ZERO_BLOCK
#define ZERO_BLOCK 256
#endif
constexpr int kBlock = ZERO_BLOCK;  // threads per block (waves of 64 lanes)

// Tuning constants of the streaming kernels (compile-time; the values are the
// measured best on the 1.5B shard).
#ifndef ZERO_ADAM_UNROLL
#define ZERO_ADAM_UNROLL 1   // 8-element chunks per lane kept in flight
#endif
#ifndef ZERO_FLAT_CPT
#define ZERO_FLAT_CPT 1      // 16-byte lines per thread in a flatten tile
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

// The 16 bytes of lane `lane + d` (d = +1 or -1 within the wave).
__device__ __forceinline__ uint4 shfl_line_down(const uint4 &x)
{
    return make_uint4(__shfl_down(x.x, 1, 64), __shfl_down(x.y, 1, 64), __shfl_down(x.z, 1, 64),
                      __shfl_down(x.w, 1, 64));
}

__device__ __forceinline__ uint4 shfl_line_up(const uint4 &x)
{
    return make_uint4(__shfl_up(x.x, 1, 64), __shfl_up(x.y, 1, 64), __shfl_up(x.z, 1, 64),
                      __shfl_up(x.w, 1, 64));
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
    const uint32_t tile = blockIdx.x;  // one tile per block: the grid is the tile count
    const uint32_t s = find_segment(a, tile);
    const uint64_t e_lo = a.seg_lo[s], e_hi = a.seg_lo[s + 1];
    const uint64_t ph = a.dst_phase;
    // full destination lines inside the segment: [c0, c1) in line units
    const uint64_t c0 = (e_lo + ph + V - 1) / V, c1 = (e_hi + ph) / V;
    const bool has_full = c1 > c0;
    const uint64_t k = tile - a.tile_lo[s];  // tile within the segment
    const char *src = a.src[s];
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
                reinterpret_cast<uint16_t *>(a.dst)[e] = v;
                if constexpr (MODE != kCopy) {
                    const double x = (double)to_f32<MODE == kStatsBF16>(v);
                    acc = fma(x, x, acc);
                }
            } else {
                reinterpret_cast<uint32_t *>(a.dst)[e] =
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
        char *dl = a.dst + (c0 * V - ph) * ES;
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
// same per-tile partial.  The loads of all its tiles are issued before any is
// summed, so a block keeps several lines per thread in flight.
constexpr int kStatsTilesPerBlock = 4;

template <bool BF16>
__global__ void __launch_bounds__(kBlock) stats_segments(FlatArgs a)
{
    constexpr int T = kStatsTilesPerBlock;
    uint4 lo[T], hi[T];
    uint32_t sb[T];
    bool line[T];
    uint16_t edge[T];
    bool has_edge[T];
    // the lines of every tile first, then the edge elements, then the sums
#pragma unroll
    for (int q = 0; q < T; ++q) {
        line[q] = has_edge[q] = false;
        sb[q] = 0;
        hi[q] = make_uint4(0, 0, 0, 0);
        const uint32_t tile = blockIdx.x * T + q;
        if (tile >= a.n_tiles)
            continue;
        const uint32_t s = find_segment(a, tile);
        const uint64_t e_lo = a.seg_lo[s], e_hi = a.seg_lo[s + 1];
        const uint64_t ph = a.dst_phase;
        const uint64_t c0 = (e_lo + ph + 7) / 8, c1 = (e_hi + ph) / 8;
        const bool has_full = c1 > c0;
        const uint64_t k = tile - a.tile_lo[s];
        const uint16_t *src = reinterpret_cast<const uint16_t *>(a.src[s]);
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
#pragma unroll
    for (int q = 0; q < T; ++q) {
        double acc = 0.0;
        if (has_edge[q]) {
            const double x = (double)to_f32<BF16>(edge[q]);
            acc = fma(x, x, acc);
        }
        if (line[q]) {
            const uint4 o = sb[q] ? shift_lines_rt(lo[q], hi[q], sb[q]) : lo[q];
            accum2<BF16>(o.x, acc);
            accum2<BF16>(o.y, acc);
            accum2<BF16>(o.z, acc);
            accum2<BF16>(o.w, acc);
        }
        const uint32_t tile = blockIdx.x * T + q;
        if (tile < a.n_tiles) {  // uniform: every thread of the block takes the barrier
            const double t = block_sum(acc);
            if (threadIdx.x == 0)
                a.part[a.tile_base + tile] = t;
        }
    }
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

// One tile per block: block b leaves the partial of tile tile0 + b.
template <bool BF16>
__global__ void __launch_bounds__(kBlock)
    stats_pass1(const uint16_t *g, uint64_t head, uint64_t nchunks, uint64_t tail_beg, uint64_t n,
                uint64_t tile0, double *part)
{
    double acc = 0.0;
    const uint64_t tile = tile0 + blockIdx.x;
    stats_tile<BF16>(g, head, nchunks, tail_beg, n, tile, acc);
    const double t = block_sum(acc);
    if (threadIdx.x == 0)
        part[tile] = t;
}

// A fixed number of partials for any n: block b sums tiles b, b + gridDim.x,
// b + 2 gridDim.x, ... and leaves one partial, part[b].
template <bool BF16>
__global__ void __launch_bounds__(kBlock)
    stats_pass1_strided(const uint16_t *g, uint64_t head, uint64_t nchunks, uint64_t tail_beg,
                        uint64_t n, uint64_t tiles, double *part)
{
    double acc = 0.0;
    for (uint64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x)
        stats_tile<BF16>(g, head, nchunks, tail_beg, n, tile, acc);
    const double t = block_sum(acc);
    if (threadIdx.x == 0)
        part[blockIdx.x] = t;
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

// ================================================================= AdamW
// Per-step scalars, computed once in fp64 by one thread.
__global__ void adam_scalars(zero_adamw hp, const zero_grad_stats_t *stats,
                             const zero_loss_scale_t *scale, zero_adam_state_t *st)
{
    if (threadIdx.x != 0 || blockIdx.x != 0)
        return;
    const uint32_t overflow = stats ? stats->overflow : 0u;
    if (overflow) {  // skipped step: nothing advances
        st->skip = 1;
        return;
    }
    const uint64_t t = st->step + 1;
    double coef = 1.0;
    if (stats && hp.max_grad_norm > 0.0) {
        const double sq = stats->sq_norm;
        if (sq > 0.0) {
            const double norm = sqrt(sq);
            if (hp.max_grad_norm < norm)
                coef = hp.max_grad_norm / norm;
        }
    }
    st->step = t;
    st->skip = 0;
    st->coef = coef;
    st->inv_scale = scale ? scale->inv_scale : hp.inv_loss_scale;
    const double bc1 = 1.0 - pow(hp.beta1, (double)t);
    const double bc2 = 1.0 - pow(hp.beta2, (double)t);
    st->bc1 = bc1;
    st->bc2 = bc2;
    st->inv_bc1 = 1.0 / bc1;
    st->inv_bc2 = 1.0 / bc2;
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

// Hyper-parameters of the element update, fp64, from the host: beta1, beta2,
// eps and lr as given, 1 - beta1, 1 - beta2 and lr * wd formed in fp64.
struct AdamHyper {
    double b1, omb1, b2, omb2, eps, lr, lrwd;
};

struct AdamArgs {
    const uint16_t *g;
    float *master, *m, *v;
    uint16_t *p;
    const zero_adam_state_t *st;
    AdamHyper h;
    uint64_t n;
    uint64_t head;     // elements [0, head) go element by element
    uint64_t nchunks;  // then nchunks chunks of 8 elements
    uint32_t g_phase;  // slot (0..7) of element `head` of g within its 16-byte line
    uint32_t p_phase;  // same for p
};

// Everything one element's update needs: the host's hyper-parameters and the
// step's device scalars (inverse loss scale, clip coefficient, bias
// corrections and their correctly rounded reciprocals).
struct Coeffs {
    AdamHyper h;
    double inv, coef, bc1, bc2, inv_bc1, inv_bc2;
};

// a / b rounded to nearest, given rb = RN(1 / b): the product a * rb is
// within one ulp of the quotient, and one fused correction with the exact
// residual a - b q0 rounds it correctly (Markstein's theorem: P. Markstein,
// "Computation of elementary functions on the IBM RISC System/6000
// processor", IBM J. Res. Dev. 34(1), 1990), for finite a and b without
// underflow, which holds here (|a| is 0 or above 2^-160, b in (0, 1]).
// SIGNED_ZERO: a may be -0, which is returned as it is (a / b keeps the sign
// of a zero dividend; the correction would give +0).
template <bool SIGNED_ZERO>
__device__ __forceinline__ double div_by(double a, double b, double rb)
{
#pragma clang fp contract(off)
    const double q0 = a * rb;
    const double r = __builtin_fma(-b, q0, a);
    const double q = __builtin_fma(r, rb, q0);
    if constexpr (SIGNED_ZERO)
        return a == 0.0 ? a : q;
    else
        return q;
}

// One element of AdamW in fp64, every operation correctly rounded and none
// fused, in the order the update is written: the fp32 results are the
// roundings of the exact fp64 sequence.
__device__ __forceinline__ void adamw_elem(const Coeffs &k, float graw, float &th, float &m,
                                           float &v)
{
#pragma clang fp contract(off)
    const double g = ((double)graw * k.inv) * k.coef;
    const double m1 = k.h.b1 * (double)m + k.h.omb1 * g;
    const double v1 = k.h.b2 * (double)v + (k.h.omb2 * g) * g;
    const double m_hat = div_by<true>(m1, k.bc1, k.inv_bc1);
    const double v_hat = div_by<false>(v1, k.bc2, k.inv_bc2);  // v1 is +0 or positive
    const double p = (double)th;
    const double p1 = (p - k.h.lrwd * p) - (k.h.lr * m_hat) / (__builtin_sqrt(v_hat) + k.h.eps);
    th = (float)p1;
    m = (float)m1;
    v = (float)v1;
}

constexpr int kAdamUnroll = ZERO_ADAM_UNROLL;

// Dynamic LDS reserved by every AdamW block, which uses none.  Of gfx950's
// 160 KiB of LDS per CU it leaves room for three blocks (twelve waves) per
// CU, below the four or five that the registers allow.  With fewer streams
// in flight at once HBM serves the kernel's five arrays faster, and three
// blocks hide the fp64 arithmetic: on the 1.5B shard 7.02 ms per step
// against 7.40 ms at two blocks per CU and 7.17 ms at four; on the 13B
// shard 57.9 ms against 61.0 and 59.2.
#ifndef ZERO_ADAM_LDS
#define ZERO_ADAM_LDS (48 * 1024)
#endif
constexpr size_t kAdamLdsReserve = ZERO_ADAM_LDS;

// Whether chunk c's right neighbour c + 1 is not held by the next lane of the
// same wave: c is on the last lane, or c + 1 is past the body.  Chunks of one
// unrolled step are consecutive across the lanes of a wave.
__device__ __forceinline__ bool edge_hi(uint64_t c, uint64_t nchunks)
{
    return threadIdx.x % 64 == 63 || c + 1 >= nchunks;
}

template <bool GBF16, bool PBF16, bool G_ALIGNED, bool P_ALIGNED>
__global__ void __launch_bounds__(kBlock) adamw_stream(AdamArgs a)
{
    const zero_adam_state_t *st = a.st;
    if (st->skip)
        return;
    const Coeffs k{a.h, st->inv_scale, st->coef, st->bc1, st->bc2, st->inv_bc1, st->inv_bc2};

    // aligned views of the body [head, head + 8 nchunks)
    float4 *th4 = reinterpret_cast<float4 *>(a.master + a.head);
    float4 *m4 = reinterpret_cast<float4 *>(a.m + a.head);
    float4 *v4 = reinterpret_cast<float4 *>(a.v + a.head);
    const uint4 *gl = reinterpret_cast<const uint4 *>(a.g + a.head - a.g_phase);
    uint16_t *pl = a.p + a.head - a.p_phase;  // aligned line holding element `head`
    const uint32_t gsb = 2 * a.g_phase;

    // One contiguous tile of kBlock * kAdamUnroll chunks per block.  Block i
    // runs on XCD i % 8, so tiles are renumbered to give each XCD (with its own
    // L2) a contiguous eighth of the shard.  Chunk j of a lane is base + j * step;
    // the loop takes a second round only if the grid was capped.
    const uint64_t stride = (uint64_t)gridDim.x * kBlock;
    const uint64_t step = kBlock;
    const uint64_t per_xcd = (gridDim.x + 7) / 8;
    const uint64_t tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const uint64_t first = tile * kBlock * kAdamUnroll + threadIdx.x;
    const uint64_t advance = stride * kAdamUnroll;
    for (uint64_t base = first; base < a.nchunks; base += advance) {
        uint4 gw[kAdamUnroll], ghi[kAdamUnroll];
        float4 th[kAdamUnroll][2], mm[kAdamUnroll][2], vv[kAdamUnroll][2];
#pragma unroll
        for (int j = 0; j < kAdamUnroll; ++j) {
            const uint64_t c = base + j * step;
            if (c < a.nchunks) {
                gw[j] = ld_stream(gl + c);
                if constexpr (!G_ALIGNED) {
                    // the next aligned line is the next lane's own line; only the
                    // last lane of the wave and the last chunk load it themselves
                    // (it holds at least one live element, so it is mapped)
                    if (edge_hi(c, a.nchunks))
                        ghi[j] = ld_stream(gl + c + 1);
                }
                th[j][0] = ld_stream(th4 + 2 * c); th[j][1] = ld_stream(th4 + 2 * c + 1);
                mm[j][0] = ld_stream(m4 + 2 * c);  mm[j][1] = ld_stream(m4 + 2 * c + 1);
                vv[j][0] = ld_stream(v4 + 2 * c);  vv[j][1] = ld_stream(v4 + 2 * c + 1);
            }
        }
#pragma unroll
        for (int j = 0; j < kAdamUnroll; ++j) {
            const uint64_t c = base + j * step;
            if (c < a.nchunks) {
                if constexpr (!G_ALIGNED) {
                    const uint4 nxt = shfl_line_down(gw[j]);
                    gw[j] = shift_lines_rt(gw[j], edge_hi(c, a.nchunks) ? ghi[j] : nxt, gsb);
                }
                const uint32_t gws[4] = {gw[j].x, gw[j].y, gw[j].z, gw[j].w};
                float *t = reinterpret_cast<float *>(th[j]);
                float *mv = reinterpret_cast<float *>(mm[j]);
                float *vw = reinterpret_cast<float *>(vv[j]);
                uint32_t ph[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t w = gws[e / 2];
                    const float graw = (e & 1) ? hi_to_f32<GBF16>(w) : to_f32<GBF16>(w & 0xffffu);
                    adamw_elem(k, graw, t[e], mv[e], vw[e]);
                    ph[e] = from_f32<PBF16>(t[e]);
                }
                st_stream(th4 + 2 * c, th[j][0]); st_stream(th4 + 2 * c + 1, th[j][1]);
                st_stream(m4 + 2 * c, mm[j][0]);  st_stream(m4 + 2 * c + 1, mm[j][1]);
                st_stream(v4 + 2 * c, vv[j][0]);  st_stream(v4 + 2 * c + 1, vv[j][1]);
                if constexpr (P_ALIGNED) {
                    store_run<0, 8>(pl + 8 * c, ph);
                } else {
                    // aligned line c holds the previous chunk's last p_phase values
                    // and this chunk's first 8 - p_phase: every lane but the first
                    // of the wave takes the former from its left neighbour and
                    // writes the whole line; the first lane writes only its head,
                    // and the lane whose right neighbour is absent writes its tail
                    const uint4 own = make_uint4(ph[0] | ph[1] << 16, ph[2] | ph[3] << 16,
                                                 ph[4] | ph[5] << 16, ph[6] | ph[7] << 16);
                    const uint4 prev = shfl_line_up(own);
                    if (threadIdx.x % 64 != 0)
                        st_stream(reinterpret_cast<uint4 *>(pl + 8 * c),
                                  shift_lines_rt(prev, own, 16 - 2 * a.p_phase));
                    else
                        store_head_rt(pl + 8 * c, ph, a.p_phase);
                    if (edge_hi(c, a.nchunks))
                        store_tail_rt(pl + 8 * c + 8, ph, a.p_phase);
                }
            }
        }
    }
    // elements outside the body, one per thread: [0, head) and the tail
    const uint64_t body_end = a.head + 8 * a.nchunks;
    const uint64_t n_edge = a.head + (a.n - body_end);
    for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < n_edge; i += stride) {
        const uint64_t e = i < a.head ? i : body_end + (i - a.head);
        float t = a.master[e], mv = a.m[e], vw = a.v[e];
        adamw_elem(k, to_f32<GBF16>(a.g[e]), t, mv, vw);
        a.master[e] = t;
        a.m[e] = mv;
        a.v[e] = vw;
        a.p[e] = (uint16_t)from_f32<PBF16>(t);
    }
}

// ------------------------------------------------- AdamW from tensor lists
// The same update over a range of the tensors' list-order flat stream, with
// every gradient read in place from its per-tensor buffer ("ZeRO: Memory
// Optimizations Toward Training Trillion Parameter Models", paper summary
// page, section ZeRO-R > CB: the gradients need no gathered copy when the
// per-tensor buffers already hold the rank's final gradients).  The segment
// table is the gather's: tiles follow the 8-element chunks of the fp32
// arrays (a notional 16-bit destination at phase (8 - head) % 8 has its lines
// exactly there), each tile inside one tensor's segment; a segment's
// elements outside whole chunks (at most 7 at each end) are updated one by
// one by the threads of its first tile.
struct AdamSegArgs {
    FlatArgs t;            // segment table (t.dst is unused)
    float *master, *m, *v; // element 0 of the range
    uint16_t *p;
    const zero_adam_state_t *st;
    AdamHyper h;
    uint64_t head;         // elements before the fp32 arrays' first 16-byte boundary
    uint32_t p_phase;      // slot (0..7) of element `head` of p within its 16-byte line
};
static_assert(sizeof(AdamSegArgs) <= 4096, "kernel arguments are limited to 4 KiB");

template <bool GBF16, bool PBF16, bool P_ALIGNED>
__global__ void __launch_bounds__(kBlock) adamw_segments(AdamSegArgs a)
{
    const zero_adam_state_t *st = a.st;
    if (st->skip)
        return;
    const Coeffs k{a.h, st->inv_scale, st->coef, st->bc1, st->bc2, st->inv_bc1, st->inv_bc2};
    // tiles renumbered so that each XCD (block i runs on XCD i % 8) streams a
    // contiguous eighth of the range; the grid is a multiple of 8
    const uint32_t per_xcd = gridDim.x / 8;
    const uint32_t tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (tile >= a.t.n_tiles)
        return;
    const uint32_t s = find_segment(a.t, tile);
    const uint64_t e_lo = a.t.seg_lo[s], e_hi = a.t.seg_lo[s + 1];
    const uint64_t ph = a.t.dst_phase;
    const uint64_t c0 = (e_lo + ph + 7) / 8, c1 = (e_hi + ph) / 8;  // whole chunks, line units
    const bool has_full = c1 > c0;
    const uint64_t kt = tile - a.t.tile_lo[s];  // tile within the segment
    const uint16_t *src = reinterpret_cast<const uint16_t *>(a.t.src[s]);  // gradient of e_lo
    if (kt == 0) {  // the segment's elements outside whole chunks, one per thread
        const uint64_t head_end = has_full ? c0 * 8 - ph : e_hi;
        const uint64_t tail_beg = has_full ? c1 * 8 - ph : e_hi;
        const uint64_t n_head = head_end - e_lo, n_tail = e_hi - tail_beg;
        if (threadIdx.x < n_head + n_tail) {
            const uint64_t e =
                threadIdx.x < n_head ? e_lo + threadIdx.x : tail_beg + (threadIdx.x - n_head);
            float t = a.master[e], mv = a.m[e], vw = a.v[e];
            adamw_elem(k, to_f32<GBF16>(ld_global(src + (e - e_lo))), t, mv, vw);
            a.master[e] = t;
            a.m[e] = mv;
            a.v[e] = vw;
            a.p[e] = (uint16_t)from_f32<PBF16>(t);
        }
    }
    if (!has_full)
        return;
    const uint64_t t_beg = kt * kFlatTileChunks;
    const uint64_t t_end = t_beg + kFlatTileChunks < c1 - c0 ? t_beg + kFlatTileChunks : c1 - c0;
    const uint64_t j = t_beg + threadIdx.x;  // this lane's chunk within the segment
    if (j >= t_end)
        return;
    // chunk of the segment's first whole line: line L holds elements
    // [8L - ph, 8L - ph + 8) = chunk L - 1 when head > 0, chunk L otherwise
    const uint64_t c = c0 - (a.head != 0) + j;
    const bool last = threadIdx.x % 64 == 63 || j + 1 >= t_end;  // no right neighbour
    // the gradients of chunk c: elements head + 8c .. + 7 of the range
    const uintptr_t g0 = (uintptr_t)(src + (a.head + 8 * (c0 - (a.head != 0)) - e_lo));
    const uint32_t gsb = (uint32_t)(g0 & 15u);  // uniform in the segment
    const uint4 *gl = reinterpret_cast<const uint4 *>(g0 - gsb) + j;
    float4 *th4 = reinterpret_cast<float4 *>(a.master + a.head);
    float4 *m4 = reinterpret_cast<float4 *>(a.m + a.head);
    float4 *v4 = reinterpret_cast<float4 *>(a.v + a.head);
    uint16_t *pl = a.p + a.head - a.p_phase;  // aligned line holding element `head`
    uint4 gw = ld_global(gl), ghi = make_uint4(0, 0, 0, 0);
    if (gsb != 0 && last)  // the next line holds live gradients of this chunk
        ghi = ld_global(gl + 1);
    float4 th[2] = {ld_stream(th4 + 2 * c), ld_stream(th4 + 2 * c + 1)};
    float4 mm[2] = {ld_stream(m4 + 2 * c), ld_stream(m4 + 2 * c + 1)};
    float4 vv[2] = {ld_stream(v4 + 2 * c), ld_stream(v4 + 2 * c + 1)};
    if (gsb != 0) {
        const uint4 nxt = shfl_line_down(gw);
        gw = shift_lines_rt(gw, last ? ghi : nxt, gsb);
    }
    const uint32_t gws[4] = {gw.x, gw.y, gw.z, gw.w};
    float *t = reinterpret_cast<float *>(th);
    float *mv = reinterpret_cast<float *>(mm);
    float *vw = reinterpret_cast<float *>(vv);
    uint32_t ph16[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t w = gws[e / 2];
        const float graw = (e & 1) ? hi_to_f32<GBF16>(w) : to_f32<GBF16>(w & 0xffffu);
        adamw_elem(k, graw, t[e], mv[e], vw[e]);
        ph16[e] = from_f32<PBF16>(t[e]);
    }
    st_stream(th4 + 2 * c, th[0]); st_stream(th4 + 2 * c + 1, th[1]);
    st_stream(m4 + 2 * c, mm[0]);  st_stream(m4 + 2 * c + 1, mm[1]);
    st_stream(v4 + 2 * c, vv[0]);  st_stream(v4 + 2 * c + 1, vv[1]);
    if constexpr (P_ALIGNED) {
        store_run<0, 8>(pl + 8 * c, ph16);
    } else {
        // as in adamw_stream: a lane with a left neighbour writes the whole line
        // it shares with it; the first lane of a wave writes its head, and a
        // lane without a right neighbour also its tail
        const uint4 own = make_uint4(ph16[0] | ph16[1] << 16, ph16[2] | ph16[3] << 16,
                                     ph16[4] | ph16[5] << 16, ph16[6] | ph16[7] << 16);
        const uint4 prev = shfl_line_up(own);
        if (threadIdx.x % 64 != 0)
            st_stream(reinterpret_cast<uint4 *>(pl + 8 * c),
                      shift_lines_rt(prev, own, 16 - 2 * a.p_phase));
        else
            store_head_rt(pl + 8 * c, ph16, a.p_phase);
        if (last)
            store_tail_rt(pl + 8 * c + 8, ph16, a.p_phase);
    }
}

// ------------------------------------------------------------ host helpers
inline bool aligned(const void *p, uintptr_t k) { return ((uintptr_t)p & (k - 1)) == 0; }

inline bool overlap(const void *a, uint64_t an, const void *b, uint64_t bn)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return an && bn && x < y + bn && y < x + an;
}

zero_status launch_status(const char *what)
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

template <int ES, int MODE>
zero_status flatten_launch(FlatArgs &a, hipStream_t stream)
{
    // one tile per block
    hipLaunchKernelGGL((flatten_segments<ES, MODE>), dim3(a.n_tiles), dim3(kBlock), 0, stream, a);
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

// Checks the tensor table and the range [range_begin, range_begin + count)
// of the flat stream; *range_end receives its end.
zero_status check_range(const char *what, const void *const *tensor_ptrs, const uint64_t *numel,
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

zero_status zero::launch_adam_scalars(const zero_adamw &hp, const zero_grad_stats_t *d_stats,
                                      const zero_loss_scale_t *d_scale,
                                      zero_adam_state_t *d_state, void *stream)
{
    hipLaunchKernelGGL(adam_scalars, dim3(1), dim3(64), 0, (hipStream_t)stream, hp, d_stats,
                       d_scale, d_state);
    return launch_status("adam step scalars");
}

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
    // one tile per block, in launches of at most kMaxLaunchBlocks blocks
    for (uint64_t t0 = 0; t0 < l.tiles; t0 += kMaxLaunchBlocks) {
        const uint32_t grid = (uint32_t)(l.tiles - t0 < kMaxLaunchBlocks ? l.tiles - t0
                                                                         : kMaxLaunchBlocks);
        if (gdt == ZERO_BF16)
            hipLaunchKernelGGL(stats_pass1<true>, dim3(grid), dim3(kBlock), 0, s, g, l.head,
                               l.nchunks, l.tail_beg, n, t0, part);
        else
            hipLaunchKernelGGL(stats_pass1<false>, dim3(grid), dim3(kBlock), 0, s, g, l.head,
                               l.nchunks, l.tail_beg, n, t0, part);
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
static_assert(kScratchPartials <= kFinalMax, "one block must finish the scratch partials");
static __device__ __align__(256) double scratch[kScratchPartials];

namespace {
// Device address of `scratch` on the current device, looked up once per device.
zero_status scratch_address(const char *what, double **out)
{
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static double *addr[kMaxDev];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
        return fail(ZERO_EDEVICE, "%s: no current HIP device (or device index %d >= %d)", what,
                    dev, kMaxDev);
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
    if (zero_status st = scratch_address(what, &part); st != ZERO_OK)
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
    if (gdt == ZERO_BF16)
        hipLaunchKernelGGL(stats_pass1_strided<true>, dim3((uint32_t)blocks), dim3(kBlock), 0, s,
                           g, l.head, l.nchunks, l.tail_beg, n, l.tiles, part);
    else
        hipLaunchKernelGGL(stats_pass1_strided<false>, dim3((uint32_t)blocks), dim3(kBlock), 0, s,
                           g, l.head, l.nchunks, l.tail_beg, n, l.tiles, part);
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

namespace {
template <bool GB, bool PB, bool GA, bool PA>
void launch_adam_variant(const AdamArgs &a, uint64_t work, hipStream_t s)
{
    auto kernel = adamw_stream<GB, PB, GA, PA>;
    const uint64_t per_block = (uint64_t)kBlock * kAdamUnroll;
    // one tile per block; the element-wise fallback keeps a resident grid
    uint32_t grid = a.nchunks ? grid_for(a.nchunks, per_block, kMaxLaunchBlocks)
                              : grid_for(work, per_block, resident_blocks(kernel, kAdamLdsReserve));
    if (a.nchunks)
        grid = (grid + 7) / 8 * 8;  // whole rounds of the 8 XCDs; spare blocks find no tile
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlock), kAdamLdsReserve, s, a);
}

template <bool GB, bool PB>
void launch_adam(const AdamArgs &a, uint64_t work, hipStream_t s)
{
    const bool ga = a.g_phase == 0, pa = a.p_phase == 0;
    if (ga && pa) launch_adam_variant<GB, PB, true, true>(a, work, s);
    else if (ga) launch_adam_variant<GB, PB, true, false>(a, work, s);
    else if (pa) launch_adam_variant<GB, PB, false, true>(a, work, s);
    else launch_adam_variant<GB, PB, false, false>(a, work, s);
}
}  // namespace

extern "C" zero_status zero_adam_step(const zero_adamw *hp, const void *grad, zero_dtype gdt,
                                      float *master, float *exp_avg, float *exp_avg_sq,
                                      void *param_out, zero_dtype pdt, uint64_t n,
                                      const zero_grad_stats_t *d_stats,
                                      const zero_loss_scale_t *d_scale, zero_adam_state_t *d_state,
                                      void *stream)
{
    if (!hp)
        return fail(ZERO_EINVAL, "zero_adam_step: NULL hyper-parameters");
    if (!d_state)
        return fail(ZERO_EINVAL, "zero_adam_step: NULL d_state");
    if ((gdt != ZERO_F16 && gdt != ZERO_BF16) || (pdt != ZERO_F16 && pdt != ZERO_BF16))
        return fail(ZERO_EINVAL, "zero_adam_step: grad and param dtypes must be F16 or BF16");
    if (zero_status hs = zero::check_adamw(*hp, d_scale == nullptr, "zero_adam_step");
        hs != ZERO_OK)
        return hs;
    if (n > 0 && (!grad || !master || !exp_avg || !exp_avg_sq || !param_out))
        return fail(ZERO_EINVAL, "zero_adam_step: NULL array with n > 0");
    if (n > UINT64_MAX / 4)
        return fail(ZERO_EINVAL, "zero_adam_step: n too large");
    if (!aligned(grad, 2) || !aligned(param_out, 2) || !aligned(master, 4) ||
        !aligned(exp_avg, 4) || !aligned(exp_avg_sq, 4) || !aligned(d_state, 8) ||
        !aligned(d_stats, 8) || !aligned(d_scale, 8))
        return fail(ZERO_EALIGN, "zero_adam_step: misaligned pointer");
    {
        const void *buf[8] = {grad, master, exp_avg, exp_avg_sq, param_out, d_state, d_stats,
                              d_scale};
        const uint64_t len[8] = {2 * n, 4 * n, 4 * n, 4 * n, 2 * n, sizeof(zero_adam_state_t),
                                 d_stats ? sizeof(zero_grad_stats_t) : 0,
                                 d_scale ? sizeof(zero_loss_scale_t) : 0};
        for (int i = 0; i < 8; ++i)
            for (int j = i + 1; j < 8; ++j)
                if (overlap(buf[i], len[i], buf[j], len[j]))
                    return fail(ZERO_EINVAL, "zero_adam_step: buffers %d and %d overlap", i, j);
    }
    hipStream_t s = (hipStream_t)stream;
    zero_status st = zero::launch_adam_scalars(*hp, d_stats, d_scale, d_state, stream);
    if (st != ZERO_OK || n == 0)
        return st;

    AdamArgs a{};
    a.g = (const uint16_t *)grad;
    a.master = master;
    a.m = exp_avg;
    a.v = exp_avg_sq;
    a.p = (uint16_t *)param_out;
    a.st = d_state;
    a.h = AdamHyper{hp->beta1, 1.0 - hp->beta1, hp->beta2, 1.0 - hp->beta2, hp->eps, hp->lr,
                    hp->lr * hp->weight_decay};
    a.n = n;
    const uintptr_t fph = ((uintptr_t)master & 15u) / 4;
    const bool same = fph == ((uintptr_t)exp_avg & 15u) / 4 && fph == ((uintptr_t)exp_avg_sq & 15u) / 4;
    if (same) {
        a.head = (4 - fph) % 4;
        if (a.head > n) a.head = n;
        a.nchunks = (n - a.head) / 8;
    } else {  // fp32 arrays at different 16-byte phases: element by element
        a.head = n;
        a.nchunks = 0;
    }
    a.g_phase = (uint32_t)((((uintptr_t)grad & 15u) / 2 + a.head) % 8);
    a.p_phase = (uint32_t)((((uintptr_t)param_out & 15u) / 2 + a.head) % 8);
    if (a.nchunks == 0) {
        a.g_phase = 0;
        a.p_phase = 0;
    }
    const uint64_t work = a.nchunks ? a.nchunks : n;
    const bool gb = gdt == ZERO_BF16, pb = pdt == ZERO_BF16;
    if (gb && pb) launch_adam<true, true>(a, work, s);
    else if (gb) launch_adam<true, false>(a, work, s);
    else if (pb) launch_adam<false, true>(a, work, s);
    else launch_adam<false, false>(a, work, s);
    return launch_status("zero_adam_step");
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
        const uint32_t grid = (t.n_tiles + kStatsTilesPerBlock - 1) / kStatsTilesPerBlock;
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

namespace {
template <bool GB, bool PB, bool PA>
zero_status launch_adam_segments(const AdamSegArgs &a, hipStream_t s)
{
    const uint32_t grid = (a.t.n_tiles + 7) / 8 * 8;  // whole rounds of the 8 XCDs
    hipLaunchKernelGGL((adamw_segments<GB, PB, PA>), dim3(grid), dim3(kBlock), kAdamLdsReserve,
                       s, a);
    return launch_status("zero_adam_step_tensors");
}
}  // namespace

extern "C" zero_status zero_adam_step_tensors(const zero_adamw *hp,
                                              const void *const *tensor_ptrs,
                                              const uint64_t *numel, uint32_t n_tensors,
                                              zero_dtype gdt, uint64_t range_begin,
                                              uint64_t count, float *master, float *exp_avg,
                                              float *exp_avg_sq, void *param_out, zero_dtype pdt,
                                              const zero_grad_stats_t *d_stats,
                                              const zero_loss_scale_t *d_scale,
                                              zero_adam_state_t *d_state, void *stream)
{
    const char *what = "zero_adam_step_tensors";
    if (!hp)
        return fail(ZERO_EINVAL, "%s: NULL hyper-parameters", what);
    if (!d_state)
        return fail(ZERO_EINVAL, "%s: NULL d_state", what);
    if ((gdt != ZERO_F16 && gdt != ZERO_BF16) || (pdt != ZERO_F16 && pdt != ZERO_BF16))
        return fail(ZERO_EINVAL, "%s: grad and param dtypes must be F16 or BF16", what);
    if (zero_status hs = zero::check_adamw(*hp, d_scale == nullptr, what); hs != ZERO_OK)
        return hs;
    uint64_t range_end;
    if (zero_status st = check_range(what, tensor_ptrs, numel, n_tensors, range_begin, count,
                                     &range_end);
        st != ZERO_OK)
        return st;
    if (count > 0 && (!master || !exp_avg || !exp_avg_sq || !param_out))
        return fail(ZERO_EINVAL, "%s: NULL array with count > 0", what);
    if (!aligned(param_out, 2) || !aligned(master, 4) || !aligned(exp_avg, 4) ||
        !aligned(exp_avg_sq, 4) || !aligned(d_state, 8) || !aligned(d_stats, 8) ||
        !aligned(d_scale, 8))
        return fail(ZERO_EALIGN, "%s: misaligned pointer", what);
    const uintptr_t fph = ((uintptr_t)master & 15u) / 4;
    if (count > 0 && (fph != ((uintptr_t)exp_avg & 15u) / 4 ||
                      fph != ((uintptr_t)exp_avg_sq & 15u) / 4))
        return fail(ZERO_EALIGN, "%s: master, exp_avg and exp_avg_sq must share their position "
                    "within 16 bytes", what);
    const void *buf[7] = {master, exp_avg, exp_avg_sq, param_out, d_state, d_stats, d_scale};
    static const char *const names[7] = {"master", "exp_avg", "exp_avg_sq", "param_out",
                                         "d_state", "d_stats", "d_scale"};
    const uint64_t len[7] = {4 * count, 4 * count, 4 * count, 2 * count,
                             sizeof(zero_adam_state_t), d_stats ? sizeof(zero_grad_stats_t) : 0,
                             d_scale ? sizeof(zero_loss_scale_t) : 0};
    for (int i = 0; i < 7; ++i)
        for (int j = i + 1; j < 7; ++j)
            if (overlap(buf[i], len[i], buf[j], len[j]))
                return fail(ZERO_EINVAL, "%s: buffers %d and %d overlap", what, i, j);
    // the tensors are checked against the outputs in segment_launches, before
    // any element kernel runs; the scalar kernel only touches d_state
    Guard guards[7];
    for (int i = 0; i < 7; ++i)
        guards[i] = Guard{buf[i], len[i], names[i]};
    hipStream_t s = (hipStream_t)stream;
    if (count == 0)
        return zero::launch_adam_scalars(*hp, d_stats, d_scale, d_state, stream);

    AdamSegArgs a{};
    a.master = master;
    a.m = exp_avg;
    a.v = exp_avg_sq;
    a.p = (uint16_t *)param_out;
    a.st = d_state;
    a.h = AdamHyper{hp->beta1, 1.0 - hp->beta1, hp->beta2, 1.0 - hp->beta2, hp->eps, hp->lr,
                    hp->lr * hp->weight_decay};
    a.head = (4 - fph) % 4;
    if (a.head > count)
        a.head = count;
    a.p_phase = (uint32_t)((((uintptr_t)param_out & 15u) / 2 + a.head) % 8);
    const bool gb = gdt == ZERO_BF16, pb = pdt == ZERO_BF16, pa = a.p_phase == 0;
    bool scalars_done = false;
    auto launch = [&](FlatArgs &t) -> zero_status {
        if (!scalars_done) {  // after every tensor has been checked
            if (zero_status st = zero::launch_adam_scalars(*hp, d_stats, d_scale, d_state, s);
                st != ZERO_OK)
                return st;
            scalars_done = true;
        }
        a.t = t;
        if (gb)
            return pb ? (pa ? launch_adam_segments<true, true, true>(a, s)
                            : launch_adam_segments<true, true, false>(a, s))
                      : (pa ? launch_adam_segments<true, false, true>(a, s)
                            : launch_adam_segments<true, false, false>(a, s));
        return pb ? (pa ? launch_adam_segments<false, true, true>(a, s)
                        : launch_adam_segments<false, true, false>(a, s))
                  : (pa ? launch_adam_segments<false, false, true>(a, s)
                        : launch_adam_segments<false, false, false>(a, s));
    };
    FlatArgs t{};
    uint64_t tiles = 0;
    return segment_launches(what, tensor_ptrs, numel, n_tensors, 2, range_begin, range_end,
                            (8 - a.head) % 8, guards, 7, t, launch, &tiles);
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
