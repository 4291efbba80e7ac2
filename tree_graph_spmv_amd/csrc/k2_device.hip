// k2_device.hip -- gfx950 kernels of the k^2-tree SpMV.
//
// Tosoni & Mencagli, "A GPU Engine for Sparse Matrix-Vector Products on
// k^2-Tree-Compressed Graphs":
//   Algorithm 1   fill y with the semiring zero, expand the frontier level by
//                 level (child j of node t gets code (F_t << 2) | b at offset
//                 off_t + j of the next level), and at the last internal level
//                 visit the leaves in place: leaf off_t + j of node t is the
//                 2x2 block at the origin decoded from (F_t << 2) | b, and
//                 each set bit q = 2*dr + dc of its signature is one cell.
//   Sec. 3.2      off_t = the popcounts of the signatures before t in the
//                 level, taken from a directory sample every 256 nodes plus
//                 the popcounts inside the block.
//   Sec. 3.4      tiles: ranges of nodes descended depth first.
//   Sec. 3.5      cached last internal level: one kernel over its nodes.
//   Sec. 3.6      left product: cell (r, c) adds x_r to y_c; batches are
//                 row-major n x B, B adjacent lanes per node.
//   Table 1       the semirings and their atomics.
//
// gfx950 mapping:
//   * workgroups of 256 threads = 4 wave64; one directory block (256 nodes)
//     per workgroup pass, so a block's offsets are one directory load plus an
//     exclusive scan of the fan-outs.  The scan uses three ballots, one per
//     bit of the fan-out (0..4), and popcounts of the lanes below; four wave
//     totals meet in LDS.
//   * the tiled descent keeps the whole frontier of a tile in LDS (two
//     buffers of tile_nodes codes); no frontier ever goes to HBM and a
//     product is one launch after the fill.
//   * a node's cells are folded per output index (the four rows, or columns,
//     of its 4x4 block) before the atomics, and a contribution equal to the
//     semiring zero (x = 0, or +inf for min-plus) issues no atomic.
//   * batches: B adjacent lanes per node, so one atomic instruction updates B
//     contiguous floats of a row (one memory request instead of B).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "k2_internal.h"

namespace k2 {

// ------------------------------------------------------------- semirings

struct PlusTimes {
    using T = float;
    // tree-only products use the band groups: every cell's contribution is an
    // atomic add that the windows absorb
    static constexpr bool kTreeBands = true;
    // window updates skip the zero tests: inputs are rarely zero, and adding
    // a zero leaves a window word as it is (windows start at +0 and never
    // hold -0)
    static constexpr bool kWindowUnchecked = true;
    static constexpr uint32_t kZeroBits = 0u;
    __device__ static T zero() { return 0.0f; }
    __device__ static bool contributes(T x) { return x != 0.0f; }
    __device__ static bool contributes_out(T v) { return v != 0.0f; }
    __device__ static T contrib(T x) { return x; }
    __device__ static T combine(T a, T b) { return a + b; }
    __device__ static void atomic(T *p, T v) {
        __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // LDS fp32 add as an integer compare-and-swap: at random window rows
    // gfx950's ds_add_f32 completes 8x fewer updates per second than this
    // loop (201 against 1599 G/s measured).  The first try
    // uses the value read just before, so it fails only when another lane
    // changed the word in between.
    __device__ static void lds_atomic(T *p, T v) {
        uint32_t *u = reinterpret_cast<uint32_t *>(p);
        uint32_t expected = __hip_atomic_load(u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        while (!__hip_atomic_compare_exchange_strong(u, &expected,
                                                     __float_as_uint(__uint_as_float(expected) + v),
                                                     __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP)) {
        }
    }
};

struct BooleanF32 {
    using T = float;
    // tree-only products take the whole rest cut, no band groups (see
    // PlusTimes and Tropical)
    static constexpr bool kTreeBands = false;
    static constexpr bool kWindowUnchecked = false;
    static constexpr uint32_t kZeroBits = 0u;
    __device__ static T zero() { return 0.0f; }
    __device__ static bool contributes(T x) { return (__float_as_uint(x) & 0x7FFFFFFFu) != 0u; }
    __device__ static bool contributes_out(T v) { return __float_as_uint(v) != 0u; }
    __device__ static T contrib(T) { return 1.0f; }
    __device__ static T combine(T a, T b) { return a > b ? a : b; }
    __device__ static void atomic(T *p, T v) {
        __hip_atomic_fetch_max(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ static void lds_atomic(T *p, T v) {
        __hip_atomic_fetch_max(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    }
};

struct BooleanU32 {
    using T = uint32_t;
    // tree-only products take the whole rest cut, no band groups (see
    // PlusTimes and Tropical)
    static constexpr bool kTreeBands = false;
    static constexpr bool kWindowUnchecked = false;
    static constexpr uint32_t kZeroBits = 0u;
    __device__ static T zero() { return 0u; }
    __device__ static bool contributes(T x) { return x != 0u; }
    __device__ static bool contributes_out(T v) { return v != 0u; }
    __device__ static T contrib(T x) { return x; }
    __device__ static T combine(T a, T b) { return a | b; }
    __device__ static void atomic(T *p, T v) {
        __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ static void lds_atomic(T *p, T v) {
        __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
};

struct Tropical {
    using T = float;
    // tree-only products take the whole rest cut, no band groups: the
    // groups' windows would absorb atomics, but contributions equal to the
    // zero (x = +inf) issue none, and relaxation steps skip most
    static constexpr bool kTreeBands = false;
    static constexpr bool kWindowUnchecked = false;
    static constexpr uint32_t kZeroBits = 0x7F800000u;   // +inf
    __device__ static T zero() { return __uint_as_float(kZeroBits); }
    __device__ static bool contributes(T x) { return x < __uint_as_float(kZeroBits); }
    __device__ static bool contributes_out(T v) { return __float_as_uint(v) != kZeroBits; }
    __device__ static T contrib(T x) { return 1.0f + x; }
    __device__ static T combine(T a, T b) { return a < b ? a : b; }
    // non-negative floats order like their bit patterns
    __device__ static void atomic(T *p, T v) {
        __hip_atomic_fetch_min(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ static void lds_atomic(T *p, T v) {
        __hip_atomic_fetch_min(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    }
};

// ------------------------------------------------------------- helpers

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Workgroups per CU the product kernels are compiled for: 8 x 4 waves fills
// the 8 wave slots of each SIMD (64 VGPRs); the leaf phase is latency-bound,
// so resident waves matter more than registers.
constexpr int kOccupancy = 8;
// Threads of the cached-level kernel's workgroups (one band tile each).
// Measured on web-like 2^27 at batch 8: 512 or 1024 threads per band keep
// fewer bands in flight per XCD (L2 hit rate 0.58 -> 0.65, a quarter fewer
// bytes read) but their waves wait at the window's closing barrier and
// collide in its compare-and-swaps: right product 11.1 -> 13.9 / 33 ms.
constexpr int kCachedThreads = 256;

__device__ __forceinline__ uint32_t nib(const uint64_t *__restrict__ w, uint64_t i) {
    return uint32_t(w[i >> 4] >> ((i & 15) * 4)) & 0xFu;
}

// even bits of v -> low half (the column index of a Morton code)
__device__ __forceinline__ uint32_t compact_even(uint64_t x) {
    x &= 0x5555555555555555ull;
    x = (x | (x >> 1)) & 0x3333333333333333ull;
    x = (x | (x >> 2)) & 0x0F0F0F0F0F0F0F0Full;
    x = (x | (x >> 4)) & 0x00FF00FF00FF00FFull;
    x = (x | (x >> 8)) & 0x0000FFFF0000FFFFull;
    x = (x | (x >> 16)) & 0x00000000FFFFFFFFull;
    return uint32_t(x);
}

// Inclusive prefix sum over the 64 lanes of a wave: four shifts within each
// row of 16 lanes (lanes shifted in from outside the row add 0), then row
// 0's total is added to row 1 and row 2's to row 3 (broadcast of lane 15),
// then lane 31's sum of rows 0-1 to rows 2 and 3 (broadcast of lane 31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xf, 0xf, true));    // row_shr:1
    v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xf, 0xf, true));    // row_shr:2
    v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xf, 0xf, true));    // row_shr:4
    v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xf, 0xf, true));    // row_shr:8
    v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x142, 0xa, 0xf, false));   // row_bcast:15
    v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x143, 0xc, 0xf, false));   // row_bcast:31
    return v;
}

// Exclusive prefix sum of f over the wave, and the wave's total.
__device__ __forceinline__ uint32_t wave_scan(uint32_t f, uint32_t &total) {
    const uint32_t incl = wave_incl_scan(f);
    total = uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
    return incl - f;
}

// Exclusive prefix sum of f over the workgroup: wave scans, then the four
// wave totals meet in LDS.
__device__ __forceinline__ uint32_t block_scan(uint32_t f, uint32_t *s_tot, uint32_t &total) {
    const unsigned wave = threadIdx.x >> 6;
    uint32_t wt;
    const uint32_t ex = wave_scan(f, wt);
    if (__lane_id() == 0) s_tot[wave] = wt;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        uint32_t v = s_tot[w];
        before += (w < int(wave)) ? v : 0u;
        tot += v;
    }
    __syncthreads();
    total = tot;
    return before + ex;
}

// Offset in level d+1 of the first child of node i of level d (i < nodes[d]):
// the directory sample of i's block plus the popcounts of the words before i
// in the block.  Computed by wave 0 and broadcast through LDS.
__device__ __forceinline__ uint32_t block_child_offset(const DevTree &t, int d, uint32_t i,
                                                       uint32_t *s_val) {
    if (threadIdx.x < 64) {
        const unsigned lane = __lane_id();
        const uint32_t blk = i >> 8;
        const uint32_t wi = i >> 4;                   // i's word
        const uint32_t w = blk * kWordsPerBlock + lane;
        uint32_t c = 0;
        if (lane < kWordsPerBlock && w <= wi) {
            uint64_t v = t.words[d][w];
            if (w == wi) {
                const unsigned sh = (i & 15) * 4;
                v = sh ? (v & ((1ull << sh) - 1)) : 0ull;
            }
            c = __popcll(v);
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) c += __shfl_xor(c, o, 16);
        if (lane == 0) *s_val = t.dir[d][blk] + c;
    }
    __syncthreads();
    const uint32_t r = *s_val;
    __syncthreads();
    return r;
}

// Offset in level d+1 of the first child of node i of level d (i < nodes[d]),
// computed by the calling wave alone: the directory sample of i's block plus
// the popcounts of the words before i in the block (lanes 0..15, one word
// each), summed across the wave.
__device__ __forceinline__ uint32_t wave_child_offset(const DevTree &t, int d, uint32_t i) {
    const unsigned lane = __lane_id();
    const uint32_t blk = i >> 8;
    const uint32_t wi = i >> 4;
    const uint32_t w = blk * kWordsPerBlock + lane;
    uint32_t c = 0;
    if (lane < kWordsPerBlock && w <= wi) {
        uint64_t v = t.words[d][w];
        if (w == wi) {
            const unsigned sh = (i & 15) * 4;
            v = sh ? (v & ((1ull << sh) - 1)) : 0ull;
        }
        c = __popcll(v);
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) c += __shfl_xor(c, o, 16);
    return __shfl(c, 0) + t.dir[d][blk];
}

// wave_child_offset for a level given by its signature words and directory.
__device__ __forceinline__ uint32_t wave_child_offset_of(const uint64_t *__restrict__ words,
                                                         const uint32_t *__restrict__ dir, uint32_t i) {
    const unsigned lane = __lane_id();
    const uint32_t blk = i >> 8;
    const uint32_t wi = i >> 4;
    const uint32_t w = blk * kWordsPerBlock + lane;
    uint32_t c = 0;
    if (lane < kWordsPerBlock && w <= wi) {
        uint64_t v = words[w];
        if (w == wi) {
            const unsigned sh = (i & 15) * 4;
            v = sh ? (v & ((1ull << sh) - 1)) : 0ull;
        }
        c = __popcll(v);
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) c += __shfl_xor(c, o, 16);
    return __shfl(c, 0) + dir[blk];
}

// Orders a wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------- kernels

// LDS of one wave's leaf segment: a round of the list of its cells, each as
// the element offsets of its input in x (input index * B) and of its output
// (output index * B in y, or relative to the tile's window).  A node has at
// most 4 leaves of 4 cells, so a segment has at most 1024 cells; they go
// through the buffer kRound at a time (one round in the common case).  Off is
// uint32_t when every offset fits, else uint64_t (half as many per round).
template <class Off, uint32_t kSlots = 512 / sizeof(Off)>
struct alignas(16) WaveCells {
    static constexpr uint32_t kRound = kSlots;
    Off xo[kRound];
    Off yo[kRound];
};

// cells whose x loads a lane issues before their atomics: as many as 64
// registers hold (64-bit offsets take twice the registers)
template <class Off>
constexpr int unroll_for() { return sizeof(Off) == 4 ? 8 : 4; }

// Output window of a tile: 'win' (LDS, or null) holds outputs [out0, out0 +
// rows) x B; cells of the tile all land inside it.
template <class T>
struct Window {
    T *win;
    uint64_t out0;
    uint32_t rows;
    bool runs;   // right products: combine runs of one output row (ring_pass)
};

// Row and column offsets within a node's 4x4 block of cell q of the leaf for
// child b, at bits 2 (4 b + q) of these words: b = 2 b1 + b0 and q = 2 q1 +
// q0 give row 2 b1 + q1 and column 2 b0 + q0.
constexpr uint32_t cell_offset_table(bool row) {
    uint32_t t = 0;
    for (uint32_t bit = 0; bit < 16; ++bit) {
        const uint32_t b = bit >> 2, q = bit & 3u;
        const uint32_t v = row ? 2u * (b >> 1) + (q >> 1) : 2u * (b & 1u) + (q & 1u);
        t |= v << (2 * bit);
    }
    return t;
}
constexpr uint32_t kCellRowTable = cell_offset_table(true);
constexpr uint32_t kCellColTable = cell_offset_table(false);

// The atomics of a lane's kUnroll cells (contributions xv, outputs yo + v of
// 'out': the LDS window when kWin, else y).  kRuns: the cells are
// consecutive in the list (ok[] a prefix), and runs of one output are
// combined into one atomic.
template <class SR, class Off, int kUnroll, bool kRuns, bool kWin>
__device__ __forceinline__ void apply_cells(const typename SR::T (&xv)[kUnroll], const Off (&yo)[kUnroll],
                                            const bool (&ok)[kUnroll], typename SR::T *__restrict__ out,
                                            uint32_t v) {
    using T = typename SR::T;
    // no zero tests where the semiring allows (window updates only)
    constexpr bool kUnchecked = kWin && SR::kWindowUnchecked;
    // plus-times window outputs o are byte offsets, the others element indexes
    char *const wv = reinterpret_cast<char *>(out) + v * uint32_t(sizeof(T));
    auto apply = [&](Off o, T c) {
        if constexpr (kWin && SR::kTreeBands) SR::lds_atomic(reinterpret_cast<T *>(wv + uint32_t(o)), c);
        else if constexpr (kWin) SR::lds_atomic(&out[o + v], c);
        else SR::atomic(&out[o + v], c);
    };
    if constexpr (kRuns) {
        T acc = SR::zero();
        Off cur = yo[0];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (ok[u]) {
                if (yo[u] != cur) {
                    if (kUnchecked || SR::contributes_out(acc)) apply(cur, acc);
                    acc = SR::zero();
                    cur = yo[u];
                }
                if (kUnchecked || SR::contributes(xv[u])) acc = SR::combine(acc, SR::contrib(xv[u]));
            }
        // ok[] is a prefix: a lane group with no cell (a pass's tail) has no
        // run, and its yo[0] is a ring slot past the queued cells
        if (ok[0] && (kUnchecked || SR::contributes_out(acc))) apply(cur, acc);
    } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (ok[u] && (kUnchecked || SR::contributes(xv[u]))) apply(yo[u], SR::contrib(xv[u]));
    }
}

// One pass over 'count' cells of a wave's ring from position 'head' (R
// slots, R a power of 2): VL lanes per cell, kUnroll cells per lane, their
// gathers issued before their atomics.  Without kRuns an instruction takes
// kUnroll-strided cells, G neighbours of the list at a time, whose x rows
// often share cache lines.  With kRuns each lane group takes kUnroll
// neighbours of the list and combines runs of equal outputs before their
// atomic: in a right product the cells of one row of a 4x4 block, and of
// horizontally adjacent blocks, are neighbours in Z order, so a row of many
// non-zeros would otherwise send several lanes of one instruction to the same
// word (serialised, and a failed compare-and-swap each).  kFull: count is
// exactly G x kUnroll (a full pass of the ring), so no slot needs a bounds
// test (about 5% fewer VALU instructions in a windowed right product).
template <class SR, class Off, bool kRuns, bool kFull = false, uint32_t kSlots>
__device__ __forceinline__ void pass_cells(const WaveCells<Off, kSlots> *wc, uint32_t head, uint32_t count,
                                           const typename SR::T *__restrict__ x,
                                           typename SR::T *__restrict__ y, uint32_t B, uint32_t VL,
                                           const Window<typename SR::T> &w) {
    using T = typename SR::T;
    constexpr uint32_t R = kSlots;
    constexpr int kUnroll = unroll_for<Off>();
    const uint32_t lane = __lane_id();
    const uint32_t G = 64 / VL, g = lane / VL, lv = lane % VL;
    // cell u of this lane is k0 + u * step
    const uint32_t step = kRuns ? 1u : G;
    for (uint32_t base = 0; base < count; base += G * kUnroll) {
        const uint32_t k0 = base + (kRuns ? g * uint32_t(kUnroll) : g);
        // slots past count repeat cell 'base' for the loads and skip the atomics
        Off xo[kUnroll], yo[kUnroll];
        bool ok[kUnroll];
        if constexpr (kFull) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const uint32_t at = (head + k0 + uint32_t(u) * step) & (R - 1u);
                ok[u] = true;
                xo[u] = wc->xo[at];
                yo[u] = wc->yo[at];
            }
        } else if constexpr (kRuns && sizeof(Off) == 4 && kUnroll == 8) {
            // a lane group's 8 cells are 8 consecutive slots from a multiple
            // of 8 (head and k0 both are: the ring advances by whole passes
            // of G x 8 cells), so they never wrap and load as 16-byte words
            const uint32_t at = (head + k0) & (R - 8u);   // R - 8: the same value, known aligned
            const uint4 xa = *reinterpret_cast<const uint4 *>(&wc->xo[at]);
            const uint4 xb = *reinterpret_cast<const uint4 *>(&wc->xo[at + 4u]);
            const uint4 ya = *reinterpret_cast<const uint4 *>(&wc->yo[at]);
            const uint4 yb = *reinterpret_cast<const uint4 *>(&wc->yo[at + 4u]);
            const Off x0 = wc->xo[(head + base) & (R - 1u)];
            const uint32_t xs[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
            const uint32_t ys[8] = {ya.x, ya.y, ya.z, ya.w, yb.x, yb.y, yb.z, yb.w};
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                ok[u] = k0 + uint32_t(u) < count;
                xo[u] = ok[u] ? Off(xs[u]) : x0;
                yo[u] = Off(ys[u]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const uint32_t k = k0 + uint32_t(u) * step;
                ok[u] = k < count;
                const uint32_t at = (head + (ok[u] ? k : base)) & (R - 1u);
                xo[u] = wc->xo[at];
                yo[u] = wc->yo[at];
            }
        }
        for (uint32_t v = lv; v < B; v += VL) {
            T xv[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) xv[u] = x[xo[u] + v];
            if (w.win) apply_cells<SR, Off, kUnroll, kRuns, true>(xv, yo, ok, w.win, v);
            else apply_cells<SR, Off, kUnroll, kRuns, false>(xv, yo, ok, y, v);
        }
    }
}

template <class SR, class Off, bool kMayRun, bool kFull = false, uint32_t kSlots>
__device__ __forceinline__ void ring_pass(const WaveCells<Off, kSlots> *wc, uint32_t head, uint32_t count,
                                          const typename SR::T *__restrict__ x,
                                          typename SR::T *__restrict__ y, uint32_t B, uint32_t VL,
                                          const Window<typename SR::T> &w) {
    if (kMayRun && w.runs) pass_cells<SR, Off, kMayRun, kFull>(wc, head, count, x, y, B, VL, w);
    else pass_cells<SR, Off, false, kFull>(wc, head, count, x, y, B, VL, w);
}

// Leaf work of one wave over a segment of up to 64 nodes of the last internal
// level; lane l holds the first row and column of node l's 4x4 block and its
// cells as a 16-bit mask (bit 4 b + q: cell q of the leaf for child b; 0: no
// node).
// Phase A (a lane per node): list the segment's cells in the wave's LDS, each
// as its x and output offsets, at positions from a wave scan of the cell
// counts.  Phase B (VL adjacent lanes per cell, one per vector): gather x for
// kUnroll cells, then apply the semiring's atomics, to the LDS window when
// the tile has one, else to y.  No workgroup barrier.
template <class SR, int DIR, class Off, uint32_t kSlots>
__device__ __forceinline__ void leaf_cells(uint32_t row0, uint32_t col0, uint32_t cells,
                                           const typename SR::T *__restrict__ x,
                                           typename SR::T *__restrict__ y, uint32_t B, uint32_t VL,
                                           Window<typename SR::T> w, WaveCells<Off, kSlots> *wc) {
    constexpr uint32_t R = kSlots;
    uint32_t total;
    const uint32_t pos0 = wave_scan(__popc(cells), total);
    const uint32_t obase = w.win ? uint32_t(w.out0) : 0u;
    // offsets of the block's first cell; a cell adds its in-block offset * B
    const Off xb = Off((DIR == K2_RIGHT) ? col0 : row0) * B;
    // plus-times window outputs as byte offsets into the window (one add
    // per update; measured slower for the packed Boolean semiring)
    const uint32_t yB = (SR::kTreeBands && w.win) ? B * uint32_t(sizeof(typename SR::T)) : B;
    const Off yb = Off(((DIR == K2_RIGHT) ? row0 : col0) - obase) * yB;
    constexpr uint32_t kInTable = (DIR == K2_RIGHT) ? kCellColTable : kCellRowTable;
    constexpr uint32_t kOutTable = (DIR == K2_RIGHT) ? kCellRowTable : kCellColTable;
    for (uint32_t round = 0; round < total; round += R) {
        // this lane's cells with list positions in [round, round + R)
        uint32_t m = cells, pos = pos0;
        while (m && pos < round + R) {
            const uint32_t sh = 2u * uint32_t(__builtin_ctz(m));
            m &= m - 1u;
            if (pos >= round) {
                wc->xo[pos - round] = xb + __umul24((kInTable >> sh) & 3u, B);
                wc->yo[pos - round] = yb + __umul24((kOutTable >> sh) & 3u, yB);
            }
            ++pos;
        }
        wave_lds_sync();
        const uint32_t n = (total - round < R) ? total - round : R;
        ring_pass<SR, Off, DIR == K2_RIGHT>(wc, 0u, n, x, y, B, VL, w);
        wave_lds_sync();
    }
}

// The cells of one segment (as for leaf_cells) queued in the wave's ring
// behind the 'fill' cells already there from 'head': whenever a full pass
// (G x kUnroll cells, at most the ring) is queued it runs, so a segment's
// last few cells wait for the next segment instead of taking a pass of
// their own.  ring_drain runs what is left at the end of a tile.
template <class SR, int DIR, class Off, uint32_t kSlots>
__device__ __forceinline__ void ring_cells(uint32_t row0, uint32_t col0, uint32_t cells,
                                           const typename SR::T *__restrict__ x,
                                           typename SR::T *__restrict__ y, uint32_t B, uint32_t VL,
                                           const Window<typename SR::T> &w, WaveCells<Off, kSlots> *wc,
                                           uint32_t &head, uint32_t &fill) {
    constexpr uint32_t R = kSlots;
    constexpr int kUnroll = unroll_for<Off>();
    uint32_t total;
    const uint32_t pos0 = wave_scan(__popc(cells), total);
    const uint32_t obase = w.win ? uint32_t(w.out0) : 0u;
    const Off xb = Off((DIR == K2_RIGHT) ? col0 : row0) * B;
    // plus-times window outputs as byte offsets into the window (one add
    // per update; measured slower for the packed Boolean semiring)
    const uint32_t yB = (SR::kTreeBands && w.win) ? B * uint32_t(sizeof(typename SR::T)) : B;
    const Off yb = Off(((DIR == K2_RIGHT) ? row0 : col0) - obase) * yB;
    constexpr uint32_t kInTable = (DIR == K2_RIGHT) ? kCellColTable : kCellRowTable;
    constexpr uint32_t kOutTable = (DIR == K2_RIGHT) ? kCellRowTable : kCellColTable;
    const uint32_t G = 64 / VL;
    const uint32_t P = (G * uint32_t(kUnroll) < R) ? G * uint32_t(kUnroll) : R;
    for (uint32_t done = 0; done < total;) {
        const uint32_t now = (total - done < R - fill) ? total - done : R - fill;
        // this lane's cells with segment positions in [done, done + now)
        uint32_t m = cells, pos = pos0;
        while (m && pos < done + now) {
            const uint32_t sh = 2u * uint32_t(__builtin_ctz(m));
            m &= m - 1u;
            if (pos >= done) {
                const uint32_t at = (head + fill + (pos - done)) & (R - 1u);
                wc->xo[at] = xb + __umul24((kInTable >> sh) & 3u, B);
                wc->yo[at] = yb + __umul24((kOutTable >> sh) & 3u, yB);
            }
            ++pos;
        }
        fill += now;
        done += now;
        wave_lds_sync();
        const bool full = P == G * uint32_t(kUnroll);
        while (fill >= P) {
            if (full) ring_pass<SR, Off, DIR == K2_RIGHT, true>(wc, head, P, x, y, B, VL, w);
            else ring_pass<SR, Off, DIR == K2_RIGHT, false>(wc, head, P, x, y, B, VL, w);
            head = (head + P) & (R - 1u);
            fill -= P;
        }
        wave_lds_sync();
    }
}

template <class SR, int DIR, class Off, uint32_t kSlots>
__device__ __forceinline__ void ring_drain(const typename SR::T *__restrict__ x, typename SR::T *__restrict__ y,
                                           uint32_t B, uint32_t VL, const Window<typename SR::T> &w,
                                           WaveCells<Off, kSlots> *wc, uint32_t &head, uint32_t &fill) {
    if (fill) ring_pass<SR, Off, DIR == K2_RIGHT>(wc, head, fill, x, y, B, VL, w);
    wave_lds_sync();
    head = 0;
    fill = 0;
}

// A node's cells as a 16-bit mask (bit 4 b + q: cell q of the leaf for
// child b) from ssh = s | p << 6 (signature s, first leaf nibble p of lo32)
// and the two leaf-level dwords holding its leaf nibbles: they are the low
// 4 * fan-out bits of (hi32:lo32) >> 4 p, in child order.
__device__ __forceinline__ uint32_t node_cells(uint32_t ssh, uint32_t lo32, uint32_t hi32) {
    const uint32_t s = ssh & 15u;
    uint32_t bits = uint32_t(((uint64_t(hi32) << 32) | lo32) >> ((ssh >> 4) & 28u));
    uint32_t cells = 0u;
#pragma unroll
    for (uint32_t b = 0; b < 4; ++b)
        if (s & (1u << b)) {
            cells |= (bits & 15u) << (4 * b);
            bits >>= 4;
        }
    return cells;
}

// leaf_cells for a lane whose node has Morton code 'code', signature s and
// first leaf 'off': its leaf nibbles come from two leaf-level dwords, loaded
// by every lane at clamped indexes (last_dw: the level's last dword), so no
// load sits under a branch.
// Cells of a 4x4 block whose input (its column in a right product, its row
// in a left one) is one of the set bits of in4 (bit c: the block's input
// origin + c), as a 16-bit cell mask (bit 4 b + q as in node_cells).
constexpr uint32_t cells_on_input(bool right, uint32_t c) {
    uint32_t m = 0;
    for (uint32_t t = 0; t < 16; ++t)
        if (((cell_offset_table(!right) >> (2 * t)) & 3u) == c) m |= 1u << t;
    return m;
}
template <int DIR>
__device__ __forceinline__ uint32_t cells_with_inputs(uint32_t in4) {
    constexpr bool kR = DIR == K2_RIGHT;
    return ((in4 & 1u) ? cells_on_input(kR, 0) : 0u) | ((in4 & 2u) ? cells_on_input(kR, 1) : 0u) |
           ((in4 & 4u) ? cells_on_input(kR, 2) : 0u) | ((in4 & 8u) ? cells_on_input(kR, 3) : 0u);
}
// The input bit array's word holding the bits of a block's 4 inputs from
// input origin in0 (a multiple of 4), and those 4 bits.
__device__ __forceinline__ uint32_t inmask_word(const uint32_t *__restrict__ inmask, uint32_t in0) {
    return inmask[in0 >> 5];
}
__device__ __forceinline__ uint32_t inmask_bits(uint32_t word, uint32_t in0) { return (word >> (in0 & 31u)) & 15u; }

template <class SR, int DIR, class Off, uint32_t kSlots>
__device__ __forceinline__ void leaf_segment(uint64_t code, uint32_t s, uint32_t off,
                                             const uint32_t *__restrict__ leaf_dw, uint32_t last_dw,
                                             const typename SR::T *__restrict__ x,
                                             typename SR::T *__restrict__ y, uint32_t B, uint32_t VL,
                                             Window<typename SR::T> w, WaveCells<Off, kSlots> *wc) {
    const uint32_t dw = (off >> 3) < last_dw ? (off >> 3) : last_dw;
    const uint32_t lo32 = leaf_dw[dw], hi32 = leaf_dw[dw < last_dw ? dw + 1u : last_dw];
    const uint32_t row0 = compact_even(code >> 1) * 4u, col0 = compact_even(code) * 4u;
    leaf_cells<SR, DIR, Off>(row0, col0, node_cells(s | ((off & 7u) << 6), lo32, hi32), x, y, B, VL, w, wc);
}

// The window of tile 'tl' for this product (no window: win = null), its LDS
// set to the semiring zero.  'use' is false when the batch is too wide for
// the planned window size.
template <class SR, int DIR, int kT = kThreads>
__device__ __forceinline__ Window<typename SR::T> open_window(const Tile &tl, typename SR::T *lds,
                                                              bool use, uint32_t B, int runs) {
    Window<typename SR::T> w{nullptr, 0, 0, runs != 0};
    if (!use || tl.win_log2 == kNoWindow) return w;
    w.win = lds;
    w.out0 = (DIR == K2_RIGHT) ? tl.win_row : tl.win_col;
    w.rows = 1u << tl.win_log2;
    const uint32_t n = w.rows * B;
    for (uint32_t e = threadIdx.x; e < n; e += kT) lds[e] = SR::zero();
    __syncthreads();
    return w;
}

// Add a tile's window to y: one coalesced pass, skipping semiring zeros.
// The only tile of its band (sole) writes y itself instead: it stores the
// window (zeros included: y was not filled) or, accumulating, combines it
// with y, with plain loads and stores.  The stores of a sole window are
// non-temporal 16-byte stores where y allows: nothing in the product reads
// them again, and they then displace less of the L2's x rows (web-like
// 2^27, batch 8: 10.70 -> 10.61 ms right, 8.70 -> 8.59 ms left).
template <class SR, int kT = kThreads>
__device__ __forceinline__ void close_window(const Window<typename SR::T> &w,
                                             typename SR::T *__restrict__ y, uint64_t n_out,
                                             uint32_t B, bool sole, int accumulate) {
    using T = typename SR::T;
    if (!w.win) return;
    __syncthreads();
    const uint64_t rows = (w.out0 + w.rows <= n_out) ? w.rows : (n_out - w.out0);
    const uint32_t n = uint32_t(rows) * B;
    T *__restrict__ out = y + w.out0 * B;
    if (sole && !accumulate) {
        if ((n & 3u) == 0 && (reinterpret_cast<uintptr_t>(out) & 15u) == 0) {
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 *src = reinterpret_cast<const u32x4 *>(w.win);
            u32x4 *dst = reinterpret_cast<u32x4 *>(out);
            for (uint32_t e = threadIdx.x; e < n / 4u; e += kT) __builtin_nontemporal_store(src[e], &dst[e]);
        } else {
            for (uint32_t e = threadIdx.x; e < n; e += kT) __builtin_nontemporal_store(w.win[e], &out[e]);
        }
    } else if (sole) {
        for (uint32_t e = threadIdx.x; e < n; e += kT) {
            const T v = w.win[e];
            if (SR::contributes_out(v)) out[e] = SR::combine(out[e], v);
        }
    } else {
        for (uint32_t e = threadIdx.x; e < n; e += kT) {
            const T v = w.win[e];
            if (SR::contributes_out(v)) SR::atomic(&out[e], v);
        }
    }
    __syncthreads();
}

// y[0..n) = value; 16-byte stores when y is 16-byte aligned.
__global__ __launch_bounds__(kThreads) void fill_kernel(uint32_t *__restrict__ y, uint64_t n,
                                                        uint32_t value, int vec) {
    const uint64_t stride = uint64_t(gridDim.x) * kThreads;
    uint64_t i = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    const uint64_t n4 = vec ? n / 4 : 0;
    uint4 v4 = make_uint4(value, value, value, value);
    uint4 *y4 = reinterpret_cast<uint4 *>(y);
    for (uint64_t k = i; k < n4; k += stride) y4[k] = v4;
    for (uint64_t k = n4 * 4 + i; k < n; k += stride) y[k] = value;
}

// Pipeline state of one segment of a cached tile in the directory ablation
// (kUseDir), in three stages: its
// descriptor (uniform: a scalar load), issued three segments ahead; the
// 64-bit signature word holding each lane's node, two segments ahead; and
// (SegLeaves) one segment ahead: the lane's node's block origin (first row
// << 32 | first column), its signature s and first-leaf nibble position p
// packed as s | p << 6, and the two leaf-level dwords that hold its leaf
// signatures (from nibble p of lo32).
// Every lane issues every load of a stage, at an index clamped into its
// array, and no load sits under a branch: the compiler then knows how many
// loads are still in flight at each use and waits only for the ones the use
// needs, so a stage's loads stay in flight while the wave works on the
// segment before.
struct SegSig {
    uint32_t lo, count, leaf;   // uniform; count = 0 past the wave's last segment
    uint64_t word;              // signature word of node lo + lane (node lo past count)
};
struct SegLeaves {
    uint64_t blk;
    uint32_t ssh, lo32, hi32;
};

__device__ __forceinline__ Seg stage_seg(const Seg *__restrict__ segs, uint32_t first, uint32_t k,
                                         uint32_t nseg) {
    Seg g{0u, 0u, 0u, 0u};
    if (k < nseg) g = segs[first + k];
    return g;
}

// With kUseDir the segment's first leaf comes from the directory on the
// device, else from the plan.
template <bool kUseDir>
__device__ __forceinline__ SegSig stage_sig(const uint32_t *__restrict__ dir, const Seg &g,
                                            const uint64_t *__restrict__ sig_words) {
    SegSig a;
    a.lo = g.lo;
    a.count = g.count;
    a.leaf = (kUseDir && g.count) ? wave_child_offset_of(sig_words, dir, g.lo) : g.leaf;
    const uint32_t lane = __lane_id();
    a.word = sig_words[(g.lo + (lane < g.count ? lane : 0u)) >> 4];
    return a;
}

// The lane's first leaf is the segment's first leaf plus the fan-outs of the
// lanes before it (a wave scan).  A node's at most 4 leaf nibbles start at
// nibble off % 8 of dword off / 8 and may reach into the next dword;
// last_dw is the leaf level's last dword.
__device__ __forceinline__ SegLeaves stage_leaves(const SegSig &a, const uint64_t *__restrict__ blocks,
                                                  const uint32_t *__restrict__ leaf_dw, uint32_t last_dw) {
    const uint32_t lane = __lane_id();
    const bool in = lane < a.count;
    const uint32_t s = in ? uint32_t(a.word >> (((a.lo + lane) & 15u) * 4u)) & 15u : 0u;
    uint32_t total;
    const uint32_t ex = wave_scan(__popc(s), total);
    const uint32_t off = a.leaf + ex;
    const uint32_t dw = (off >> 3) < last_dw ? (off >> 3) : last_dw;
    SegLeaves b;
    b.blk = blocks[a.lo + (in ? lane : 0u)];
    b.ssh = s | ((off & 7u) << 6);
    b.lo32 = leaf_dw[dw];
    b.hi32 = leaf_dw[dw < last_dw ? dw + 1u : last_dw];
    return b;
}

// A segment's nodes with their cells kept since the matrix was created:
// the lane's node's block origin and its cells (0 past the segment).
struct SegNodes {
    uint64_t blk;
    uint32_t cells;
};
template <bool kPacked>
__device__ __forceinline__ SegNodes stage_nodes(const Seg &g, const uint64_t *__restrict__ blocks,
                                                const uint32_t *__restrict__ nodew) {
    const uint32_t lane = __lane_id();
    const bool in = lane < g.count;
    const uint32_t i = g.lo + (in ? lane : 0u);
    SegNodes d;
    const uint32_t wv = nodew[i];
    if constexpr (kPacked) {
        // the block's place in the segment's quadrant, whose first row and
        // column the segment holds
        d.blk = (uint64_t(g.leaf + ((wv >> 14) & 0x3FCu)) << 32) | (g.pad + ((wv >> 22) & 0x3FCu));
    } else {
        d.blk = blocks[i];
    }
    d.cells = in ? (wv & 0xFFFFu) : 0u;
    return d;
}

// The input bit array of a product: bit i of word i / 32 is set when input
// row i has a contributing vector (one of x[i B .. i B + B - 1] is not the
// semiring's zero); rows past n_in read 0.  A wave writes the two words of
// its 64 rows from one ballot.
template <class SR>
__global__ __launch_bounds__(kThreads) void inmask_kernel(const typename SR::T *__restrict__ x, uint64_t n_in,
                                                          uint32_t B, uint32_t *__restrict__ mask) {
    const uint64_t stride = uint64_t(gridDim.x) * kThreads;
    const uint64_t n_words = (n_in + 31) / 32;
    for (uint64_t i0 = uint64_t(blockIdx.x) * kThreads + (threadIdx.x & ~63u); i0 < n_in; i0 += stride) {
        const uint64_t i = i0 + __lane_id();
        bool c = false;
        if (i < n_in)
            for (uint32_t v = 0; v < B; ++v) c = c || SR::contributes(x[i * B + v]);
        const uint64_t bal = __ballot(c);
        if (__lane_id() == 0) {
            mask[i0 >> 5] = uint32_t(bal);
            if ((i0 >> 5) + 1 < n_words) mask[(i0 >> 5) + 1] = uint32_t(bal >> 32);
        }
    }
}

// One product over the cached last internal level (Sec. 3.5): each workgroup
// takes a tile, a list of segments of up to 64 nodes of that level; wave w
// takes segments w, w + 4, ...  With the node words kept since creation
// (!kUseDir) a wave works on three of its segments at once: while it lists
// the cells of one, the node words (and, unless kPacked, the block origins)
// of the next and the descriptor of the one after are in flight; kPacked
// segments carry their quadrant's origin, so the node words alone give each
// block's origin.  With kUseDir (the directory ablation) the wave reads the
// signatures, the directory and the leaves instead, four segments at once.
// A band's owner tile (code_off = 1) then adds the band's strays
// (strays[stray_off[band] .. stray_off[band + 1]): each with its cells, its
// output coordinate in the band and its input block) to the same window.
// kSlots: the cell ring of each wave (one full pass).  kFilter (the max /
// or / min semirings): the listing keeps only the cells whose input row has
// a contributing vector (inmask), so the passes gather x for those alone;
// the pipeline then loads each segment's node words two segments ahead and
// its input bits one ahead, and each stray group's records two groups ahead
// and their input bits one ahead.
template <class SR, int DIR, class Off, bool kUseDir, bool kPacked, int kT, uint32_t kSlots, bool kFilter>
__global__ __launch_bounds__(kT, kOccupancy * kThreads / kT) void cached_kernel(
    const uint64_t *__restrict__ sig_words, const uint32_t *__restrict__ leaf_dw, uint32_t last_dw,
    const uint32_t *__restrict__ dir, const Tile *__restrict__ tiles, uint32_t n_tiles, const Seg *__restrict__ segs,
    const uint64_t *__restrict__ blocks, const uint32_t *__restrict__ nodew, const StrayRec *__restrict__ strays,
    const uint32_t *__restrict__ stray_off, const typename SR::T *__restrict__ x,
    typename SR::T *__restrict__ y, uint32_t B, uint32_t VL, uint64_t n_out, int use_window,
    int accumulate, int runs, const uint32_t *__restrict__ inmask) {
    using T = typename SR::T;
    extern __shared__ __attribute__((aligned(16))) uint64_t s_dyn[];   // the window (16-byte reads when stored)
    constexpr int kW = kT / 64;
    __shared__ WaveCells<Off, kSlots> s_cells[kW];
    // uniform, so that segment descriptors are scalar loads
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    WaveCells<Off, kSlots> *wc = &s_cells[wave];
    for (uint32_t ti = blockIdx.x; ti < n_tiles; ti += gridDim.x) {
        const Tile tl = tiles[ti];
        const Window<T> w = open_window<SR, DIR, kT>(tl, reinterpret_cast<T *>(s_dyn), use_window, B, runs);
        const uint32_t nseg = tl.count;
        uint32_t ring_head = 0, ring_fill = 0;   // the wave's queued cells
        uint32_t k = wave;
        // a node's input origin (its block's first column, right; row, left)
        auto in0_of = [&](const SegNodes &d) { return DIR == K2_RIGHT ? uint32_t(d.blk) : uint32_t(d.blk >> 32); };
        if constexpr (!kUseDir && kFilter) {
            // descriptor three segments ahead, node words two, input bits one
            Seg g2 = stage_seg(segs, tl.first, k + 2 * kW, nseg);
            SegNodes d0 = stage_nodes<kPacked>(stage_seg(segs, tl.first, k, nseg), blocks, nodew);
            SegNodes d1 = stage_nodes<kPacked>(stage_seg(segs, tl.first, k + kW, nseg), blocks, nodew);
            uint32_t m0 = inmask_word(inmask, in0_of(d0));
            for (; k < nseg; k += kW) {
                const Seg g3 = stage_seg(segs, tl.first, k + 3 * kW, nseg);
                const SegNodes d2 = stage_nodes<kPacked>(g2, blocks, nodew);
                const uint32_t m1 = inmask_word(inmask, in0_of(d1));
                const uint32_t cells = d0.cells & cells_with_inputs<DIR>(inmask_bits(m0, in0_of(d0)));
                ring_cells<SR, DIR, Off>(uint32_t(d0.blk >> 32), uint32_t(d0.blk), cells, x, y, B, VL, w, wc,
                                         ring_head, ring_fill);
                d0 = d1;
                d1 = d2;
                m0 = m1;
                g2 = g3;
            }
        } else if constexpr (!kUseDir) {
            // the nodes' cells kept since creation: two stages, a descriptor
            // two segments ahead and the nodes one ahead
            Seg g1 = stage_seg(segs, tl.first, k + kW, nseg);
            SegNodes d0 = stage_nodes<kPacked>(stage_seg(segs, tl.first, k, nseg), blocks, nodew);
            for (; k < nseg; k += kW) {
                const Seg g2 = stage_seg(segs, tl.first, k + 2 * kW, nseg);
                const SegNodes d1 = stage_nodes<kPacked>(g1, blocks, nodew);
                ring_cells<SR, DIR, Off>(uint32_t(d0.blk >> 32), uint32_t(d0.blk), d0.cells, x, y, B, VL, w, wc,
                                         ring_head, ring_fill);
                d0 = d1;
                g1 = g2;
            }
        } else {
        Seg g2 = stage_seg(segs, tl.first, k + 2 * kW, nseg);
        SegSig a1 = stage_sig<kUseDir>(dir, stage_seg(segs, tl.first, k + kW, nseg), sig_words);
        SegLeaves b0 = stage_leaves(stage_sig<kUseDir>(dir, stage_seg(segs, tl.first, k, nseg), sig_words),
                                    blocks, leaf_dw, last_dw);
        for (; k < nseg; k += kW) {
            const Seg g3 = stage_seg(segs, tl.first, k + 3 * kW, nseg);
            const SegSig a2 = stage_sig<kUseDir>(dir, g2, sig_words);
            const SegLeaves b1 = stage_leaves(a1, blocks, leaf_dw, last_dw);
            ring_cells<SR, DIR, Off>(uint32_t(b0.blk >> 32), uint32_t(b0.blk),
                                     node_cells(b0.ssh, b0.lo32, b0.hi32), x, y, B, VL, w, wc, ring_head,
                                     ring_fill);
            b0 = b1;
            a1 = a2;
            g2 = g3;
        }
        }
        if ((tl.code_off & 1u) && strays && tl.win_log2 != kNoWindow) {
            // the band's owner tile: its strays, 64 per wave at a time
            const uint32_t band0 = (DIR == K2_RIGHT) ? tl.win_row : tl.win_col;
            const uint32_t band = band0 >> tl.win_log2;
            const uint32_t s0 = stray_off[band], s1 = stray_off[band + 1];
            const uint32_t lane = __lane_id();
            // each group's records load while the wave works on the group
            // before; every call has at < s1, and lanes past the band's last
            // record read that record (no branch around the load)
            auto rec = [&](uint32_t at) { return strays[at + lane < s1 ? at + lane : s1 - 1u]; };
            uint32_t b = s0 + wave * 64u;
            if (kFilter && b < s1) {
                // records two groups ahead, their input bits one ahead
                StrayRec r = rec(b), r1 = rec(b + kT < s1 ? b + kT : b);
                uint32_t m0 = inmask_word(inmask, uint32_t(r.in()));
                for (; b < s1; b += kT) {
                    const StrayRec r2 = rec(b + 2 * kT < s1 ? b + 2 * kT : b);
                    const uint32_t m1 = inmask_word(inmask, uint32_t(r1.in()));
                    const bool in = b + lane < s1;
                    const uint32_t o = band0 + r.out_in_band(), i = uint32_t(r.in());
                    const uint32_t cells = in ? r.cells() & cells_with_inputs<DIR>(inmask_bits(m0, i)) : 0u;
                    ring_cells<SR, DIR, Off>(DIR == K2_RIGHT ? o : i, DIR == K2_RIGHT ? i : o, cells, x, y, B, VL,
                                             w, wc, ring_head, ring_fill);
                    r = r1;
                    r1 = r2;
                    m0 = m1;
                }
            } else if (b < s1) {
                StrayRec r = rec(b);
                for (; b < s1; b += kT) {
                    const StrayRec rn = rec(b + kT < s1 ? b + kT : b);
                    const bool in = b + lane < s1;
                    const uint32_t o = band0 + r.out_in_band(), i = uint32_t(r.in());
                    ring_cells<SR, DIR, Off>(DIR == K2_RIGHT ? o : i, DIR == K2_RIGHT ? i : o, in ? r.cells() : 0u,
                                             x, y, B, VL, w, wc, ring_head, ring_fill);
                    r = rn;
                }
            }
        }
        ring_drain<SR, DIR, Off>(x, y, B, VL, w, wc, ring_head, ring_fill);
        close_window<SR, kT>(w, y, n_out, B, (tl.code_off & 2u) != 0, accumulate);
    }
}

// Tree-only band groups (Sec. 3.4 tiles over the dense quadrants of one
// row / column band, into one LDS window): each wave takes sub-tiles w, w +
// 4, ... of its workgroup's group and descends each on its own, level by
// level, with wave scans and a frontier of at most 'cap' nodes per level in
// the wave's LDS, so no workgroup barrier is needed before the window's
// flush.  Frontier entries are Morton codes relative to the sub-tile's
// window quadrant (at most 2 log2 Q bits); the leaf level's cells go through
// the wave's ring as in the cached kernel.  Offsets: planned (bases, the
// sub-tile's first child on each level) or, without them, the directory.
template <class SR, int DIR, class Off>
__global__ __launch_bounds__(kThreads, kOccupancy) void band_kernel(
    DevTree t, const Tile *__restrict__ groups, const Tile *__restrict__ subs, uint32_t n_groups,
    const uint64_t *__restrict__ tile_codes, const uint32_t *__restrict__ bases, uint32_t cap,
    const typename SR::T *__restrict__ x, typename SR::T *__restrict__ y, uint32_t B, uint32_t VL,
    uint64_t n_out, int use_window, int runs) {
    using T = typename SR::T;
    extern __shared__ uint64_t s_dyn[];   // kWaves frontiers of 2 cap codes, then the window
    __shared__ WaveCells<Off> s_cells[kWaves];
    const int last = t.levels - 2;
    const uint32_t lane = __lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t *front = reinterpret_cast<uint32_t *>(s_dyn) + size_t(wave) * 2u * cap;
    T *s_win = reinterpret_cast<T *>(reinterpret_cast<uint32_t *>(s_dyn) + size_t(kWaves) * 2u * cap);
    WaveCells<Off> *wc = &s_cells[wave];
    const uint32_t *__restrict__ leaf_dw = reinterpret_cast<const uint32_t *>(t.words[last + 1]);
    const uint32_t last_dw = uint32_t((uint64_t(t.nodes[last + 1]) + 15u) / 16u * 2u - 1u);
    for (uint32_t gi = blockIdx.x; gi < n_groups; gi += gridDim.x) {
        const Tile gr = groups[gi];
        const Window<T> w = open_window<SR, DIR>(gr, s_win, use_window, B, runs);
        const int hq = t.levels - int(gr.win_log2);   // the window quadrants' level
        uint32_t ring_head = 0, ring_fill = 0;
        for (uint32_t si = wave; si < gr.count; si += kWaves) {
            const Tile tl = subs[gr.first + si];
            int d = int(tl.level);
            uint32_t lo = tl.first, cnt = tl.count;
            // the sub-tile's quadrant: the level-hq prefix of its codes
            const uint64_t qc = tile_codes[tl.code_off] >> (2 * (d - hq));
            uint32_t *cur = front, *nxt = front + cap;
            // the signature word of node start + lane of level dd (clamped):
            // a level's first chunk is loaded while the level above is
            // expanded, since its first node (the planned base) is known
            auto first_word = [&](int dd, uint32_t start) {
                const uint32_t last_node = t.nodes[dd] - 1u;
                return t.words[dd][(start + lane < last_node ? start + lane : last_node) >> 4];
            };
            uint64_t wpre = first_word(d, lo);
            for (uint32_t i = lane; i < cnt; i += 64)
                cur[i] = uint32_t(tile_codes[tl.code_off + i] - (qc << (2 * (d - hq))));
            wave_lds_sync();
            // nibble of node lo + i (i = s0 + lane) from the chunk's word
            auto sig_of = [&](const uint64_t *__restrict__ wd, uint32_t s0, bool valid) {
                const uint32_t i = s0 + lane;
                const uint64_t word = s0 == 0 ? wpre : wd[(lo + (valid ? i : s0)) >> 4];
                return valid ? uint32_t(word >> (((lo + i) & 15u) * 4u)) & 15u : 0u;
            };
            while (d < last) {
                const uint32_t base = bases ? bases[tl.base_off + uint32_t(d - int(tl.level))]
                                            : wave_child_offset(t, d, lo);
                const uint64_t wnext = first_word(d + 1, base);
                const uint64_t *__restrict__ wd = t.words[d];
                uint32_t running = 0;
                for (uint32_t s0 = 0; s0 < cnt; s0 += 64) {
                    const uint32_t i = s0 + lane;
                    const bool valid = i < cnt;
                    const uint32_t sg = sig_of(wd, s0, valid);
                    uint32_t total;
                    const uint32_t ex = wave_scan(__popc(sg), total);
                    if (sg) {
                        const uint32_t c2 = cur[i] << 2;
                        uint32_t p = running + ex;
#pragma unroll
                        for (uint32_t b = 0; b < 4; ++b)
                            if (sg & (1u << b)) nxt[p++] = c2 | b;
                    }
                    running += total;
                }
                wave_lds_sync();
                uint32_t *tmp = cur;
                cur = nxt;
                nxt = tmp;
                lo = base;
                cnt = running;
                wpre = wnext;
                ++d;
            }
            // the last internal level: each node's cells into the ring
            const uint32_t leaf0 = bases ? bases[tl.base_off + uint32_t(last - int(tl.level))]
                                         : wave_child_offset(t, last, lo);
            const uint64_t *__restrict__ wd = t.words[last];
            const int sh = int(gr.win_log2);
            const uint32_t qrow = uint32_t(compact_even(qc >> 1)) << sh, qcol = uint32_t(compact_even(qc)) << sh;
            uint32_t running = 0;
            for (uint32_t s0 = 0; s0 < cnt; s0 += 64) {
                const uint32_t i = s0 + lane;
                const bool valid = i < cnt;
                const uint32_t sg = sig_of(wd, s0, valid);
                const uint32_t rel = valid ? cur[i] : 0u;
                uint32_t total;
                const uint32_t ex = wave_scan(__popc(sg), total);
                const uint32_t off = leaf0 + running + ex;
                const uint32_t dw = (off >> 3) < last_dw ? (off >> 3) : last_dw;
                const uint32_t lo32 = leaf_dw[dw], hi32 = leaf_dw[dw < last_dw ? dw + 1u : last_dw];
                ring_cells<SR, DIR, Off>(qrow + compact_even(uint64_t(rel) >> 1) * 4u,
                                         qcol + compact_even(rel) * 4u,
                                         node_cells(sg | ((off & 7u) << 6), lo32, hi32), x, y, B, VL, w, wc,
                                         ring_head, ring_fill);
                running += total;
            }
            wave_lds_sync();
        }
        ring_drain<SR, DIR, Off>(x, y, B, VL, w, wc, ring_head, ring_fill);
        close_window<SR>(w, y, n_out, B, false, 1);
    }
}

// Whether v lies in one of the n sorted disjoint ranges r[k] = (lo << 32) | hi.
__device__ __forceinline__ bool in_ranges(const uint64_t *__restrict__ r, uint32_t n, uint32_t v) {
    uint32_t a = 0, b = n;
    while (a < b) {   // the first range ending after v
        const uint32_t mid = (a + b) >> 1;
        if (uint32_t(r[mid]) <= v) a = mid + 1;
        else b = mid;
    }
    return a < n && uint32_t(r[a] >> 32) <= v;
}

// Tree-only rest tiles (a second depth-first cut of Sec. 3.4, taken in
// output-block order): wave w of workgroup g takes entry 4 g + w of 'order'
// (an index into the cut), or of 'take' (an index and the ranges to skip),
// then the entries a whole grid of waves further on, and descends each tile
// on its own as band_kernel does, with frontiers of at most 'cap' absolute
// Morton codes per level in the wave's LDS.  A 'take' entry skips the
// last-internal-level ranges skips[skip_row ..] (skip_count of them; their
// fan-outs still count towards the leaf offsets).  Outputs go straight to y
// (no window), so no workgroup barrier at all.
template <class SR, int DIR, class Off, bool kFilter = false>
__global__ __launch_bounds__(kThreads, kOccupancy) void rest_kernel(
    DevTree t, const RestTile *__restrict__ cut, const uint32_t *__restrict__ order,
    const RestTake *__restrict__ take, uint32_t n_tiles, const uint64_t *__restrict__ skips,
    const uint64_t *__restrict__ tile_codes,
    const uint32_t *__restrict__ bases, uint32_t cap, const typename SR::T *__restrict__ x,
    typename SR::T *__restrict__ y, uint32_t B, uint32_t VL, int runs, const uint32_t *__restrict__ inmask) {
    using T = typename SR::T;
    extern __shared__ uint64_t s_dyn[];   // kWaves frontiers of 2 cap codes
    __shared__ WaveCells<Off> s_cells[kWaves];
    const int last = t.levels - 2;
    const uint32_t lane = __lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint64_t *front = s_dyn + size_t(wave) * 2u * cap;
    WaveCells<Off> *wc = &s_cells[wave];
    const uint32_t *__restrict__ leaf_dw = reinterpret_cast<const uint32_t *>(t.words[last + 1]);
    const uint32_t last_dw = uint32_t((uint64_t(t.nodes[last + 1]) + 15u) / 16u * 2u - 1u);
    const Window<T> w{nullptr, 0, 0, runs != 0};
    uint32_t ring_head = 0, ring_fill = 0;
    for (uint32_t ti = blockIdx.x * kWaves + wave; ti < n_tiles; ti += gridDim.x * kWaves) {
        uint32_t idx, skip_row = 0, nskip = 0;
        if (take) {
            const RestTake tk = take[ti];
            idx = tk.tile;
            skip_row = tk.skip_row;
            nskip = tk.skip_count;
        } else {
            idx = order[ti];
        }
        const RestTile tl = cut[idx];
        const int d0 = int(tl.level());
        int d = d0;
        uint32_t lo = tl.first, cnt = tl.count();
        uint64_t *cur = front, *nxt = front + cap;
        // the signature word of node start + lane of level dd (clamped): a
        // level's first chunk is loaded while the level above is expanded
        auto first_word = [&](int dd, uint32_t start) {
            const uint32_t last_node = t.nodes[dd] - 1u;
            return t.words[dd][(start + lane < last_node ? start + lane : last_node) >> 4];
        };
        uint64_t wpre = first_word(d, lo);
        for (uint32_t i = lane; i < cnt; i += 64) cur[i] = tile_codes[tl.code_off + i];
        wave_lds_sync();
        auto sig_of = [&](const uint64_t *__restrict__ wd, uint32_t s0, bool valid) {
            const uint32_t i = s0 + lane;
            const uint64_t word = s0 == 0 ? wpre : wd[(lo + (valid ? i : s0)) >> 4];
            return valid ? uint32_t(word >> (((lo + i) & 15u) * 4u)) & 15u : 0u;
        };
        while (d < last) {
            const uint32_t base = bases ? bases[tl.base_off + uint32_t(d - d0)]
                                        : wave_child_offset(t, d, lo);
            const uint64_t wnext = first_word(d + 1, base);
            const uint64_t *__restrict__ wd = t.words[d];
            uint32_t running = 0;
            for (uint32_t s0 = 0; s0 < cnt; s0 += 64) {
                const uint32_t i = s0 + lane;
                const bool valid = i < cnt;
                const uint32_t sg = sig_of(wd, s0, valid);
                uint32_t total;
                const uint32_t ex = wave_scan(__popc(sg), total);
                if (sg) {
                    const uint64_t c2 = cur[i] << 2;
                    uint32_t p = running + ex;
#pragma unroll
                    for (uint32_t b = 0; b < 4; ++b)
                        if (sg & (1u << b)) nxt[p++] = c2 | b;
                }
                running += total;
            }
            wave_lds_sync();
            uint64_t *tmp = cur;
            cur = nxt;
            nxt = tmp;
            lo = base;
            cnt = running;
            wpre = wnext;
            ++d;
        }
        // the last internal level: each node's cells into the ring
        const uint32_t leaf0 = bases ? bases[tl.base_off + uint32_t(last - d0)]
                                     : wave_child_offset(t, last, lo);
        const uint64_t *__restrict__ wd = t.words[last];
        uint32_t running = 0;
        for (uint32_t s0 = 0; s0 < cnt; s0 += 64) {
            const uint32_t i = s0 + lane;
            const bool valid = i < cnt;
            const uint32_t sg = sig_of(wd, s0, valid);
            const uint64_t code = valid ? cur[i] : 0ull;
            uint32_t total;
            const uint32_t ex = wave_scan(__popc(sg), total);
            const bool skip = valid && nskip && in_ranges(skips + skip_row, nskip, lo + i);
            const uint32_t off = leaf0 + running + ex;
            const uint32_t dw = (off >> 3) < last_dw ? (off >> 3) : last_dw;
            const uint32_t lo32 = leaf_dw[dw], hi32 = leaf_dw[dw < last_dw ? dw + 1u : last_dw];
            const uint32_t row0 = compact_even(code >> 1) * 4u, col0 = compact_even(code) * 4u;
            uint32_t cells = skip ? 0u : node_cells(sg | ((off & 7u) << 6), lo32, hi32);
            if constexpr (kFilter) {
                // only the cells whose input row has a contributing vector
                const uint32_t in0 = DIR == K2_RIGHT ? col0 : row0;
                cells &= cells_with_inputs<DIR>(inmask_bits(inmask_word(inmask, in0), in0));
            }
            ring_cells<SR, DIR, Off>(row0, col0, cells, x, y, B, VL, w, wc, ring_head, ring_fill);
            running += total;
        }
        wave_lds_sync();
    }
    ring_drain<SR, DIR, Off>(x, y, B, VL, w, wc, ring_head, ring_fill);
}

// Signature words w0 .. w0 + n - 1 of level d (indexes clamped to the
// last readable word, words_end[d] - 1), n <= kThreads * kStagedPerThread:
// loaded into
// registers by load_level_words, so that they stay in flight while the
// workgroup works on the level above, then written to LDS.
constexpr uint32_t kStagedPerThread = (4096u / 16u + 1u + kThreads - 1u) / kThreads;
__device__ __forceinline__ void load_level_words(const DevTree &t, int d, uint32_t w0, uint32_t n,
                                                 uint64_t (&v)[kStagedPerThread]) {
    const uint32_t end = t.words_end[d];
#pragma unroll
    for (uint32_t j = 0; j < kStagedPerThread; ++j) {
        const uint32_t k = threadIdx.x + j * kThreads;
        const uint32_t wi = w0 + (k < n ? k : 0u);
        v[j] = end ? t.words[d][wi < end ? wi : end - 1u] : 0ull;
    }
}
__device__ __forceinline__ void store_level_words(uint64_t *sig, uint32_t n, const uint64_t (&v)[kStagedPerThread]) {
#pragma unroll
    for (uint32_t j = 0; j < kStagedPerThread; ++j) {
        const uint32_t k = threadIdx.x + j * kThreads;
        if (k < n) sig[k] = v[j];
    }
}
// the nibble of node a (absolute index on its level) from staged words
// starting at word w0
__device__ __forceinline__ uint32_t staged_nib(const uint64_t *sig, uint32_t w0, uint32_t a) {
    return uint32_t(sig[(a >> 4) - w0] >> ((a & 15u) * 4u)) & 0xFu;
}

// One product by tiled descent (Algorithm 1 with the tiles of Sec. 3.4): each
// workgroup takes a tile, expands it level by level inside LDS, then visits
// the leaves of its last-internal-level nodes in place, with the semiring's
// atomics straight to y.  With 'emit' set the kernel writes the last level's
// block origins instead (building the cached level, Sec. 3.5).
template <class SR, int DIR, bool EMIT, class Off>
__global__ __launch_bounds__(kThreads, kOccupancy) void descent_kernel(
    DevTree t, const Tile *__restrict__ tiles, uint32_t n_tiles, const uint64_t *__restrict__ tile_codes,
    uint32_t cap, const typename SR::T *__restrict__ x, typename SR::T *__restrict__ y, uint32_t B,
    uint32_t VL, uint64_t *__restrict__ emit, const uint32_t *__restrict__ bases, int runs) {
    using T = typename SR::T;
    // 2 * cap codes (the frontier's two levels), then two buffers of
    // cap / 16 + 1 signature words
    extern __shared__ uint64_t s_front[];
    __shared__ uint32_t s_tot[kWaves];
    __shared__ uint32_t s_segtot[4096 / 64];   // scan offsets: fan-out per leaf segment
    __shared__ uint32_t s_val;
    __shared__ WaveCells<Off> s_cells[kWaves];
    const int last = t.levels - 2;
    const uint32_t lane = __lane_id(), wave = threadIdx.x >> 6;
    const Window<T> w{nullptr, 0, 0, !EMIT && runs != 0};
    const uint32_t sw = cap / 16u + 1u;   // words holding any cap consecutive nodes' nibbles
    for (uint32_t ti = blockIdx.x; ti < n_tiles; ti += gridDim.x) {
        const Tile tl = tiles[ti];
        int d = int(tl.level);
        uint32_t lo = tl.first, cnt = tl.count;
        uint64_t *cur = s_front, *nxt = s_front + cap;
        // A level's signature words are staged in LDS while the level above
        // expands, so no level waits on a global load in its scan loop.
        uint64_t *sig = s_front + 2u * cap, *sig_next = sig + sw;
        uint32_t w0 = lo >> 4;
        {
            uint64_t v[kStagedPerThread];
            load_level_words(t, d, w0, sw, v);
            store_level_words(sig, sw, v);
        }
        for (uint32_t i = threadIdx.x; i < cnt; i += kThreads) cur[i] = tile_codes[tl.code_off + i];
        __syncthreads();
        while (d < last) {
            const uint32_t base = bases ? bases[tl.base_off + uint32_t(d - int(tl.level))]
                                        : block_child_offset(t, d, lo, &s_val);
            const uint32_t w1 = base >> 4;
            uint64_t pre[kStagedPerThread];
            load_level_words(t, d + 1, w1, sw, pre);
            uint32_t running = 0;
            for (uint32_t s0 = 0; s0 < cnt; s0 += kThreads) {
                const uint32_t i = s0 + threadIdx.x;
                const bool valid = i < cnt;
                const uint32_t s = valid ? staged_nib(sig, w0, lo + i) : 0u;
                uint32_t total;
                const uint32_t ex = block_scan(__popc(s), s_tot, total);
                if (s) {
                    const uint64_t c2 = cur[i] << 2;
                    uint32_t p = running + ex;
#pragma unroll
                    for (uint32_t b = 0; b < 4; ++b)
                        if (s & (1u << b)) nxt[p++] = c2 | b;
                }
                running += total;
            }
            store_level_words(sig_next, sw, pre);
            __syncthreads();
            uint64_t *tmp = cur;
            cur = nxt;
            nxt = tmp;
            tmp = sig;
            sig = sig_next;
            sig_next = tmp;
            w0 = w1;
            lo = base;
            cnt = running;
            ++d;
        }
        if (EMIT) {
            for (uint32_t i = threadIdx.x; i < cnt; i += kThreads)
                emit[uint64_t(lo) + i] = (uint64_t(compact_even(cur[i] >> 1) * 4u) << 32) |
                                         (compact_even(cur[i]) * 4u);
        } else {
            const uint32_t *__restrict__ leaf_dw = reinterpret_cast<const uint32_t *>(t.words[last + 1]);
            const uint32_t last_dw = uint32_t((uint64_t(t.nodes[last + 1]) + 15u) / 16u * 2u - 1u);
            uint32_t leaf0 = 0;
            if (bases) {
                // scan offsets: the tile's first leaf, plus the fan-outs of the
                // 64-node segments before each segment
                leaf0 = bases[tl.base_off + uint32_t(last - int(tl.level))];
                for (uint32_t seg = wave * 64; seg < cnt; seg += kThreads) {
                    const uint32_t i = seg + lane;
                    const uint32_t s = i < cnt ? staged_nib(sig, w0, lo + i) : 0u;
                    uint32_t total;
                    wave_scan(__popc(s), total);
                    if (lane == 0) s_segtot[seg >> 6] = total;
                }
                __syncthreads();
            }
            for (uint32_t seg = wave * 64; seg < cnt; seg += kThreads) {
                const uint32_t i = seg + lane;
                const bool valid = i < cnt;
                const uint32_t s = staged_nib(sig, w0, lo + (valid ? i : seg)) & (valid ? 15u : 0u);
                const uint64_t code = valid ? cur[i] : 0ull;
                uint32_t base = leaf0;
                if (bases) {
                    for (uint32_t k = 0; k < (seg >> 6); ++k) base += s_segtot[k];
                } else {
                    base = wave_child_offset(t, last, lo + seg);
                }
                uint32_t total;
                const uint32_t ex = wave_scan(__popc(s), total);
                leaf_segment<SR, DIR, Off>(code, s, base + ex, leaf_dw, last_dw, x, y, B, VL, w, &s_cells[wave]);
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------- search

// Multi-source search (Sec. 5.8): dense tables of n vertices x S sources.
// The frontier F, the reached set V and the product output y hold W = S/32
// (rounded up) words per vertex, bit j % 32 of word j / 32 for source j;
// dist is n x S int32.

// The search's packed words (F, V, y and the level planes, contiguous) = 0.
__global__ __launch_bounds__(kThreads) void bfs_init_kernel(uint32_t *__restrict__ words, uint64_t n_words) {
    const uint64_t stride = uint64_t(gridDim.x) * kThreads;
    for (uint64_t i = uint64_t(blockIdx.x) * kThreads + threadIdx.x; i < n_words; i += stride) words[i] = 0u;
}

// Source j starts at level 0 in the frontier and the reached set.
__global__ __launch_bounds__(kThreads) void bfs_seed_kernel(const uint32_t *__restrict__ src, uint32_t S,
                                                            uint32_t W, uint32_t *__restrict__ F,
                                                            uint32_t *__restrict__ V) {
    const uint32_t j = blockIdx.x * kThreads + threadIdx.x;
    if (j >= S) return;
    const uint64_t v = src[j];
    const uint32_t bit = 1u << (j & 31u);
    atomicOr(&F[v * W + (j >> 5)], bit);
    atomicOr(&V[v * W + (j >> 5)], bit);
}

// After the level's product y = A (or, and) F: the newly reached bits are
// y & ~V; they become the next frontier and join V.  y is left zero for the
// next product, which accumulates into it.  The number of newly reached
// (vertex, source) pairs is added to *count.  A lane takes a word.  With
// planes (levels below 2^kBfsPlanes) the level is recorded by or-ing the
// fresh bits into plane p (n_words words from planes + p n_words) for each
// set bit p of the level: whole-word stores of the packed layout.  Without,
// the distances are stored: a word's sources are 32 adjacent entries of its
// vertex's row of dist, so the wave writes them together, two fresh words
// per store (lanes 0-31 and 32-63, a lane per source).
__global__ __launch_bounds__(kThreads) void bfs_mark_kernel(uint32_t *__restrict__ y,
                                                            uint32_t *__restrict__ V,
                                                            uint32_t *__restrict__ F,
                                                            uint32_t *__restrict__ planes,
                                                            int32_t *__restrict__ dist, uint64_t n_words,
                                                            uint32_t W, uint32_t S, int32_t level,
                                                            unsigned long long *__restrict__ count) {
    const uint64_t stride = uint64_t(gridDim.x) * kThreads;
    const uint32_t lane = __lane_id();
    uint32_t found = 0;
    // e0: the wave's first word (uniform, so the shuffles below see every lane)
    for (uint64_t e0 = uint64_t(blockIdx.x) * kThreads + (threadIdx.x & ~63u); e0 < n_words; e0 += stride) {
        const uint64_t e = e0 + lane;
        uint32_t fresh = 0u;
        if (e < n_words) {
            const uint32_t yw = y[e];
            if (yw) {
                y[e] = 0u;
                const uint32_t seen = V[e];
                fresh = yw & ~seen;
                if (fresh) {
                    V[e] = seen | fresh;
                    if (planes)
                        for (uint32_t p = 0; p < kBfsPlanes; ++p)
                            if ((uint32_t(level) >> p) & 1u) planes[p * n_words + e] |= fresh;
                }
            }
            F[e] = fresh;
        }
        found += uint32_t(__popc(fresh));
        if (planes) continue;
        uint64_t pending = __ballot(fresh != 0u);
        while (pending) {
            const uint32_t a = uint32_t(__builtin_ctzll(pending));
            pending &= pending - 1u;
            const uint32_t b = pending ? uint32_t(__builtin_ctzll(pending)) : a;
            const bool second = pending != 0u;
            if (second) pending &= pending - 1u;
            const uint32_t from = lane < 32u ? a : b;
            const uint32_t fw = uint32_t(__shfl(int(fresh), int(from)));
            const uint32_t bit = lane & 31u;
            if ((lane < 32u || second) && ((fw >> bit) & 1u)) {
                const uint64_t we = e0 + from;
                const uint32_t j = uint32_t(we % W) * 32u + bit;
                if (j < S) dist[(we / W) * S + j] = level;
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) found += __shfl_xor(found, o);
    if (lane == 0 && found) atomicAdd(count, (unsigned long long)found);
}

// The distance table from the reached set and the level planes: entry (v, j)
// is -1 where bit j of v's words in V is clear, else the level the planes
// hold (0 for the sources).  A lane takes a word and writes its (up to) 32
// entries, the word's segment of its vertex's row: 16-byte stores when
// 'vec4' (S a multiple of 4 and dist 16-byte aligned), so every 128-byte
// segment is written whole.
__global__ __launch_bounds__(kThreads) void bfs_dist_kernel(int32_t *__restrict__ dist,
                                                            const uint32_t *__restrict__ V,
                                                            const uint32_t *__restrict__ planes,
                                                            uint64_t n_words, uint32_t W, uint32_t S,
                                                            int vec4) {
    const uint64_t stride = uint64_t(gridDim.x) * kThreads;
    for (uint64_t e = uint64_t(blockIdx.x) * kThreads + threadIdx.x; e < n_words; e += stride) {
        const uint32_t vw = V[e];
        uint32_t pl[kBfsPlanes];
#pragma unroll
        for (uint32_t p = 0; p < kBfsPlanes; ++p) pl[p] = planes[p * n_words + e];
        const uint64_t v = W == 1u ? e : e / W;
        const uint32_t j0 = uint32_t(e - v * W) * 32u;
        const uint32_t nj = S - j0 < 32u ? S - j0 : 32u;
        int32_t *__restrict__ row = dist + v * S + j0;
        auto entry = [&](uint32_t b) -> int32_t {
            int32_t d = 0;
#pragma unroll
            for (uint32_t p = 0; p < kBfsPlanes; ++p) d |= int32_t((pl[p] >> b) & 1u) << p;
            return ((vw >> b) & 1u) ? d : -1;
        };
        if (vec4 && nj == 32u) {
#pragma unroll
            for (uint32_t q = 0; q < 8u; ++q)
                reinterpret_cast<int4 *>(row)[q] =
                    make_int4(entry(4u * q), entry(4u * q + 1u), entry(4u * q + 2u), entry(4u * q + 3u));
        } else {
            for (uint32_t b = 0; b < nj; ++b) row[b] = entry(b);
        }
    }
}

// bfs_dist_kernel when the sources fill whole words (S = 32 W) and dist is
// 16-byte aligned: word e's entries are dist[32 e .. 32 e + 32), so thread q
// writes entries 4 q .. 4 q + 3 of word q / 8 with one 16-byte store and a
// wave writes 1 KB of consecutive entries; a thread takes two such chunks a
// grid apart per round, their loads issued together.
__global__ __launch_bounds__(kThreads) void bfs_dist32_kernel(int32_t *__restrict__ dist,
                                                              const uint32_t *__restrict__ V,
                                                              const uint32_t *__restrict__ planes,
                                                              uint64_t n_words) {
    const uint64_t grid = uint64_t(gridDim.x) * kThreads, n = n_words * 8u;
    for (uint64_t q0 = uint64_t(blockIdx.x) * kThreads + threadIdx.x; q0 < n; q0 += 2u * grid) {
        uint32_t vw[2], pl[2][kBfsPlanes];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint64_t q = q0 + uint64_t(k) * grid;
            const uint64_t e = (q < n ? q : q0) >> 3;
            const uint32_t b0 = uint32_t(q & 7u) * 4u;
            vw[k] = V[e] >> b0;
#pragma unroll
            for (uint32_t p = 0; p < kBfsPlanes; ++p) pl[k][p] = planes[p * n_words + e] >> b0;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint64_t q = q0 + uint64_t(k) * grid;
            if (q >= n) break;
            int32_t d[4];
#pragma unroll
            for (uint32_t b = 0; b < 4u; ++b) {
                int32_t l = 0;
#pragma unroll
                for (uint32_t p = 0; p < kBfsPlanes; ++p) l |= int32_t((pl[k][p] >> b) & 1u) << p;
                d[b] = ((vw[k] >> b) & 1u) ? l : -1;
            }
            reinterpret_cast<int4 *>(dist)[q] = make_int4(d[0], d[1], d[2], d[3]);
        }
    }
}

// ------------------------------------------------------------- strays

// Grouping the strays by band when a matrix is created: one wave per stray
// segment, a lane per node.  The band is the node's first output >> qlog.
__global__ __launch_bounds__(kThreads) void stray_count_kernel(const Seg *__restrict__ segs, uint32_t n_segs,
                                                               const uint64_t *__restrict__ blocks, int dir,
                                                               uint32_t qlog, uint32_t *__restrict__ counts) {
    const uint32_t lane = __lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (uint32_t k = blockIdx.x * kWaves + wave; k < n_segs; k += gridDim.x * kWaves) {
        const Seg sg = segs[k];
        if (lane < sg.count) {
            const uint64_t blk = blocks[sg.lo + lane];
            const uint32_t o = dir == K2_RIGHT ? uint32_t(blk >> 32) : uint32_t(blk);
            atomicAdd(&counts[o >> qlog], 1u);
        }
    }
}

// Each stray's record at its band's cursor (advanced), with its cells from
// its leaves: its first leaf is the segment's plus the fan-outs of the nodes
// before it.
__global__ __launch_bounds__(kThreads) void stray_scatter_kernel(DevTree t, const Seg *__restrict__ segs,
                                                                 uint32_t n_segs,
                                                                 const uint64_t *__restrict__ blocks, int dir,
                                                                 uint32_t qlog, uint32_t *__restrict__ cursor,
                                                                 StrayRec *__restrict__ out) {
    const uint32_t lane = __lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t *__restrict__ sig_words = t.words[t.levels - 2];
    const uint32_t *__restrict__ leaf_dw = reinterpret_cast<const uint32_t *>(t.words[t.levels - 1]);
    const uint32_t last_dw = uint32_t((uint64_t(t.nodes[t.levels - 1]) + 15u) / 16u * 2u - 1u);
    for (uint32_t k = blockIdx.x * kWaves + wave; k < n_segs; k += gridDim.x * kWaves) {
        const Seg sg = segs[k];
        const bool in = lane < sg.count;
        const uint32_t s = in ? nib(sig_words, uint64_t(sg.lo) + lane) : 0u;
        uint32_t total;
        const uint32_t ex = wave_scan(__popc(s), total);
        if (in) {
            const uint64_t blk = blocks[sg.lo + lane];
            const uint32_t off = sg.leaf + ex;
            const uint32_t dw = (off >> 3) < last_dw ? (off >> 3) : last_dw;
            const uint32_t cells = node_cells(s | ((off & 7u) << 6), leaf_dw[dw],
                                              leaf_dw[dw < last_dw ? dw + 1u : last_dw]);
            const uint32_t o = dir == K2_RIGHT ? uint32_t(blk >> 32) : uint32_t(blk);
            const uint32_t i = dir == K2_RIGHT ? uint32_t(blk) : uint32_t(blk >> 32);
            const uint32_t pos = atomicAdd(&cursor[o >> qlog], 1u);
            out[pos] = StrayRec::make(cells, o & ((1u << qlog) - 1u), i);
        }
    }
}

// The node word of every node of the given segments of the cached level:
// its cells from its leaves and, with qlog > 0, its block's place in its
// 2^qlog-sided quadrant; the segment's (leaf, pad) then become the quadrant's
// first row and column, and status bit 0 is set when a segment's nodes lie
// in more than one quadrant.  One wave per segment, a lane per node.
__global__ __launch_bounds__(kThreads) void node_cells_kernel(DevTree t, Seg *__restrict__ segs, uint32_t n_segs,
                                                              const uint64_t *__restrict__ blocks, uint32_t qlog,
                                                              uint32_t *__restrict__ out,
                                                              uint32_t *__restrict__ status) {
    const uint32_t lane = __lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t *__restrict__ sig_words = t.words[t.levels - 2];
    const uint32_t *__restrict__ leaf_dw = reinterpret_cast<const uint32_t *>(t.words[t.levels - 1]);
    const uint32_t last_dw = uint32_t((uint64_t(t.nodes[t.levels - 1]) + 15u) / 16u * 2u - 1u);
    for (uint32_t k = blockIdx.x * kWaves + wave; k < n_segs; k += gridDim.x * kWaves) {
        const Seg sg = segs[k];
        const bool in = lane < sg.count;
        const uint32_t s = in ? nib(sig_words, uint64_t(sg.lo) + lane) : 0u;
        uint32_t total;
        const uint32_t ex = wave_scan(__popc(s), total);
        uint32_t word = 0u, qr = 0u, qc = 0u;
        if (in) {
            const uint32_t off = sg.leaf + ex;
            const uint32_t dw = (off >> 3) < last_dw ? (off >> 3) : last_dw;
            word = node_cells(s | ((off & 7u) << 6), leaf_dw[dw], leaf_dw[dw < last_dw ? dw + 1u : last_dw]);
            if (qlog) {
                const uint64_t blk = blocks[sg.lo + lane];
                const uint32_t r0 = uint32_t(blk >> 32), c0 = uint32_t(blk), m = (1u << qlog) - 1u;
                qr = r0 & ~m;
                qc = c0 & ~m;
                word |= ((r0 & m) >> 2) << 16 | ((c0 & m) >> 2) << 24;
            }
            out[sg.lo + lane] = word;
        }
        if (qlog) {
            // lane 0 holds a node (count >= 1): every node in its quadrant?
            const uint32_t r = __builtin_amdgcn_readfirstlane(qr), c = __builtin_amdgcn_readfirstlane(qc);
            if (in && (qr != r || qc != c)) atomicOr(status, 1u);
            if (lane == 0) {
                segs[k].leaf = r;
                segs[k].pad = c;
            }
        }
    }
}

// ------------------------------------------------------------- launchers

namespace {

// Lanes per cell: B rounded up to a power of 2 (at most 64).  Plus-times
// right products take at least 4: neighbouring cells of a list (Z order)
// often share a row, and with 64 cells per instruction their LDS float adds
// (compare-and-swap loops) keep colliding and retrying (B = 1: 35 ms
// against 14 ms for the left product at 2^27).  The other semirings' atomics
// (max, or, min) resolve collisions in one instruction, so they take B lanes
// (packed Boolean R-MAT 2^24 tree-only: 7.54 -> 6.66 ms); cached products
// then size the ring to a full pass (run_cached).
template <class SR>
uint32_t lanes_per_node(uint32_t B, int dir, bool) {
    uint32_t v = (dir == K2_RIGHT && SR::kTreeBands) ? 4u : 1u;
    while (v < B && v < 64) v <<= 1;
    return v;
}

// One workgroup per tile up to 2^20 workgroups, then a grid-stride loop; the
// cap is a multiple of 8, so a tile runs on the XCD its position names (tile
// lists ordered for the XCDs rely on it).
uint32_t grid_for(uint64_t blocks) {
    const uint64_t cap = 1u << 20;
    return uint32_t(blocks < cap ? (blocks ? blocks : 1) : cap);
}

// Whether products with batch B use the planned windows, and their LDS bytes:
// whenever the window (Q outputs x B) fits one workgroup's LDS beside the
// kernel's other LDS ('other' bytes: its cell rings and frontiers); beyond
// window_batch vectors fewer workgroups share a CU.
size_t window_bytes(const Matrix &m, uint32_t B, size_t other, int *use) {
    const size_t bytes = m.plan.window_log2 >= 0 ? (size_t(1) << m.plan.window_log2) * B * 4 : 0;
    *use = (m.window_elems > 0 && bytes > 0 && bytes + other <= m.lds_per_block) ? 1 : 0;
    return *use ? bytes : 0;
}

// LDS of the cached kernel beside its window (the waves' cell rings), and of
// the band kernel (the rings and the waves' two frontier levels of band_cap
// relative codes).
template <class Off, uint32_t kSlots = 512 / sizeof(Off)>
size_t cached_other_lds() { return sizeof(WaveCells<Off, kSlots>) * (kCachedThreads / 64); }
template <class Off>
size_t band_other_lds(const Matrix &m) {
    return sizeof(WaveCells<Off>) * kWaves + size_t(kWaves) * 2 * m.plan.band_cap * sizeof(uint32_t);
}

int set_lds_limit(const void *k, size_t lds) {
    if (lds <= 48 * 1024) return hipSuccess;
    return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
}

// Cell offsets (index * B + vector) fit 32 bits when every index times B does.
bool narrow_offsets(const Matrix &m, uint32_t B) {
    return uint64_t(m.n_rows > m.n_cols ? m.n_rows : m.n_cols) * B <= 0xFFFFFFFFull;
}

// The input bit array of a product over x (n_in rows of B vectors).
template <class SR>
int launch_inmask(const Matrix &m, uint64_t n_in, uint32_t B, const void *x, hipStream_t st) {
    const uint64_t waves = (n_in + 63) / 64;
    const uint64_t blocks = (waves + kWaves - 1) / kWaves;
    const uint32_t g = uint32_t(blocks < 8192 ? (blocks ? blocks : 1) : 8192);
    hipLaunchKernelGGL(inmask_kernel<SR>, dim3(g), dim3(kThreads), 0, st, static_cast<const typename SR::T *>(x),
                       n_in, B, m.d_inmask);
    return hipGetLastError();
}

// One launch of the cached kernel with kSlots ring slots per wave.
template <class SR, int DIR, class Off, uint32_t kSlots>
int run_cached_with(const Matrix &m, uint32_t B, uint32_t VL, const void *x, void *y, int accumulate,
                    bool want_filter, hipStream_t st) {
    using T = typename SR::T;
    const uint32_t n_tiles = uint32_t(m.plan.cached_tiles[DIR].size());
    const uint32_t grid = grid_for(n_tiles);
    int use = 0;
    const size_t lds = window_bytes(m, B, cached_other_lds<Off, kSlots>(), &use);
    const uint64_t n_out = DIR == K2_RIGHT ? m.n_rows : m.n_cols;
    const bool use_dir = m.plan.use_directory;
    // the max / or / min semirings list only the cells whose input row has a
    // contributing vector (plus-times inputs are rarely zero)
    constexpr bool kF = !SR::kWindowUnchecked;
    const bool filter = kF && !use_dir && want_filter;
    auto k = use_dir    ? cached_kernel<SR, DIR, Off, true, false, kCachedThreads, kSlots, false>
             : m.packed ? (filter ? cached_kernel<SR, DIR, Off, false, true, kCachedThreads, kSlots, kF>
                                  : cached_kernel<SR, DIR, Off, false, true, kCachedThreads, kSlots, false>)
                        : (filter ? cached_kernel<SR, DIR, Off, false, false, kCachedThreads, kSlots, kF>
                                  : cached_kernel<SR, DIR, Off, false, false, kCachedThreads, kSlots, false>);
    if (filter) {
        const int e0 = launch_inmask<SR>(m, DIR == K2_RIGHT ? m.n_cols : m.n_rows, B, x, st);
        if (e0 != hipSuccess) return e0;
    }
    int e = set_lds_limit(reinterpret_cast<const void *>(k), lds);
    if (e != hipSuccess) return e;
    const int d = m.levels - 2;
    const uint32_t last_dw = uint32_t((uint64_t(m.dev.nodes[d + 1]) + 15u) / 16u * 2u - 1u);
    hipLaunchKernelGGL(k, dim3(grid), dim3(kCachedThreads), lds, st, m.dev.words[d],
                       reinterpret_cast<const uint32_t *>(m.dev.words[d + 1]), last_dw, m.dev.dir[d],
                       m.d_cached_tiles[DIR], n_tiles,
                       m.d_cached_segs[DIR], m.d_cached, use_dir ? nullptr : m.d_nodew, m.d_strays[DIR],
                       m.d_stray_off[DIR],
                       static_cast<const T *>(x),
                       static_cast<T *>(y), B, VL, n_out, use, accumulate, m.plan.row_runs ? 1 : 0,
                       filter ? m.d_inmask : nullptr);
    return hipGetLastError();
}

// The wave's ring holds one full pass, 64 / VL lane groups x kUnroll cells:
// with one or two lanes per cell (batches 1 and 2) a 128-slot ring would let
// a lane load 2 or 4 cells per pass, too few gathers in flight (web-like
// 2^20 left, R-MAT 2^22 tropical: the 512-slot ring with one lane per cell
// measured 0.84 -> 0.58 ms); at B = 1 its 16 KB per workgroup still leave
// eight workgroups per CU.
template <class SR, int DIR, class Off>
int run_cached(const Matrix &m, uint32_t B, const void *x, void *y, int accumulate, bool filter, hipStream_t st) {
    if (m.plan.cached_tiles[DIR].empty()) return hipSuccess;
    const uint32_t VL = lanes_per_node<SR>(B, DIR, true);
    constexpr uint32_t k1 = 512 / sizeof(Off);
    if constexpr (!(DIR == K2_RIGHT && SR::kTreeBands)) {   // those take 4 lanes or more
        if (VL == 1) return run_cached_with<SR, DIR, Off, 4 * k1>(m, B, VL, x, y, accumulate, filter, st);
        if (VL == 2) return run_cached_with<SR, DIR, Off, 2 * k1>(m, B, VL, x, y, accumulate, filter, st);
    }
    return run_cached_with<SR, DIR, Off, k1>(m, B, VL, x, y, accumulate, filter, st);
}

// Descent tiles, depth first, a workgroup each; LDS: the frontier's two
// levels of 'cap' codes.
template <class SR, int DIR, bool EMIT, class Off>
int run_tiles(const DevTree &t, const Tile *tiles, size_t n, const uint64_t *codes, const uint32_t *bases,
              uint32_t cap, const void *x, void *y, uint32_t B, uint64_t *emit, bool row_runs, hipStream_t st) {
    using T = typename SR::T;
    if (n == 0) return hipSuccess;
    auto k = descent_kernel<SR, DIR, EMIT, Off>;
    const size_t lds = (size_t(2) * cap + 2u * (cap / 16u + 1u)) * sizeof(uint64_t);
    int e = set_lds_limit(reinterpret_cast<const void *>(k), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(grid_for(n)), dim3(kThreads), lds, st, t, tiles, uint32_t(n), codes, cap,
                       static_cast<const T *>(x), static_cast<T *>(y), B, lanes_per_node<SR>(B, DIR, false), emit, bases,
                       row_runs ? 1 : 0);
    return hipGetLastError();
}

template <class SR, int DIR, bool EMIT, class Off = uint32_t>
int run_descent(const Matrix &m, uint32_t B, const void *x, void *y, uint64_t *emit,
                hipStream_t st, bool want_filter = true) {
    using T = typename SR::T;
    const uint32_t VL = lanes_per_node<SR>(B, DIR, false);
    const uint64_t n_out = DIR == K2_RIGHT ? m.n_rows : m.n_cols;
    const Plan &p = m.plan;
    // the max / or / min semirings: the leaf level keeps only the cells whose
    // input row has a contributing vector (the input bit array, built first)
    const bool filter = !EMIT && !SR::kWindowUnchecked && want_filter && m.d_inmask;
    if (filter) {
        const int e0 = launch_inmask<SR>(m, DIR == K2_RIGHT ? m.n_cols : m.n_rows, B, x, st);
        if (e0 != hipSuccess) return e0;
    }
    const uint32_t *inmask = filter ? m.d_inmask : nullptr;
    if (EMIT)   // the cached level's block origins: the depth-first tiles
        return run_tiles<SR, DIR, EMIT, Off>(m.dev, m.d_tiles, p.tiles.size(), m.d_codes, m.d_bases, p.tile_nodes,
                                             x, y, B, emit, p.row_runs, st);
    // a list of tiles of at most rest_cap nodes per level, a wave each
    auto waves = [&](const RestTake *take, size_t n) -> int {
        if (n == 0) return hipSuccess;
        auto kr = inmask ? rest_kernel<SR, DIR, Off, !SR::kWindowUnchecked> : rest_kernel<SR, DIR, Off, false>;
        const size_t lds = size_t(kWaves) * 2 * p.rest_cap * sizeof(uint64_t);
        int e = set_lds_limit(reinterpret_cast<const void *>(kr), lds);
        if (e != hipSuccess) return e;
        // the whole cut: at most two rounds of resident workgroups (eight
        // per CU on 256 CUs), so that each wave takes a run of tiles and its
        // cell ring fills across them instead of draining a short pass after
        // every tile (R-MAT 2^22 tropical 0.93 / 0.91 -> 0.85 / 0.82 ms,
        // packed Boolean 2^24 6.47 -> 5.90 ms); after band groups a wave per
        // tile as before
        constexpr uint64_t kRestGrid = 2 * 8 * 256;
        const uint64_t blocks = (n + kWaves - 1) / kWaves;
        const uint32_t grid = take ? grid_for(blocks) : uint32_t(blocks < kRestGrid ? blocks : kRestGrid);
        hipLaunchKernelGGL(kr, dim3(grid), dim3(kThreads), lds, st, m.dev,
                           m.d_rest, m.d_rest_order[DIR], take, uint32_t(n), m.d_skip[DIR], m.d_codes, m.d_bases,
                           p.rest_cap,
                           static_cast<const T *>(x), static_cast<T *>(y), B, VL, p.row_runs ? 1 : 0, inmask);
        return hipGetLastError();
    };
    // the rest tiles the band groups leave, each skipping what the groups
    // cover; or all of them, skips ignored: the whole tree
    auto rest = [&](bool after_groups) -> int {
        return after_groups ? waves(m.d_rest_take[DIR], p.rest_take[DIR].size())
                            : waves(nullptr, p.rest_order[DIR].size());
    };
    int use = 0;
    const size_t wb = SR::kTreeBands ? window_bytes(m, B, band_other_lds<Off>(m), &use) : 0;
    if (use && !p.band_groups[DIR].empty()) {
        // the bands' dense quadrants into their windows, then the rest
        auto kb = band_kernel<SR, DIR, Off>;
        const size_t lds = size_t(kWaves) * 2 * p.band_cap * sizeof(uint32_t) + wb;
        int e = set_lds_limit(reinterpret_cast<const void *>(kb), lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kb, dim3(grid_for(p.band_groups[DIR].size())), dim3(kThreads), lds, st, m.dev,
                           m.d_band_groups[DIR], m.d_band_sub[DIR], uint32_t(p.band_groups[DIR].size()),
                           m.d_codes, m.d_bases, p.band_cap, static_cast<const T *>(x),
                           static_cast<T *>(y), B, VL, n_out, 1, p.row_runs ? 1 : 0);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return rest(true);
    }
    // No band groups, or no windows for them (the max / or / min semirings,
    // or a batch too wide): the whole second cut, each tile descended by one
    // wave without workgroup barriers.  (Measured on R-MAT 2^22 tropical
    // against the workgroup descent of the depth-first tiles: 1.26 -> 0.91
    // ms right, 1.19 -> 0.90 left; the groups' sub-tiles plus the rest
    // tiles with their skips, a wave each, took 1.52.)
    return rest(false);
}

template <int DIR>
int dispatch_cached(const Matrix &m, int semiring, uint32_t B, const void *x, void *y, int acc, bool f,
                    hipStream_t st) {
    switch (semiring) {
    case K2_PLUS_TIMES_F32: return narrow_offsets(m, B) ? run_cached<PlusTimes, DIR, uint32_t>(m, B, x, y, acc, f, st)
                                                         : run_cached<PlusTimes, DIR, uint64_t>(m, B, x, y, acc, f, st);
    case K2_BOOLEAN_F32: return narrow_offsets(m, B) ? run_cached<BooleanF32, DIR, uint32_t>(m, B, x, y, acc, f, st)
                                                         : run_cached<BooleanF32, DIR, uint64_t>(m, B, x, y, acc, f, st);
    case K2_BOOLEAN_U32X32: return narrow_offsets(m, B) ? run_cached<BooleanU32, DIR, uint32_t>(m, B, x, y, acc, f, st)
                                                         : run_cached<BooleanU32, DIR, uint64_t>(m, B, x, y, acc, f, st);
    case K2_TROPICAL_F32: return narrow_offsets(m, B) ? run_cached<Tropical, DIR, uint32_t>(m, B, x, y, acc, f, st)
                                                         : run_cached<Tropical, DIR, uint64_t>(m, B, x, y, acc, f, st);
    }
    return hipErrorInvalidValue;
}

template <int DIR>
int dispatch_descent(const Matrix &m, int semiring, uint32_t B, const void *x, void *y, bool f,
                     hipStream_t st) {
    switch (semiring) {
    case K2_PLUS_TIMES_F32: return narrow_offsets(m, B)
                   ? run_descent<PlusTimes, DIR, false, uint32_t>(m, B, x, y, nullptr, st, f)
                   : run_descent<PlusTimes, DIR, false, uint64_t>(m, B, x, y, nullptr, st, f);
    case K2_BOOLEAN_F32: return narrow_offsets(m, B)
                   ? run_descent<BooleanF32, DIR, false, uint32_t>(m, B, x, y, nullptr, st, f)
                   : run_descent<BooleanF32, DIR, false, uint64_t>(m, B, x, y, nullptr, st, f);
    case K2_BOOLEAN_U32X32: return narrow_offsets(m, B)
                   ? run_descent<BooleanU32, DIR, false, uint32_t>(m, B, x, y, nullptr, st, f)
                   : run_descent<BooleanU32, DIR, false, uint64_t>(m, B, x, y, nullptr, st, f);
    case K2_TROPICAL_F32: return narrow_offsets(m, B)
                   ? run_descent<Tropical, DIR, false, uint32_t>(m, B, x, y, nullptr, st, f)
                   : run_descent<Tropical, DIR, false, uint64_t>(m, B, x, y, nullptr, st, f);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int launch_fill(void *y, uint64_t n_words32, uint32_t value, void *stream) {
    if (n_words32 == 0) return hipSuccess;
    const uint64_t blocks = (n_words32 / 4 + kThreads - 1) / kThreads;
    const uint32_t grid = uint32_t(blocks < 8192 ? (blocks ? blocks : 1) : 8192);
    const int vec = (reinterpret_cast<uintptr_t>(y) & 15) == 0;
    hipLaunchKernelGGL(fill_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint32_t *>(y), n_words32, value, vec);
    return hipGetLastError();
}

int launch_cached(const Matrix &m, int dir, int semiring, uint32_t batch, const void *x, void *y,
                  int accumulate, void *stream, bool filter) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    return dir == K2_RIGHT ? dispatch_cached<K2_RIGHT>(m, semiring, batch, x, y, accumulate, filter, st)
                           : dispatch_cached<K2_LEFT>(m, semiring, batch, x, y, accumulate, filter, st);
}

bool cached_writes_all(const Matrix &m, int dir, uint32_t batch) {
    int use = 0;
    window_bytes(m, batch, narrow_offsets(m, batch) ? cached_other_lds<uint32_t>() : cached_other_lds<uint64_t>(),
                 &use);
    return use && m.plan.bands_cover[dir] && !m.plan.cached_tiles[dir].empty();
}

int launch_descent(const Matrix &m, int dir, int semiring, uint32_t batch, const void *x, void *y,
                   uint64_t *emit_codes, void *stream, bool filter) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (emit_codes) return run_descent<BooleanU32, K2_RIGHT, true>(m, 1, nullptr, nullptr, emit_codes, st);
    return dir == K2_RIGHT ? dispatch_descent<K2_RIGHT>(m, semiring, batch, x, y, filter, st)
                           : dispatch_descent<K2_LEFT>(m, semiring, batch, x, y, filter, st);
}

template <int DIR>
int dispatch_tiles(const DevTree &t, const Tile *tiles, size_t n, const uint64_t *codes, const uint32_t *bases,
                   uint32_t cap, bool narrow, bool row_runs, int semiring, uint32_t B, const void *x, void *y,
                   hipStream_t st) {
    switch (semiring) {
    case K2_PLUS_TIMES_F32:
        return narrow ? run_tiles<PlusTimes, DIR, false, uint32_t>(t, tiles, n, codes, bases, cap, x, y, B, nullptr,
                                                                   row_runs, st)
                      : run_tiles<PlusTimes, DIR, false, uint64_t>(t, tiles, n, codes, bases, cap, x, y, B, nullptr,
                                                                   row_runs, st);
    case K2_BOOLEAN_F32:
        return narrow ? run_tiles<BooleanF32, DIR, false, uint32_t>(t, tiles, n, codes, bases, cap, x, y, B,
                                                                    nullptr, row_runs, st)
                      : run_tiles<BooleanF32, DIR, false, uint64_t>(t, tiles, n, codes, bases, cap, x, y, B,
                                                                    nullptr, row_runs, st);
    case K2_BOOLEAN_U32X32:
        return narrow ? run_tiles<BooleanU32, DIR, false, uint32_t>(t, tiles, n, codes, bases, cap, x, y, B,
                                                                    nullptr, row_runs, st)
                      : run_tiles<BooleanU32, DIR, false, uint64_t>(t, tiles, n, codes, bases, cap, x, y, B,
                                                                    nullptr, row_runs, st);
    case K2_TROPICAL_F32:
        return narrow ? run_tiles<Tropical, DIR, false, uint32_t>(t, tiles, n, codes, bases, cap, x, y, B, nullptr,
                                                                  row_runs, st)
                      : run_tiles<Tropical, DIR, false, uint64_t>(t, tiles, n, codes, bases, cap, x, y, B, nullptr,
                                                                  row_runs, st);
    }
    return hipErrorInvalidValue;
}

int launch_descent_tiles(const DevTree &t, const Tile *tiles, size_t n_tiles, const uint64_t *codes,
                         const uint32_t *bases, uint32_t cap, uint32_t n_rows, uint32_t n_cols, bool row_runs,
                         int dir, int semiring, uint32_t batch, const void *x, void *y, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool narrow = uint64_t(n_rows > n_cols ? n_rows : n_cols) * batch <= 0xFFFFFFFFull;
    return dir == K2_RIGHT
               ? dispatch_tiles<K2_RIGHT>(t, tiles, n_tiles, codes, bases, cap, narrow, row_runs, semiring, batch,
                                          x, y, st)
               : dispatch_tiles<K2_LEFT>(t, tiles, n_tiles, codes, bases, cap, narrow, row_runs, semiring, batch, x,
                                         y, st);
}

static uint32_t stray_grid(uint32_t n_segs) {
    const uint32_t b = (n_segs + kWaves - 1) / kWaves;
    return b < 65536 ? (b ? b : 1) : 65536;
}

int launch_stray_count(const Matrix &m, int dir, const Seg *segs, uint32_t n_segs, uint32_t *counts,
                       void *stream) {
    if (n_segs == 0) return hipSuccess;
    hipLaunchKernelGGL(stray_count_kernel, dim3(stray_grid(n_segs)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), segs, n_segs, m.d_cached, dir,
                       uint32_t(m.plan.window_log2), counts);
    return hipGetLastError();
}

int launch_stray_scatter(const Matrix &m, int dir, const Seg *segs, uint32_t n_segs, uint32_t *cursor,
                         StrayRec *out, void *stream) {
    if (n_segs == 0) return hipSuccess;
    hipLaunchKernelGGL(stray_scatter_kernel, dim3(stray_grid(n_segs)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), m.dev, segs, n_segs, m.d_cached, dir,
                       uint32_t(m.plan.window_log2), cursor, out);
    return hipGetLastError();
}

int launch_node_cells(const Matrix &m, Seg *segs, uint32_t n_segs, int qlog, uint32_t *status, void *stream) {
    if (n_segs == 0) return hipSuccess;
    hipLaunchKernelGGL(node_cells_kernel, dim3(stray_grid(n_segs)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), m.dev, segs, n_segs, m.d_cached, uint32_t(qlog),
                       m.d_nodew, status);
    return hipGetLastError();
}

const char *hip_error_text(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

// ------------------------------------------------------------- scratch

// Workspace of k2_bfs_noalloc, for callers that cannot allocate device
// memory: a fixed array in the library's code object, which every GPU the
// library runs on holds until the process ends.  Host code never uses the
// name itself (on the host it is a stand-in, not a device address): the
// device address comes from hipGetSymbolAddress, once per device, and is
// passed to the kernels like any workspace.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

int noalloc_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *per_device[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {   // first call on this device, with it current
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

}  // namespace k2

namespace k2 {

static uint32_t small_grid(uint64_t items) {
    const uint64_t b = (items + kThreads - 1) / kThreads;
    return uint32_t(b < 8192 ? (b ? b : 1) : 8192);
}

int launch_bfs_init(uint32_t *words, uint64_t n_words, void *stream) {
    hipLaunchKernelGGL(bfs_init_kernel, dim3(small_grid(n_words)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), words, n_words);
    return hipGetLastError();
}

int launch_bfs_seed(const uint32_t *src, uint32_t S, uint32_t W, uint32_t *F, uint32_t *V, void *stream) {
    hipLaunchKernelGGL(bfs_seed_kernel, dim3((S + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), src, S, W, F, V);
    return hipGetLastError();
}

int launch_bfs_mark(uint32_t *y, uint32_t *V, uint32_t *F, uint32_t *planes, int32_t *dist, uint64_t n_words,
                    uint32_t W, uint32_t S, int32_t level, unsigned long long *count, void *stream) {
    hipLaunchKernelGGL(bfs_mark_kernel, dim3(small_grid(n_words)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), y, V, F, planes, dist, n_words, W, S, level, count);
    return hipGetLastError();
}

int launch_bfs_dist(int32_t *dist, const uint32_t *V, const uint32_t *planes, uint64_t n_words, uint32_t W,
                    uint32_t S, void *stream) {
    const bool aligned = reinterpret_cast<uintptr_t>(dist) % 16u == 0u;
    if (aligned && S == 32u * W) {
        hipLaunchKernelGGL(bfs_dist32_kernel, dim3(small_grid(n_words * 8u)), dim3(kThreads), 0,
                           static_cast<hipStream_t>(stream), dist, V, planes, n_words);
        return hipGetLastError();
    }
    const int vec4 = (S % 4u == 0u) && aligned;
    hipLaunchKernelGGL(bfs_dist_kernel, dim3(small_grid(n_words)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), dist, V, planes, n_words, W, S, vec4);
    return hipGetLastError();
}

}  // namespace k2
