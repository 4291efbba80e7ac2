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

#include "k2_internal.h"

namespace k2 {

// ------------------------------------------------------------- semirings

struct PlusTimes {
    using T = float;
    static constexpr uint32_t kZeroBits = 0u;
    __device__ static T zero() { return 0.0f; }
    __device__ static bool contributes(T x) { return x != 0.0f; }
    __device__ static T contrib(T x) { return x; }
    __device__ static T combine(T a, T b) { return a + b; }
    __device__ static void atomic(T *p, T v) {
        __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
};

struct BooleanF32 {
    using T = float;
    static constexpr uint32_t kZeroBits = 0u;
    __device__ static T zero() { return 0.0f; }
    __device__ static bool contributes(T x) { return (__float_as_uint(x) & 0x7FFFFFFFu) != 0u; }
    __device__ static T contrib(T) { return 1.0f; }
    __device__ static T combine(T a, T b) { return a > b ? a : b; }
    __device__ static void atomic(T *p, T v) {
        __hip_atomic_fetch_max(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
};

struct BooleanU32 {
    using T = uint32_t;
    static constexpr uint32_t kZeroBits = 0u;
    __device__ static T zero() { return 0u; }
    __device__ static bool contributes(T x) { return x != 0u; }
    __device__ static T contrib(T x) { return x; }
    __device__ static T combine(T a, T b) { return a | b; }
    __device__ static void atomic(T *p, T v) {
        __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
};

struct Tropical {
    using T = float;
    static constexpr uint32_t kZeroBits = 0x7F800000u;   // +inf
    __device__ static T zero() { return __uint_as_float(kZeroBits); }
    __device__ static bool contributes(T x) { return x < __uint_as_float(kZeroBits); }
    __device__ static T contrib(T x) { return 1.0f + x; }
    __device__ static T combine(T a, T b) { return a < b ? a : b; }
    // non-negative floats order like their bit patterns
    __device__ static void atomic(T *p, T v) {
        __hip_atomic_fetch_min(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
};

// ------------------------------------------------------------- helpers

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

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

// Exclusive prefix sum over the workgroup of f in [0, 7] (fan-outs are 0..4).
__device__ __forceinline__ uint32_t block_scan_small(uint32_t f, uint32_t *s_tot, uint32_t &total) {
    const unsigned lane = __lane_id();
    const unsigned wave = threadIdx.x >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint64_t b0 = __ballot(f & 1u), b1 = __ballot(f & 2u), b2 = __ballot(f & 4u);
    const uint32_t ex = __popcll(b0 & below) + 2u * __popcll(b1 & below) + 4u * __popcll(b2 & below);
    const uint32_t wt = __popcll(b0) + 2u * __popcll(b1) + 4u * __popcll(b2);
    if (lane == 0) s_tot[wave] = wt;
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

// The cells of one node of the last internal level: code F, signature s, first
// leaf 'off'.  Folds the contributions per output index of the node's 4x4
// block, then one atomic per touched output.  Vectors v = v0, v0+step, ...
template <class SR, int DIR>
__device__ __forceinline__ void leaf_node(uint64_t code, uint32_t s, uint32_t off,
                                          const uint64_t *__restrict__ leaf_words,
                                          const typename SR::T *__restrict__ x,
                                          typename SR::T *__restrict__ y, uint32_t B, uint32_t v0,
                                          uint32_t step) {
    using T = typename SR::T;
    if (s == 0) return;
    const uint64_t R4 = compact_even(code >> 1), C4 = compact_even(code);   // 4x4 block
    uint32_t lam[4];
    uint32_t quad[4];
    int nl = 0;
#pragma unroll
    for (uint32_t b = 0; b < 4; ++b)
        if (s & (1u << b)) {
            lam[nl] = nib(leaf_words, uint64_t(off) + uint64_t(nl));
            quad[nl] = b;
            ++nl;
        }
    const uint64_t in_base = (DIR == K2_RIGHT) ? 4 * C4 : 4 * R4;
    const uint64_t out_base = (DIR == K2_RIGHT) ? 4 * R4 : 4 * C4;
    for (uint32_t v = v0; v < B; v += step) {
        T acc[4];
        bool any[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc[k] = SR::zero();
            any[k] = false;
        }
        for (int l = 0; l < nl; ++l) {
            const uint32_t b = quad[l], lm = lam[l];
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q) {
                if (!(lm & (1u << q))) continue;
                const uint32_t r = 2 * (b >> 1) + (q >> 1);   // row within the 4x4 block
                const uint32_t c = 2 * (b & 1) + (q & 1);     // column within the block
                const uint32_t in_l = (DIR == K2_RIGHT) ? c : r;
                const uint32_t out_l = (DIR == K2_RIGHT) ? r : c;
                const T xv = x[(in_base + in_l) * B + v];
                if (SR::contributes(xv)) {
                    acc[out_l] = SR::combine(acc[out_l], SR::contrib(xv));
                    any[out_l] = true;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (any[k]) SR::atomic(&y[(out_base + k) * B + v], acc[k]);
    }
}

// ------------------------------------------------------------- kernels

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

// Node data of one 256-node pass, for the batched leaf work.
struct PassNodes {
    uint64_t code[kThreads];
    uint32_t off[kThreads];
    uint8_t sig[kThreads];
};

// Leaf work of a pass of 256 nodes whose (code, s, off) each thread holds.
template <class SR, int DIR, bool VL1>
__device__ __forceinline__ void leaf_pass(uint64_t code, uint32_t s, uint32_t off,
                                          const uint64_t *__restrict__ leaf_words,
                                          const typename SR::T *__restrict__ x,
                                          typename SR::T *__restrict__ y, uint32_t B, uint32_t VL,
                                          PassNodes *s_nodes) {
    if (VL1) {
        leaf_node<SR, DIR>(code, s, off, leaf_words, x, y, B, 0, 1);
        return;
    }
    s_nodes->code[threadIdx.x] = code;
    s_nodes->off[threadIdx.x] = off;
    s_nodes->sig[threadIdx.x] = uint8_t(s);
    __syncthreads();
    const uint32_t groups = kThreads / VL;
    const uint32_t g = threadIdx.x / VL, lv = threadIdx.x % VL;
    for (uint32_t k = g; k < kThreads; k += groups)
        leaf_node<SR, DIR>(s_nodes->code[k], s_nodes->sig[k], s_nodes->off[k], leaf_words, x, y, B,
                           lv, VL);
    __syncthreads();
}

// One product over the cached last internal level (Sec. 3.5): pass p covers
// nodes [256p, 256p + 256) of level l-2, one directory block.
template <class SR, int DIR, bool VL1>
__global__ __launch_bounds__(kThreads) void cached_kernel(DevTree t,
                                                          const uint64_t *__restrict__ codes,
                                                          const typename SR::T *__restrict__ x,
                                                          typename SR::T *__restrict__ y,
                                                          uint32_t B, uint32_t VL) {
    __shared__ uint32_t s_tot[kWaves];
    __shared__ PassNodes s_nodes;
    const int d = t.levels - 2;
    const uint32_t N = t.nodes[d];
    const uint32_t nblocks = (N + kThreads - 1) / kThreads;
    const uint64_t *__restrict__ sig_words = t.words[d];
    const uint64_t *__restrict__ leaf_words = t.words[d + 1];
    const uint32_t *__restrict__ dir = t.dir[d];
    for (uint32_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
        const uint32_t i = blk * kThreads + threadIdx.x;
        const bool valid = i < N;
        const uint32_t s = valid ? nib(sig_words, i) : 0u;
        const uint64_t code = valid ? codes[i] : 0ull;
        uint32_t total;
        const uint32_t ex = block_scan_small(__popc(s), s_tot, total);
        const uint32_t off = dir[blk] + ex;
        leaf_pass<SR, DIR, VL1>(code, s, off, leaf_words, x, y, B, VL, &s_nodes);
    }
}

// One product by tiled descent (Algorithm 1 with the tiles of Sec. 3.4): each
// workgroup takes a tile and expands it level by level inside LDS, then visits
// the leaves of its last-internal-level nodes in place.  With 'emit' set it
// writes those nodes' codes instead (building the cached level, Sec. 3.5).
template <class SR, int DIR, bool VL1, bool EMIT>
__global__ __launch_bounds__(kThreads) void descent_kernel(DevTree t, const Tile *__restrict__ tiles,
                                                           uint32_t n_tiles,
                                                           const uint64_t *__restrict__ tile_codes,
                                                           uint32_t cap,
                                                           const typename SR::T *__restrict__ x,
                                                           typename SR::T *__restrict__ y,
                                                           uint32_t B, uint32_t VL,
                                                           uint64_t *__restrict__ emit) {
    extern __shared__ uint64_t s_front[];   // 2 * cap codes
    __shared__ uint32_t s_tot[kWaves];
    __shared__ uint32_t s_val;
    __shared__ PassNodes s_nodes;
    const int last = t.levels - 2;
    for (uint32_t ti = blockIdx.x; ti < n_tiles; ti += gridDim.x) {
        const Tile tl = tiles[ti];
        int d = int(tl.level);
        uint32_t lo = tl.first, cnt = tl.count;
        uint64_t *cur = s_front, *nxt = s_front + cap;
        for (uint32_t i = threadIdx.x; i < cnt; i += kThreads) cur[i] = tile_codes[tl.code_off + i];
        __syncthreads();
        while (d < last) {
            const uint32_t base = block_child_offset(t, d, lo, &s_val);
            const uint64_t *__restrict__ w = t.words[d];
            uint32_t running = 0;
            for (uint32_t s0 = 0; s0 < cnt; s0 += kThreads) {
                const uint32_t i = s0 + threadIdx.x;
                const bool valid = i < cnt;
                const uint32_t s = valid ? nib(w, uint64_t(lo) + i) : 0u;
                uint32_t total;
                const uint32_t ex = block_scan_small(__popc(s), s_tot, total);
                if (s) {
                    const uint64_t c2 = cur[i] << 2;
                    uint32_t p = running + ex;
#pragma unroll
                    for (uint32_t b = 0; b < 4; ++b)
                        if (s & (1u << b)) nxt[p++] = c2 | b;
                }
                running += total;
            }
            __syncthreads();
            uint64_t *tmp = cur;
            cur = nxt;
            nxt = tmp;
            lo = base;
            cnt = running;
            ++d;
        }
        if (EMIT) {
            for (uint32_t i = threadIdx.x; i < cnt; i += kThreads) emit[uint64_t(lo) + i] = cur[i];
        } else {
            const uint32_t base = block_child_offset(t, last, lo, &s_val);
            const uint64_t *__restrict__ w = t.words[last];
            const uint64_t *__restrict__ leaf_words = t.words[last + 1];
            uint32_t running = 0;
            for (uint32_t s0 = 0; s0 < cnt; s0 += kThreads) {
                const uint32_t i = s0 + threadIdx.x;
                const bool valid = i < cnt;
                const uint32_t s = valid ? nib(w, uint64_t(lo) + i) : 0u;
                const uint64_t code = valid ? cur[i] : 0ull;
                uint32_t total;
                const uint32_t ex = block_scan_small(__popc(s), s_tot, total);
                leaf_pass<SR, DIR, VL1>(code, s, base + running + ex, leaf_words, x, y, B, VL,
                                        &s_nodes);
                running += total;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------- launchers

namespace {

uint32_t lanes_per_node(uint32_t B) {
    uint32_t v = 1;
    while (v < B && v < 64) v <<= 1;
    return v;
}

uint32_t grid_for(uint64_t blocks) {
    const uint64_t cap = 1u << 20;
    return uint32_t(blocks < cap ? (blocks ? blocks : 1) : cap);
}

template <class SR, int DIR>
int run_cached(const Matrix &m, uint32_t B, const void *x, void *y, hipStream_t st) {
    using T = typename SR::T;
    const uint32_t N = m.dev.nodes[m.levels - 2];
    if (N == 0) return hipSuccess;
    const uint32_t VL = lanes_per_node(B);
    const uint32_t grid = grid_for((N + kThreads - 1) / kThreads);
    if (VL == 1)
        hipLaunchKernelGGL((cached_kernel<SR, DIR, true>), dim3(grid), dim3(kThreads), 0, st, m.dev,
                           m.d_cached, static_cast<const T *>(x), static_cast<T *>(y), B, VL);
    else
        hipLaunchKernelGGL((cached_kernel<SR, DIR, false>), dim3(grid), dim3(kThreads), 0, st,
                           m.dev, m.d_cached, static_cast<const T *>(x), static_cast<T *>(y), B, VL);
    return hipGetLastError();
}

template <class SR, int DIR, bool EMIT>
int run_descent(const Matrix &m, uint32_t B, const void *x, void *y, uint64_t *emit,
                hipStream_t st) {
    using T = typename SR::T;
    const uint32_t n_tiles = uint32_t(m.plan.tiles.size());
    if (n_tiles == 0) return hipSuccess;
    const uint32_t cap = m.plan.tile_nodes;
    const size_t lds = size_t(2) * cap * sizeof(uint64_t);
    const uint32_t VL = lanes_per_node(B);
    const uint32_t grid = grid_for(n_tiles);
    auto kv1 = descent_kernel<SR, DIR, true, EMIT>;
    auto kvn = descent_kernel<SR, DIR, false, EMIT>;
    auto k = (VL == 1) ? kv1 : kvn;
    if (lds > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3(grid), dim3(kThreads), lds, st, m.dev, m.d_tiles, n_tiles, m.d_codes,
                       cap, static_cast<const T *>(x), static_cast<T *>(y), B, VL, emit);
    return hipGetLastError();
}

template <int DIR>
int dispatch_cached(const Matrix &m, int semiring, uint32_t B, const void *x, void *y,
                    hipStream_t st) {
    switch (semiring) {
    case K2_PLUS_TIMES_F32: return run_cached<PlusTimes, DIR>(m, B, x, y, st);
    case K2_BOOLEAN_F32: return run_cached<BooleanF32, DIR>(m, B, x, y, st);
    case K2_BOOLEAN_U32X32: return run_cached<BooleanU32, DIR>(m, B, x, y, st);
    case K2_TROPICAL_F32: return run_cached<Tropical, DIR>(m, B, x, y, st);
    }
    return hipErrorInvalidValue;
}

template <int DIR>
int dispatch_descent(const Matrix &m, int semiring, uint32_t B, const void *x, void *y,
                     hipStream_t st) {
    switch (semiring) {
    case K2_PLUS_TIMES_F32: return run_descent<PlusTimes, DIR, false>(m, B, x, y, nullptr, st);
    case K2_BOOLEAN_F32: return run_descent<BooleanF32, DIR, false>(m, B, x, y, nullptr, st);
    case K2_BOOLEAN_U32X32: return run_descent<BooleanU32, DIR, false>(m, B, x, y, nullptr, st);
    case K2_TROPICAL_F32: return run_descent<Tropical, DIR, false>(m, B, x, y, nullptr, st);
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
                  void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    return dir == K2_RIGHT ? dispatch_cached<K2_RIGHT>(m, semiring, batch, x, y, st)
                           : dispatch_cached<K2_LEFT>(m, semiring, batch, x, y, st);
}

int launch_descent(const Matrix &m, int dir, int semiring, uint32_t batch, const void *x, void *y,
                   uint64_t *emit_codes, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (emit_codes) return run_descent<BooleanU32, K2_RIGHT, true>(m, 1, nullptr, nullptr, emit_codes, st);
    return dir == K2_RIGHT ? dispatch_descent<K2_RIGHT>(m, semiring, batch, x, y, st)
                           : dispatch_descent<K2_LEFT>(m, semiring, batch, x, y, st);
}

const char *hip_error_text(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

}  // namespace k2
