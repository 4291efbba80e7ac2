// k2_probe.hip -- ceiling microbenchmarks of gfx950 for the product's
// memory operations.
//
// Tosoni & Mencagli, "A GPU Engine for Sparse Matrix-Vector Products on
// k^2-Tree-Compressed Graphs", Sec. 5.6 and Table 4: the engine is placed
// against two measured ceilings, the copy bandwidth and the rate of vector
// updates y_o += x_i (consecutive entries with atomics or plain stores,
// scattered entries with atomics).  The kernels here measure those, plus the
// operations the MI355X kernels are built from: random row gathers of x (a
// batch row of B floats) and LDS window updates (native float add against
// an integer compare-and-swap).  Every kernel stays inside the buffers the
// host passes (sizes checked in k2_probe_run); each is timed with HIP events
// on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/k2probe.h"

namespace {

constexpr int kThreads = 256;

// counter-based hash (the splitmix64 output function), for LDS addresses
__device__ __forceinline__ uint32_t mix32(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return uint32_t(z ^ (z >> 31));
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4 *__restrict__ a, uint4 *__restrict__ b,
                                                        uint64_t n4) {
    const uint64_t stride = uint64_t(gridDim.x) * kThreads;
    for (uint64_t i = uint64_t(blockIdx.x) * kThreads + threadIdx.x; i < n4; i += stride) b[i] = a[i];
}

// every element read once; one sum per thread written (n_threads floats)
__global__ __launch_bounds__(kThreads) void read_kernel(const uint4 *__restrict__ a, float *__restrict__ out,
                                                        uint64_t n4) {
    const uint64_t stride = uint64_t(gridDim.x) * kThreads;
    const uint64_t t = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    float s = 0.0f;
    for (uint64_t i = t; i < n4; i += stride) {
        const uint4 v = a[i];
        s += __uint_as_float(v.x) + __uint_as_float(v.y) + __uint_as_float(v.z) + __uint_as_float(v.w);
    }
    out[t] = s;
}

__global__ __launch_bounds__(kThreads) void write_kernel(uint4 *__restrict__ b, uint64_t n4) {
    const uint64_t stride = uint64_t(gridDim.x) * kThreads;
    const uint4 v = make_uint4(0x3F800000u, 0x3F800000u, 0x3F800000u, 0x3F800000u);
    for (uint64_t i = uint64_t(blockIdx.x) * kThreads + threadIdx.x; i < n4; i += stride) b[i] = v;
}

// y[o] += x[i] for consecutive o = i, with a device-scope atomic add or a
// plain load and store
template <bool kAtomic>
__global__ __launch_bounds__(kThreads) void update_seq_kernel(const float *__restrict__ x, float *__restrict__ y,
                                                              uint64_t n) {
    const uint64_t stride = uint64_t(gridDim.x) * kThreads;
    for (uint64_t i = uint64_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride) {
        if (kAtomic) __hip_atomic_fetch_add(&y[i], x[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else y[i] = y[i] + x[i];
    }
}

// Random rows of R floats (R a power of 2, at most 64): row k of the list
// idx[k] (< rows).  Gather: lane group g of R lanes adds x[idx[k] * R + v]
// over its rows and writes one sum per lane.  Scatter: y[idx[k] * R + v] +=
// x[k * R + v] with device-scope atomics (one request per row and
// instruction, like a batch row's update).
// kPolicy: 0 plain loads; 1 non-temporal loads (nt); 2 buffer loads with
// the sc0 and nt bits; 3 buffer loads with sc0 and sc1 (x under 4 GiB)
template <int kPolicy>
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(const float *__restrict__ x,
                                                               const uint32_t *__restrict__ idx, uint64_t n_idx,
                                                               uint32_t R, float *__restrict__ out) {
    __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(x), 0, 0xFFFFFFFF,
                                                                    0x00020000);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t G = 64u / R, g = lane / R, v = lane % R;
    const uint64_t wave = (uint64_t(blockIdx.x) * kThreads + threadIdx.x) >> 6;
    const uint64_t waves = (uint64_t(gridDim.x) * kThreads) >> 6;
    float s = 0.0f;
    // 8 rows in flight per lane group
    for (uint64_t k0 = wave * G * 8u; k0 < n_idx; k0 += waves * G * 8u) {
        float v8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint64_t k = k0 + uint64_t(u) * G + g;
            const uint32_t r = idx[k < n_idx ? k : k0];
            if constexpr (kPolicy == 0) v8[u] = x[uint64_t(r) * R + v];
            else if constexpr (kPolicy == 1) v8[u] = __builtin_nontemporal_load(&x[uint64_t(r) * R + v]);
            else if constexpr (kPolicy == 2)
                v8[u] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (r * R + v) * 4u, 0, 3);
            else v8[u] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (r * R + v) * 4u, 0, 17);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) s += (k0 + uint64_t(u) * G + g < n_idx) ? v8[u] : 0.0f;
    }
    out[uint64_t(blockIdx.x) * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void scatter_rows_kernel(const float *__restrict__ x,
                                                                const uint32_t *__restrict__ idx, uint64_t n_idx,
                                                                uint32_t R, float *__restrict__ y) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t G = 64u / R, g = lane / R, v = lane % R;
    const uint64_t wave = (uint64_t(blockIdx.x) * kThreads + threadIdx.x) >> 6;
    const uint64_t waves = (uint64_t(gridDim.x) * kThreads) >> 6;
    for (uint64_t k = wave * G + g; k < n_idx; k += waves * G)
        __hip_atomic_fetch_add(&y[uint64_t(idx[k]) * R + v], x[k * R + v], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

// LDS window updates: each workgroup holds a window of W floats (W a power
// of 2); lane group g of R lanes updates row h(g, step) of the window, v
// its vector, 'reps' times, then the window is added to out once.
template <int kMode>   // 0: native float add, 1: integer compare-and-swap, 2: integer add
__global__ __launch_bounds__(kThreads) void lds_update_kernel(float *__restrict__ out, uint32_t W, uint32_t R,
                                                              uint32_t reps) {
    extern __shared__ float win[];
    for (uint32_t e = threadIdx.x; e < W; e += kThreads) win[e] = 0.0f;
    __syncthreads();
    const uint32_t lane = threadIdx.x & 63u, g = threadIdx.x / R, v = lane % R;
    const uint32_t rows_mask = W / R - 1u;
    const float one = 1.0f;
    for (uint32_t s = 0; s < reps; ++s) {
        const uint32_t row = mix32((uint64_t(blockIdx.x) << 40) ^ (uint64_t(g) << 20) ^ s) & rows_mask;
        float *p = &win[row * R + v];
        if constexpr (kMode == 0) {
            __hip_atomic_fetch_add(p, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        } else if constexpr (kMode == 1) {
            uint32_t *u = reinterpret_cast<uint32_t *>(p);
            uint32_t expected = __hip_atomic_load(u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            while (!__hip_atomic_compare_exchange_strong(u, &expected, __float_as_uint(__uint_as_float(expected) + one),
                                                         __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_WORKGROUP)) {
            }
        } else {
            __hip_atomic_fetch_add(reinterpret_cast<uint32_t *>(p), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    __syncthreads();
    float s = 0.0f;
    for (uint32_t e = threadIdx.x; e < W; e += kThreads) s += win[e];
    out[uint64_t(blockIdx.x) * kThreads + threadIdx.x] = s;
}

uint32_t grid_of(uint64_t items, uint32_t cap) {
    const uint64_t b = (items + kThreads - 1) / kThreads;
    return uint32_t(b < cap ? (b ? b : 1) : cap);
}

}  // namespace

extern "C" k2_status k2_probe_run(int32_t kind, const void *d_a, void *d_b, const uint32_t *d_idx, uint64_t n,
                                  uint64_t b_elems, uint32_t row_elems, uint32_t reps, void *stream, float *ms) {
    if (!ms || !d_b) return K2_E_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint32_t R = row_elems;
    const bool r_ok = R >= 1 && R <= 64 && (R & (R - 1)) == 0;
    const uint32_t big = 256u * 8u * 16u;   // 16 waves per SIMD's worth of workgroups x 16
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return K2_E_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return K2_E_HIP;
    }
    k2_status rc = K2_OK;
    (void)hipEventRecord(e0, st);
    switch (kind) {
    case K2_PROBE_COPY:
        if (!d_a || n % 4 || b_elems < n) { rc = K2_E_INVALID_ARG; break; }
        hipLaunchKernelGGL(copy_kernel, dim3(grid_of(n / 4, big)), dim3(kThreads), 0, st,
                           static_cast<const uint4 *>(d_a), static_cast<uint4 *>(d_b), n / 4);
        break;
    case K2_PROBE_READ:
        if (!d_a || n % 4 || b_elems < uint64_t(grid_of(n / 4, big)) * kThreads) { rc = K2_E_INVALID_ARG; break; }
        hipLaunchKernelGGL(read_kernel, dim3(grid_of(n / 4, big)), dim3(kThreads), 0, st,
                           static_cast<const uint4 *>(d_a), static_cast<float *>(d_b), n / 4);
        break;
    case K2_PROBE_WRITE:
        if (n % 4 || b_elems < n) { rc = K2_E_INVALID_ARG; break; }
        hipLaunchKernelGGL(write_kernel, dim3(grid_of(n / 4, big)), dim3(kThreads), 0, st,
                           static_cast<uint4 *>(d_b), n / 4);
        break;
    case K2_PROBE_UPDATE_SEQ_ATOMIC:
    case K2_PROBE_UPDATE_SEQ_STORE:
        if (!d_a || b_elems < n) { rc = K2_E_INVALID_ARG; break; }
        if (kind == K2_PROBE_UPDATE_SEQ_ATOMIC)
            hipLaunchKernelGGL(update_seq_kernel<true>, dim3(grid_of(n, big)), dim3(kThreads), 0, st,
                               static_cast<const float *>(d_a), static_cast<float *>(d_b), n);
        else
            hipLaunchKernelGGL(update_seq_kernel<false>, dim3(grid_of(n, big)), dim3(kThreads), 0, st,
                               static_cast<const float *>(d_a), static_cast<float *>(d_b), n);
        break;
    case K2_PROBE_GATHER_ROWS:
    case K2_PROBE_GATHER_ROWS_NT:
    case K2_PROBE_GATHER_ROWS_BUF_NT:
    case K2_PROBE_GATHER_ROWS_BUF_SYS: {
        // d_a: x of reps rows of R floats (reps is the row count here); d_b:
        // one float per thread of the grid; d_idx: n row indexes < reps
        if (!d_a || !d_idx || !r_ok) { rc = K2_E_INVALID_ARG; break; }
        if (kind >= K2_PROBE_GATHER_ROWS_BUF_NT && uint64_t(reps) * R * 4u > (1ull << 32)) {
            rc = K2_E_INVALID_ARG;   // buffer offsets are 32-bit
            break;
        }
        const uint32_t grid = grid_of(n * R / 8, big);
        if (b_elems < uint64_t(grid) * kThreads) { rc = K2_E_INVALID_ARG; break; }
        auto k = kind == K2_PROBE_GATHER_ROWS      ? gather_rows_kernel<0>
                 : kind == K2_PROBE_GATHER_ROWS_NT ? gather_rows_kernel<1>
                 : kind == K2_PROBE_GATHER_ROWS_BUF_NT ? gather_rows_kernel<2>
                                                       : gather_rows_kernel<3>;
        hipLaunchKernelGGL(k, dim3(grid), dim3(kThreads), 0, st, static_cast<const float *>(d_a), d_idx, n, R,
                           static_cast<float *>(d_b));
        break;
    }
    case K2_PROBE_SCATTER_ROWS_ATOMIC: {
        // d_a: n rows of R floats; d_b: y of b_elems / R rows; d_idx: n row
        // indexes, each < b_elems / R (the caller's promise, as for a product)
        if (!d_a || !d_idx || !r_ok || b_elems < R) { rc = K2_E_INVALID_ARG; break; }
        hipLaunchKernelGGL(scatter_rows_kernel, dim3(grid_of(n * R, big)), dim3(kThreads), 0, st,
                           static_cast<const float *>(d_a), d_idx, n, R, static_cast<float *>(d_b));
        break;
    }
    case K2_PROBE_LDS_ADD_F32:
    case K2_PROBE_LDS_CAS_F32:
    case K2_PROBE_LDS_ADD_U32: {
        // n workgroups, each with a window of 512 rows of R floats
        const uint32_t W = R * 512u;
        if (!r_ok || n == 0 || n > (1u << 20) || W * 4u > 65536u || b_elems < n * kThreads) {
            rc = K2_E_INVALID_ARG;
            break;
        }
        const size_t lds = size_t(W) * 4u;
        if (kind == K2_PROBE_LDS_ADD_F32)
            hipLaunchKernelGGL(lds_update_kernel<0>, dim3(uint32_t(n)), dim3(kThreads), lds, st,
                               static_cast<float *>(d_b), W, R, reps);
        else if (kind == K2_PROBE_LDS_CAS_F32)
            hipLaunchKernelGGL(lds_update_kernel<1>, dim3(uint32_t(n)), dim3(kThreads), lds, st,
                               static_cast<float *>(d_b), W, R, reps);
        else
            hipLaunchKernelGGL(lds_update_kernel<2>, dim3(uint32_t(n)), dim3(kThreads), lds, st,
                               static_cast<float *>(d_b), W, R, reps);
        break;
    }
    default:
        rc = K2_E_INVALID_ARG;
    }
    if (rc == K2_OK) {
        if (hipGetLastError() != hipSuccess) rc = K2_E_HIP;
        (void)hipEventRecord(e1, st);
        if (rc == K2_OK && hipEventSynchronize(e1) != hipSuccess) rc = K2_E_HIP;
        if (rc == K2_OK && hipEventElapsedTime(ms, e0, e1) != hipSuccess) rc = K2_E_HIP;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return rc;
}
