/*
 * k2probe.h -- ceiling microbenchmarks of the GPU the library runs on.
 *
 * Tosoni & Mencagli, "A GPU Engine for Sparse Matrix-Vector Products on
 * k^2-Tree-Compressed Graphs", Sec. 5.6 and Table 4, place the engine
 * against two measured ceilings: the copy bandwidth and the rate of vector
 * updates y_o += x_i (consecutive entries with atomics or plain stores,
 * scattered entries with atomics).  k2_probe_run measures those on the
 * device, and the operations the MI355X kernels are built from: random
 * gathers and atomic scatters of batch rows, and LDS window updates.
 */
#ifndef K2PROBE_H
#define K2PROBE_H

#include "k2spmv.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
    K2_PROBE_COPY = 0,                /* b[i] = a[i], i < n (n % 4 == 0, b_elems >= n) */
    K2_PROBE_READ = 1,                /* every a[i] read once, one sum per thread into b */
    K2_PROBE_WRITE = 2,               /* b[i] = 1.0f, i < n */
    K2_PROBE_UPDATE_SEQ_ATOMIC = 3,   /* b[i] += a[i] with device-scope atomic adds */
    K2_PROBE_UPDATE_SEQ_STORE = 4,    /* b[i] = b[i] + a[i] with plain loads and stores */
    K2_PROBE_GATHER_ROWS = 5,         /* rows idx[k] (k < n) of R floats gathered from a
                                         (reps rows), summed per lane into b */
    K2_PROBE_SCATTER_ROWS_ATOMIC = 6, /* b[idx[k] R + v] += a[k R + v], atomic adds */
    K2_PROBE_LDS_ADD_F32 = 7,         /* LDS window updates, native float atomic add */
    K2_PROBE_LDS_CAS_F32 = 8,         /* LDS window updates, integer compare-and-swap loop */
    K2_PROBE_LDS_ADD_U32 = 9,         /* LDS window updates, integer atomic add */
    K2_PROBE_GATHER_ROWS_NT = 10,     /* as GATHER_ROWS with non-temporal loads */
    K2_PROBE_GATHER_ROWS_BUF_NT = 11, /* as GATHER_ROWS with buffer loads, sc0 and nt (x < 4 GiB) */
    K2_PROBE_GATHER_ROWS_BUF_SYS = 12 /* as GATHER_ROWS with buffer loads, sc0 and sc1 (x < 4 GiB) */
};

/* One timed launch of probe 'kind' on 'stream'; *ms receives its duration
   between two HIP events (Sec. 4: products timed between two events).
   d_a (input, device), d_b (output, device, b_elems floats), d_idx (device
   uint32 row indexes, for the row probes), n (elements, rows, or for the LDS
   probes the workgroup count), row_elems R (floats per row, a power of 2 up
   to 64; the LDS window holds 512 rows of R floats), reps (the gather
   probe's row count of a; the LDS probes' updates per lane).  Index
   contents are the caller's promise, as in a product.  Synchronizes the
   stream.  Errors: K2_E_INVALID_ARG (a size or kind outside the above),
   K2_E_HIP. */
k2_status k2_probe_run(int32_t kind, const void *d_a, void *d_b, const uint32_t *d_idx, uint64_t n,
                       uint64_t b_elems, uint32_t row_elems, uint32_t reps, void *stream, float *ms);

#ifdef __cplusplus
}
#endif

#endif /* K2PROBE_H */
