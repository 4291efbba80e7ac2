/*
 * k2_oracle.c -- plain, slow, CPU reference for k^2-tree SpMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library
 * and its Python binding) may include, link, load or call this file; only
 * the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code with the library.
 *
 * Source: Tosoni & Mencagli, "A GPU Engine for Sparse Matrix-Vector
 * Products on k^2-Tree-Compressed Graphs" (arXiv:2611.03610v1).
 *   - Sec. 2.1 (The k^2-tree): the tree of the recursive 2x2 decomposition
 *     of an n x n Boolean matrix, n = 2^l; a node's 4-bit signature has bit
 *     b = 2*b1 + b0 set iff quadrant b is non-empty (b1 = lower half of the
 *     rows, b0 = right half of the columns); signatures concatenated in
 *     level order; children found by rank.
 *   - Sec. 2.2 and Table 1: the semiring product y_i = (+)_{j: A_ij = 1} w (x) x_j.
 *   - Sec. 3.2: the sampled directory, one child offset every S nodes.
 *
 * What this file does, deliberately without cleverness:
 *   build   -- deduplicate the edges, then split the matrix recursively,
 *              breadth first, by scanning each node's own edge list for
 *              each of its four quadrants.  Children are appended in
 *              quadrant order, which is level order.
 *   export  -- per level, node i's signature in bits 4(i mod 16)..+3 of
 *              64-bit word floor(i/16) (least significant nibble first).
 *   product -- descend from the root; the j-th child of node t of level d is
 *              node (sum of popcounts of the signatures before t) + j of level
 *              d+1 (rank), its block origin is the parent's plus the
 *              quadrant's half-size offsets; at the leaf level every set bit
 *              q = 2*dr + dc is the cell (r0+dr, c0+dc).
 *   edges   -- the same product straight from the definition over the
 *              deduplicated edge list (no tree at all).
 *   bfs     -- Sec. 5.8's multi-source search (hop distances from several
 *              sources, one level per product) as a plain queue search per
 *              source over adjacency lists of the edge list.
 *
 * Readings where the pages are silent (shared with the library's contract):
 *   - l = max(2, ceil(log2(max(n_rows, n_cols)))), so a last internal level
 *     l-2 >= 0 exists; an empty matrix has a root of signature 0 and no
 *     other nodes.
 *   - Duplicated edges count once (a Boolean matrix is a set).
 *   - Tropical infinity is IEEE +inf; the contribution 1 + x_j is one fp32
 *     addition rounded to nearest even; min is exact.
 *   - Plus-times accumulates in fp64 from the fp32 inputs.
 *   - y is overwritten, starting from the semiring zero.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define ORC_OK 0
#define ORC_E_ARG (-1)
#define ORC_E_RANGE (-2)
#define ORC_E_OOM (-3)

/* semiring ids (the tests pass these numbers) */
#define ORC_PLUS_TIMES 0   /* x f32, y f64, w = 1 */
#define ORC_BOOLEAN_F32 1  /* x f32, y f32 in {0, 1} */
#define ORC_BOOLEAN_U32 2  /* x u32, y u32, bitwise or (32 vectors per word) */
#define ORC_TROPICAL 3     /* x f32 >= 0 or +inf, y f32, min and + */

#define ORC_RIGHT 0        /* y = A x  : y[r] (+)= x[c] */
#define ORC_LEFT 1         /* y = x^T A: y[c] (+)= x[r] */

typedef struct orc_tree {
    int levels;          /* l */
    uint64_t n;          /* 2^l */
    uint32_t n_rows, n_cols;
    uint64_t nnz;        /* distinct cells */
    uint64_t *nodes;     /* nodes[d], d = 0..l-1 */
    uint64_t **words;    /* words[d][k], ceil(nodes[d]/16) words */
    uint64_t **before;   /* before[d][k] = set bits in words[d][0..k-1] */
} orc_tree;

/* ---------------------------------------------------------------- helpers */

static int bit_count(uint64_t v) {
    int c = 0;
    while (v) { c += (int)(v & 1u); v >>= 1; }
    return c;
}

static int cmp_u64(const void *a, const void *b) {
    uint64_t x = *(const uint64_t *)a, y = *(const uint64_t *)b;
    return (x > y) - (x < y);
}

static uint64_t n_words_for(uint64_t nodes) { return (nodes + 15) / 16; }

static unsigned nibble_of(const orc_tree *t, int d, uint64_t i) {
    return (unsigned)((t->words[d][i / 16] >> (4 * (i % 16))) & 0xFu);
}

/* Number of set bits in the signatures of nodes 0..i-1 of level d. */
static uint64_t rank_before(const orc_tree *t, int d, uint64_t i) {
    uint64_t w = i / 16;
    unsigned sh = (unsigned)(4 * (i % 16));
    uint64_t part = sh ? (t->words[d][w] & ((1ull << sh) - 1)) : 0;
    return t->before[d][w] + (uint64_t)bit_count(part);
}

/* Deduplicated cells as (row << 32 | col), ascending.  Returns count. */
static int dedupe(const uint32_t *rows, const uint32_t *cols, uint64_t m,
                  uint32_t n_rows, uint32_t n_cols, uint64_t **out, uint64_t *out_m) {
    uint64_t *key = (uint64_t *)malloc((m ? m : 1) * sizeof(uint64_t));
    if (!key) return ORC_E_OOM;
    for (uint64_t e = 0; e < m; e++) {
        if (rows[e] >= n_rows || cols[e] >= n_cols) { free(key); return ORC_E_RANGE; }
        key[e] = ((uint64_t)rows[e] << 32) | cols[e];
    }
    qsort(key, m, sizeof(uint64_t), cmp_u64);
    uint64_t u = 0;
    for (uint64_t e = 0; e < m; e++)
        if (u == 0 || key[e] != key[u - 1]) key[u++] = key[e];
    *out = key;
    *out_m = u;
    return ORC_OK;
}

/* ------------------------------------------------------------------ build */

typedef struct { uint32_t r0, c0; uint64_t lo, hi; } orc_node;  /* edges [lo,hi) */

void orc_free(orc_tree *t) {
    if (!t) return;
    for (int d = 0; d < t->levels; d++) {
        if (t->words) free(t->words[d]);
        if (t->before) free(t->before[d]);
    }
    free(t->words); free(t->before); free(t->nodes); free(t);
}

int orc_build(const uint32_t *rows, const uint32_t *cols, uint64_t m,
              uint32_t n_rows, uint32_t n_cols, orc_tree **out) {
    *out = NULL;
    if (n_rows == 0 || n_cols == 0) return ORC_E_ARG;
    uint64_t *cell = NULL, nnz = 0;
    int rc = dedupe(rows, cols, m, n_rows, n_cols, &cell, &nnz);
    if (rc) return rc;

    uint32_t dim = n_rows > n_cols ? n_rows : n_cols;
    int l = 0;
    while ((1ull << l) < dim) l++;
    if (l < 2) l = 2;

    orc_tree *t = (orc_tree *)calloc(1, sizeof(orc_tree));
    t->levels = l; t->n = 1ull << l; t->n_rows = n_rows; t->n_cols = n_cols; t->nnz = nnz;
    t->nodes = (uint64_t *)calloc((size_t)l, sizeof(uint64_t));
    t->words = (uint64_t **)calloc((size_t)l, sizeof(uint64_t *));
    t->before = (uint64_t **)calloc((size_t)l, sizeof(uint64_t *));

    /* Edges are partitioned in place, level by level; each node owns a
       contiguous segment of 'cell'.  'tmp' holds one node's four buckets. */
    uint64_t *tmp = (uint64_t *)malloc((nnz ? nnz : 1) * sizeof(uint64_t));
    orc_node *cur = (orc_node *)malloc(sizeof(orc_node));
    uint64_t n_cur = 1;
    cur[0].r0 = 0; cur[0].c0 = 0; cur[0].lo = 0; cur[0].hi = nnz;

    for (int d = 0; d < l; d++) {
        uint64_t half = t->n >> (d + 1);          /* quadrant side of a level-d node */
        t->nodes[d] = n_cur;
        t->words[d] = (uint64_t *)calloc((size_t)(n_words_for(n_cur) + 1), sizeof(uint64_t));
        /* children of this level, at most 4 per node */
        orc_node *nxt = NULL;
        uint64_t n_nxt = 0;
        if (d + 1 < l) nxt = (orc_node *)malloc((size_t)(4 * n_cur + 1) * sizeof(orc_node));
        for (uint64_t i = 0; i < n_cur; i++) {
            orc_node nd = cur[i];
            uint64_t count[4] = {0, 0, 0, 0};
            for (uint64_t e = nd.lo; e < nd.hi; e++) {
                uint32_t r = (uint32_t)(cell[e] >> 32), c = (uint32_t)cell[e];
                int b1 = (uint64_t)(r - nd.r0) >= half;   /* lower half of the rows */
                int b0 = (uint64_t)(c - nd.c0) >= half;   /* right half of the columns */
                count[2 * b1 + b0]++;
            }
            /* stable split into the four quadrant buckets, in order b = 0..3 */
            uint64_t start[4];
            start[0] = nd.lo;
            for (int b = 1; b < 4; b++) start[b] = start[b - 1] + count[b - 1];
            uint64_t fill[4] = {start[0], start[1], start[2], start[3]};
            for (uint64_t e = nd.lo; e < nd.hi; e++) {
                uint32_t r = (uint32_t)(cell[e] >> 32), c = (uint32_t)cell[e];
                int b = 2 * ((uint64_t)(r - nd.r0) >= half) + ((uint64_t)(c - nd.c0) >= half);
                tmp[fill[b]++] = cell[e];
            }
            for (uint64_t e = nd.lo; e < nd.hi; e++) cell[e] = tmp[e];
            unsigned sig = 0;
            for (int b = 0; b < 4; b++) {
                if (count[b] == 0) continue;
                sig |= 1u << b;
                if (nxt) {
                    orc_node ch;
                    ch.r0 = nd.r0 + (uint32_t)((b >> 1) * half);
                    ch.c0 = nd.c0 + (uint32_t)((b & 1) * half);
                    ch.lo = start[b];
                    ch.hi = start[b] + count[b];
                    nxt[n_nxt++] = ch;
                }
            }
            t->words[d][i / 16] |= (uint64_t)sig << (4 * (i % 16));
        }
        free(cur);
        cur = nxt;
        n_cur = n_nxt;
        if (!cur) { n_cur = 0; cur = (orc_node *)malloc(sizeof(orc_node)); }
    }
    free(cur); free(tmp); free(cell);

    for (int d = 0; d < l; d++) {
        uint64_t nw = n_words_for(t->nodes[d]);
        t->before[d] = (uint64_t *)calloc((size_t)(nw + 1), sizeof(uint64_t));
        uint64_t acc = 0;
        for (uint64_t k = 0; k <= nw; k++) {
            t->before[d][k] = acc;
            if (k < nw) acc += (uint64_t)bit_count(t->words[d][k]);
        }
    }
    *out = t;
    return ORC_OK;
}

/* ----------------------------------------------------------- accessors */

int orc_levels(const orc_tree *t) { return t->levels; }
uint64_t orc_nnz(const orc_tree *t) { return t->nnz; }
uint64_t orc_level_nodes(const orc_tree *t, int d) { return t->nodes[d]; }
uint64_t orc_level_nwords(const orc_tree *t, int d) { return n_words_for(t->nodes[d]); }

void orc_level_words(const orc_tree *t, int d, uint64_t *out) {
    memcpy(out, t->words[d], (size_t)n_words_for(t->nodes[d]) * sizeof(uint64_t));
}

/* Offset of the first child of every node of level d (by rank). */
void orc_child_offsets(const orc_tree *t, int d, uint64_t *out) {
    for (uint64_t i = 0; i < t->nodes[d]; i++) out[i] = rank_before(t, d, i);
}

/* Sampled directory of level d: entry k = offset of the first child of node
   k*S, i.e. the set bits of the signatures of nodes 0..k*S-1 (Sec. 3.2). */
void orc_directory(const orc_tree *t, int d, uint64_t S, uint64_t *out) {
    uint64_t nb = (t->nodes[d] + S - 1) / S;
    for (uint64_t k = 0; k < nb; k++) {
        uint64_t acc = 0;
        for (uint64_t u = 0; u < k * S; u++) acc += (uint64_t)bit_count(nibble_of(t, d, u));
        out[k] = acc;
    }
}

/* --------------------------------------------------------------- descent */

typedef struct {
    const orc_tree *t;
    int dir, semiring;
    uint32_t B;
    const void *x;
    void *y;
    /* band restriction: only output indices in [band_lo, band_hi) */
    uint64_t band_lo, band_hi;
    /* cell enumeration mode */
    uint32_t *cell_r, *cell_c;
    uint64_t n_cells;
} orc_walk;

static void apply_cell(orc_walk *w, uint64_t r, uint64_t c) {
    if (w->cell_r) {
        w->cell_r[w->n_cells] = (uint32_t)r;
        w->cell_c[w->n_cells] = (uint32_t)c;
        w->n_cells++;
        return;
    }
    uint64_t o = (w->dir == ORC_RIGHT) ? r : c;   /* output index */
    uint64_t s = (w->dir == ORC_RIGHT) ? c : r;   /* input index */
    if (o < w->band_lo || o >= w->band_hi) return;
    for (uint32_t v = 0; v < w->B; v++) {
        uint64_t io = o * w->B + v, is = s * w->B + v;
        switch (w->semiring) {
        case ORC_PLUS_TIMES: {
            double *y = (double *)w->y;
            y[io] += (double)((const float *)w->x)[is];
            break;
        }
        case ORC_BOOLEAN_F32: {
            float *y = (float *)w->y;
            if (((const float *)w->x)[is] != 0.0f) y[io] = 1.0f;
            break;
        }
        case ORC_BOOLEAN_U32: {
            uint32_t *y = (uint32_t *)w->y;
            y[io] |= ((const uint32_t *)w->x)[is];
            break;
        }
        case ORC_TROPICAL: {
            float *y = (float *)w->y;
            volatile float contrib = 1.0f + ((const float *)w->x)[is];
            if (contrib < y[io]) y[io] = contrib;
            break;
        }
        }
    }
}

static void walk(orc_walk *w, int d, uint64_t node, uint64_t r0, uint64_t c0) {
    const orc_tree *t = w->t;
    unsigned s = nibble_of(t, d, node);
    uint64_t size = t->n >> d;                  /* side of this node's block */
    /* prune blocks outside the output band */
    if (!w->cell_r) {
        uint64_t o0 = (w->dir == ORC_RIGHT) ? r0 : c0;
        if (o0 + size <= w->band_lo || o0 >= w->band_hi) return;
    }
    if (d == t->levels - 1) {
        for (unsigned q = 0; q < 4; q++)
            if (s & (1u << q)) apply_cell(w, r0 + (q >> 1), c0 + (q & 1));
        return;
    }
    uint64_t first = rank_before(t, d, node);
    uint64_t half = size / 2, j = 0;
    for (unsigned b = 0; b < 4; b++) {
        if (!(s & (1u << b))) continue;
        walk(w, d + 1, first + j, r0 + (b >> 1) * half, c0 + (b & 1) * half);
        j++;
    }
}

static size_t elem_size(int semiring) { return semiring == ORC_PLUS_TIMES ? 8 : 4; }

static void fill_zero(int semiring, void *y, uint64_t count) {
    if (semiring == ORC_TROPICAL) {
        float *f = (float *)y;
        for (uint64_t i = 0; i < count; i++) f[i] = INFINITY;
    } else {
        memset(y, 0, (size_t)count * elem_size(semiring));
    }
}

/* Cells of the matrix, enumerated by descent (row/col arrays of nnz). */
uint64_t orc_cells(const orc_tree *t, uint32_t *rows, uint32_t *cols) {
    orc_walk w;
    memset(&w, 0, sizeof w);
    w.t = t; w.cell_r = rows; w.cell_c = cols;
    if (t->nodes[0]) walk(&w, 0, 0, 0, 0);
    return w.n_cells;
}

/* y = A x (dir RIGHT) or y^T = x^T A (dir LEFT) by naive descent.  x and y
   are row-major (length x B).  Work is split into 'threads' disjoint bands
   of output indices; each band descends from the root on its own. */
int orc_spmv(const orc_tree *t, int dir, int semiring, uint32_t B,
             const void *x, void *y, int threads) {
    if (B == 0 || (dir != ORC_RIGHT && dir != ORC_LEFT) || semiring < 0 || semiring > 3)
        return ORC_E_ARG;
    uint64_t n_out = (dir == ORC_RIGHT) ? t->n_rows : t->n_cols;
    fill_zero(semiring, y, n_out * B);
    if (threads < 1) threads = 1;
    uint64_t band = (t->n + (uint64_t)threads - 1) / (uint64_t)threads;
    #pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
    for (int p = 0; p < threads; p++) {
        orc_walk w;
        memset(&w, 0, sizeof w);
        w.t = t; w.dir = dir; w.semiring = semiring; w.B = B; w.x = x; w.y = y;
        w.band_lo = (uint64_t)p * band;
        w.band_hi = w.band_lo + band;
        if (t->nodes[0]) walk(&w, 0, 0, 0, 0);
    }
    return ORC_OK;
}

/* The product from its definition over the deduplicated edge list. */
static void edge_apply(int dir, int semiring, uint32_t B, const void *x, void *y,
                       uint64_t o, uint64_t s, uint64_t o_slot) {
    (void)o;
    for (uint32_t v = 0; v < B; v++) {
        uint64_t io = o_slot * B + v, is = s * B + v;
        switch (semiring) {
        case ORC_PLUS_TIMES: ((double *)y)[io] += (double)((const float *)x)[is]; break;
        case ORC_BOOLEAN_F32: if (((const float *)x)[is] != 0.0f) ((float *)y)[io] = 1.0f; break;
        case ORC_BOOLEAN_U32: ((uint32_t *)y)[io] |= ((const uint32_t *)x)[is]; break;
        case ORC_TROPICAL: {
            volatile float contrib = 1.0f + ((const float *)x)[is];
            if (contrib < ((float *)y)[io]) ((float *)y)[io] = contrib;
            break;
        }
        }
    }
    (void)dir;
}

int orc_spmv_edges(const uint32_t *rows, const uint32_t *cols, uint64_t m,
                   uint32_t n_rows, uint32_t n_cols, int dir, int semiring, uint32_t B,
                   const void *x, void *y) {
    if (B == 0 || (dir != ORC_RIGHT && dir != ORC_LEFT) || semiring < 0 || semiring > 3)
        return ORC_E_ARG;
    uint64_t *cell = NULL, nnz = 0;
    int rc = dedupe(rows, cols, m, n_rows, n_cols, &cell, &nnz);
    if (rc) return rc;
    uint64_t n_out = (dir == ORC_RIGHT) ? n_rows : n_cols;
    fill_zero(semiring, y, n_out * B);
    for (uint64_t e = 0; e < nnz; e++) {
        uint64_t r = cell[e] >> 32, c = (uint32_t)cell[e];
        uint64_t o = (dir == ORC_RIGHT) ? r : c, s = (dir == ORC_RIGHT) ? c : r;
        edge_apply(dir, semiring, B, x, y, o, s, o);
    }
    free(cell);
    return ORC_OK;
}

/* Selected outputs only, from the definition: y_sample[k] is output index
   sample[k] (sample entries distinct).  Used where the whole product is too
   large for the other routines. */
int orc_spmv_sample(const uint32_t *rows, const uint32_t *cols, uint64_t m,
                    uint32_t n_rows, uint32_t n_cols, int dir, int semiring, uint32_t B,
                    const void *x, const uint32_t *sample, uint64_t n_sample, void *y_sample) {
    if (B == 0 || (dir != ORC_RIGHT && dir != ORC_LEFT) || semiring < 0 || semiring > 3)
        return ORC_E_ARG;
    uint64_t n_out = (dir == ORC_RIGHT) ? n_rows : n_cols;
    int64_t *slot = (int64_t *)malloc((size_t)n_out * sizeof(int64_t));
    if (!slot) return ORC_E_OOM;
    for (uint64_t i = 0; i < n_out; i++) slot[i] = -1;
    for (uint64_t k = 0; k < n_sample; k++) {
        if (sample[k] >= n_out) { free(slot); return ORC_E_RANGE; }
        slot[sample[k]] = (int64_t)k;
    }
    /* collect the sampled outputs' cells, then deduplicate them */
    uint64_t cap = 1024, n_sel = 0;
    uint64_t *sel = (uint64_t *)malloc(cap * sizeof(uint64_t));
    for (uint64_t e = 0; e < m; e++) {
        if (rows[e] >= n_rows || cols[e] >= n_cols) { free(slot); free(sel); return ORC_E_RANGE; }
        uint64_t o = (dir == ORC_RIGHT) ? rows[e] : cols[e];
        if (slot[o] < 0) continue;
        if (n_sel == cap) { cap *= 2; sel = (uint64_t *)realloc(sel, cap * sizeof(uint64_t)); }
        sel[n_sel++] = ((uint64_t)rows[e] << 32) | cols[e];
    }
    qsort(sel, n_sel, sizeof(uint64_t), cmp_u64);
    fill_zero(semiring, y_sample, n_sample * B);
    for (uint64_t e = 0; e < n_sel; e++) {
        if (e > 0 && sel[e] == sel[e - 1]) continue;
        uint64_t r = sel[e] >> 32, c = (uint32_t)sel[e];
        uint64_t o = (dir == ORC_RIGHT) ? r : c, s = (dir == ORC_RIGHT) ? c : r;
        edge_apply(dir, semiring, B, x, y_sample, o, s, (uint64_t)slot[o]);
    }
    free(sel); free(slot);
    return ORC_OK;
}

/* ---- multi-source search (Sec. 5.8) ----------------------------------
 * Hop distances from several sources of a square n x n matrix, one level
 * per step, as the paper's search computes them by iterating the batched
 * Boolean product to its fixed point.  A step in direction RIGHT reaches row
 * r from column c for every cell (r, c) (the right product's y[r] gathers
 * x[c]); LEFT reaches column c from row r.  dist[v * n_src + j] is the hop
 * count from sources[j] to v, 0 at the source, -1 when v is not reached
 * within max_levels steps.  Written as a plain queue search per source over
 * adjacency lists built from the edge list; duplicated edges are harmless. */
int orc_bfs(const uint32_t *rows, const uint32_t *cols, uint64_t m, uint32_t n, int dir,
            const uint32_t *sources, uint32_t n_src, uint32_t max_levels, int32_t *dist) {
    if ((m && (!rows || !cols)) || (n_src && (!sources || !dist)) || n == 0) return ORC_E_ARG;
    if (dir != ORC_RIGHT && dir != ORC_LEFT) return ORC_E_ARG;
    for (uint32_t j = 0; j < n_src; j++)
        if (sources[j] >= n) return ORC_E_RANGE;
    uint64_t *start = (uint64_t *)calloc((size_t)n + 1, sizeof(uint64_t));
    uint32_t *adj = (uint32_t *)malloc((size_t)(m ? m : 1) * sizeof(uint32_t));
    if (!start || !adj) { free(start); free(adj); return ORC_E_OOM; }
    for (uint64_t e = 0; e < m; e++) {
        if (rows[e] >= n || cols[e] >= n) { free(start); free(adj); return ORC_E_RANGE; }
        uint32_t from = (dir == ORC_RIGHT) ? cols[e] : rows[e];
        start[from + 1]++;
    }
    for (uint64_t v = 0; v < n; v++) start[v + 1] += start[v];
    uint64_t *fillp = (uint64_t *)malloc((size_t)n * sizeof(uint64_t));
    if (!fillp) { free(start); free(adj); return ORC_E_OOM; }
    memcpy(fillp, start, (size_t)n * sizeof(uint64_t));
    for (uint64_t e = 0; e < m; e++) {
        uint32_t from = (dir == ORC_RIGHT) ? cols[e] : rows[e];
        uint32_t to = (dir == ORC_RIGHT) ? rows[e] : cols[e];
        adj[fillp[from]++] = to;
    }
    free(fillp);
    for (uint64_t k = 0; k < (uint64_t)n * n_src; k++) dist[k] = -1;
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < (int64_t)n_src; j++) {
        uint32_t *queue = (uint32_t *)malloc((size_t)n * sizeof(uint32_t));
        if (!queue) {
#pragma omp critical
            err = ORC_E_OOM;
            continue;
        }
        uint64_t head = 0, tail = 0;
        uint32_t s = sources[j];
        dist[(uint64_t)s * n_src + (uint64_t)j] = 0;
        queue[tail++] = s;
        while (head < tail) {
            uint32_t u = queue[head++];
            int32_t du = dist[(uint64_t)u * n_src + (uint64_t)j];
            if ((uint32_t)du >= max_levels) continue;
            for (uint64_t a = start[u]; a < start[u + 1]; a++) {
                uint32_t v = adj[a];
                int32_t *dv = &dist[(uint64_t)v * n_src + (uint64_t)j];
                if (*dv < 0) {
                    *dv = du + 1;
                    queue[tail++] = v;
                }
            }
        }
        free(queue);
    }
    free(start); free(adj);
    return err;
}
