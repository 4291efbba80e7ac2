/*
 * k2spmv.h -- C ABI of a k^2-tree SpMV library for the AMD Instinct MI355X
 * (gfx950, CDNA4).
 *
 * The operations follow Tosoni & Mencagli, "A GPU Engine for Sparse
 * Matrix-Vector Products on k^2-Tree-Compressed Graphs" (arXiv:2611.03610v1):
 *   - the k^2-tree with k = 2 of a Boolean matrix (Sec. 2.1),
 *   - the semiring products y = A x and y^T = x^T A (Sec. 2.2, Table 1,
 *     Sec. 3.6), for one vector or a row-major batch (Sec. 3.6),
 *   - the level-synchronous traversal with child offsets from popcount
 *     prefix sums seeded by a sampled directory (Sec. 3, Algorithm 1,
 *     Sec. 3.2), tiled so that its scratch is fixed before a product runs
 *     (Sec. 3.4), and the optional cached last internal level (Sec. 3.5),
 *   - the device memory of a product, known after construction and before
 *     any kernel runs (Sec. 1 and Sec. 3.4).
 *
 * Conventions
 *   - Every call returns a k2_status and never throws.  Invalid input is
 *     rejected before anything is written.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are HIP
 *     device memory (for instance from torch.empty(..., device="cuda")).
 *   - Streams are passed as void* and are hipStream_t values; NULL means the
 *     default (null) stream.
 *   - A matrix is n_rows x n_cols; the tree pads it to n x n, n = 2^l,
 *     l = max(2, ceil(log2(max(n_rows, n_cols)))).  Padding costs nothing.
 *   - Vectors are row-major: a batch of B vectors over n entries is n*B
 *     elements, entry i of vector v at [i*B + v].  Right product: x has
 *     n_cols*B elements and y n_rows*B; left product: swapped.
 *   - Products overwrite y (it starts from the semiring zero).
 */
#ifndef K2SPMV_H
#define K2SPMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    K2_OK = 0,
    K2_E_INVALID_ARG = 1,     /* null pointer, bad enum, batch 0, ... */
    K2_E_INDEX_RANGE = 2,     /* an edge index >= its dimension */
    K2_E_ARENA_TOO_SMALL = 3, /* arena smaller than the estimate */
    K2_E_HOST_OOM = 4,        /* host allocation failed */
    K2_E_HIP = 5,             /* a HIP runtime call failed (see k2_last_hip_error) */
    K2_E_UNSUPPORTED = 6      /* size or option outside what this build handles */
} k2_status;

/* Table 1 of the pages: plus-times (w = 1, atomic add), Boolean (or-and,
   contribution [x_j != 0], atomic max on the bit patterns of 0 and 1),
   tropical (min-plus, w = 1, contribution 1 + x_j rounded to fp32, atomic
   min on bit patterns; x must be >= 0 or +inf, zero element +inf).
   K2_BOOLEAN_U32X32 packs 32 Boolean vectors per uint32 word (bit v of word
   i is entry i of vector v) and accumulates with bitwise or. */
typedef enum {
    K2_PLUS_TIMES_F32 = 0,
    K2_BOOLEAN_F32 = 1,
    K2_BOOLEAN_U32X32 = 2,
    K2_TROPICAL_F32 = 3
} k2_semiring;

/* Sec. 3.6: the left product reads the same tree and swaps the decoded
   coordinates at the leaves, so cell (r, c) adds x_r to y_c. */
typedef enum { K2_RIGHT = 0, K2_LEFT = 1 } k2_direction;

/* Which traversal a product uses (Sec. 3.5).  AUTO: the cached last internal
   level when the matrix holds it, else the tree-only descent. */
typedef enum { K2_MODE_AUTO = 0, K2_MODE_TREE_ONLY = 1, K2_MODE_CACHED = 2 } k2_mode;

/* Flag or-ed into the mode of k2_spmv: skip the fill and accumulate into the
   caller's y (y = y (+) A x), for products summed over several matrices or
   steps that update a running vector. */
#define K2_SPMV_ACCUMULATE 0x100

typedef struct {
    /* Tiled descent (Sec. 3.4): a tile is a contiguous node range whose
       subtree holds at most tile_nodes nodes on every level; one workgroup
       descends a tile with its frontier in LDS (the cached level's creation,
       streamed products).  Tree-only products cut their band sub-tiles and
       rest tiles at min(tile_nodes, 256) nodes per level instead, one wave
       each.  256..4096, power of 2.  Default 1024. */
    uint32_t tile_nodes;
    /* Host-side top (Sec. 3.4): the device starts from the deepest level with
       at most host_top_max nodes (never below the last internal level).
       Default 65536. */
    uint32_t host_top_max;
    /* Keep the last internal level's nodes on the device (Sec. 3.5, "k2+F"),
       12 bytes per node: the block coordinates their Morton codes encode (8
       bytes, the pages' cached codes) and a 4-byte node word with the
       node's cells as its leaves give them and, when every cached tile has
       a band window of at most 1024 rows, the block's place inside its
       window's quadrant; a product then reads neither the level's
       signatures nor its leaves, and with band windows only the node words.
       Default 0. */
    int32_t cache_last_level;
    /* Order of the cached-level tiles for the MI355X's 8 XCDs (each with
       its own L2; workgroup b runs on XCD b % 8).  The tiles are kept in
       order of output blocks (about 16 MB of y each); with 1, the band tiles
       of a block and its sparse tiles are each cut into 8 runs of about
       equal work and run k goes to positions k, k + 8, ..., so each XCD
       takes neighbouring bands (their shared x columns in its own L2) while
       all XCDs stay in one block of y.  Padding tiles (count 0) even out
       the lists.  0 keeps the block order.  Descent tiles keep their Z
       order either way.  Default 1. */
    int32_t xcd_remap;
    /* Output windows for products over the cached level and for tree-only
       plus-times products (their band groups): Q is the largest
       power of 2 with Q * window_batch <= window_elems (at most 16384
       elements of 4 bytes; 0 disables).  A tile made of the dense Q x Q
       quadrants of one row band (right products) or column band (left
       products) accumulates its outputs in LDS and adds them to y once (a
       band's only cached tile stores them instead).
       Products with more than window_batch vectors use the same windows
       while Q x batch elements fit one workgroup's LDS (fewer workgroups per
       CU), else direct atomics everywhere.  Defaults 4096 and 8. */
    uint32_t window_elems;
    uint32_t window_batch;
    /* Where the kernels get child offsets (Sec. 3.2, "ChildOffset"; the
       ablation of Sec. 5.5 compares the two):
       K2_OFFSETS_DIRECTORY: on the device, from the directory (one sample per
         256 nodes of each internal level) plus the popcounts of at most 16
         signature words: per descent tile and level, and per 64-node segment
         of the cached level.
       K2_OFFSETS_SCAN: from exclusive prefix sums of the fan-outs: the host
         plan holds each descent tile's first child offset on every level it
         spans and each cached segment's first leaf; the kernels scan the
         fan-outs inside tiles and segments.  No directory is uploaded.
       K2_OFFSETS_AUTO: K2_OFFSETS_SCAN (measured at least as fast on gfx950
         for every workload here, single and batched).  Default AUTO. */
    int32_t offsets;
    /* With windows and a cached level: 1 gives every row band (right
       products) or column band (left) that holds nodes outside the dense
       quadrants a windowed tile, and those nodes are added to their band's
       window too (strays), instead of one y atomic per cell from separate
       sparse tiles.  k2_matrix_create groups the strays by band on the
       device (8 bytes per stray node and direction: its block's coordinates
       and its cells, read from its leaves once).  0: sparse tiles.
       Default 1. */
    int32_t band_strays;
    /* Nodes of the last internal level per windowed cached tile (Sec. 3.4's
       tiles over the cached level, Sec. 3.5).  A band holding more is cut
       into several tiles that each add their window to y with atomics after
       the fill; a band of one tile stores its window.  64..2^30.
       Default 65536. */
    uint32_t band_tile_nodes;
} k2_plan_opts;

enum { K2_OFFSETS_AUTO = 0, K2_OFFSETS_DIRECTORY = 1, K2_OFFSETS_SCAN = 2 };

/* Device bytes of a matrix and of one product, by part; 'arena' is what
   k2_matrix_create needs, 'vectors' the caller's x and y for the semiring
   and batch asked about, 'total' = arena + vectors. */
typedef struct {
    uint64_t tree;        /* signatures of the levels the device reads */
    uint64_t directory;   /* offset source: one uint32 per 256 nodes of each
                             internal level (directory), or the planned first
                             child offsets of the descent tiles (scan) */
    uint64_t top_codes;   /* Morton codes of the tile starts (host top + splits) */
    uint64_t tiles;       /* the tile plan */
    uint64_t cached_codes;/* 12 bytes per node of the last internal level (block
                             coordinates and node words), plus 8 per stray node
                             and direction (band_strays), or 0 */
    uint64_t scratch;     /* transient product memory: a bit per input row
                             (max(n_rows, n_cols) bits) that products of the
                             max / or / min semirings rebuild from x (the
                             frontiers live in LDS) */
    uint64_t alignment;   /* padding between parts */
    uint64_t arena;       /* sum of the above */
    uint64_t vectors;     /* x and y */
    uint64_t total;       /* arena + vectors */
} k2_mem_breakdown;

typedef struct {
    uint32_t n_rows, n_cols;
    uint32_t levels;      /* l */
    uint32_t top_level;   /* d0 for the default plan options */
    uint64_t nnz;         /* distinct non-zeros */
    uint64_t nodes;       /* all levels */
} k2_tree_info_t;

typedef struct k2_tree k2_tree;
typedef struct k2_matrix k2_matrix;
typedef struct k2_stream k2_stream;

/* Fill 'opts' with the defaults above: the tile size and host top of the
   tiled descent (Sec. 3.4), the offset source (Sec. 3.2) and the settings the
   ablation of Sec. 5.5 varies, at the values measured best on gfx950.
   Errors: K2_E_INVALID_ARG (null). */
k2_status k2_plan_defaults(k2_plan_opts *opts);

/* Build the tree of the Boolean matrix whose non-zeros are the pairs
   (rows[e], cols[e]), e < n_edges (host arrays; copied, not kept).
   Duplicate pairs count once.  n_threads = 0 uses the host's cores (at most
   64).  *out is a host object owned by the caller (k2_tree_free).
   Errors: K2_E_INVALID_ARG (null pointer with n_edges > 0, n_rows or n_cols
   zero), K2_E_INDEX_RANGE (rows[e] >= n_rows or cols[e] >= n_cols),
   K2_E_UNSUPPORTED (a level with 2^32 or more nodes), K2_E_HOST_OOM.
   (Sec. 2.1; construction on the host as in Sec. 5.1.) */
k2_status k2_build(const uint32_t *rows, const uint32_t *cols, uint64_t n_edges,
                   uint32_t n_rows, uint32_t n_cols, uint32_t n_threads, k2_tree **out);

/* Release a tree built by k2_build (null is ignored).  A tree is built once
   and serves any number of products (Sec. 4 and Sec. 5.1: compress once,
   multiply many times); a matrix made from it by k2_matrix_create keeps no
   pointer to it and may outlive it, a stream plan (k2_stream_create) may
   not. */
void k2_tree_free(k2_tree *tree);

/* Sizes of a tree (host): the dimensions, l with n = 2^l (Sec. 2.1: the
   matrix padded to n x n), the host-top level d0 the default options give
   (Sec. 3.4: the deepest level with at most 2^16 nodes, never below l-2),
   the distinct non-zeros and the node count of all levels (Table 2 reports
   these sizes per graph).  Errors: K2_E_INVALID_ARG (null). */
k2_status k2_tree_info(const k2_tree *tree, k2_tree_info_t *out);

/* Node count of every level in level order (Sec. 2.1; the popcount of level
   d's signatures is the node count of level d+1), nodes[0..levels-1] (host
   array of 'levels' entries from k2_tree_info).  Errors: K2_E_INVALID_ARG. */
k2_status k2_tree_level_nodes(const k2_tree *tree, uint64_t *nodes);

/* Canonical export of level 'level' (Sec. 2.1: one signature per nibble, in
   level order): node i's signature in bits 4*(i%16)..4*(i%16)+3 of word
   i/16, unused high nibbles zero.  'words' is a host array of n_words >=
   ceil(nodes/16) entries.  Errors: K2_E_INVALID_ARG. */
k2_status k2_tree_level_words(const k2_tree *tree, uint32_t level, uint64_t *words,
                              uint64_t n_words);

/* Sampled directory of internal level 'level' (Sec. 3.2, S = 256): entry k
   is the offset in level+1 of the first child of node 256*k.  'out' is a host
   array of ceil(nodes/256) entries.  Errors: K2_E_INVALID_ARG (leaf level). */
k2_status k2_tree_directory(const k2_tree *tree, uint32_t level, uint32_t *out, uint64_t n_out);

/* Device bytes of a matrix created with 'opts' plus the x and y of a product
   over 'semiring' with 'batch' vectors (words, for K2_BOOLEAN_U32X32).
   Host only: no HIP call.  The arena k2_matrix_create needs is out->arena.
   (Sec. 1 and 3.4: memory fixed by the tree and the tile size.) */
k2_status k2_estimate_device_bytes(const k2_tree *tree, const k2_plan_opts *opts,
                                   k2_semiring semiring, uint32_t batch,
                                   k2_mem_breakdown *out);

/* The tile plans a matrix created with 'opts' would use (host only, no HIP
   call; Sec. 3.4).  which = 0: the descent tiles (depth first) and their
   start codes (all codes of the plan); 1 / 2: the cached-level tiles of
   right / left products and their segments (empty unless
   opts->cache_last_level); for tree-only right / left products, 3 / 4: the
   rest tiles and their skip ranges, 5 / 6: the band groups, 7 / 8: the
   band groups' tiles, 9 / 10: the stray segments of right / left products.
   Reports the host-top level d0, the number of tiles and of aux entries
   (see k2_plan_tiles).  Errors: K2_E_INVALID_ARG. */
k2_status k2_plan_info(const k2_tree *tree, const k2_plan_opts *opts, int32_t which,
                       uint32_t *top_level, uint64_t *n_tiles, uint64_t *n_aux);

/* The tiles themselves (Sec. 3.4, Fig. 2: tiles descended depth first), in
   the order the kernels take them.
   tiles[8k..8k+7] = (first, count, level, code index, window row, window
   column, log2 of the window side or 0xFFFFFFFF for no window, base index).
   With scan offsets a tile's (descent, band or rest tile) first child
   offsets on levels level .. l-2 (the last its first leaf) are entries
   base index .. of the plan's offsets (k2_plan_offsets); otherwise the base
   index is 0.
   which = 0: 'count' nodes of 'level' from node 'first', whose Morton codes
   (row bit above column bit per level, 2*level bits) are aux[code index ..].
   Tree-only right / left products take, when windows are planned and the
   batch fits them, first the band groups (which = 5 / 6), each a workgroup's
   job: 'count' tiles from tile 'first' of list 7 / 8 (descent tiles as for
   0, over the dense quadrants of one row / column band), sharing the
   group's window (fields 4-6); then the rest tiles (which = 3 / 4) that
   the groups do not cover whole.  The rest tiles are a second depth-first
   cut like 0 with at most min(tile_nodes, 256) nodes per level (each a
   wave's job), in order of output block (2^k rows / columns, 2^k *
   window_batch * 4 the largest power of 2 <= 16 MB; a tile's block is its
   first node's); after band groups a tile skips the last-internal-level
   nodes they cover: 'window column' ranges from aux index 'window row',
   each aux[r] = (first node << 32) | end node, or 0xFFFFFFFF in 'window
   column' for a tile they cover whole.  Products without band groups (the
   max / or / min semirings, a batch too wide for the windows, no windows
   planned) take every rest tile, skipping nothing: the whole second cut.
   which = 1 / 2: 'count' segments of the last internal level from segment
   'first'; segment r is aux[2r] = (first node << 32) | node count (1..64)
   and aux[2r + 1] = the leaf-level index of its first node's first child.
   With band_strays, a tile of 1 / 2 whose code index has bit 0 set owns its
   band (row band for 1, column band for 2, from the window fields) and also
   adds the band's strays: the nodes of the segments of which = 9 / 10 (no
   tiles; aux as for 1 / 2) whose block's first row (9) or column (10) lies
   in it.  Bit 1 of the code index marks the band's only tile, which stores
   its window to y instead of adding it.
   Host arrays of 8*n_tiles and n_aux entries (sizes from k2_plan_info).
   Errors: K2_E_INVALID_ARG. */
k2_status k2_plan_tiles(const k2_tree *tree, const k2_plan_opts *opts, int32_t which,
                        uint32_t *tiles, uint64_t n_tiles, uint64_t *aux, uint64_t n_aux);

/* The scan offsets of the plan's tiles (host only: descent, band and rest
   tiles): with K2_OFFSETS_SCAN (or AUTO), tile k's first child offsets on
   levels tiles[k].level .. l-2 are bases[base index of tile k ..] (Sec. 3.2: the
   exclusive prefix sums of the fan-outs, sampled at the tile starts); empty
   with K2_OFFSETS_DIRECTORY.  *n_total receives the count; bases may be
   null to ask only for it, else it must hold n_bases >= that many entries.
   Errors: K2_E_INVALID_ARG. */
k2_status k2_plan_offsets(const k2_tree *tree, const k2_plan_opts *opts, uint32_t *bases,
                          uint64_t n_bases, uint64_t *n_total);

/* Upload a tree into the caller's device arena and return a matrix handle:
   the levels from the host top down (Sec. 2.1, Sec. 3.4), the offset source
   (Sec. 3.2: the directory, or the planned prefix sums) and the tile plan,
   which depend on the tree alone and are made once, before any product
   (Sec. 3.4).  The device memory is what k2_estimate_device_bytes returned
   (Sec. 1: known after construction, before any kernel runs): d_arena is a
   caller-owned device buffer of arena_bytes >= that estimate's arena,
   256-byte aligned, and must outlive the matrix; the library allocates no
   device memory.  If opts->cache_last_level, the last internal level's nodes
   are computed here, once, by a descent on the device and kept as the block
   coordinates their Morton codes encode (Sec. 3.5: the cached frontier, 8
   bytes per node).  Runs on 'stream' and synchronizes it before returning.
   Errors: K2_E_INVALID_ARG (null, bad options, unaligned arena),
   K2_E_ARENA_TOO_SMALL, K2_E_HOST_OOM, K2_E_HIP (nothing of the matrix is
   kept; the arena's content is then undefined). */
k2_status k2_matrix_create(const k2_tree *tree, const k2_plan_opts *opts, void *d_arena,
                           uint64_t arena_bytes, void *stream, k2_matrix **out);

/* y = A x (K2_RIGHT) or y^T = x^T A (K2_LEFT) over 'semiring' for 'batch'
   row-major vectors (Algorithm 1), asynchronously on 'stream'.  d_x and d_y
   are device arrays of the lengths given at the top of this file (float, or
   uint32 for K2_BOOLEAN_U32X32); they must not overlap.  y is overwritten.
   'mode' picks the traversal (k2_mode), optionally or-ed with
   K2_SPMV_ACCUMULATE.  Products of the max / or / min semirings first
   mark, in the matrix's arena, the input rows with a contributing vector
   and then list only those rows' cells: two such products of one matrix
   must not run at the same time (on different streams).  Errors
   (nothing launched):
   K2_E_INVALID_ARG (null, batch 0, bad enum, K2_MODE_CACHED without cached
   codes), K2_E_HIP (launch failure). */
k2_status k2_spmv(k2_matrix *matrix, k2_direction direction, k2_semiring semiring,
                  uint32_t batch, int32_t mode, const void *d_x, void *d_y, void *stream);

/* Kernel timing (Sec. 4: products timed on the device between two events),
   with HIP events on the product's stream.  While enabled, every
   k2_spmv records an event before the fill, between the fill and the main
   kernel, and after the main kernel; k2_matrix_last_timing waits for the
   last product and returns the fill and main-kernel durations in ms (the
   fill time is 0 under K2_SPMV_ACCUMULATE).  Errors: K2_E_INVALID_ARG
   (timing off or no product yet), K2_E_HIP. */
k2_status k2_matrix_set_timing(k2_matrix *matrix, int32_t enable);
k2_status k2_matrix_last_timing(k2_matrix *matrix, float *fill_ms, float *kernel_ms);

/* Release a matrix handle and its host-side plan.  The device arena stays
   the caller's (Sec. 1: the arena was sized before any kernel ran), and
   products still queued on a stream must finish first: destroy does not
   synchronize.  Null is ignored.  Errors: none (K2_OK). */
k2_status k2_matrix_destroy(k2_matrix *matrix);

/* Description of the plan a matrix uses (host): its host-top level d0 and
   descent tile count (Sec. 3.4), and whether it keeps the cached last
   internal level (Sec. 3.5): *cached = 0 no, 1 yes, 2 yes and its products
   read only the 4-byte node words (every cached tile has a band window of
   at most 1024 rows; see cache_last_level).  Errors: K2_E_INVALID_ARG
   (null). */
k2_status k2_matrix_info(const k2_matrix *matrix, uint32_t *top_level, uint64_t *n_tiles,
                         int32_t *cached);

/* Copy level 'level' of the device-resident tree back to the host in the
   export layout of k2_tree_level_words (Sec. 2.1: one signature per nibble,
   level order; synchronous; for verification).
   Levels above the top level are not on the device: K2_E_INVALID_ARG. */
k2_status k2_matrix_level_words(const k2_matrix *matrix, uint32_t level, uint64_t *words,
                                uint64_t n_words, void *stream);

/* Copy the cached last internal level back to the host (synchronous):
   blocks[i] = (first row << 32) | first column of the 4x4 block of node i of
   level l-2, the coordinates its Morton code encodes (Sec. 3.5 keeps that
   level's codes; the device keeps them decoded, 8 bytes either way).
   Errors: K2_E_INVALID_ARG if not cached or n_blocks is too small. */
k2_status k2_matrix_cached_blocks(const k2_matrix *matrix, uint64_t *blocks, uint64_t n_blocks,
                                  void *stream);

/* Multi-source search to the fixed point (Sec. 5.8, Table 6): hop distances
   from n_sources sources of a square matrix at once, one level per batched
   Boolean product.  A level's product runs in 'direction' (K2_RIGHT: row r
   is reached from column c for a cell (r, c); K2_LEFT: column c from row r)
   over the packed frontier of the previous level (32 sources per uint32,
   K2_BOOLEAN_U32X32 with batch ceil(n_sources / 32)), with the matrix's
   cached level when it has one; a marking kernel keeps the entries not
   reached before as the next frontier and records their level: as bit
   planes of the packed words for levels below 64 (plane p holds bit p of the
   level), from which one pass writes the whole distance table at the end
   (or before level 64, whose marking then stores distances directly).  The
   search stops after a level that reaches nothing new, or after max_levels
   levels.
     sources            host array of n_sources vertex ids (< n; repeats are
                        independent searches)
     d_dist             device n x n_sources int32, row-major: d_dist[v *
                        n_sources + j] = hops from sources[j] to v, -1 if not
                        reached (overwritten)
     d_workspace        device, 256-byte aligned, k2_bfs_workspace_bytes bytes
                        (caller-owned; the library allocates nothing): 9
                        arrays of n ceil(n_sources / 32) words (frontier,
                        reached set, product output, 6 level planes), a
                        count and the sources
     levels             out: the last level that reached a new entry
     reached_per_level  optional host array of max_levels entries: entries
                        reached at each level run (the last run level's is 0
                        when the search converged)
   Synchronous: the host reads one count per level and the call returns once
   the distance table is written.  Errors:
   K2_E_INVALID_ARG (null, non-square matrix, no sources, small or unaligned
   workspace), K2_E_INDEX_RANGE (a source >= n), K2_E_HIP. */
k2_status k2_bfs_workspace_bytes(const k2_matrix *matrix, uint32_t n_sources, uint64_t *bytes);
k2_status k2_bfs(k2_matrix *matrix, k2_direction direction, const uint32_t *sources, uint32_t n_sources,
                 uint32_t max_levels, int32_t *d_dist, void *d_workspace, uint64_t workspace_bytes,
                 void *stream, uint32_t *levels, uint64_t *reached_per_level);

/* Bytes of the library's fixed scratch array (64 MiB), the workspace of
   k2_bfs_noalloc. */
#define K2_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* k2_bfs for callers that cannot allocate device memory (code that must not
   call hipMalloc: tight serving loops, harnesses that forbid allocation):
   the same search and results, with no workspace argument.  Its workspace
   (k2_bfs_workspace_bytes of this matrix and n_sources, at most
   K2_NOALLOC_SCRATCH_BYTES) is a fixed array inside the library's code
   object, which each GPU the library runs on holds from the library's load
   until the process ends; its device address is looked up on the first
   call on each device.  The call allocates no memory: the caller passes the
   matrix, the sources (host) and d_dist (device, n x n_sources int32, as for
   k2_bfs).  Every call on a GPU uses that GPU's one array and leaves its
   last contents there (the search clears what must start at zero), so
   calls that overlap on one GPU, from several threads or streams, race and
   must be serialized by the caller.  Synchronous like k2_bfs.
   Errors: as k2_bfs, plus K2_E_UNSUPPORTED when the workspace of this
   search (about 36 n ceil(n_sources / 32) bytes) exceeds
   K2_NOALLOC_SCRATCH_BYTES; nothing runs then. */
k2_status k2_bfs_noalloc(k2_matrix *matrix, k2_direction direction, const uint32_t *sources,
                         uint32_t n_sources, uint32_t max_levels, int32_t *d_dist, void *stream,
                         uint32_t *levels, uint64_t *reached_per_level);

/* Out-of-core products (Sec. 7, the paper's direction for trees larger than
   device memory): the tree stays in host memory and each product streams it
   through a caller-owned device staging buffer, chunk by chunk.

   k2_stream_create plans the depth-first descent tiles of 'tree' with
   'opts' (tile_nodes and host_top_max are used; the tiles always carry
   planned scan offsets; no cached level, no windows) and cuts them, in
   order, into chunks of consecutive tiles whose staged data fits half of
   staging_bytes (products alternate between the two halves, copying one
   chunk while the previous one is descended): per level the span of node
   words the chunk's tiles reach (plus one word), then its tiles, start
   codes and scan offsets, each part 256-byte aligned.  It also keeps a
   page-locked host copy of the tree's words and the chunks' metadata
   (hipHostMalloc; the size of the tree) for asynchronous copies; where that
   allocation fails, products copy from the tree itself.  'tree' must
   outlive the stream.  Errors: K2_E_INVALID_ARG, K2_E_ARENA_TOO_SMALL (one
   tile does not fit half the staging), K2_E_HOST_OOM. */
k2_status k2_stream_create(const k2_tree *tree, const k2_plan_opts *opts, uint64_t staging_bytes,
                           k2_stream **out);

/* Chunk count, the largest chunk's staged bytes (a product needs a staging
   buffer of twice this) and the bytes one product copies to the device
   (Sec. 7; host only).  Errors: K2_E_INVALID_ARG (null). */
k2_status k2_stream_info(const k2_stream *stream_plan, uint64_t *n_chunks, uint64_t *max_chunk_bytes,
                         uint64_t *staged_bytes);

/* Chunk 'chunk' of a stream plan (Sec. 7; host only): its tiles
   [*first_tile, *end_tile) of the plan's descent
   tiles (k2_plan_tiles which = 0, same options) and, for levels 0 ..
   n_levels-1, the first staged word and the staged word count (0: none).
   Errors: K2_E_INVALID_ARG. */
k2_status k2_stream_chunk(const k2_stream *stream_plan, uint64_t chunk, uint64_t *first_tile,
                          uint64_t *end_tile, uint64_t *lo_words, uint64_t *n_words, uint32_t n_levels);

/* One product of Sec. 7 (the tree in host memory, streamed to the device)
   as k2_spmv (direction, semiring, batch, device x and y, flags
   0 or K2_SPMV_ACCUMULATE), tree-only, with the tree streamed: per chunk its
   level words, tiles, codes and offsets are copied from host memory into
   one half of d_staging (256-byte aligned, at least 2 max_chunk_bytes) on a
   copy stream of the library's, and the chunk's tiles are descended from
   there on 'stream'; events keep a half's copies behind the last kernel that
   read it and each kernel behind its copies, so copies overlap the kernel of
   the chunk before.  Asynchronous like k2_spmv; products of one stream plan
   must not run concurrently.
   Errors: K2_E_INVALID_ARG (null, small or unaligned staging, overlapping
   x and y), K2_E_HIP. */
k2_status k2_stream_spmv(k2_stream *stream_plan, k2_direction direction, k2_semiring semiring,
                         uint32_t batch, int32_t flags, const void *d_x, void *d_y, void *d_staging,
                         uint64_t staging_bytes, void *stream);

/* Release a stream plan of Sec. 7 and its page-locked host copy (null is
   ignored); products still queued on a stream must finish first. */
void k2_stream_destroy(k2_stream *stream_plan);

/* Text of a status code.  The pages define no API; every call here checks
   its arguments on the host and returns a code before any kernel runs, as
   the plan and device memory of a product are fixed before it (Sec. 1,
   Sec. 3.4).  Never null; unknown codes give "unknown status". */
const char *k2_status_string(k2_status status);

/* Text of the last HIP error this thread saw (empty string if none), behind
   a K2_E_HIP status of any call (Sec. 4: products run on the device through
   the runtime, whose errors surface here). */
const char *k2_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* K2SPMV_H */
