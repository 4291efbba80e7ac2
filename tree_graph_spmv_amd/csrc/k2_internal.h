// k2_internal.h -- structures shared by the host runtime and the HIP kernels.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/k2spmv.h"

// Functions of the structures below that both the host code and the HIP
// kernels call.
#if defined(__HIP__)
#define K2_HD __host__ __device__
#else
#define K2_HD
#endif

namespace k2 {

constexpr int kMaxLevels = 32;     // n <= 2^32
constexpr uint32_t kDirBlock = 256;  // directory sample S (Sec. 3.2)
constexpr uint32_t kWordsPerBlock = kDirBlock / 16;

// Host tree: per level, node count and packed signatures (16 per word, node i
// at bits 4*(i%16)); per internal level, the S = 256 directory.
struct HostTree {
    uint32_t n_rows = 0, n_cols = 0;
    int levels = 0;
    uint64_t nnz = 0;
    std::vector<uint64_t> nodes;                 // [levels]
    std::vector<std::vector<uint64_t>> words;    // [levels][ceil(nodes/16)]
    std::vector<std::vector<uint32_t>> dir;      // [levels-1][ceil(nodes/256)]
};

inline unsigned nibble(const std::vector<uint64_t> &w, uint64_t i) {
    return unsigned(w[i >> 4] >> ((i & 15) * 4)) & 0xFu;
}

// Offset in level d+1 of the first child of node i of level d, from the
// directory plus the popcounts of the words before i in its block.
uint64_t child_offset(const HostTree &t, int d, uint64_t i);

// One tile: 'count' consecutive nodes of level 'level' starting at node
// 'first'; for descent tiles their codes are codes[code_off ..].  A tile with
// a window (win_log2 != kNoWindow) lies inside the 2^win_log2 x 2^win_log2
// quadrant at (win_row, win_col) and accumulates its outputs in LDS.
constexpr uint32_t kNoWindow = 0xFFFFFFFFu;
struct Tile {
    uint32_t first;
    uint32_t count;
    uint32_t level;
    uint32_t code_off;
    uint32_t win_row;
    uint32_t win_col;
    uint32_t win_log2;
    uint32_t base_off;   // descent tiles with scan offsets: index into tile_bases
};
static_assert(sizeof(Tile) == 32, "tile layout");

// A tile of the second depth-first cut (tree-only rest tiles, a wave's job):
// 'count' (at most 256) nodes of 'level' from node 'first', their codes at
// code_off, their scan offsets at base_off.  The cut is shared by both
// directions; each direction orders it through a list of indexes.
struct RestTile {
    uint32_t first;
    uint32_t code_off;
    uint32_t base_off;
    uint32_t shape;   // count | level << 16
    K2_HD uint32_t count() const { return shape & 0xFFFFu; }
    K2_HD uint32_t level() const { return shape >> 16; }
};
static_assert(sizeof(RestTile) == 16, "rest tile layout");

// A rest tile that band groups cover in part: its index in the cut and its
// skip ranges (skip_count ranges from skip_row of the direction's list).
struct RestTake {
    uint32_t tile;
    uint32_t skip_row;
    uint32_t skip_count;
    uint32_t unused;
};
static_assert(sizeof(RestTake) == 16, "rest take layout");

// A segment of a cached tile: up to kSegNodes consecutive nodes of the last
// internal level, one wave's job, with the level-order index of the first
// node's first child (its first leaf), so the kernel needs no rank query.
constexpr uint32_t kSegNodes = 64;
struct Seg {
    uint32_t lo;
    uint32_t count;
    uint32_t leaf;
    uint32_t pad;
};
static_assert(sizeof(Seg) == 16, "segment layout");

// A stray: a node of the cached level outside the dense quadrants, stored
// again with its band's other strays so that a band tile can add its cells to
// the band's window, in 8 bytes: its cells as read from its leaves when the
// matrix is created (bit 4 b + q: cell q of the leaf for child b; bits
// 48-63), so that a product reads no leaf at a stray's random position; its
// block's output coordinate relative to the band, in blocks (bits 36-47; a
// band has at most 16384 outputs, 4096 blocks); and its block's input
// coordinate, in blocks (bits 0-35).  Outputs are rows for right products
// (row bands) and columns for left products.
struct StrayRec {
    uint64_t bits;
    K2_HD static StrayRec make(uint32_t cells, uint32_t out_in_band, uint64_t in) {
        return StrayRec{(uint64_t(cells) << 48) | (uint64_t(out_in_band >> 2) << 36) | (in >> 2)};
    }
    K2_HD uint32_t cells() const { return uint32_t(bits >> 48); }
    K2_HD uint32_t out_in_band() const { return uint32_t((bits >> 36) & 0xFFFu) << 2; }
    K2_HD uint64_t in() const { return (bits & 0xFFFFFFFFFull) << 2; }
};
static_assert(sizeof(StrayRec) == 8, "stray layout");

// The plan of a matrix: host top level, descent tiles in depth-first order and
// the codes their first level starts from, and per product direction the
// tiles of the cached level (a cached tile is 'count' segments starting at
// cached_segs[dir][first]).
struct Plan {
    int top_level = 0;                 // d0
    uint32_t tile_nodes = 0;
    int window_log2 = -1;              // quadrant side of the windows, -1: none
    std::vector<uint64_t> codes;       // tile start codes
    std::vector<Tile> tiles;           // descent tiles
    std::vector<Tile> cached_tiles[2];
    std::vector<Seg> cached_segs[2];
    // offset source: true = the directory on the device; false = planned
    // prefix sums (tile_bases, and the segments' first leaves)
    bool use_directory = false;
    // scan offsets: descent tile k's first child offset on each level it
    // spans, tile_bases[tiles[k].base_off + (d - tiles[k].level)] for d = level ..
    // last internal level (the last entry is its first leaf)
    std::vector<uint32_t> tile_bases;
    // Tree-only products, per direction.  Band groups (when windows are
    // planned): a group (first, count = its sub-tiles in band_sub[dir], window
    // fields) descends the dense quadrants of one row / column band into one
    // LDS window, with frontiers of at most band_cap nodes.  The rest: a
    // second depth-first cut with at most rest_cap nodes per level, in
    // rest_cut, taken in output-block order (rest_order[dir]).  After band
    // groups, plus-times products take the tiles rest_take[dir] lists (those
    // the groups do not cover whole, in block order), each skipping the
    // last-internal-level nodes listed for it in skip[dir] (ranges
    // (lo << 32) | hi, sorted); products without groups take rest_order[dir]
    // whole: the whole second cut.
    uint32_t band_cap = 0;
    // rest tiles hold at most rest_cap nodes per level (a wave's frontier)
    uint32_t rest_cap = 0;
    std::vector<Tile> band_groups[2], band_sub[2];
    std::vector<RestTile> rest_cut;
    std::vector<uint32_t> rest_order[2];
    std::vector<RestTake> rest_take[2];
    std::vector<uint64_t> skip[2];
    // Strays (cached level, band_strays): per direction the segments of the
    // nodes outside every band tile's ranges, and the number of bands of
    // 2^window_log2 outputs.  Every band holding strays has one cached tile
    // with code_off = 1 that adds them (the band's owner tile); matrix
    // creation groups the strays by band on the device.
    // code_off bit 0 marks a band's owner tile, bit 1 a band's only tile
    // (it stores its window into y instead of adding it); bands_cover: every
    // band has exactly one tile, so a windowed product writes all of y.
    std::vector<Seg> stray_segs[2];
    uint64_t stray_nodes[2] = {0, 0};
    uint32_t n_bands[2] = {0, 0};
    bool bands_cover[2] = {false, false};
    // Right products combine runs of one output row among neighbouring
    // cells (the leaves show many row pairs and few column pairs).
    bool row_runs = false;
};

k2_status make_plan(const HostTree &t, const k2_plan_opts &o, Plan *out);
int top_level_for(const HostTree &t, uint32_t host_top_max);

// Arena layout of a matrix (byte offsets from the arena base).
struct Layout {
    uint64_t words_off[kMaxLevels] = {};   // level words (levels >= top)
    uint64_t dir_off[kMaxLevels] = {};     // directories (internal levels >= top)
    uint64_t codes_off = 0, tiles_off = 0, cached_off = 0, bases_off = 0;
    uint64_t groups_off[2] = {0, 0}, sub_off[2] = {0, 0}, skip_off[2] = {0, 0};
    uint64_t rest_off = 0, order_off[2] = {0, 0}, take_off[2] = {0, 0};
    uint64_t cached_tiles_off[2] = {0, 0}, cached_segs_off[2] = {0, 0};
    uint64_t stray_segs_off[2] = {0, 0}, stray_off_off[2] = {0, 0}, stray_cur_off[2] = {0, 0};
    uint64_t strays_off[2] = {0, 0};
    // per node of the cached level, its node word: its cells (bits 0-15) and,
    // with packed nodes, its block's row and column inside its Q x Q quadrant
    // (in blocks of 4, bits 16-23 and 24-31)
    uint64_t cells_off = 0;
    uint64_t status_off = 0;               // creation checks (4 bytes)
    uint64_t inmask_off = 0;               // input bit array of exact-semiring cached products
    k2_mem_breakdown mem = {};
};

void layout_for(const HostTree &t, int top_level, const Plan &plan, bool cached, Layout *out);

// ------------------------------------------------------------ device view

// Everything a kernel needs to address the tree, passed by value.
struct DevTree {
    const uint64_t *words[kMaxLevels];   // per level (nullptr above the top)
    const uint32_t *dir[kMaxLevels];     // per internal level
    uint32_t nodes[kMaxLevels];
    // one past the last word index of words[d] that may be read: the level's
    // word count, or the end of the staged range in out-of-core products
    uint32_t words_end[kMaxLevels];
    int levels;
    int top_level;
};

struct Matrix {
    DevTree dev;
    HostTree const *host_shape = nullptr;  // not kept; shape copied below
    uint32_t n_rows = 0, n_cols = 0;
    int levels = 0;
    std::vector<uint64_t> nodes;
    Plan plan;
    Layout layout;
    char *arena = nullptr;
    const uint64_t *d_codes = nullptr;   // tile start codes
    const Tile *d_tiles = nullptr;
    const uint32_t *d_bases = nullptr;   // scan offsets of the descent tiles, or null
    const Tile *d_band_groups[2] = {nullptr, nullptr}, *d_band_sub[2] = {nullptr, nullptr};
    const RestTile *d_rest = nullptr;
    const uint32_t *d_rest_order[2] = {nullptr, nullptr};
    const uint64_t *d_skip[2] = {nullptr, nullptr};
    const RestTake *d_rest_take[2] = {nullptr, nullptr};
    const Tile *d_cached_tiles[2] = {nullptr, nullptr};
    const Seg *d_cached_segs[2] = {nullptr, nullptr};
    const StrayRec *d_strays[2] = {nullptr, nullptr};   // grouped by band
    const uint32_t *d_stray_off[2] = {nullptr, nullptr}; // band b: d_strays[off[b] .. off[b + 1])
    uint64_t *d_cached = nullptr;        // last internal level codes or null
    uint32_t *d_nodew = nullptr;         // their node words (cells: bit 4 b + q, cell q of the leaf for child b)
    // Cached products of the max / or / min semirings first mark the input
    // rows with a contributing vector here (a bit each), so that the
    // listing drops the cells of the others before any x gather.
    uint32_t *d_inmask = nullptr;
    // Packed nodes: every cached segment lies in one Q x Q quadrant (Q = 2^
    // plan.window_log2 <= 1024), whose origin its Seg holds in (leaf, pad);
    // a product then reads 4 bytes per node (the node word) instead of 10.
    bool packed = false;
    uint32_t window_elems = 0, window_batch = 0;
    size_t lds_per_block = 0;    // LDS bytes of one workgroup (windows and the kernels' own)
    bool cached = false;
    // kernel timing (events created on first enable)
    void *ev[3] = {nullptr, nullptr, nullptr};
    bool timing = false, timed_once = false, last_accumulate = false;
};

// Kernel launchers (k2_device.hip).  Return hipError_t as int.
int launch_fill(void *y, uint64_t n_words32, uint32_t value, void *stream);
// Multi-source search: a level below 2^kBfsPlanes is recorded as bit planes
// of the packed words (plane p holds bit p of each entry's level); the
// distance table is written from them once.
constexpr uint32_t kBfsPlanes = 6;
int launch_bfs_init(uint32_t *words, uint64_t n_words, void *stream);
int launch_bfs_seed(const uint32_t *src, uint32_t S, uint32_t W, uint32_t *F, uint32_t *V, void *stream);
int launch_bfs_mark(uint32_t *y, uint32_t *V, uint32_t *F, uint32_t *planes, int32_t *dist, uint64_t n_words,
                    uint32_t W, uint32_t S, int32_t level, unsigned long long *count, void *stream);
int launch_bfs_dist(int32_t *dist, const uint32_t *V, const uint32_t *planes, uint64_t n_words, uint32_t W,
                    uint32_t S, void *stream);
// Descent tiles over a tree given by 't' alone (a streamed chunk: its level
// words staged on the device), with scan offsets 'bases'.
int launch_descent_tiles(const DevTree &t, const Tile *tiles, size_t n_tiles, const uint64_t *codes,
                         const uint32_t *bases, uint32_t cap, uint32_t n_rows, uint32_t n_cols, bool row_runs,
                         int dir, int semiring, uint32_t batch, const void *x, void *y, void *stream);
int launch_descent(const Matrix &m, int dir, int semiring, uint32_t batch, const void *x, void *y,
                   uint64_t *emit_codes, void *stream, bool filter = true);
// filter (max / or / min semirings): list only the cells whose input row
// has a contributing vector (worth it unless most rows have one)
int launch_cached(const Matrix &m, int dir, int semiring, uint32_t batch, const void *x, void *y,
                  int accumulate, void *stream, bool filter = true);
// Whether a cached product of this batch writes every element of y itself
// (windows in use and every band its own tile's), so y needs no fill.
bool cached_writes_all(const Matrix &m, int dir, uint32_t batch);
// Strays of direction dir (Plan::stray_segs): count per band into counts
// (n_bands entries, zeroed by the caller), or with 'cursor' (each band's
// first slot, advanced) write each stray's record to 'out'.
int launch_stray_count(const Matrix &m, int dir, const Seg *segs, uint32_t n_segs, uint32_t *counts,
                       void *stream);
int launch_stray_scatter(const Matrix &m, int dir, const Seg *segs, uint32_t n_segs, uint32_t *cursor,
                         StrayRec *out, void *stream);
// The node words of the nodes of the cached level that the segments cover,
// their cells read from their leaves, into m.d_nodew.  With qlog (> 0) the
// words also hold each block's place in its 2^qlog-sided quadrant, each
// segment's (leaf, pad) are overwritten with its quadrant's first row and
// column, and *status gets bit 0 set if a segment's nodes span quadrants.
int launch_node_cells(const Matrix &m, Seg *segs, uint32_t n_segs, int qlog, uint32_t *status, void *stream);
const char *hip_error_text(int err);
// The device address of the library's fixed scratch array on the current
// device (k2_bfs_noalloc's workspace, K2_NOALLOC_SCRATCH_BYTES bytes),
// looked up once per device.
constexpr uint64_t kNoAllocScratchBytes = K2_NOALLOC_SCRATCH_BYTES;
int noalloc_scratch(void **ptr);

void set_hip_error(int err, const char *where);

}  // namespace k2
