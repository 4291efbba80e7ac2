// k2_plan.cpp -- host top, tile plans and device-memory layout.
//
// Tosoni & Mencagli, Sec. 3.4: kernel launches cost more than the first tiny
// levels, so the host expands the top of the tree and the device starts from
// the deepest level with at most 2^16 nodes; in level order the children of a
// contiguous node range form a contiguous range, so each level can be cut
// into tiles descended depth first, which bounds the scratch; the tile
// sequence depends only on the tree, so the host plans it before any product.
//
// Descent tiles.  A tile is one workgroup's job: a range of consecutive nodes
// of some level whose descendants on every level down to the last internal
// one number at most tile_nodes (levels never shrink with depth, so bounding
// the last internal level bounds them all).  The workgroup holds the tile's
// frontier in LDS, so a product needs no frontier memory in HBM.  Tiles are
// cut greedily; a node whose subtree is too large is replaced by its children
// (at most four), recursively, which keeps the tiles in depth-first (Z) order.
// The tile start codes are the Morton codes of the first nodes, taken from the
// host-top expansion or from a split parent.
//
// Cached tiles (for the kernel that reads the cached codes of the last
// internal level, Sec. 3.5) are lists of node ranges of that level, one list
// per product direction, cut into segments of at most 64 nodes (a wave's
// job) that carry their first leaf's index, which the planner finds with the
// same directory query the descent uses.
//
// Windows.  Every node of a Q x Q quadrant (a node of level h = l - log2 Q)
// has its rows and its columns inside the quadrant's Q.  A quadrant holding
// many nodes is dense.  For the cached level the dense quadrants of one row
// band (right product) or one column band (left product) are gathered into
// one tile whose window is that band: the workgroup accumulates the band's
// outputs in LDS (Q outputs x B vectors) and adds them to y once at the end,
// so each band's part of y costs one coalesced pass instead of one atomic
// per cell.  With band_strays the nodes outside the dense quadrants (strays)
// join their band's window too: every band holding some gets a tile, and the
// device groups the strays by band when the matrix is created (their bands
// come from the block origins it computes).  Otherwise the sparse rest keeps
// one y atomic per cell, in separate tiles.  (The kernels also
// accept windows on descent tiles; planning one per dense quadrant made many
// small tiles and measured slower, so descent tiles carry none.)
#include <algorithm>
#include <atomic>
#include <thread>

#include "k2_internal.h"

namespace k2 {

int top_level_for(const HostTree &t, uint32_t host_top_max) {
    int d0 = 0;
    for (int d = 0; d <= t.levels - 2; ++d)
        if (t.nodes[d] <= host_top_max) d0 = d;
    return d0;
}

namespace {

inline uint32_t even_bits(uint64_t x) {
    x &= 0x5555555555555555ull;
    x = (x | (x >> 1)) & 0x3333333333333333ull;
    x = (x | (x >> 2)) & 0x0F0F0F0F0F0F0F0Full;
    x = (x | (x >> 4)) & 0x00FF00FF00FF00FFull;
    x = (x | (x >> 8)) & 0x0000FFFF0000FFFFull;
    x = (x | (x >> 16)) & 0x00000000FFFFFFFFull;
    return uint32_t(x);
}

struct Planner {
    const HostTree &t;
    uint64_t C;
    Plan &p;
    int last;           // last internal level
    uint64_t cached_C;  // nodes per cached tile without a window
    uint64_t band_cap = 65536;                    // nodes per windowed cached tile
    static constexpr uint64_t kSparseTile = 8192; // nodes per sparse cached tile beside bands
    std::vector<Tile> *sink = nullptr;            // where range() puts tiles (p.tiles if null)
    std::vector<uint64_t> sink_weight;            // last-internal-level nodes of the sink's tiles
    std::vector<uint64_t> sink_lo2;               // first last-internal-level node of the sink's tiles
    static constexpr uint64_t kGroupCap = 8192;   // last-internal-level nodes per band group

    // Descendant index on level 'to' of boundary 'i' of level d.
    uint64_t down(int d, uint64_t i, int to) const {
        for (int e = d; e < to; ++e) i = child_offset(t, e, i);
        return i;
    }

    void split(int d, uint64_t node, uint64_t code, const Tile &win) {
        uint64_t c0 = child_offset(t, d, node), c1 = child_offset(t, d, node + 1);
        unsigned s = nibble(t.words[d], node);
        uint64_t code_base = p.codes.size();
        for (unsigned b = 0; b < 4; ++b)
            if (s & (1u << b)) p.codes.push_back((code << 2) | b);
        range(d + 1, c0, c1, code_base, win);
    }

    // Descent tiles over nodes [a, b) of level d (codes at
    // p.codes[code_base + i - a]), all with the window fields of 'win'.
    // bound[k] (optional) is node a + k's first descendant on the last
    // internal level, for k = 0..b-a.
    void range(int d, uint64_t a, uint64_t b, uint64_t code_base, const Tile &win,
               const std::vector<uint64_t> *known = nullptr) {
        std::vector<uint64_t> bound;
        if (known) {
            bound = *known;
        } else {
            bound.resize(b - a + 1);
            for (uint64_t i = a; i <= b; ++i) bound[i - a] = down(d, i, last);
        }
        uint64_t i = a;
        while (i < b) {
            if (bound[i + 1 - a] - bound[i - a] > C) {
                split(d, i, p.codes[code_base + (i - a)], win);
                ++i;
                continue;
            }
            uint64_t j = i + 1;
            while (j < b && bound[j + 1 - a] - bound[i - a] <= C) ++j;
            Tile tl = win;
            tl.first = uint32_t(i);
            tl.count = uint32_t(j - i);
            tl.level = uint32_t(d);
            tl.code_off = uint32_t(code_base + (i - a));
            if (sink) {
                sink->push_back(tl);
                sink_weight.push_back(bound[j - a] - bound[i - a]);
                sink_lo2.push_back(bound[i - a]);
            } else {
                p.tiles.push_back(tl);
            }
            i = j;
        }
    }

    // Appends the segments of nodes [lo, lo + count) of the last internal level.
    static void push_segs(std::vector<Seg> &to, uint64_t lo, uint64_t count) {
        for (uint64_t i = 0; i < count; i += kSegNodes)
            to.push_back({uint32_t(lo + i), uint32_t(std::min<uint64_t>(kSegNodes, count - i)), 0u, 0u});
    }
    void push_segs(int dir, uint64_t lo, uint64_t count) { push_segs(p.cached_segs[dir], lo, count); }

    // Cached tiles of direction dir over nodes [lo, hi) of the last internal
    // level, no window: 'per' nodes per tile (cached_C if 0).
    void cached_run(int dir, uint64_t lo, uint64_t hi, uint64_t per = 0) {
        if (!per) per = cached_C;
        for (uint64_t i = lo; i < hi; i += per) {
            Tile tl{};
            tl.first = uint32_t(p.cached_segs[dir].size());
            tl.level = uint32_t(last);
            tl.win_log2 = kNoWindow;
            push_segs(dir, i, std::min(per, hi - i));
            tl.count = uint32_t(p.cached_segs[dir].size() - tl.first);
            p.cached_tiles[dir].push_back(tl);
        }
    }

    // Cached tiles of direction dir over the node ranges 'ranges' of one
    // band, all with the band's window; at most band_cap nodes per tile.
    void cached_band(int dir, const std::vector<Seg> &ranges, const Tile &win) {
        Tile tl = win;
        tl.first = uint32_t(p.cached_segs[dir].size());
        tl.level = uint32_t(last);
        uint64_t nodes = 0;
        auto close = [&]() {
            tl.count = uint32_t(p.cached_segs[dir].size() - tl.first);
            if (tl.count) p.cached_tiles[dir].push_back(tl);
            tl.first = uint32_t(p.cached_segs[dir].size());
            nodes = 0;
        };
        for (Seg sg : ranges) {
            while (sg.count > 0) {
                uint64_t take = std::min<uint64_t>(sg.count, band_cap - nodes);
                push_segs(dir, sg.lo, take);
                nodes += take;
                sg.lo += uint32_t(take);
                sg.count -= uint32_t(take);
                if (nodes == band_cap) close();
            }
        }
        close();
    }

    // First leaf of every segment's first node, in parallel.
    void set_leaves(std::vector<Seg> &sg) {
        const size_t n = sg.size();
        const unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
        std::vector<std::thread> pool;
        for (unsigned k = 0; k < nt; ++k)
            pool.emplace_back([&, k]() {
                for (size_t i = n * k / nt; i < n * (k + 1) / nt; ++i)
                    sg[i].leaf = uint32_t(child_offset(t, last, sg[i].lo));
            });
        for (auto &th : pool) th.join();
    }
};

Tile no_window() {
    Tile w{};
    w.win_log2 = kNoWindow;
    return w;
}

// log2 of the rows (right products) or columns (left) of an output block:
// about 16 MB of y at window_batch vectors, at least 2^min_log2.
int block_log2(const k2_plan_opts &o, int min_log2) {
    int kb = min_log2;
    const uint64_t wb = o.window_batch ? o.window_batch : 1;
    while (kb < 30 && (2ull << kb) * wb * 4 <= (16ull << 20)) ++kb;
    return kb;
}

Tile window_of(uint64_t code, int h, int L) {
    Tile w{};
    const int sh = L - h;                       // log2 of the quadrant side
    w.win_row = uint32_t(uint64_t(even_bits(code >> 1)) << sh);
    w.win_col = uint32_t(uint64_t(even_bits(code)) << sh);
    w.win_log2 = uint32_t(sh);
    return w;
}

}  // namespace

namespace {

// A piece of the last internal level in depth-first order: the subtree(s) of
// nodes [a, b) of level 'level' (codes in Units::codes from 'code_idx'),
// covering nodes [lo2, hi2) of the last internal level; dense units are
// single quadrants of the window level.
struct Unit {
    int level;
    uint64_t a, b, code_idx, lo2, hi2;
    bool dense;
    uint64_t qcode;   // Morton code of the quadrant (dense units)
};

// Workgroup b of a launch runs on XCD b % 8, and each of the 8 XCDs has its
// own L2.  Neighbouring tiles in Z order share rows and columns (a row band's
// tiles gather x from overlapping column windows), so they should run on one
// XCD.  The tiles of each group [group[g], group[g+1]) are cut into 8 runs of
// about equal weight; XCD k's list is its run of every group in turn, and
// list k's j-th tile goes to position 8 j + k.  Shorter lists are padded with
// empty tiles (count 0), so the length is a multiple of 8.
void xcd_order(std::vector<Tile> &tiles, const std::vector<uint64_t> &weight,
               const std::vector<size_t> &group, uint32_t pad_level) {
    constexpr int kXcds = 8;
    std::vector<Tile> list[kXcds];
    for (size_t g = 0; g + 1 < group.size(); ++g) {
        const size_t a = group[g], b = group[g + 1];
        uint64_t total = 0;
        for (size_t i = a; i < b; ++i) total += weight[i];
        uint64_t acc = 0;
        for (size_t i = a; i < b; ++i) {
            // the run whose share of the group's weight holds this tile's middle
            const uint64_t mid = acc + weight[i] / 2;
            const int k = total ? int(std::min<uint64_t>(kXcds - 1, mid * kXcds / total)) : 0;
            list[k].push_back(tiles[i]);
            acc += weight[i];
        }
    }
    size_t len = 0;
    for (auto &l : list) len = std::max(len, l.size());
    Tile pad{};
    pad.level = pad_level;
    pad.win_log2 = kNoWindow;
    std::vector<Tile> out(len * kXcds, pad);
    for (int k = 0; k < kXcds; ++k)
        for (size_t j = 0; j < list[k].size(); ++j) out[j * kXcds + size_t(k)] = list[k][j];
    tiles.swap(out);
}

}  // namespace

k2_status make_plan(const HostTree &t, const k2_plan_opts &o, Plan *out) {
    Plan &p = *out;
    p = Plan();
    p.top_level = top_level_for(t, o.host_top_max);
    p.tile_nodes = o.tile_nodes;
    const int L = t.levels, last = L - 2, d0 = p.top_level;
    if (L < 2 || t.nodes[last] == 0) return K2_OK;   // empty matrix: no tiles

    // host-top expansion: Morton codes of levels 0..d0, parent code then b1b0
    std::vector<std::vector<uint64_t>> codes(size_t(d0) + 1);
    codes[0].assign(1, 0);
    for (int d = 0; d < d0; ++d) {
        codes[d + 1].reserve(t.nodes[d + 1]);
        for (uint64_t i = 0; i < t.nodes[d]; ++i) {
            unsigned s = nibble(t.words[d], i);
            for (unsigned b = 0; b < 4; ++b)
                if (s & (1u << b)) codes[d + 1].push_back((codes[d][i] << 2) | b);
        }
    }
    p.codes = codes[d0];

    const uint64_t n2 = t.nodes[last];
    {   // row pairs and column pairs of cells inside the leaves (2 x 2
        // blocks): a matrix whose rows hold runs of neighbouring non-zeros
        // (many row pairs, few column pairs) gains from combining runs of
        // one row in right products; one whose pairs are balanced loses the
        // x locality the interleaved order gives (measured: web-like 2^27,
        // 10% of cells in row pairs, 0.4% in column pairs: 8.5 against 19.6
        // ms at B = 1 with runs; R-MAT 2^22, 2.3% each: 1.08 against 0.97)
        const std::vector<uint64_t> &lw = t.words[L - 1];
        const unsigned nth = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
        std::vector<uint64_t> cnt(3 * size_t(nth), 0);
        std::vector<std::thread> pool;
        for (unsigned k = 0; k < nth; ++k)
            pool.emplace_back([&, k]() {
                uint64_t cells = 0, rows = 0, cols = 0;
                for (size_t i = lw.size() * k / nth; i < lw.size() * (k + 1) / nth; ++i) {
                    const uint64_t w = lw[i];
                    cells += uint64_t(__builtin_popcountll(w));
                    rows += uint64_t(__builtin_popcountll(w & (w >> 1) & 0x5555555555555555ull));
                    cols += uint64_t(__builtin_popcountll(w & (w >> 2) & 0x3333333333333333ull));
                }
                cnt[3 * k] = cells;
                cnt[3 * k + 1] = rows;
                cnt[3 * k + 2] = cols;
            });
        for (auto &th : pool) th.join();
        uint64_t cells = 0, rows = 0, cols = 0;
        for (unsigned k = 0; k < nth; ++k) {
            cells += cnt[3 * k];
            rows += cnt[3 * k + 1];
            cols += cnt[3 * k + 2];
        }
        p.row_runs = 2 * rows * 50 >= cells && rows >= 4 * cols && rows > 0;
    }
    uint64_t cc = n2 / 2048;                      // enough tiles to fill the GPU
    cc = std::max<uint64_t>(256, std::min<uint64_t>(16384, cc));
    cc = (cc + 255) & ~uint64_t(255);
    Planner pl{t, o.tile_nodes, p, last, cc};
    pl.band_cap = o.band_tile_nodes;

    // window quadrants: side Q with Q * window_batch <= window_elems
    int qlog = -1;
    if (o.window_elems > 0 && o.window_batch > 0) {
        uint64_t q = uint64_t(o.window_elems) / o.window_batch;
        while (q > 1 && (q & (q - 1))) q &= q - 1;
        if (q >= 4) qlog = 0;
        while (qlog >= 0 && (2ull << qlog) <= q) ++qlog;
    }
    p.window_log2 = -1;
    // descent tiles: the plain depth-first cut (windowed descent tiles, one
    // per dense quadrant, measured slower: many small tiles)
    pl.range(d0, 0, t.nodes[d0], 0, no_window());
    // order of a tile list per direction: by output block of the tile's first
    // node, then depth first, so the tiles in flight update one slice of y
    // (its lines stay in the last-level cache while the atomics land)
    auto block_order = [&](const std::vector<Tile> &tiles, int dir, std::vector<uint32_t> &order) {
        const int kb = block_log2(o, 0);
        std::vector<std::pair<uint64_t, uint32_t>> key(tiles.size());
        for (size_t i = 0; i < tiles.size(); ++i) {
            const Tile &tl = tiles[i];
            const uint64_t code = p.codes[tl.code_off];
            const uint64_t c = dir == K2_RIGHT ? even_bits(code >> 1) : even_bits(code);
            key[i] = {(c << (L - int(tl.level))) >> kb, uint32_t(i)};
        }
        std::stable_sort(key.begin(), key.end(), [](const auto &x, const auto &y) { return x.first < y.first; });
        order.resize(key.size());
        for (size_t i = 0; i < key.size(); ++i) order[i] = key[i].second;
    };
    p.use_directory = o.offsets == K2_OFFSETS_DIRECTORY;
    // scan offsets of a tile list: each tile's first child on every level it
    // spans, by following its first node down (the host's rank query),
    // appended to tile_bases
    auto plan_bases = [&](std::vector<Tile> &tiles) -> k2_status {
        if (p.use_directory) return K2_OK;
        uint64_t total = p.tile_bases.size();
        for (Tile &tl : tiles) {
            tl.base_off = uint32_t(total);
            total += uint64_t(last - int(tl.level) + 1);
        }
        if (total >= (1ull << 32)) return K2_E_UNSUPPORTED;
        p.tile_bases.resize(total);
        const size_t nt = tiles.size();
        const unsigned nth = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
        std::vector<std::thread> pool;
        for (unsigned k = 0; k < nth; ++k)
            pool.emplace_back([&, k]() {
                for (size_t i = nt * k / nth; i < nt * (k + 1) / nth; ++i) {
                    const Tile &tl = tiles[i];
                    uint64_t node = tl.first;
                    for (int d = int(tl.level); d <= last; ++d) {
                        node = child_offset(t, d, node);
                        p.tile_bases[tl.base_off + uint32_t(d - int(tl.level))] = uint32_t(node);
                    }
                }
            });
        for (auto &th : pool) th.join();
        return K2_OK;
    };
    if (plan_bases(p.tiles) != K2_OK) return K2_E_UNSUPPORTED;
    // rest tiles of tree-only plus-times products (a wave's job): the same
    // depth-first cut with at most rest_cap nodes per level, in block order.
    // Threads cut chunks of the top level (a tile never spans two chunks);
    // the chunks' split codes are appended to the plan's codes in order.
    p.rest_cap = std::min<uint32_t>(o.tile_nodes, 256);
    std::vector<Tile> rest_cut;
    std::vector<uint64_t> rest_w, rest_lo2;
    std::vector<uint32_t> rest_order[2];
    {
        struct Part {
            Plan plan;   // only its codes: the chunk's top codes, then its splits
            std::vector<Tile> tiles;
            std::vector<uint64_t> w, lo2;
        };
        const uint64_t ntop = t.nodes[d0];
        const unsigned nth = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
        const uint64_t nparts = std::min<uint64_t>(ntop, uint64_t(nth) * 16);
        std::vector<Part> parts(nparts);
        std::atomic<uint64_t> next{0};
        auto worker = [&]() {
            for (;;) {
                const uint64_t c = next.fetch_add(1);
                if (c >= nparts) return;
                const uint64_t a = ntop * c / nparts, b = ntop * (c + 1) / nparts;
                Part &pt = parts[c];
                pt.plan.codes.assign(codes[d0].begin() + int64_t(a), codes[d0].begin() + int64_t(b));
                Planner q{t, p.rest_cap, pt.plan, last, cc};
                q.sink = &pt.tiles;
                q.range(d0, a, b, 0, no_window());
                pt.w.swap(q.sink_weight);
                pt.lo2.swap(q.sink_lo2);
            }
        };
        std::vector<std::thread> pool;
        for (unsigned k = 0; k < nth; ++k) pool.emplace_back(worker);
        for (auto &th : pool) th.join();
        for (Part &pt : parts) {
            const uint64_t off = p.codes.size();
            if (off + pt.plan.codes.size() >= (1ull << 32)) return K2_E_UNSUPPORTED;
            p.codes.insert(p.codes.end(), pt.plan.codes.begin(), pt.plan.codes.end());
            for (Tile tl : pt.tiles) {
                tl.code_off = uint32_t(tl.code_off + off);
                rest_cut.push_back(tl);
            }
            rest_w.insert(rest_w.end(), pt.w.begin(), pt.w.end());
            rest_lo2.insert(rest_lo2.end(), pt.lo2.begin(), pt.lo2.end());
        }
        for (int dir = 0; dir < 2; ++dir) block_order(rest_cut, dir, rest_order[dir]);
        if (plan_bases(rest_cut) != K2_OK) return K2_E_UNSUPPORTED;
        p.rest_cut.reserve(rest_cut.size());
        for (const Tile &tl : rest_cut) p.rest_cut.push_back({tl.first, tl.code_off, tl.base_off, tl.count | (tl.level << 16)});
        for (int dir = 0; dir < 2; ++dir) p.rest_order[dir] = rest_order[dir];
    }
    // group boundaries: tile indexes where a new group starts (and the end)
    auto order_cached = [&](int dir, std::vector<size_t> groups) {
        pl.set_leaves(p.cached_segs[dir]);
        pl.set_leaves(p.stray_segs[dir]);
        if (!o.xcd_remap) return;
        std::vector<uint64_t> w;
        for (const Tile &tl : p.cached_tiles[dir]) {
            uint64_t nodes = 64;   // a tile's fixed cost, in nodes
            for (uint32_t r = 0; r < tl.count; ++r) nodes += p.cached_segs[dir][tl.first + r].count;
            nodes += 8 * tl.count;   // a segment's fixed cost
            w.push_back(nodes);
        }
        xcd_order(p.cached_tiles[dir], w, groups, uint32_t(last));
    };
    const bool cache = o.cache_last_level != 0;
    p.band_cap = std::min<uint32_t>(o.tile_nodes, 256);   // per-wave frontiers (band kernel)
    // Tree-only plus-times products after band groups: the rest tiles in
    // block order that the last-internal-level ranges 'wr' (sorted, those
    // the groups cover) do not cover whole, each with its ranges to skip.
    auto rest_plain = [&](int dir, const std::vector<std::pair<uint64_t, uint64_t>> &wr) {
        if (wr.empty()) return;
        for (uint32_t idx : rest_order[dir]) {
            const uint64_t a = rest_lo2[idx], b = a + rest_w[idx];
            auto it = std::lower_bound(wr.begin(), wr.end(), a,
                                       [](const std::pair<uint64_t, uint64_t> &r, uint64_t v) { return r.second <= v; });
            RestTake tk{idx, uint32_t(p.skip[dir].size()), 0, 0};
            uint64_t covered = 0;
            for (; it != wr.end() && it->first < b; ++it) {
                const uint64_t lo = std::max(a, it->first), hi = std::min(b, it->second);
                p.skip[dir].push_back((lo << 32) | hi);
                covered += hi - lo;
                ++tk.skip_count;
            }
            if (covered == b - a && b > a) p.skip[dir].resize(tk.skip_row);   // wholly inside band groups
            else p.rest_take[dir].push_back(tk);
        }
    };
    // Scan offsets of the band groups' sub-tiles (the rest tiles are copies of
    // the rest cut and share its offsets).
    auto finish = [&]() -> k2_status {
        for (int dir = 0; dir < 2; ++dir)
            if (plan_bases(p.band_sub[dir]) != K2_OK) return K2_E_UNSUPPORTED;
        if (p.codes.size() >= (1ull << 32)) return K2_E_UNSUPPORTED;
        return K2_OK;
    };
    if (qlog < 0) {
        if (cache)
            for (int dir = 0; dir < 2; ++dir) {
                pl.cached_run(dir, 0, n2);
                order_cached(dir, {0, p.cached_tiles[dir].size()});
            }
        return finish();
    }
    const int h = std::max(0, L - qlog);            // quadrant level
    p.window_log2 = L - h;
    const uint64_t side = 1ull << (L - h);
    const uint64_t dense = std::max<uint64_t>(16, side / 16);   // nodes of level l-2

    // ---- units, in depth-first order
    std::vector<Unit> units;
    std::vector<uint64_t> ucodes;
    if (h <= d0) {
        // quadrants at or above the host top: each is a contiguous range of top nodes
        for (uint64_t q = 0; q < t.nodes[h]; ++q) {
            uint64_t a0 = pl.down(h, q, d0), b0 = pl.down(h, q + 1, d0);
            Unit u{d0, a0, b0, ucodes.size(), pl.down(d0, a0, last), pl.down(d0, b0, last), false,
                   codes[h][q]};
            u.dense = u.hi2 - u.lo2 >= dense;
            ucodes.insert(ucodes.end(), codes[d0].begin() + int64_t(a0), codes[d0].begin() + int64_t(b0));
            units.push_back(u);
        }
    } else {
        // Walk down from the host top.  A subtree with fewer than 'dense' nodes
        // on the last internal level holds no dense quadrant and stays whole;
        // larger ones are split down to level h.  The top nodes are walked in
        // parallel, in chunks whose units are concatenated in order.
        struct Item {
            int d;
            uint64_t node, code, lo2, hi2;
        };
        const uint64_t ntop = t.nodes[d0];
        const int nt = int(std::min<uint64_t>(uint64_t(std::max(1u, std::thread::hardware_concurrency())),
                                              std::min<uint64_t>(64, ntop)));
        std::atomic<uint64_t> next_chunk{0};
        const uint64_t chunk = std::max<uint64_t>(1, ntop / (uint64_t(nt) * 16));
        std::vector<std::vector<Unit>> chunk_units((ntop + chunk - 1) / chunk);
        std::vector<std::vector<uint64_t>> chunk_codes(chunk_units.size());
        auto worker = [&]() {
            std::vector<Item> stack;
            for (;;) {
                const uint64_t c = next_chunk.fetch_add(1);
                if (c >= chunk_units.size()) return;
                std::vector<Unit> &us = chunk_units[c];
                std::vector<uint64_t> &cs = chunk_codes[c];
                const uint64_t i0 = c * chunk, i1 = std::min(ntop, i0 + chunk);
                for (uint64_t i = i1; i-- > i0;)
                    stack.push_back({d0, i, codes[d0][i], pl.down(d0, i, last), pl.down(d0, i + 1, last)});
                while (!stack.empty()) {
                    Item it = stack.back();
                    stack.pop_back();
                    const uint64_t desc = it.hi2 - it.lo2;
                    if (it.d == h || desc < dense) {
                        us.push_back({it.d, it.node, it.node + 1, cs.size(), it.lo2, it.hi2,
                                      it.d == h && desc >= dense, it.code});
                        cs.push_back(it.code);
                        continue;
                    }
                    const uint64_t c0 = child_offset(t, it.d, it.node);
                    const unsigned sg = nibble(t.words[it.d], it.node);
                    Item ch[4];
                    int nc = 0;
                    for (unsigned b = 0; b < 4; ++b)
                        if (sg & (1u << b)) {
                            ch[nc].d = it.d + 1;
                            ch[nc].node = c0 + uint64_t(nc);
                            ch[nc].code = (it.code << 2) | b;
                            ++nc;
                        }
                    // first and last boundaries are the parent's
                    ch[0].lo2 = it.lo2;
                    for (int k = 1; k < nc; ++k) ch[k].lo2 = ch[k - 1].hi2 = pl.down(it.d + 1, ch[k].node, last);
                    ch[nc - 1].hi2 = it.hi2;
                    for (int k = nc - 1; k >= 0; --k) stack.push_back(ch[k]);
                }
            }
        };
        std::vector<std::thread> pool;
        for (int k = 0; k < nt; ++k) pool.emplace_back(worker);
        for (auto &th : pool) th.join();
        for (size_t c = 0; c < chunk_units.size(); ++c) {
            const uint64_t base = ucodes.size();
            for (Unit u : chunk_units[c]) {
                u.code_idx += base;
                units.push_back(u);
            }
            ucodes.insert(ucodes.end(), chunk_codes[c].begin(), chunk_codes[c].end());
        }
    }

    // ---- cached tiles, per direction: windowed bands and the sparse rest,
    // merged in order of output blocks of 2^kb rows (right products) or
    // columns (left), about 16 MB of y each at window_batch vectors.  The
    // tiles in flight then update one narrow slice of y, whose lines the
    // chip's last-level cache can hold while their atomics arrive.
    const uint64_t band_min = std::max<uint64_t>(64, side * o.window_batch / 32);
    const int kb = block_log2(o, L - h);
    const bool strays = cache && o.band_strays != 0;
    for (int dir = 0; dir < 2; ++dir) {
        const uint64_t n_out = dir == K2_RIGHT ? t.n_rows : t.n_cols;
        const uint64_t n_bands = (n_out + side - 1) >> (L - h);
        if (strays && n_bands >= (1ull << 32)) return K2_E_UNSUPPORTED;
        std::vector<char> has_tile(strays ? n_bands : 0, 0);
        // output coordinate of a quadrant's first cell
        auto out_of = [&](uint64_t code, int level) -> uint64_t {
            const uint64_t c = dir == K2_RIGHT ? even_bits(code >> 1) : even_bits(code);
            return c << (L - level);
        };
        // band of each dense unit: its row band (right) or column band (left)
        std::vector<std::pair<uint64_t, uint32_t>> dense_units;   // (band, unit index)
        for (size_t i = 0; i < units.size(); ++i)
            if (units[i].dense) {
                uint64_t code = units[i].qcode;
                uint64_t band = dir == K2_RIGHT ? even_bits(code >> 1) : even_bits(code);
                dense_units.push_back({band, uint32_t(i)});
            }
        std::stable_sort(dense_units.begin(), dense_units.end(),
                         [](const auto &x, const auto &y) { return x.first < y.first; });
        std::vector<char> windowed(units.size(), 0);
        std::vector<std::pair<uint64_t, Tile>> keyed;    // (output block, cached tile)
        std::vector<std::pair<uint64_t, Tile>> dkeyed;   // (output block, band group)
        for (size_t i = 0; i < dense_units.size();) {
            size_t j = i;
            uint64_t total = 0;
            while (j < dense_units.size() && dense_units[j].first == dense_units[i].first) {
                const Unit &u = units[dense_units[j].second];
                total += u.hi2 - u.lo2;
                ++j;
            }
            if (total >= band_min) {
                std::vector<Seg> ranges;
                for (size_t k = i; k < j; ++k) {
                    const Unit &u = units[dense_units[k].second];
                    windowed[dense_units[k].second] = 1;
                    ranges.push_back({uint32_t(u.lo2), uint32_t(u.hi2 - u.lo2), 0u, 0u});
                }
                Tile w = window_of(units[dense_units[i].second].qcode, h, L);
                const uint64_t key = (dense_units[i].first << (L - h)) >> kb;
                if (cache) {
                    const size_t t0 = p.cached_tiles[dir].size();
                    pl.cached_band(dir, ranges, w);
                    if (strays && p.cached_tiles[dir].size() > t0) {
                        p.cached_tiles[dir][t0].code_off = 1;   // the band's owner tile
                        has_tile[dense_units[i].first] = 1;
                    }
                    for (size_t t = t0; t < p.cached_tiles[dir].size(); ++t) keyed.push_back({key, p.cached_tiles[dir][t]});
                    p.cached_tiles[dir].resize(t0);
                }
                // the band's groups for tree-only products: its quadrants'
                // subtrees cut into sub-tiles of at most band_cap nodes, and
                // those into groups of at most kGroupCap nodes (one window
                // flush each), so dense bands still spread over the GPU
                const size_t s0 = p.band_sub[dir].size();
                const uint64_t C0 = pl.C;
                pl.C = p.band_cap;
                pl.sink = &p.band_sub[dir];
                pl.sink_weight.clear();
                pl.sink_lo2.clear();
                for (size_t k = i; k < j; ++k) {
                    const Unit &u = units[dense_units[k].second];
                    const uint64_t cb = p.codes.size();
                    p.codes.insert(p.codes.end(), ucodes.begin() + int64_t(u.code_idx),
                                   ucodes.begin() + int64_t(u.code_idx + (u.b - u.a)));
                    pl.range(u.level, u.a, u.b, cb, no_window());
                }
                pl.sink = nullptr;
                pl.C = C0;
                Tile g = w;
                g.level = uint32_t(last);
                g.first = uint32_t(s0);
                uint64_t acc = 0;
                for (size_t q = 0; q < pl.sink_weight.size(); ++q) {
                    if (acc > 0 && acc + pl.sink_weight[q] > Planner::kGroupCap) {
                        g.count = uint32_t(s0 + q - g.first);
                        dkeyed.push_back({key, g});
                        g.first = uint32_t(s0 + q);
                        acc = 0;
                    }
                    acc += pl.sink_weight[q];
                }
                g.count = uint32_t(p.band_sub[dir].size() - g.first);
                if (g.count) dkeyed.push_back({key, g});
            }
            i = j;
        }
        // tree-only products: band groups in block order, then the rest.
        // Groups pay for their sequential descents only when the windows
        // cover most of the level (measured: web-like 2^27, 84% covered, 30%
        // faster; R-MAT, mostly sparse, 2-3x slower), so below half the
        // level every tile stays a rest tile.
        std::vector<std::pair<uint64_t, uint64_t>> wr;
        uint64_t in_bands = 0;
        for (size_t i = 0; i < units.size(); ++i)
            if (windowed[i]) {
                wr.push_back({units[i].lo2, units[i].hi2});
                in_bands += units[i].hi2 - units[i].lo2;
            }
        if (2 * in_bands >= n2) {
            std::stable_sort(dkeyed.begin(), dkeyed.end(),
                             [](const auto &x, const auto &y) { return x.first < y.first; });
            for (const auto &kg : dkeyed) p.band_groups[dir].push_back(kg.second);
        } else {
            wr.clear();
            p.band_sub[dir].clear();
        }
        rest_plain(dir, wr);
        if (!cache) continue;
        if (strays) {
            // strays: the runs of level l-2 outside the band tiles, and an
            // owner tile (no segments) for every band they may reach that
            // has none; a unit's nodes lie in its quadrant, whose output
            // range gives the bands
            std::vector<uint32_t> reach(n_bands + 1, 0);   // difference array
            uint64_t run_lo = 0, run_hi = 0;
            bool in_run = false;
            for (size_t i = 0; i < units.size(); ++i) {
                if (windowed[i]) continue;
                const Unit &u = units[i];
                const int lev = h <= d0 ? h : u.level;
                const uint64_t first = out_of(u.qcode, lev), span = 1ull << (L - lev);
                const uint64_t b0 = first >> (L - h);
                const uint64_t b1 = std::min(n_bands, ((first + span - 1) >> (L - h)) + 1);
                if (b0 < b1) {
                    ++reach[b0];
                    --reach[b1];
                }
                if (in_run && u.lo2 == run_hi) {
                    run_hi = u.hi2;
                    continue;
                }
                if (in_run) Planner::push_segs(p.stray_segs[dir], run_lo, run_hi - run_lo);
                in_run = true;
                run_lo = u.lo2;
                run_hi = u.hi2;
            }
            if (in_run) Planner::push_segs(p.stray_segs[dir], run_lo, run_hi - run_lo);
            for (const Seg &sg : p.stray_segs[dir]) p.stray_nodes[dir] += sg.count;
            p.n_bands[dir] = uint32_t(n_bands);
            // up to 2^20 bands every band gets a tile, so the bands cover y
            const bool all_bands = n_bands <= (1u << 20);
            uint32_t live = 0;
            for (uint64_t b = 0; b < n_bands; ++b) {
                live += reach[b];
                if ((!live && !all_bands) || has_tile[b]) continue;
                Tile w{};
                (dir == K2_RIGHT ? w.win_row : w.win_col) = uint32_t(b << (L - h));
                w.win_log2 = uint32_t(L - h);
                w.level = uint32_t(last);
                w.first = uint32_t(p.cached_segs[dir].size());
                w.count = 0;
                w.code_off = 1;
                keyed.push_back({(b << (L - h)) >> kb, w});
            }
            // a band with one tile: that tile alone writes the band's part of
            // y (code_off bit 1), so it may store its window instead of
            // adding it atomically; when every band is such, the cached
            // product writes all of y and needs no fill
            std::vector<uint32_t> per_band(n_bands, 0);
            auto band_of = [&](const Tile &tl) {
                return uint64_t(dir == K2_RIGHT ? tl.win_row : tl.win_col) >> tl.win_log2;
            };
            for (const auto &kt : keyed) ++per_band[band_of(kt.second)];
            bool every = all_bands;
            for (uint64_t b = 0; b < n_bands; ++b) every = every && per_band[b] == 1;
            for (auto &kt : keyed)
                if (per_band[band_of(kt.second)] == 1) kt.second.code_off |= 2u;
            p.bands_cover[dir] = every;
        }
        // the sparse rest in depth-first order: contiguous runs of level l-2
        // within one output block
        uint64_t run_lo = 0, run_hi = 0, run_key = 0;
        bool in_run = false;
        auto flush = [&]() {
            const size_t t0 = p.cached_tiles[dir].size();
            pl.cached_run(dir, run_lo, run_hi, Planner::kSparseTile);
            for (size_t t = t0; t < p.cached_tiles[dir].size(); ++t) keyed.push_back({run_key, p.cached_tiles[dir][t]});
            p.cached_tiles[dir].resize(t0);
        };
        for (size_t i = 0; i < units.size() && !strays; ++i) {
            if (windowed[i]) continue;
            const Unit &u = units[i];
            const uint64_t key = out_of(ucodes[u.code_idx], u.level) >> kb;
            if (in_run && u.lo2 == run_hi && key == run_key) {
                run_hi = u.hi2;
                continue;
            }
            if (in_run) flush();
            in_run = true;
            run_lo = u.lo2;
            run_hi = u.hi2;
            run_key = key;
        }
        if (in_run) flush();
        std::stable_sort(keyed.begin(), keyed.end(),
                         [](const auto &x, const auto &y) { return x.first < y.first; });
        // with XCD order, the bands of an output block are one group and its
        // sparse tiles another: all XCDs stay in the block (y in the
        // last-level cache) and each takes a run of neighbouring bands (their
        // shared x columns in its own L2) and an eighth of the sparse tiles
        std::vector<size_t> groups{0};
        for (size_t i = 0; i < keyed.size(); ++i) {
            if (i && (keyed[i].first != keyed[i - 1].first ||
                      (keyed[i].second.win_log2 == kNoWindow) != (keyed[i - 1].second.win_log2 == kNoWindow)))
                groups.push_back(i);
            p.cached_tiles[dir].push_back(keyed[i].second);
        }
        groups.push_back(keyed.size());
        order_cached(dir, groups);
    }
    return finish();
}

static uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

void layout_for(const HostTree &t, int top, const Plan &plan, bool cached, Layout *out) {
    Layout &l = *out;
    l = Layout();
    uint64_t off = 0, raw = 0;
    auto take = [&](uint64_t bytes, uint64_t &field_bytes) {
        uint64_t at = off;
        off = align256(off + bytes);
        raw += bytes;
        field_bytes += bytes;
        return at;
    };
    for (int d = top; d < t.levels; ++d)
        l.words_off[d] = take(8 * ((t.nodes[d] + 15) / 16), l.mem.tree);
    for (int d = top; d + 1 < t.levels; ++d)
        l.dir_off[d] = take(plan.use_directory ? 4 * ((t.nodes[d] + kDirBlock - 1) / kDirBlock) : 0,
                            l.mem.directory);
    l.bases_off = take(4 * plan.tile_bases.size(), l.mem.directory);
    l.codes_off = take(8 * plan.codes.size(), l.mem.top_codes);
    l.tiles_off = take(sizeof(Tile) * plan.tiles.size(), l.mem.tiles);
    for (int dir = 0; dir < 2; ++dir) {
        l.groups_off[dir] = take(sizeof(Tile) * plan.band_groups[dir].size(), l.mem.tiles);
        l.sub_off[dir] = take(sizeof(Tile) * plan.band_sub[dir].size(), l.mem.tiles);
        l.order_off[dir] = take(4 * plan.rest_order[dir].size(), l.mem.tiles);
        l.take_off[dir] = take(sizeof(RestTake) * plan.rest_take[dir].size(), l.mem.tiles);
        l.skip_off[dir] = take(8 * plan.skip[dir].size(), l.mem.tiles);
    }
    l.rest_off = take(sizeof(RestTile) * plan.rest_cut.size(), l.mem.tiles);
    for (int dir = 0; dir < 2; ++dir) {
        l.cached_tiles_off[dir] = take(cached ? sizeof(Tile) * plan.cached_tiles[dir].size() : 0, l.mem.tiles);
        l.cached_segs_off[dir] = take(cached ? sizeof(Seg) * plan.cached_segs[dir].size() : 0, l.mem.tiles);
        // strays: their segments, each band's first record and a cursor per
        // band (used while grouping), and the records (copies of cached-level
        // entries, counted with the cached codes)
        const bool st = cached && plan.n_bands[dir] > 0;
        l.stray_segs_off[dir] = take(st ? sizeof(Seg) * plan.stray_segs[dir].size() : 0, l.mem.tiles);
        l.stray_off_off[dir] = take(st ? 4 * (uint64_t(plan.n_bands[dir]) + 1) : 0, l.mem.tiles);
        l.stray_cur_off[dir] = take(st ? 4 * uint64_t(plan.n_bands[dir]) : 0, l.mem.tiles);
        l.strays_off[dir] = take(st ? sizeof(StrayRec) * plan.stray_nodes[dir] : 0, l.mem.cached_codes);
    }
    l.cached_off = take(cached ? 8 * t.nodes[t.levels - 2] : 0, l.mem.cached_codes);
    l.cells_off = take(cached ? 4 * t.nodes[t.levels - 2] : 0, l.mem.cached_codes);
    l.status_off = take(cached ? 4 : 0, l.mem.tiles);
    // products of the max / or / min semirings: a bit per input row (does
    // any of its vectors contribute), rebuilt by every such product
    l.mem.scratch = 0;
    const uint64_t nmax = t.n_rows > t.n_cols ? t.n_rows : t.n_cols;
    l.inmask_off = take(4 * ((nmax + 31) / 32), l.mem.scratch);
    l.mem.alignment = off - raw;
    l.mem.arena = off;
}

}  // namespace k2
