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
// Cached tiles cover the last internal level in order, as ranges of at most
// a few thousand nodes, for the kernel that reads the cached codes (Sec. 3.5).
//
// Windows.  Every node of a Q x Q quadrant (a node of level h = l - log2 Q)
// has its rows and its columns inside the quadrant's Q.  When such a quadrant
// holds many nodes, its tiles get a window: the workgroup accumulates its
// outputs in LDS (Q outputs x B vectors) and adds them to y once at the end,
// so the y atomics of a dense region become LDS atomics plus one coalesced
// pass.  Tiles never straddle a windowed quadrant; the sparse rest keeps one
// y atomic per cell.
#include <algorithm>

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
    uint64_t cached_C;  // nodes per cached tile

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
    void range(int d, uint64_t a, uint64_t b, uint64_t code_base, const Tile &win) {
        std::vector<uint64_t> bound(b - a + 1);
        for (uint64_t i = a; i <= b; ++i) bound[i - a] = down(d, i, last);
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
            p.tiles.push_back(tl);
            i = j;
        }
    }

    // Cached tiles over nodes [lo, hi) of the last internal level.
    void cached(uint64_t lo, uint64_t hi, const Tile &win) {
        for (uint64_t i = lo; i < hi; i += cached_C) {
            Tile tl = win;
            tl.first = uint32_t(i);
            tl.count = uint32_t(std::min(cached_C, hi - i));
            tl.level = uint32_t(last);
            tl.code_off = 0;
            p.cached_tiles.push_back(tl);
        }
    }
};

Tile no_window() {
    Tile w{};
    w.win_log2 = kNoWindow;
    return w;
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
    uint64_t cc = n2 / 2048;                      // enough tiles to fill the GPU
    cc = std::max<uint64_t>(256, std::min<uint64_t>(16384, cc));
    cc = (cc + 255) & ~uint64_t(255);
    Planner pl{t, o.tile_nodes, p, last, cc};

    // window quadrants: side Q with Q * window_batch <= window_elems
    int qlog = -1;
    if (o.window_elems > 0 && o.window_batch > 0) {
        uint64_t q = uint64_t(o.window_elems) / o.window_batch;
        while (q > 1 && (q & (q - 1))) q &= q - 1;
        if (q >= 4) qlog = 0;
        while (qlog >= 0 && (2ull << qlog) <= q) ++qlog;
    }
    p.window_log2 = -1;
    if (qlog < 0) {
        pl.range(d0, 0, t.nodes[d0], 0, no_window());
        pl.cached(0, n2, no_window());
        return K2_OK;
    }
    const int h = std::max(0, L - qlog);           // quadrant level
    p.window_log2 = L - h;
    const uint64_t dense = std::max<uint64_t>(16, (1ull << (L - h)) / 8);   // nodes of level l-2

    if (h <= d0) {
        // quadrants at or above the host top: each is a contiguous range of top nodes
        uint64_t run_a = 0, run_lo2 = 0;
        bool in_run = false;
        for (uint64_t q = 0; q < t.nodes[h]; ++q) {
            uint64_t a0 = pl.down(h, q, d0), b0 = pl.down(h, q + 1, d0);
            uint64_t lo2 = pl.down(d0, a0, last), hi2 = pl.down(d0, b0, last);
            if (hi2 - lo2 >= dense) {
                if (in_run) {
                    pl.range(d0, run_a, a0, run_a, no_window());
                    pl.cached(run_lo2, lo2, no_window());
                    in_run = false;
                }
                Tile w = window_of(codes[h][q], h, L);
                pl.range(d0, a0, b0, a0, w);
                pl.cached(lo2, hi2, w);
            } else if (!in_run) {
                in_run = true;
                run_a = a0;
                run_lo2 = lo2;
            }
        }
        if (in_run) {
            pl.range(d0, run_a, t.nodes[d0], run_a, no_window());
            pl.cached(run_lo2, n2, no_window());
        }
    } else {
        // Walk down from the host top.  A subtree with fewer than 'dense' nodes
        // on the last internal level holds no dense quadrant and stays sparse;
        // larger ones are split down to level h, whose dense nodes get windows.
        // Consecutive sparse subtrees of one level, adjacent in it, form one run.
        struct Run {
            int level = -1;
            uint64_t a = 0, b = 0, code_base = 0, lo2 = 0, hi2 = 0;
        } run;
        auto flush_run = [&]() {
            if (run.level < 0) return;
            pl.range(run.level, run.a, run.b, run.code_base, no_window());
            pl.cached(run.lo2, run.hi2, no_window());
            run.level = -1;
        };
        auto add_sparse = [&](int d, uint64_t node, uint64_t code, uint64_t lo2, uint64_t hi2) {
            if (run.level == d && run.b == node) {
                p.codes.push_back(code);
                run.b = node + 1;
                run.hi2 = hi2;
                return;
            }
            flush_run();
            run.level = d;
            run.a = node;
            run.b = node + 1;
            run.code_base = p.codes.size();
            p.codes.push_back(code);
            run.lo2 = lo2;
            run.hi2 = hi2;
        };
        // explicit stack of (level, node, code), children pushed in reverse
        struct Item {
            int d;
            uint64_t node, code;
        };
        std::vector<Item> stack;
        for (uint64_t i = t.nodes[d0]; i-- > 0;) stack.push_back({d0, i, codes[d0][i]});
        while (!stack.empty()) {
            Item it = stack.back();
            stack.pop_back();
            uint64_t lo2 = pl.down(it.d, it.node, last), hi2 = pl.down(it.d, it.node + 1, last);
            uint64_t desc = hi2 - lo2;
            if (it.d == h) {
                if (desc >= dense) {
                    flush_run();
                    Tile w = window_of(it.code, h, L);
                    uint64_t base = p.codes.size();
                    p.codes.push_back(it.code);
                    pl.range(h, it.node, it.node + 1, base, w);
                    pl.cached(lo2, hi2, w);
                } else {
                    add_sparse(it.d, it.node, it.code, lo2, hi2);
                }
            } else if (desc < dense) {
                add_sparse(it.d, it.node, it.code, lo2, hi2);
            } else {
                uint64_t c0 = child_offset(t, it.d, it.node);
                unsigned s = nibble(t.words[it.d], it.node);
                uint64_t ch[4];
                int nc = 0;
                for (unsigned b = 0; b < 4; ++b)
                    if (s & (1u << b)) ch[nc++] = (it.code << 2) | b;
                for (int k = nc - 1; k >= 0; --k)
                    stack.push_back({it.d + 1, c0 + uint64_t(k), ch[k]});
            }
        }
        flush_run();
    }
    if (p.codes.size() >= (1ull << 32)) return K2_E_UNSUPPORTED;
    return K2_OK;
}

static uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

void layout_for(const HostTree &t, int top, uint64_t n_codes, uint64_t n_tiles, uint64_t n_cached_tiles,
                bool cached, Layout *out) {
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
        l.dir_off[d] = take(4 * ((t.nodes[d] + kDirBlock - 1) / kDirBlock), l.mem.directory);
    l.codes_off = take(8 * n_codes, l.mem.top_codes);
    l.tiles_off = take(sizeof(Tile) * n_tiles, l.mem.tiles);
    l.cached_tiles_off = take(cached ? sizeof(Tile) * n_cached_tiles : 0, l.mem.tiles);
    l.cached_off = take(cached ? 8 * t.nodes[t.levels - 2] : 0, l.mem.cached_codes);
    l.mem.scratch = 0;
    l.mem.alignment = off - raw;
    l.mem.arena = off;
}

}  // namespace k2
