// k2_plan.cpp -- host top, tile plan and device-memory layout.
//
// Tosoni & Mencagli, Sec. 3.4: kernel launches cost more than the first tiny
// levels, so the host expands the top of the tree and the device starts from
// the deepest level with at most 2^16 nodes; in level order the children of a
// contiguous node range form a contiguous range, so each level can be cut
// into tiles descended depth first, which bounds the scratch; the tile
// sequence depends only on the tree, so the host plans it before any product.
//
// Here a tile is one workgroup's job: a range of consecutive nodes of some
// level whose descendants on every level down to the last internal one number
// at most tile_nodes (levels never shrink with depth, so bounding the last
// internal level bounds them all).  The workgroup holds the tile's frontier in
// LDS, so the product needs no frontier memory in HBM at all.  Tiles are cut
// greedily from the host-top level; a node whose subtree is too large is
// replaced by its children (at most four), recursively, which keeps the tiles
// in depth-first (Z) order.  The tile start codes are the Morton codes of the
// first nodes, taken from the host-top expansion or from a split parent.
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

struct Planner {
    const HostTree &t;
    uint64_t C;
    Plan &p;
    int last;   // last internal level

    // Descendant index on the last internal level of boundary 'i' of level d.
    uint64_t down(int d, uint64_t i) const {
        for (int e = d; e < last; ++e) i = child_offset(t, e, i);
        return i;
    }

    void split(int d, uint64_t node, uint64_t code) {
        uint64_t c0 = child_offset(t, d, node), c1 = child_offset(t, d, node + 1);
        unsigned s = nibble(t.words[d], node);
        uint64_t code_base = p.codes.size();
        for (unsigned b = 0; b < 4; ++b)
            if (s & (1u << b)) p.codes.push_back((code << 2) | b);
        range(d + 1, c0, c1, code_base);
    }

    // Cut nodes [a, b) of level d (codes at p.codes[code_base + i - a]).
    void range(int d, uint64_t a, uint64_t b, uint64_t code_base) {
        std::vector<uint64_t> bound(b - a + 1);
        for (uint64_t i = a; i <= b; ++i) bound[i - a] = down(d, i);
        uint64_t i = a;
        while (i < b) {
            if (bound[i + 1 - a] - bound[i - a] > C) {
                split(d, i, p.codes[code_base + (i - a)]);
                ++i;
                continue;
            }
            uint64_t j = i + 1;
            while (j < b && bound[j + 1 - a] - bound[i - a] <= C) ++j;
            Tile tl;
            tl.first = uint32_t(i);
            tl.count = uint32_t(j - i);
            tl.level = uint32_t(d);
            tl.code_off = uint32_t(code_base + (i - a));
            p.tiles.push_back(tl);
            i = j;
        }
    }
};

}  // namespace

k2_status make_plan(const HostTree &t, const k2_plan_opts &o, Plan *out) {
    Plan &p = *out;
    p = Plan();
    p.top_level = top_level_for(t, o.host_top_max);
    p.tile_nodes = o.tile_nodes;
    const int L = t.levels;
    if (L < 2 || t.nodes[L - 2] == 0) return K2_OK;   // empty matrix: no tiles

    // host-top expansion: Morton codes of level d0, parent code then b1b0
    std::vector<uint64_t> codes(1, 0), next;
    for (int d = 0; d < p.top_level; ++d) {
        next.clear();
        next.reserve(t.nodes[d + 1]);
        for (uint64_t i = 0; i < t.nodes[d]; ++i) {
            unsigned s = nibble(t.words[d], i);
            for (unsigned b = 0; b < 4; ++b)
                if (s & (1u << b)) next.push_back((codes[i] << 2) | b);
        }
        codes.swap(next);
    }
    p.codes = codes;
    Planner pl{t, o.tile_nodes, p, L - 2};
    pl.range(p.top_level, 0, t.nodes[p.top_level], 0);
    if (p.codes.size() >= (1ull << 32)) return K2_E_UNSUPPORTED;
    return K2_OK;
}

static uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

void layout_for(const HostTree &t, int top, uint64_t n_codes, uint64_t n_tiles, bool cached,
                Layout *out) {
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
    l.cached_off = take(cached ? 8 * t.nodes[t.levels - 2] : 0, l.mem.cached_codes);
    l.mem.scratch = 0;
    l.mem.alignment = off - raw;
    l.mem.arena = off;
}

}  // namespace k2
