// k2_api.cpp -- the C ABI declared in include/k2spmv.h.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <memory>
#include <mutex>
#include <thread>

#include "k2_internal.h"

struct k2_tree {
    k2::HostTree t;
    // the last plan computed, and the options it was made for
    std::mutex plan_mu;
    bool have_plan = false;
    k2_plan_opts plan_opts{};
    k2::Plan plan;
};

struct k2_matrix {
    k2::Matrix m;
};

// A streamed (out-of-core) product plan: the descent tiles cut into chunks
// whose staged data fits the staging buffer.
struct k2_stream {
    struct Chunk {
        uint64_t t0 = 0, t1 = 0;            // tiles [t0, t1) of 'tiles'
        uint64_t lo_word[k2::kMaxLevels];   // first staged word per level
        uint64_t n_words[k2::kMaxLevels];   // staged words per level (0: none)
        uint64_t word_off[k2::kMaxLevels];  // byte offset in the staging buffer
        uint64_t tiles_off = 0, codes_off = 0, bases_off = 0, bytes = 0;
        std::vector<k2::Tile> tiles;        // code_off / base_off relative to the chunk
        std::vector<uint64_t> codes;
        std::vector<uint32_t> bases;
    };
    const k2_tree *tree = nullptr;
    uint32_t tile_nodes = 0;
    bool row_runs = false;
    std::vector<Chunk> chunks;
    uint64_t max_bytes = 0, staged_bytes = 0;
    // pinned host copy: every level's words at pin_words[d], then each
    // chunk's tiles, codes and offsets laid out as in the staging buffer
    char *pinned = nullptr;
    uint64_t pin_words[k2::kMaxLevels] = {};
    std::vector<uint64_t> pin_meta;   // per chunk, offset of its metadata block
    // copies run on their own stream, one staging half ahead of the kernels
    hipStream_t copy_stream = nullptr;
    hipEvent_t copied[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr}, start = nullptr;
    ~k2_stream() {
        for (hipEvent_t e : {copied[0], copied[1], done[0], done[1], start})
            if (e) (void)hipEventDestroy(e);
        if (copy_stream) (void)hipStreamDestroy(copy_stream);
        if (pinned) (void)hipHostFree(pinned);
    }
};

namespace k2 {
k2_status build_tree(const uint32_t *rows, const uint32_t *cols, uint64_t m, uint32_t n_rows,
                     uint32_t n_cols, int nt, HostTree *out);

static thread_local std::string g_hip_error;

void set_hip_error(int err, const char *where) {
    g_hip_error = std::string(where) + ": " + hip_error_text(err);
}
}  // namespace k2

using namespace k2;

namespace {

bool valid_opts(const k2_plan_opts &o) {
    if (o.tile_nodes < 256 || o.tile_nodes > 4096) return false;
    if (o.tile_nodes & (o.tile_nodes - 1)) return false;
    if (o.window_elems > 16384) return false;
    if (o.offsets < K2_OFFSETS_AUTO || o.offsets > K2_OFFSETS_SCAN) return false;
    if (o.band_tile_nodes < 64 || o.band_tile_nodes > (1u << 30)) return false;
    return true;
}

uint64_t vector_bytes(const HostTree &t, uint32_t batch) {
    return (uint64_t(t.n_rows) + uint64_t(t.n_cols)) * uint64_t(batch) * 4ull;
}

bool same_opts(const k2_plan_opts &a, const k2_plan_opts &b) {
    return a.tile_nodes == b.tile_nodes && a.host_top_max == b.host_top_max &&
           a.window_elems == b.window_elems && a.window_batch == b.window_batch &&
           (a.cache_last_level != 0) == (b.cache_last_level != 0) &&
           (a.xcd_remap != 0) == (b.xcd_remap != 0) &&
           (a.offsets == K2_OFFSETS_DIRECTORY) == (b.offsets == K2_OFFSETS_DIRECTORY) &&
           (a.band_strays != 0) == (b.band_strays != 0) && a.band_tile_nodes == b.band_tile_nodes;
}

// The plan of 'tree' for 'o', computed once per option set.
k2_status plan_of(const k2_tree *tree, const k2_plan_opts &o, Plan *out) {
    k2_tree *t = const_cast<k2_tree *>(tree);
    std::lock_guard<std::mutex> lock(t->plan_mu);
    if (!t->have_plan || !same_opts(t->plan_opts, o)) {
        t->have_plan = false;
        k2_status st = make_plan(t->t, o, &t->plan);
        if (st != K2_OK) return st;
        t->plan_opts = o;
        t->have_plan = true;
    }
    *out = t->plan;
    return K2_OK;
}

k2_status estimate(const k2_tree *tree, const k2_plan_opts &o, Plan *plan, Layout *lay) {
    const HostTree &t = tree->t;
    k2_status st = plan_of(tree, o, plan);
    if (st != K2_OK) return st;
    bool cached = o.cache_last_level != 0 && t.nodes[t.levels - 2] > 0;
    layout_for(t, plan->top_level, *plan, cached, lay);
    return K2_OK;
}

#define HIP_TRY(call, where)                                        \
    do {                                                            \
        hipError_t e_ = (call);                                     \
        if (e_ != hipSuccess) {                                     \
            set_hip_error(int(e_), where);                          \
            return K2_E_HIP;                                        \
        }                                                           \
    } while (0)

}  // namespace

extern "C" {

k2_status k2_plan_defaults(k2_plan_opts *opts) {
    if (!opts) return K2_E_INVALID_ARG;
    opts->tile_nodes = 1024;
    opts->host_top_max = 1u << 16;
    opts->cache_last_level = 0;
    opts->xcd_remap = 1;
    opts->window_elems = 4096;
    opts->window_batch = 8;
    opts->offsets = K2_OFFSETS_AUTO;
    opts->band_strays = 1;
    opts->band_tile_nodes = 65536;
    return K2_OK;
}

k2_status k2_build(const uint32_t *rows, const uint32_t *cols, uint64_t n_edges, uint32_t n_rows,
                   uint32_t n_cols, uint32_t n_threads, k2_tree **out) {
    if (!out) return K2_E_INVALID_ARG;
    *out = nullptr;
    if (n_rows == 0 || n_cols == 0) return K2_E_INVALID_ARG;
    if (n_edges > 0 && (!rows || !cols)) return K2_E_INVALID_ARG;
    int nt = int(n_threads);
    if (nt <= 0) nt = int(std::min<unsigned>(64, std::max(1u, std::thread::hardware_concurrency())));
    nt = std::min(nt, 64);
    k2_tree *t = new (std::nothrow) k2_tree();
    if (!t) return K2_E_HOST_OOM;
    k2_status st;
    try {
        st = build_tree(rows, cols, n_edges, n_rows, n_cols, nt, &t->t);
    } catch (const std::bad_alloc &) {
        st = K2_E_HOST_OOM;
    }
    if (st != K2_OK) {
        delete t;
        return st;
    }
    *out = t;
    return K2_OK;
}

void k2_tree_free(k2_tree *tree) { delete tree; }

k2_status k2_tree_info(const k2_tree *tree, k2_tree_info_t *out) {
    if (!tree || !out) return K2_E_INVALID_ARG;
    const HostTree &t = tree->t;
    out->n_rows = t.n_rows;
    out->n_cols = t.n_cols;
    out->levels = uint32_t(t.levels);
    out->top_level = uint32_t(top_level_for(t, 1u << 16));
    out->nnz = t.nnz;
    uint64_t n = 0;
    for (uint64_t v : t.nodes) n += v;
    out->nodes = n;
    return K2_OK;
}

k2_status k2_tree_level_nodes(const k2_tree *tree, uint64_t *nodes) {
    if (!tree || !nodes) return K2_E_INVALID_ARG;
    std::copy(tree->t.nodes.begin(), tree->t.nodes.end(), nodes);
    return K2_OK;
}

k2_status k2_tree_level_words(const k2_tree *tree, uint32_t level, uint64_t *words, uint64_t n_words) {
    if (!tree || !words || level >= uint32_t(tree->t.levels)) return K2_E_INVALID_ARG;
    const std::vector<uint64_t> &w = tree->t.words[level];
    if (n_words < w.size()) return K2_E_INVALID_ARG;
    std::copy(w.begin(), w.end(), words);
    std::fill(words + w.size(), words + n_words, 0ull);
    return K2_OK;
}

k2_status k2_tree_directory(const k2_tree *tree, uint32_t level, uint32_t *out, uint64_t n_out) {
    if (!tree || !out || level + 1 >= uint32_t(tree->t.levels)) return K2_E_INVALID_ARG;
    const std::vector<uint32_t> &D = tree->t.dir[level];
    if (n_out < D.size()) return K2_E_INVALID_ARG;
    std::copy(D.begin(), D.end(), out);
    return K2_OK;
}

k2_status k2_estimate_device_bytes(const k2_tree *tree, const k2_plan_opts *opts,
                                   k2_semiring semiring, uint32_t batch, k2_mem_breakdown *out) {
    if (!tree || !opts || !out || batch == 0) return K2_E_INVALID_ARG;
    if (int(semiring) < 0 || int(semiring) > 3 || !valid_opts(*opts)) return K2_E_INVALID_ARG;
    Plan plan;
    Layout lay;
    k2_status st;
    try {
        st = estimate(tree, *opts, &plan, &lay);
    } catch (const std::bad_alloc &) {
        return K2_E_HOST_OOM;
    }
    if (st != K2_OK) return st;
    *out = lay.mem;
    out->vectors = vector_bytes(tree->t, batch);
    out->total = out->arena + out->vectors;
    return K2_OK;
}

}  // extern "C"

namespace {

// The tile list and aux entry count k2_plan_tiles exports for 'which'.
// The rest tiles of a direction are built into 'tmp' in its block order,
// with their skip ranges after band groups (0xFFFFFFFF: covered whole).
void plan_list(const Plan &p, int which, std::vector<Tile> &tmp, const std::vector<Tile> **list,
               uint64_t *naux) {
    switch (which) {
    case 0: *list = &p.tiles; *naux = p.codes.size(); break;
    case 1: case 2: *list = &p.cached_tiles[which - 1]; *naux = 2 * p.cached_segs[which - 1].size(); break;
    case 3: case 4: {
        const int dir = which - 3;
        const std::vector<RestTake> &take = p.rest_take[dir];
        const bool groups = !p.band_groups[dir].empty();
        size_t t = 0;
        tmp.clear();
        tmp.reserve(p.rest_order[dir].size());
        for (uint32_t idx : p.rest_order[dir]) {
            const RestTile &rt = p.rest_cut[idx];
            Tile tl{rt.first, rt.count(), rt.level(), rt.code_off, 0, 0, 0xFFFFFFFFu, rt.base_off};
            if (t < take.size() && take[t].tile == idx) {
                tl.win_row = take[t].skip_row;
                tl.win_col = take[t].skip_count;
                ++t;
            } else if (groups) {
                tl.win_col = 0xFFFFFFFFu;
            }
            tmp.push_back(tl);
        }
        *list = &tmp;
        *naux = p.skip[dir].size();
        break;
    }
    case 5: case 6: *list = &p.band_groups[which - 5]; *naux = 0; break;
    case 7: case 8: *list = &p.band_sub[which - 7]; *naux = 0; break;
    default: {
        static const std::vector<Tile> none;
        *list = &none;
        *naux = 2 * p.stray_segs[which - 9].size();
    }
    }
}

}  // namespace

extern "C" {

k2_status k2_plan_info(const k2_tree *tree, const k2_plan_opts *opts, int32_t which,
                       uint32_t *top_level, uint64_t *n_tiles, uint64_t *n_aux) {
    if (!tree || !opts || !valid_opts(*opts) || which < 0 || which > 10) return K2_E_INVALID_ARG;
    Plan plan;
    k2_status st;
    try {
        st = plan_of(tree, *opts, &plan);
    } catch (const std::bad_alloc &) {
        return K2_E_HOST_OOM;
    }
    if (st != K2_OK) return st;
    if (top_level) *top_level = uint32_t(plan.top_level);
    std::vector<Tile> tmp;
    const std::vector<Tile> *list = nullptr;
    uint64_t naux = 0;
    plan_list(plan, which, tmp, &list, &naux);
    if (n_tiles) *n_tiles = list->size();
    if (n_aux) *n_aux = naux;
    return K2_OK;
}

k2_status k2_plan_tiles(const k2_tree *tree, const k2_plan_opts *opts, int32_t which, uint32_t *tiles,
                        uint64_t n_tiles, uint64_t *aux, uint64_t n_aux) {
    if (!tree || !opts || !valid_opts(*opts) || which < 0 || which > 10) return K2_E_INVALID_ARG;
    Plan plan;
    k2_status st;
    try {
        st = plan_of(tree, *opts, &plan);
    } catch (const std::bad_alloc &) {
        return K2_E_HOST_OOM;
    }
    if (st != K2_OK) return st;
    std::vector<Tile> tmp;
    const std::vector<Tile> *lp = nullptr;
    uint64_t naux = 0;
    plan_list(plan, which, tmp, &lp, &naux);
    const std::vector<Tile> &list = *lp;
    if (n_tiles < list.size() || n_aux < naux) return K2_E_INVALID_ARG;
    if ((!tiles && !list.empty()) || (!aux && naux)) return K2_E_INVALID_ARG;
    for (size_t k = 0; k < list.size(); ++k) {
        const Tile &tl = list[k];
        const uint32_t v[8] = {tl.first, tl.count, tl.level, tl.code_off,
                               tl.win_row, tl.win_col, tl.win_log2, tl.base_off};
        std::copy(v, v + 8, tiles + 8 * k);
    }
    if (which == 0) {
        std::copy(plan.codes.begin(), plan.codes.end(), aux);
    } else if (which == 3 || which == 4) {
        std::copy(plan.skip[which - 3].begin(), plan.skip[which - 3].end(), aux);
    } else if (which == 1 || which == 2 || which == 9 || which == 10) {
        const std::vector<Seg> &sg = which <= 2 ? plan.cached_segs[which - 1] : plan.stray_segs[which - 9];
        for (size_t k = 0; k < sg.size(); ++k) {
            aux[2 * k] = (uint64_t(sg[k].lo) << 32) | sg[k].count;
            aux[2 * k + 1] = sg[k].leaf;
        }
    }
    return K2_OK;
}

k2_status k2_plan_offsets(const k2_tree *tree, const k2_plan_opts *opts, uint32_t *bases,
                          uint64_t n_bases, uint64_t *n_total) {
    if (!tree || !opts || !valid_opts(*opts)) return K2_E_INVALID_ARG;
    Plan plan;
    k2_status st;
    try {
        st = plan_of(tree, *opts, &plan);
    } catch (const std::bad_alloc &) {
        return K2_E_HOST_OOM;
    }
    if (st != K2_OK) return st;
    if (n_total) *n_total = plan.tile_bases.size();
    if (!bases) return K2_OK;
    if (n_bases < plan.tile_bases.size()) return K2_E_INVALID_ARG;
    std::copy(plan.tile_bases.begin(), plan.tile_bases.end(), bases);
    return K2_OK;
}

namespace {

// Strays of direction dir grouped by band, once the block origins are on the
// device: count per band, prefix sums on the host, then each stray's record
// at its band's cursor.  Every band with strays must have an owner tile.
k2_status group_strays(Matrix &m, int dir, hipStream_t st) {
    const Plan &pn = m.plan;
    const uint32_t nb = pn.n_bands[dir];
    if (nb == 0) return K2_OK;
    const std::vector<Seg> &sg = pn.stray_segs[dir];
    Seg *d_segs = reinterpret_cast<Seg *>(m.arena + m.layout.stray_segs_off[dir]);
    uint32_t *d_off = reinterpret_cast<uint32_t *>(m.arena + m.layout.stray_off_off[dir]);
    uint32_t *d_cur = reinterpret_cast<uint32_t *>(m.arena + m.layout.stray_cur_off[dir]);
    StrayRec *d_rec = reinterpret_cast<StrayRec *>(m.arena + m.layout.strays_off[dir]);
    if (pn.stray_nodes[dir] >= (1ull << 32) || sg.size() >= (1ull << 32)) return K2_E_UNSUPPORTED;
    std::vector<uint32_t> cnt(nb), off(size_t(nb) + 1);
    hipError_t e = hipSuccess;
    if (!sg.empty()) e = hipMemcpyAsync(d_segs, sg.data(), sg.size() * sizeof(Seg), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemsetAsync(d_cur, 0, size_t(nb) * 4, st);
    if (e == hipSuccess) e = hipError_t(launch_stray_count(m, dir, d_segs, uint32_t(sg.size()), d_cur, st));
    if (e == hipSuccess) e = hipMemcpyAsync(cnt.data(), d_cur, size_t(nb) * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        set_hip_error(int(e), "count strays");
        return K2_E_HIP;
    }
    std::vector<char> owner(nb, 0);
    for (const Tile &tl : pn.cached_tiles[dir])
        if (tl.code_off && tl.win_log2 != kNoWindow) {
            const uint64_t b = uint64_t(dir == K2_RIGHT ? tl.win_row : tl.win_col) >> tl.win_log2;
            if (b < nb) owner[b] = 1;
        }
    uint64_t total = 0;
    for (uint32_t b = 0; b < nb; ++b) {
        if (cnt[b] && !owner[b]) return K2_E_UNSUPPORTED;   // planner invariant
        off[b] = uint32_t(total);
        total += cnt[b];
    }
    off[nb] = uint32_t(total);
    if (total != pn.stray_nodes[dir]) return K2_E_UNSUPPORTED;
    e = hipMemcpyAsync(d_off, off.data(), off.size() * 4, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(d_cur, off.data(), size_t(nb) * 4, hipMemcpyHostToDevice, st);
    if (e == hipSuccess)
        e = hipError_t(launch_stray_scatter(m, dir, d_segs, uint32_t(sg.size()), d_cur, d_rec, st));
    if (e == hipSuccess) e = hipStreamSynchronize(st);   // before off goes away
    if (e != hipSuccess) {
        set_hip_error(int(e), "group strays");
        return K2_E_HIP;
    }
    m.d_strays[dir] = d_rec;
    m.d_stray_off[dir] = d_off;
    return K2_OK;
}

}  // namespace

k2_status k2_matrix_create(const k2_tree *tree, const k2_plan_opts *opts, void *d_arena,
                           uint64_t arena_bytes, void *stream, k2_matrix **out) {
    if (!tree || !opts || !out || !d_arena) return K2_E_INVALID_ARG;
    *out = nullptr;
    if (!valid_opts(*opts) || (reinterpret_cast<uintptr_t>(d_arena) & 255)) return K2_E_INVALID_ARG;
    const HostTree &t = tree->t;
    k2_matrix *mx = new (std::nothrow) k2_matrix();
    if (!mx) return K2_E_HOST_OOM;
    Matrix &m = mx->m;
    k2_status st;
    try {
        st = estimate(tree, *opts, &m.plan, &m.layout);
    } catch (const std::bad_alloc &) {
        st = K2_E_HOST_OOM;
    }
    if (st != K2_OK) {
        delete mx;
        return st;
    }
    if (arena_bytes < m.layout.mem.arena) {
        delete mx;
        return K2_E_ARENA_TOO_SMALL;
    }
    m.arena = static_cast<char *>(d_arena);
    m.n_rows = t.n_rows;
    m.n_cols = t.n_cols;
    m.levels = t.levels;
    m.nodes = t.nodes;
    m.cached = opts->cache_last_level != 0 && t.nodes[t.levels - 2] > 0;
    m.window_elems = m.plan.window_log2 >= 0 ? opts->window_elems : 0;
    m.window_batch = opts->window_batch;
    {   // the window shares a workgroup's LDS with the kernels' own (cell rings, frontiers)
        int dev = 0, lds = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess) {
            set_hip_error(int(e), "LDS size");
            delete mx;
            return K2_E_HIP;
        }
        m.lds_per_block = lds > 0 ? size_t(lds) : 0;
    }
    std::memset(&m.dev, 0, sizeof(m.dev));
    m.dev.levels = t.levels;
    m.dev.top_level = m.plan.top_level;
    m.d_inmask = reinterpret_cast<uint32_t *>(m.arena + m.layout.inmask_off);
    hipStream_t st_h = static_cast<hipStream_t>(stream);
    auto fail = [&](k2_status s) {
        delete mx;
        return s;
    };
    for (int d = 0; d < t.levels; ++d) m.dev.nodes[d] = uint32_t(t.nodes[d]);
    for (int d = m.plan.top_level; d < t.levels; ++d) {
        char *p = m.arena + m.layout.words_off[d];
        m.dev.words[d] = reinterpret_cast<const uint64_t *>(p);
        m.dev.words_end[d] = uint32_t(t.words[d].size());
        if (!t.words[d].empty()) {
            hipError_t e = hipMemcpyAsync(p, t.words[d].data(), t.words[d].size() * 8,
                                          hipMemcpyHostToDevice, st_h);
            if (e != hipSuccess) {
                set_hip_error(int(e), "upload tree");
                return fail(K2_E_HIP);
            }
        }
    }
    for (int d = m.plan.top_level; d + 1 < t.levels && m.plan.use_directory; ++d) {
        char *p = m.arena + m.layout.dir_off[d];
        m.dev.dir[d] = reinterpret_cast<const uint32_t *>(p);
        if (!t.dir[d].empty()) {
            hipError_t e = hipMemcpyAsync(p, t.dir[d].data(), t.dir[d].size() * 4,
                                          hipMemcpyHostToDevice, st_h);
            if (e != hipSuccess) {
                set_hip_error(int(e), "upload directory");
                return fail(K2_E_HIP);
            }
        }
    }
    m.d_codes = reinterpret_cast<const uint64_t *>(m.arena + m.layout.codes_off);
    m.d_tiles = reinterpret_cast<const Tile *>(m.arena + m.layout.tiles_off);
    if (!m.plan.codes.empty()) {
        hipError_t e = hipMemcpyAsync(const_cast<uint64_t *>(m.d_codes), m.plan.codes.data(),
                                      m.plan.codes.size() * 8, hipMemcpyHostToDevice, st_h);
        if (e != hipSuccess) {
            set_hip_error(int(e), "upload tile codes");
            return fail(K2_E_HIP);
        }
    }
    if (!m.plan.tile_bases.empty()) {
        m.d_bases = reinterpret_cast<const uint32_t *>(m.arena + m.layout.bases_off);
        hipError_t e = hipMemcpyAsync(const_cast<uint32_t *>(m.d_bases), m.plan.tile_bases.data(),
                                      m.plan.tile_bases.size() * 4, hipMemcpyHostToDevice, st_h);
        if (e != hipSuccess) {
            set_hip_error(int(e), "upload tile offsets");
            return fail(K2_E_HIP);
        }
    }
    {
        auto up = [&](uint64_t off, const void *src, uint64_t bytes) -> const char * {
            if (!bytes) return nullptr;
            char *dst = m.arena + off;
            hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, st_h);
            if (e != hipSuccess) {
                set_hip_error(int(e), "upload tree-only plan");
                return reinterpret_cast<const char *>(1);
            }
            return dst;
        };
        const char *bad = reinterpret_cast<const char *>(1);
        const Plan &pn = m.plan;
        const char *r = up(m.layout.rest_off, pn.rest_cut.data(), pn.rest_cut.size() * sizeof(RestTile));
        if (r == bad) return fail(K2_E_HIP);
        m.d_rest = reinterpret_cast<const RestTile *>(r);
        for (int dir = 0; dir < 2; ++dir) {
            const char *g = up(m.layout.groups_off[dir], pn.band_groups[dir].data(),
                               pn.band_groups[dir].size() * sizeof(Tile));
            const char *sb = up(m.layout.sub_off[dir], pn.band_sub[dir].data(), pn.band_sub[dir].size() * sizeof(Tile));
            const char *o = up(m.layout.order_off[dir], pn.rest_order[dir].data(), pn.rest_order[dir].size() * 4);
            const char *tk = up(m.layout.take_off[dir], pn.rest_take[dir].data(),
                                pn.rest_take[dir].size() * sizeof(RestTake));
            const char *k = up(m.layout.skip_off[dir], pn.skip[dir].data(), pn.skip[dir].size() * 8);
            if (g == bad || sb == bad || o == bad || tk == bad || k == bad) return fail(K2_E_HIP);
            m.d_band_groups[dir] = reinterpret_cast<const Tile *>(g);
            m.d_band_sub[dir] = reinterpret_cast<const Tile *>(sb);
            m.d_rest_order[dir] = reinterpret_cast<const uint32_t *>(o);
            m.d_rest_take[dir] = reinterpret_cast<const RestTake *>(tk);
            m.d_skip[dir] = reinterpret_cast<const uint64_t *>(k);
        }
    }
    if (!m.plan.tiles.empty()) {
        hipError_t e = hipMemcpyAsync(const_cast<Tile *>(m.d_tiles), m.plan.tiles.data(),
                                      m.plan.tiles.size() * sizeof(Tile), hipMemcpyHostToDevice, st_h);
        if (e != hipSuccess) {
            set_hip_error(int(e), "upload tiles");
            return fail(K2_E_HIP);
        }
    }
    if (m.cached) {
        for (int dir = 0; dir < 2; ++dir) {
            m.d_cached_tiles[dir] = reinterpret_cast<const Tile *>(m.arena + m.layout.cached_tiles_off[dir]);
            m.d_cached_segs[dir] = reinterpret_cast<const Seg *>(m.arena + m.layout.cached_segs_off[dir]);
            const std::vector<Tile> &tl = m.plan.cached_tiles[dir];
            const std::vector<Seg> &sg = m.plan.cached_segs[dir];
            hipError_t e = hipSuccess;
            if (!tl.empty())
                e = hipMemcpyAsync(const_cast<Tile *>(m.d_cached_tiles[dir]), tl.data(), tl.size() * sizeof(Tile),
                                   hipMemcpyHostToDevice, st_h);
            if (e == hipSuccess && !sg.empty())
                e = hipMemcpyAsync(const_cast<Seg *>(m.d_cached_segs[dir]), sg.data(), sg.size() * sizeof(Seg),
                                   hipMemcpyHostToDevice, st_h);
            if (e != hipSuccess) {
                set_hip_error(int(e), "upload cached tiles");
                return fail(K2_E_HIP);
            }
        }
        m.d_cached = reinterpret_cast<uint64_t *>(m.arena + m.layout.cached_off);
        int e = launch_descent(m, K2_RIGHT, K2_BOOLEAN_U32X32, 1, nullptr, nullptr, m.d_cached, stream);
        if (e != hipSuccess) {
            set_hip_error(e, "cache last internal level");
            return fail(K2_E_HIP);
        }
        m.d_nodew = reinterpret_cast<uint32_t *>(m.arena + m.layout.cells_off);

        uint32_t *status = reinterpret_cast<uint32_t *>(m.arena + m.layout.status_off);
        // packed node words when every cached tile with segments has a
        // window of at most 1024 rows (a block's place in its quadrant then
        // takes 2 x 8 bits; the XCD order's padding tiles hold none)
        bool packed = !m.plan.use_directory && m.plan.window_log2 >= 2 && m.plan.window_log2 <= 10;
        for (int dir = 0; dir < 2 && packed; ++dir)
            for (const Tile &tl : m.plan.cached_tiles[dir])
                if (tl.count && tl.win_log2 != uint32_t(m.plan.window_log2)) {
                    packed = false;
                    break;
                }
        hipError_t es = hipMemsetAsync(status, 0, 4, st_h);
        if (es != hipSuccess) {
            set_hip_error(int(es), "cached cells");
            return fail(K2_E_HIP);
        }
        for (int dir = 0; dir < 2; ++dir) {
            const int ec = launch_node_cells(m, const_cast<Seg *>(m.d_cached_segs[dir]),
                                             uint32_t(m.plan.cached_segs[dir].size()), packed ? m.plan.window_log2 : 0,
                                             status, stream);
            if (ec != hipSuccess) {
                set_hip_error(ec, "cached cells");
                return fail(K2_E_HIP);
            }
        }
        if (packed) {
            // every segment inside one quadrant, as the plan cuts them (else
            // the products keep reading the 8-byte block origins)
            uint32_t st = 1;
            es = hipMemcpyAsync(&st, status, 4, hipMemcpyDeviceToHost, st_h);
            if (es == hipSuccess) es = hipStreamSynchronize(st_h);
            if (es != hipSuccess) {
                set_hip_error(int(es), "cached cells");
                return fail(K2_E_HIP);
            }
            m.packed = st == 0;
        }
        for (int dir = 0; dir < 2; ++dir) {
            const k2_status s = group_strays(m, dir, st_h);
            if (s != K2_OK) return fail(s);
        }
    }
    hipError_t e = hipStreamSynchronize(st_h);
    if (e != hipSuccess) {
        set_hip_error(int(e), "matrix create");
        return fail(K2_E_HIP);
    }
    *out = mx;
    return K2_OK;
}

k2_status k2_spmv(k2_matrix *matrix, k2_direction direction, k2_semiring semiring, uint32_t batch,
                  int32_t mode, const void *d_x, void *d_y, void *stream) {
    if (!matrix || !d_x || !d_y || batch == 0) return K2_E_INVALID_ARG;
    if (int(direction) != K2_RIGHT && int(direction) != K2_LEFT) return K2_E_INVALID_ARG;
    if (int(semiring) < 0 || int(semiring) > 3) return K2_E_INVALID_ARG;
    Matrix &m = matrix->m;
    const bool accumulate = (mode & K2_SPMV_ACCUMULATE) != 0;
    mode &= ~int32_t(K2_SPMV_ACCUMULATE);
    if (mode == K2_MODE_AUTO) mode = m.cached ? K2_MODE_CACHED : K2_MODE_TREE_ONLY;
    if (mode != K2_MODE_TREE_ONLY && mode != K2_MODE_CACHED) return K2_E_INVALID_ARG;
    const bool empty = m.nodes[m.levels - 2] == 0;
    if (mode == K2_MODE_CACHED && !m.cached && !empty) return K2_E_INVALID_ARG;
    const uint64_t n_out = direction == K2_RIGHT ? m.n_rows : m.n_cols;
    const uint64_t n_in = direction == K2_RIGHT ? m.n_cols : m.n_rows;
    {   // x and y must not overlap
        const char *xb = static_cast<const char *>(d_x), *yb = static_cast<const char *>(d_y);
        const uint64_t xl = n_in * batch * 4, yl = n_out * batch * 4;
        if (xb < yb + yl && yb < xb + xl) return K2_E_INVALID_ARG;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (m.timing) HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(m.ev[0]), st), "timing");
    const uint32_t zero = semiring == K2_TROPICAL_F32 ? 0x7F800000u : 0u;
    // a cached product whose bands cover y writes every element itself
    const bool fill = !accumulate && !(mode == K2_MODE_CACHED && !empty && cached_writes_all(m, direction, batch));
    int e = fill ? launch_fill(d_y, n_out * batch, zero, stream) : int(hipSuccess);
    if (e != hipSuccess) {
        set_hip_error(e, "fill");
        return K2_E_HIP;
    }
    if (m.timing) HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(m.ev[1]), st), "timing");
    if (!empty)
        e = (mode == K2_MODE_CACHED)
                ? launch_cached(m, direction, semiring, batch, d_x, d_y, accumulate ? 1 : 0, stream)
                : launch_descent(m, direction, semiring, batch, d_x, d_y, nullptr, stream);
    if (e != hipSuccess) {
        set_hip_error(e, "spmv");
        return K2_E_HIP;
    }
    if (m.timing) {
        HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(m.ev[2]), st), "timing");
        m.timed_once = true;
        m.last_accumulate = accumulate;
    }
    return K2_OK;
}

k2_status k2_matrix_set_timing(k2_matrix *matrix, int32_t enable) {
    if (!matrix) return K2_E_INVALID_ARG;
    Matrix &m = matrix->m;
    if (enable && !m.ev[0]) {
        for (int k = 0; k < 3; ++k) {
            hipEvent_t ev;
            HIP_TRY(hipEventCreate(&ev), "timing events");
            m.ev[k] = ev;
        }
    }
    m.timing = enable != 0;
    m.timed_once = false;
    return K2_OK;
}

k2_status k2_matrix_last_timing(k2_matrix *matrix, float *fill_ms, float *kernel_ms) {
    if (!matrix) return K2_E_INVALID_ARG;
    Matrix &m = matrix->m;
    if (!m.timing || !m.timed_once) return K2_E_INVALID_ARG;
    hipEvent_t e0 = static_cast<hipEvent_t>(m.ev[0]), e1 = static_cast<hipEvent_t>(m.ev[1]),
               e2 = static_cast<hipEvent_t>(m.ev[2]);
    HIP_TRY(hipEventSynchronize(e2), "timing");
    float a = 0, b = 0;
    HIP_TRY(hipEventElapsedTime(&a, e0, e1), "timing");
    HIP_TRY(hipEventElapsedTime(&b, e1, e2), "timing");
    if (fill_ms) *fill_ms = m.last_accumulate ? 0.0f : a;
    if (kernel_ms) *kernel_ms = b;
    return K2_OK;
}

k2_status k2_matrix_destroy(k2_matrix *matrix) {
    if (!matrix) return K2_OK;
    for (int k = 0; k < 3; ++k)
        if (matrix->m.ev[k]) (void)hipEventDestroy(static_cast<hipEvent_t>(matrix->m.ev[k]));
    delete matrix;
    return K2_OK;
}

k2_status k2_matrix_info(const k2_matrix *matrix, uint32_t *top_level, uint64_t *n_tiles,
                         int32_t *cached) {
    if (!matrix) return K2_E_INVALID_ARG;
    if (top_level) *top_level = uint32_t(matrix->m.plan.top_level);
    if (n_tiles) *n_tiles = matrix->m.plan.tiles.size();
    if (cached) *cached = matrix->m.cached ? (matrix->m.packed ? 2 : 1) : 0;
    return K2_OK;
}

k2_status k2_matrix_level_words(const k2_matrix *matrix, uint32_t level, uint64_t *words,
                                uint64_t n_words, void *stream) {
    if (!matrix || !words) return K2_E_INVALID_ARG;
    const Matrix &m = matrix->m;
    if (level >= uint32_t(m.levels) || int(level) < m.plan.top_level) return K2_E_INVALID_ARG;
    const uint64_t nw = (m.nodes[level] + 15) / 16;
    if (n_words < nw) return K2_E_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (nw) HIP_TRY(hipMemcpyAsync(words, m.dev.words[level], nw * 8, hipMemcpyDeviceToHost, st),
                    "read tree");
    HIP_TRY(hipStreamSynchronize(st), "read tree");
    std::fill(words + nw, words + n_words, 0ull);
    return K2_OK;
}

k2_status k2_matrix_cached_blocks(const k2_matrix *matrix, uint64_t *blocks, uint64_t n_blocks,
                                  void *stream) {
    if (!matrix || !blocks) return K2_E_INVALID_ARG;
    const Matrix &m = matrix->m;
    if (!m.cached) return K2_E_INVALID_ARG;
    const uint64_t n = m.nodes[m.levels - 2];
    if (n_blocks < n) return K2_E_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    HIP_TRY(hipMemcpyAsync(blocks, m.d_cached, n * 8, hipMemcpyDeviceToHost, st), "read blocks");
    HIP_TRY(hipStreamSynchronize(st), "read blocks");
    return K2_OK;
}

namespace {

// Workspace of a search: frontier, reached set and product output (n W
// words each), the per-level count, the sources.
// Search workspace: F, V, y and the kBfsPlanes level planes (n W words
// each, contiguous: the init kernel clears them at once), the level count
// and the sources.
struct BfsSpace {
    uint64_t words_off[3 + kBfsPlanes], count_off, src_off, bytes;
};

BfsSpace bfs_space(uint64_t n, uint32_t S) {
    const uint64_t W = (uint64_t(S) + 31) / 32;
    auto a256 = [](uint64_t v) { return (v + 255) & ~uint64_t(255); };
    BfsSpace b{};
    uint64_t off = 0;
    for (uint32_t k = 0; k < 3 + kBfsPlanes; ++k) {
        b.words_off[k] = off;
        off += n * W * 4;
    }
    off = a256(off);
    b.count_off = off;
    off = a256(off + 8);
    b.src_off = off;
    b.bytes = a256(off + uint64_t(S) * 4);
    return b;
}

}  // namespace

k2_status k2_bfs_workspace_bytes(const k2_matrix *matrix, uint32_t n_sources, uint64_t *bytes) {
    if (!matrix || !bytes || n_sources == 0) return K2_E_INVALID_ARG;
    *bytes = bfs_space(matrix->m.n_rows, n_sources).bytes;
    return K2_OK;
}

namespace {

// Arguments of a search, checked on the host before anything runs.
k2_status bfs_check(k2_matrix *matrix, k2_direction direction, const uint32_t *sources, uint32_t n_sources,
                    const int32_t *d_dist, const uint32_t *levels) {
    if (!matrix || !sources || n_sources == 0 || !d_dist || !levels) return K2_E_INVALID_ARG;
    if (int(direction) != K2_RIGHT && int(direction) != K2_LEFT) return K2_E_INVALID_ARG;
    const Matrix &m = matrix->m;
    if (m.n_rows != m.n_cols) return K2_E_INVALID_ARG;
    for (uint32_t j = 0; j < n_sources; ++j)
        if (sources[j] >= m.n_rows) return K2_E_INDEX_RANGE;
    return K2_OK;
}

// The search of k2_bfs over a checked workspace of at least
// bfs_space(n, n_sources).bytes bytes.
k2_status bfs_run(Matrix &m, k2_direction direction, const uint32_t *sources, uint32_t n_sources,
                  uint32_t max_levels, int32_t *d_dist, void *d_workspace, void *stream, uint32_t *levels,
                  uint64_t *reached_per_level) {
    const uint64_t n = m.n_rows;
    const BfsSpace sp = bfs_space(n, n_sources);
    const uint32_t W = (n_sources + 31) / 32;
    char *ws = static_cast<char *>(d_workspace);
    uint32_t *F = reinterpret_cast<uint32_t *>(ws + sp.words_off[0]);
    uint32_t *V = reinterpret_cast<uint32_t *>(ws + sp.words_off[1]);
    uint32_t *Y = reinterpret_cast<uint32_t *>(ws + sp.words_off[2]);
    uint32_t *planes = reinterpret_cast<uint32_t *>(ws + sp.words_off[3]);
    auto *count = reinterpret_cast<unsigned long long *>(ws + sp.count_off);
    uint32_t *src = reinterpret_cast<uint32_t *>(ws + sp.src_off);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool empty = m.nodes[m.levels - 2] == 0;
    HIP_TRY(hipMemcpyAsync(src, sources, uint64_t(n_sources) * 4, hipMemcpyHostToDevice, st), "search sources");
    int e = launch_bfs_init(F, (3 + uint64_t(kBfsPlanes)) * n * W, stream);
    if (e == hipSuccess) e = launch_bfs_seed(src, n_sources, W, F, V, stream);
    if (e != hipSuccess) {
        set_hip_error(e, "search init");
        return K2_E_HIP;
    }
    // levels below 2^kBfsPlanes go to the planes; the distance table is
    // written from them once, at the end or before the first deeper level,
    // whose marking then stores distances itself
    bool table = false;
    *levels = 0;
    // (vertex, source) pairs in the frontier: the products list only the
    // cells of frontier rows while fewer than half the rows can hold one
    unsigned long long frontier = n_sources;
    for (uint32_t level = 1; level <= max_levels && level < 0x7FFFFFFFu; ++level) {
        HIP_TRY(hipMemsetAsync(count, 0, 8, st), "search count");
        if (!table && level >= (1u << kBfsPlanes)) {
            e = launch_bfs_dist(d_dist, V, planes, n * W, W, n_sources, stream);
            table = true;
        }
        if (!empty && e == hipSuccess)
            e = m.cached ? launch_cached(m, direction, K2_BOOLEAN_U32X32, W, F, Y, 1, stream, frontier < n / 2)
                         : launch_descent(m, direction, K2_BOOLEAN_U32X32, W, F, Y, nullptr, stream,
                                          frontier < n / 2);
        if (e == hipSuccess)
            e = launch_bfs_mark(Y, V, F, table ? nullptr : planes, d_dist, n * W, W, n_sources, int32_t(level),
                                count, stream);
        if (e != hipSuccess) {
            set_hip_error(e, "search level");
            return K2_E_HIP;
        }
        unsigned long long found = 0;
        HIP_TRY(hipMemcpyAsync(&found, count, 8, hipMemcpyDeviceToHost, st), "search count");
        HIP_TRY(hipStreamSynchronize(st), "search level");
        if (reached_per_level) reached_per_level[level - 1] = found;
        frontier = found;
        if (found == 0) break;
        *levels = level;
    }
    if (!table) {
        e = launch_bfs_dist(d_dist, V, planes, n * W, W, n_sources, stream);
        if (e != hipSuccess) {
            set_hip_error(e, "search distances");
            return K2_E_HIP;
        }
        HIP_TRY(hipStreamSynchronize(st), "search distances");
    }
    return K2_OK;
}

}  // namespace

k2_status k2_bfs(k2_matrix *matrix, k2_direction direction, const uint32_t *sources, uint32_t n_sources,
                 uint32_t max_levels, int32_t *d_dist, void *d_workspace, uint64_t workspace_bytes,
                 void *stream, uint32_t *levels, uint64_t *reached_per_level) {
    k2_status st = bfs_check(matrix, direction, sources, n_sources, d_dist, levels);
    if (st != K2_OK) return st;
    if (!d_workspace) return K2_E_INVALID_ARG;
    const BfsSpace sp = bfs_space(matrix->m.n_rows, n_sources);
    if (workspace_bytes < sp.bytes || (reinterpret_cast<uintptr_t>(d_workspace) & 255)) return K2_E_INVALID_ARG;
    return bfs_run(matrix->m, direction, sources, n_sources, max_levels, d_dist, d_workspace, stream, levels,
                   reached_per_level);
}

k2_status k2_bfs_noalloc(k2_matrix *matrix, k2_direction direction, const uint32_t *sources, uint32_t n_sources,
                         uint32_t max_levels, int32_t *d_dist, void *stream, uint32_t *levels,
                         uint64_t *reached_per_level) {
    k2_status st = bfs_check(matrix, direction, sources, n_sources, d_dist, levels);
    if (st != K2_OK) return st;
    if (bfs_space(matrix->m.n_rows, n_sources).bytes > kNoAllocScratchBytes) return K2_E_UNSUPPORTED;
    void *ws = nullptr;
    const int e = noalloc_scratch(&ws);
    if (e != hipSuccess) {
        set_hip_error(e, "search scratch");
        return K2_E_HIP;
    }
    return bfs_run(matrix->m, direction, sources, n_sources, max_levels, d_dist, ws, stream, levels,
                   reached_per_level);
}

k2_status k2_stream_create(const k2_tree *tree, const k2_plan_opts *opts, uint64_t staging_bytes,
                           k2_stream **out) {
    if (!tree || !out) return K2_E_INVALID_ARG;
    k2_plan_opts o;
    k2_plan_defaults(&o);
    if (opts) o = *opts;
    o.cache_last_level = 0;
    o.offsets = K2_OFFSETS_SCAN;   // every tile carries its own child offsets
    o.window_elems = 0;
    if (!valid_opts(o)) return K2_E_INVALID_ARG;
    const HostTree &t = tree->t;
    const int L = t.levels;
    std::unique_ptr<k2_stream> s(new (std::nothrow) k2_stream);
    if (!s) return K2_E_HOST_OOM;
    s->tree = tree;
    s->tile_nodes = o.tile_nodes;
    if (L < 2 || t.nodes[L - 2] == 0) {   // empty matrix: nothing to stream
        *out = s.release();
        return K2_OK;
    }
    Plan p;
    try {
        k2_status st = make_plan(t, o, &p);
        if (st != K2_OK) return st;
    } catch (const std::bad_alloc &) {
        return K2_E_HOST_OOM;
    }
    s->row_runs = p.row_runs;
    const int last = L - 2;
    auto a256 = [](uint64_t v) { return (v + 255) & ~uint64_t(255); };
    // tile k's node range on every level from its own to the leaves
    auto ranges = [&](size_t k, uint64_t *tlo, uint64_t *thi) {
        const Tile &tl = p.tiles[k];
        uint64_t a = tl.first, b = uint64_t(tl.first) + tl.count;
        for (int d = int(tl.level); d < L; ++d) {
            tlo[d] = a;
            thi[d] = b;
            if (d < L - 1) {
                a = p.tile_bases[tl.base_off + uint32_t(d - int(tl.level))];
                b = child_offset(t, d, b);
            }
        }
    };
    // greedy chunks of consecutive tiles: per level the span of their ranges
    // (plus one word: the leaf reads take the next dword), then the chunk's
    // tiles, codes and scan offsets
    const size_t nt = p.tiles.size();
    uint64_t clo[kMaxLevels], chi[kMaxLevels], tlo[kMaxLevels], thi[kMaxLevels];
    bool used[kMaxLevels];
    auto span_words = [&](int d, uint64_t a, uint64_t b, uint64_t *w0) {
        *w0 = a >> 4;
        return std::min<uint64_t>((b + 15) / 16 + 1, (t.nodes[d] + 15) / 16) - *w0;
    };
    size_t k = 0;
    while (k < nt) {
        std::fill(used, used + kMaxLevels, false);
        uint64_t ncodes = 0, nbases = 0;
        size_t j = k;
        for (; j < nt; ++j) {
            const Tile &tl = p.tiles[j];
            ranges(j, tlo, thi);
            uint64_t bytes = 0;
            for (int d = 0; d < L; ++d) {
                const bool in = d >= int(tl.level);
                if (!used[d] && !in) continue;
                const uint64_t a = !used[d] ? tlo[d] : in ? std::min(clo[d], tlo[d]) : clo[d];
                const uint64_t b = !used[d] ? thi[d] : in ? std::max(chi[d], thi[d]) : chi[d];
                uint64_t w0;
                bytes += a256(8 * span_words(d, a, b, &w0));
            }
            const uint64_t nc = ncodes + tl.count, nb = nbases + uint64_t(last - int(tl.level) + 1);
            bytes += a256(sizeof(Tile) * (j - k + 1)) + a256(8 * nc) + a256(4 * nb);
            if (bytes > staging_bytes / 2) break;   // two halves: copies run one chunk ahead
            for (int d = int(tl.level); d < L; ++d) {
                clo[d] = used[d] ? std::min(clo[d], tlo[d]) : tlo[d];
                chi[d] = used[d] ? std::max(chi[d], thi[d]) : thi[d];
                used[d] = true;
            }
            ncodes = nc;
            nbases = nb;
        }
        if (j == k) return K2_E_ARENA_TOO_SMALL;   // one tile does not fit
        k2_stream::Chunk c;
        c.t0 = k;
        c.t1 = j;
        uint64_t off = 0;
        for (int d = 0; d < kMaxLevels; ++d) {
            c.lo_word[d] = c.n_words[d] = c.word_off[d] = 0;
            if (d >= L || !used[d]) continue;
            c.n_words[d] = span_words(d, clo[d], chi[d], &c.lo_word[d]);
            c.word_off[d] = off;
            off += a256(8 * c.n_words[d]);
        }
        for (size_t q = k; q < j; ++q) {
            Tile tl = p.tiles[q];
            const uint64_t nb = uint64_t(last - int(tl.level) + 1);
            c.codes.insert(c.codes.end(), p.codes.begin() + int64_t(tl.code_off),
                           p.codes.begin() + int64_t(tl.code_off + tl.count));
            c.bases.insert(c.bases.end(), p.tile_bases.begin() + int64_t(tl.base_off),
                           p.tile_bases.begin() + int64_t(tl.base_off + nb));
            tl.code_off = uint32_t(c.codes.size() - tl.count);
            tl.base_off = uint32_t(c.bases.size() - nb);
            c.tiles.push_back(tl);
        }
        c.tiles_off = off;
        off += a256(sizeof(Tile) * c.tiles.size());
        c.codes_off = off;
        off += a256(8 * c.codes.size());
        c.bases_off = off;
        off += a256(4 * c.bases.size());
        c.bytes = off;
        s->max_bytes = std::max(s->max_bytes, off);
        s->staged_bytes += off;
        s->chunks.push_back(std::move(c));
        k = j;
    }
    // the pinned host copy the products copy from (asynchronous copies need
    // page-locked memory); without it they copy from the tree's own words
    uint64_t pin_bytes = 0;
    for (int d = 0; d < L; ++d) {
        s->pin_words[d] = pin_bytes;
        pin_bytes += a256(8 * t.words[d].size());
    }
    for (const k2_stream::Chunk &c : s->chunks) {
        s->pin_meta.push_back(pin_bytes);
        pin_bytes += c.bytes - c.tiles_off;
    }
    void *pin = nullptr;
    if (hipHostMalloc(&pin, pin_bytes, hipHostMallocDefault) == hipSuccess && pin) {
        s->pinned = static_cast<char *>(pin);
        for (int d = 0; d < L; ++d)
            std::memcpy(s->pinned + s->pin_words[d], t.words[d].data(), 8 * t.words[d].size());
        for (size_t q = 0; q < s->chunks.size(); ++q) {
            const k2_stream::Chunk &c = s->chunks[q];
            char *m = s->pinned + s->pin_meta[q];
            std::memcpy(m, c.tiles.data(), sizeof(Tile) * c.tiles.size());
            std::memcpy(m + (c.codes_off - c.tiles_off), c.codes.data(), 8 * c.codes.size());
            std::memcpy(m + (c.bases_off - c.tiles_off), c.bases.data(), 4 * c.bases.size());
        }
    }
    *out = s.release();
    return K2_OK;
}

k2_status k2_stream_info(const k2_stream *s, uint64_t *n_chunks, uint64_t *max_chunk_bytes,
                         uint64_t *staged_bytes) {
    if (!s) return K2_E_INVALID_ARG;
    if (n_chunks) *n_chunks = s->chunks.size();
    if (max_chunk_bytes) *max_chunk_bytes = s->max_bytes;
    if (staged_bytes) *staged_bytes = s->staged_bytes;
    return K2_OK;
}

k2_status k2_stream_chunk(const k2_stream *s, uint64_t chunk, uint64_t *first_tile, uint64_t *end_tile,
                          uint64_t *lo_words, uint64_t *n_words, uint32_t n_levels) {
    if (!s || chunk >= s->chunks.size() || !first_tile || !end_tile) return K2_E_INVALID_ARG;
    const k2_stream::Chunk &c = s->chunks[chunk];
    *first_tile = c.t0;
    *end_tile = c.t1;
    for (uint32_t d = 0; d < n_levels && d < uint32_t(kMaxLevels); ++d) {
        if (lo_words) lo_words[d] = c.lo_word[d];
        if (n_words) n_words[d] = c.n_words[d];
    }
    return K2_OK;
}

k2_status k2_stream_spmv(k2_stream *s, k2_direction direction, k2_semiring semiring, uint32_t batch,
                         int32_t flags, const void *d_x, void *d_y, void *d_staging, uint64_t staging_bytes,
                         void *stream) {
    if (!s || !d_x || !d_y || batch == 0) return K2_E_INVALID_ARG;
    if (int(direction) != K2_RIGHT && int(direction) != K2_LEFT) return K2_E_INVALID_ARG;
    if (int(semiring) < 0 || int(semiring) > 3) return K2_E_INVALID_ARG;
    if ((flags & ~int32_t(K2_SPMV_ACCUMULATE)) != 0) return K2_E_INVALID_ARG;
    if (!s->chunks.empty() && (!d_staging || staging_bytes < 2 * s->max_bytes ||
                               (reinterpret_cast<uintptr_t>(d_staging) & 255)))
        return K2_E_INVALID_ARG;
    const HostTree &t = s->tree->t;
    const uint64_t n_out = direction == K2_RIGHT ? t.n_rows : t.n_cols;
    const uint64_t n_in = direction == K2_RIGHT ? t.n_cols : t.n_rows;
    {   // x and y must not overlap
        const char *xb = static_cast<const char *>(d_x), *yb = static_cast<const char *>(d_y);
        const uint64_t xl = n_in * batch * 4, yl = n_out * batch * 4;
        if (xb < yb + yl && yb < xb + xl) return K2_E_INVALID_ARG;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    int e = hipSuccess;
    if (!(flags & K2_SPMV_ACCUMULATE)) {
        e = launch_fill(d_y, n_out * batch, semiring == K2_TROPICAL_F32 ? 0x7F800000u : 0u, stream);
        if (e != hipSuccess) {
            set_hip_error(e, "fill");
            return K2_E_HIP;
        }
    }
    if (s->chunks.empty()) return K2_OK;
    if (!s->copy_stream) {
        HIP_TRY(hipStreamCreateWithFlags(&s->copy_stream, hipStreamNonBlocking), "stream copies");
        for (hipEvent_t *e : {&s->copied[0], &s->copied[1], &s->done[0], &s->done[1], &s->start})
            HIP_TRY(hipEventCreateWithFlags(e, hipEventDisableTiming), "stream events");
    }
    // the copies start after what the caller queued before this product
    HIP_TRY(hipEventRecord(s->start, st), "stream events");
    HIP_TRY(hipStreamWaitEvent(s->copy_stream, s->start, 0), "stream events");
    char *stage = static_cast<char *>(d_staging);
    for (size_t q = 0; q < s->chunks.size(); ++q) {
        const k2_stream::Chunk &c = s->chunks[q];
        const int h = int(q & 1);
        char *half = stage + uint64_t(h) * s->max_bytes;
        // the half's last kernel (this product's or an earlier one's) is done
        HIP_TRY(hipStreamWaitEvent(s->copy_stream, s->done[h], 0), "stream events");
        DevTree dv{};
        dv.levels = t.levels;
        dv.top_level = 0;
        for (int d = 0; d < t.levels; ++d) {
            dv.nodes[d] = uint32_t(t.nodes[d]);
            if (!c.n_words[d]) continue;
            const void *src = s->pinned ? static_cast<const void *>(s->pinned + s->pin_words[d] + 8 * c.lo_word[d])
                                        : static_cast<const void *>(t.words[d].data() + c.lo_word[d]);
            HIP_TRY(hipMemcpyAsync(half + c.word_off[d], src, 8 * c.n_words[d], hipMemcpyHostToDevice,
                                   s->copy_stream),
                    "stream level words");
            // offset so that the kernels' absolute word indexes land in the staged range
            dv.words[d] = reinterpret_cast<const uint64_t *>(half + c.word_off[d]) - c.lo_word[d];
            dv.words_end[d] = uint32_t(c.lo_word[d] + c.n_words[d]);
        }
        if (s->pinned) {
            HIP_TRY(hipMemcpyAsync(half + c.tiles_off, s->pinned + s->pin_meta[q], c.bytes - c.tiles_off,
                                   hipMemcpyHostToDevice, s->copy_stream),
                    "stream tiles");
        } else {
            HIP_TRY(hipMemcpyAsync(half + c.tiles_off, c.tiles.data(), sizeof(Tile) * c.tiles.size(),
                                   hipMemcpyHostToDevice, s->copy_stream),
                    "stream tiles");
            HIP_TRY(hipMemcpyAsync(half + c.codes_off, c.codes.data(), 8 * c.codes.size(), hipMemcpyHostToDevice,
                                   s->copy_stream),
                    "stream codes");
            HIP_TRY(hipMemcpyAsync(half + c.bases_off, c.bases.data(), 4 * c.bases.size(), hipMemcpyHostToDevice,
                                   s->copy_stream),
                    "stream offsets");
        }
        HIP_TRY(hipEventRecord(s->copied[h], s->copy_stream), "stream events");
        HIP_TRY(hipStreamWaitEvent(st, s->copied[h], 0), "stream events");
        e = launch_descent_tiles(dv, reinterpret_cast<const Tile *>(half + c.tiles_off), c.tiles.size(),
                                 reinterpret_cast<const uint64_t *>(half + c.codes_off),
                                 reinterpret_cast<const uint32_t *>(half + c.bases_off), s->tile_nodes, t.n_rows,
                                 t.n_cols, s->row_runs, direction, semiring, batch, d_x, d_y, stream);
        if (e != hipSuccess) {
            set_hip_error(e, "stream spmv");
            return K2_E_HIP;
        }
        HIP_TRY(hipEventRecord(s->done[h], st), "stream events");
    }
    return K2_OK;
}

void k2_stream_destroy(k2_stream *s) { delete s; }

const char *k2_status_string(k2_status status) {
    switch (status) {
    case K2_OK: return "ok";
    case K2_E_INVALID_ARG: return "invalid argument";
    case K2_E_INDEX_RANGE: return "edge index out of range";
    case K2_E_ARENA_TOO_SMALL: return "device arena smaller than the estimate";
    case K2_E_HOST_OOM: return "host out of memory";
    case K2_E_HIP: return "HIP runtime error";
    case K2_E_UNSUPPORTED: return "unsupported size or option";
    }
    return "unknown status";
}

const char *k2_last_hip_error(void) { return g_hip_error.c_str(); }

}  // extern "C"
