// k2_build.cpp -- host construction of the k^2-tree (k = 2).
//
// Tosoni & Mencagli, "A GPU Engine for Sparse Matrix-Vector Products on
// k^2-Tree-Compressed Graphs", Sec. 2.1: the tree of the recursive 2x2
// decomposition; bit b = 2*b1 + b0 of a node's signature is set iff quadrant b
// (b1: lower rows, b0: right columns) is non-empty; signatures in level order.
// Fig. 1 shows that level order is the order of the nodes' Morton codes, the
// quadrant digits b1b0 of the path from the root.
//
// So the builder sorts the cells by their Morton key (row bit above column bit
// at every level) and reads every level off the sorted, deduplicated keys in
// one pass: the nodes of level d are the distinct key prefixes of d digits,
// and the signature of a node collects digit d of the keys below it.  Between
// two consecutive keys the first differing digit g says which levels start a
// new node (d > g) and which node gains a new bit (d = g).  The pass runs on
// contiguous chunks of keys in parallel; node indices come from per-chunk
// counts, and the words shared by two chunks are merged with atomic or.
// Sec. 5.1 builds on one host core; this builder uses all of them.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <new>
#include <thread>

#include "k2_internal.h"

namespace k2 {

namespace {

template <class F>
void parallel_chunks(int nt, uint64_t n, F f) {
    if (nt <= 1 || n < 4096) {
        f(0, n, 0);
        return;
    }
    std::vector<std::thread> th;
    th.reserve(nt);
    for (int t = 0; t < nt; ++t) {
        uint64_t b = n * uint64_t(t) / uint64_t(nt), e = n * uint64_t(t + 1) / uint64_t(nt);
        th.emplace_back([=] { f(b, e, t); });
    }
    for (auto &x : th) x.join();
}

// bit i of v -> bit 2i
inline uint64_t spread_bits(uint32_t v) {
    uint64_t x = v;
    x = (x | (x << 16)) & 0x0000FFFF0000FFFFull;
    x = (x | (x << 8)) & 0x00FF00FF00FF00FFull;
    x = (x | (x << 4)) & 0x0F0F0F0F0F0F0F0Full;
    x = (x | (x << 2)) & 0x3333333333333333ull;
    x = (x | (x << 1)) & 0x5555555555555555ull;
    return x;
}

struct Buf {
    uint64_t *p = nullptr;
    ~Buf() { std::free(p); }
    bool alloc(uint64_t n) {
        p = static_cast<uint64_t *>(std::malloc((n ? n : 1) * sizeof(uint64_t)));
        return p != nullptr;
    }
};

// LSD radix sort of n keys on their low 'bits' bits, 8 bits per pass.
bool radix_sort(uint64_t *&a, uint64_t n, int bits, int nt) {
    if (n < (1u << 16)) {
        std::sort(a, a + n);
        return true;
    }
    uint64_t *b = static_cast<uint64_t *>(std::malloc(n * sizeof(uint64_t)));
    if (!b) return false;
    std::vector<uint64_t> hist(size_t(nt) * 256);
    for (int shift = 0; shift < bits; shift += 8) {
        std::fill(hist.begin(), hist.end(), 0);
        parallel_chunks(nt, n, [&](uint64_t s, uint64_t e, int t) {
            uint64_t *h = &hist[size_t(t) * 256];
            for (uint64_t i = s; i < e; ++i) h[(a[i] >> shift) & 255]++;
        });
        // skip a pass whose digit is constant
        bool constant = false;
        for (int dgt = 0; dgt < 256 && !constant; ++dgt) {
            uint64_t tot = 0;
            for (int t = 0; t < nt; ++t) tot += hist[size_t(t) * 256 + dgt];
            if (tot == n) constant = true;
        }
        if (constant) continue;
        uint64_t run = 0;
        for (int dgt = 0; dgt < 256; ++dgt)
            for (int t = 0; t < nt; ++t) {
                uint64_t c = hist[size_t(t) * 256 + dgt];
                hist[size_t(t) * 256 + dgt] = run;
                run += c;
            }
        parallel_chunks(nt, n, [&](uint64_t s, uint64_t e, int t) {
            uint64_t *h = &hist[size_t(t) * 256];
            for (uint64_t i = s; i < e; ++i) b[h[(a[i] >> shift) & 255]++] = a[i];
        });
        std::swap(a, b);
    }
    std::free(b);
    return true;
}

}  // namespace

uint64_t child_offset(const HostTree &t, int d, uint64_t i) {
    if (i >= t.nodes[d]) return t.nodes[d + 1];
    uint64_t blk = i / kDirBlock;
    uint64_t acc = t.dir[d][blk];
    const std::vector<uint64_t> &w = t.words[d];
    for (uint64_t k = blk * kWordsPerBlock; k < i / 16; ++k) acc += uint64_t(__builtin_popcountll(w[k]));
    unsigned sh = unsigned(i % 16) * 4;
    if (sh) acc += uint64_t(__builtin_popcountll(w[i / 16] & ((1ull << sh) - 1)));
    return acc;
}

// Directory of every internal level: entry k = set bits in nodes [0, 256k).
static void build_directories(HostTree &t, int nt) {
    t.dir.assign(t.levels > 1 ? t.levels - 1 : 0, {});
    for (int d = 0; d + 1 < t.levels; ++d) {
        uint64_t nb = (t.nodes[d] + kDirBlock - 1) / kDirBlock;
        std::vector<uint32_t> &D = t.dir[d];
        D.assign(nb, 0);
        const std::vector<uint64_t> &w = t.words[d];
        std::vector<uint64_t> blocksum(nb);
        parallel_chunks(nt, nb, [&](uint64_t s, uint64_t e, int) {
            for (uint64_t k = s; k < e; ++k) {
                uint64_t acc = 0;
                uint64_t w0 = k * kWordsPerBlock, w1 = std::min<uint64_t>(w0 + kWordsPerBlock, w.size());
                for (uint64_t j = w0; j < w1; ++j) acc += uint64_t(__builtin_popcountll(w[j]));
                blocksum[k] = acc;
            }
        });
        uint64_t run = 0;
        for (uint64_t k = 0; k < nb; ++k) {
            D[k] = uint32_t(run);
            run += blocksum[k];
        }
    }
}

k2_status build_tree(const uint32_t *rows, const uint32_t *cols, uint64_t m, uint32_t n_rows,
                     uint32_t n_cols, int nt, HostTree *out) {
    HostTree &t = *out;
    t = HostTree();
    t.n_rows = n_rows;
    t.n_cols = n_cols;
    uint32_t dim = std::max(n_rows, n_cols);
    int L = 0;
    while ((1ull << L) < dim) ++L;
    if (L < 2) L = 2;
    t.levels = L;

    // Morton keys, with the range check
    Buf keys;
    if (!keys.alloc(m)) return K2_E_HOST_OOM;
    std::atomic<bool> bad{false};
    parallel_chunks(nt, m, [&](uint64_t s, uint64_t e, int) {
        bool b = false;
        for (uint64_t i = s; i < e; ++i) {
            uint32_t r = rows[i], c = cols[i];
            b |= (r >= n_rows) | (c >= n_cols);
            keys.p[i] = (spread_bits(r) << 1) | spread_bits(c);
        }
        if (b) bad = true;
    });
    if (bad) return K2_E_INDEX_RANGE;
    if (!radix_sort(keys.p, m, 2 * L, nt)) return K2_E_HOST_OOM;

    // deduplicate (parallel: count, then compact)
    uint64_t nnz = 0;
    {
        std::vector<uint64_t> cnt(size_t(nt) + 1, 0);
        parallel_chunks(nt, m, [&](uint64_t s, uint64_t e, int th) {
            uint64_t c = 0;
            for (uint64_t i = s; i < e; ++i) c += (i == 0 || keys.p[i] != keys.p[i - 1]);
            cnt[size_t(th) + 1] = c;
        });
        for (int th = 0; th < nt; ++th) cnt[size_t(th) + 1] += cnt[size_t(th)];
        Buf uniq;
        if (!uniq.alloc(m)) return K2_E_HOST_OOM;
        parallel_chunks(nt, m, [&](uint64_t s, uint64_t e, int th) {
            uint64_t o = cnt[size_t(th)];
            for (uint64_t i = s; i < e; ++i)
                if (i == 0 || keys.p[i] != keys.p[i - 1]) uniq.p[o++] = keys.p[i];
        });
        nnz = cnt[size_t(nt)];
        std::swap(keys.p, uniq.p);
    }
    t.nnz = nnz;

    t.nodes.assign(L, 0);
    t.words.assign(L, {});
    if (nnz == 0) {
        t.nodes[0] = 1;
        t.words[0].assign(1, 0);
        build_directories(t, nt);
        return K2_OK;
    }

    // first differing digit between key i and key i-1 (-1 for the first key)
    auto first_diff = [&](uint64_t i) -> int {
        if (i == 0) return -1;
        uint64_t x = keys.p[i] ^ keys.p[i - 1];
        int hb = 63 - __builtin_clzll(x);
        return (L - 1) - hb / 2;
    };

    int P = (nnz < 4096) ? 1 : nt;
    std::vector<uint64_t> cnt(size_t(P) * L, 0);
    parallel_chunks(P, nnz, [&](uint64_t s, uint64_t e, int p) {
        std::vector<uint64_t> h(size_t(L) + 1, 0);
        for (uint64_t i = s; i < e; ++i) h[size_t(first_diff(i) + 1)]++;
        uint64_t run = 0;
        for (int d = 0; d < L; ++d) {
            run += h[size_t(d)];
            cnt[size_t(p) * L + d] = run;   // keys starting a node of level d
        }
    });
    std::vector<uint64_t> base(size_t(P) * L, 0);
    for (int d = 0; d < L; ++d) {
        uint64_t run = 0;
        for (int p = 0; p < P; ++p) {
            base[size_t(p) * L + d] = run;
            run += cnt[size_t(p) * L + d];
        }
        t.nodes[d] = run;
        if (run >= (1ull << 32)) return K2_E_UNSUPPORTED;
    }
    for (int d = 0; d < L; ++d) {
        uint64_t nw = (t.nodes[d] + 15) / 16;
        try {
            t.words[d].assign(nw, 0);
        } catch (const std::bad_alloc &) {
            return K2_E_HOST_OOM;
        }
    }

    parallel_chunks(P, nnz, [&](uint64_t s, uint64_t e, int p) {
        int64_t cur[kMaxLevels];
        uint64_t acc_w[kMaxLevels], acc_v[kMaxLevels];
        for (int d = 0; d < L; ++d) {
            cur[d] = int64_t(base[size_t(p) * L + d]) - 1;
            acc_w[d] = UINT64_MAX;
            acc_v[d] = 0;
        }
        auto flush = [&](int d) {
            if (acc_w[d] != UINT64_MAX && acc_v[d])
                __atomic_fetch_or(&t.words[d][acc_w[d]], acc_v[d], __ATOMIC_RELAXED);
            acc_v[d] = 0;
        };
        for (uint64_t i = s; i < e; ++i) {
            int g = first_diff(i);
            uint64_t key = keys.p[i];
            for (int d = (g < 0 ? 0 : g); d < L; ++d) {
                if (d > g) ++cur[d];
                unsigned digit = unsigned(key >> (2 * (L - 1 - d))) & 3u;
                uint64_t node = uint64_t(cur[d]);
                uint64_t w = node >> 4;
                if (w != acc_w[d]) {
                    flush(d);
                    acc_w[d] = w;
                }
                acc_v[d] |= uint64_t(1u << digit) << ((node & 15) * 4);
            }
        }
        for (int d = 0; d < L; ++d) flush(d);
    });
    build_directories(t, nt);
    return K2_OK;
}

}  // namespace k2
