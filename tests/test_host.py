"""Host logic of the library, checked on the CPU against the oracle.

* k2_build: every level's packed signatures and the S = 256 directory equal
  the oracle's, on several shapes and densities.
* Tile plans (k2_plan_*): descent tiles and cached-level tiles cover the last
  internal level exactly once, in order; no descent tile's subtree exceeds
  tile_nodes; tile start codes are the Morton codes of their nodes; every
  cell below a windowed tile lies inside its window.
* k2_estimate_device_bytes: the parts add up and follow the sizes of the
  levels, directories and cached codes.
* Errors: out-of-range edges, bad options.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth
import tree_graph_spmv_amd as k2


def rand_edges(seed, n_rows, n_cols, m):
    rng = np.random.default_rng(seed)
    return (rng.integers(0, n_rows, m).astype(np.uint32), rng.integers(0, n_cols, m).astype(np.uint32))


def banded(seed, n, m, width):
    rng = np.random.default_rng(seed)
    r = rng.integers(0, n, m)
    c = np.clip(r + rng.integers(-width, width + 1, m), 0, n - 1)
    far = rng.random(m) < 0.1
    c[far] = rng.integers(0, n, far.sum())
    return r.astype(np.uint32), c.astype(np.uint32)


CASES = {
    "rmat12": lambda: (*synth.rmat(12, 32768, seed=12), 4096, 4096),
    "rmat14": lambda: (*synth.rmat(14, 200000, seed=4), 2 ** 14, 2 ** 14),
    "banded": lambda: (*banded(3, 50000, 300000, 300), 50000, 50000),
    "rect": lambda: (*rand_edges(5, 3000, 700, 20000), 3000, 700),
    "tiny": lambda: (np.array([0, 1, 2], np.uint32), np.array([2, 0, 1], np.uint32), 3, 3),
    "dense64": lambda: (*[a.ravel().astype(np.uint32) for a in np.meshgrid(np.arange(64), np.arange(64),
                                                                             indexing="ij")], 64, 64),
}


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    r, c, nr, nc = CASES[request.param]()
    return request.param, r, c, nr, nc, k2.Tree(r, c, nr, nc), oracle.OracleTree(r, c, nr, nc)


def test_build_threads(case):
    """The tree does not depend on how many threads build it."""
    name, r, c, nr, nc, t, o = case
    for th in (1, 3):
        t1 = k2.Tree(r, c, nr, nc, n_threads=th)
        assert t1.level_nodes() == t.level_nodes()
        for d in range(t.levels):
            assert np.array_equal(t1.level_words(d), t.level_words(d)), (name, th, d)


def test_build_matches_oracle(case):
    name, r, c, nr, nc, t, o = case
    assert t.levels == o.levels and t.nnz == o.nnz
    assert t.level_nodes() == o.level_nodes()
    for d in range(t.levels):
        assert np.array_equal(t.level_words(d), o.level_words(d)), (name, d)
    for d in range(t.levels - 1):
        assert np.array_equal(t.directory(d).astype(np.uint64), o.directory(d, 256)), (name, d)


def oracle_codes(o, upto):
    """Morton codes of every level 0..upto, by expanding the oracle's tree."""
    codes = [np.zeros(1, np.uint64)]
    for d in range(upto):
        sig = o.signatures(d)
        nxt = []
        for i, s in enumerate(sig.tolist()):
            for b in range(4):
                if s >> b & 1:
                    nxt.append((int(codes[d][i]) << 2) | b)
        codes.append(np.array(nxt, np.uint64))
    return codes


def check_xcd_order(ordered, plain):
    """An XCD-ordered tile list holds the plain list's tiles once each; the
    tiles at positions k, k + 8, ... (XCD k) keep the plain order; every
    other entry is padding (count 0, not a band's owner)."""
    assert len(ordered) % 8 == 0
    index = {tuple(int(v) for v in tl): i for i, tl in enumerate(plain)}
    assert len(index) == len(plain)
    seen = []
    for k in range(8):
        pos = [index[tuple(int(v) for v in tl)] for tl in ordered[k::8] if int(tl[1]) or int(tl[3])]
        assert pos == sorted(pos), "an XCD's tiles keep the plain order"
        seen += pos
    assert sorted(seen) == list(range(len(plain)))


def check_plan(o, cells_r, cells_c, top, tiles, codes, cached, opts, all_codes, strays=None):
    """cached: {1: (tiles, ranges) of right products, 2: of left products};
    strays: {1: stray segments of right products, 2: of left products}."""
    L = o.levels
    last = L - 2
    nodes = o.level_nodes()
    offs = [o.child_offsets(d) for d in range(L - 1)]

    def down(d, i):
        while d < last:
            i = int(offs[d][i]) if i < nodes[d] else nodes[d + 1]
            d += 1
        return i

    # cells of the last-internal-level range [a, b): leaves [off(a), off(b)),
    # whose cells come consecutively in the oracle's enumeration
    leaf_pop = np.array([bin(int(s)).count("1") for s in o.signatures(L - 1)], np.int64)

    def leaf_of(i):   # first child of node i of the last internal level
        return int(offs[last][i]) if i < nodes[last] else nodes[L - 1]
    cell_start = np.concatenate([[0], np.cumsum(leaf_pop)])

    def cells_of(a, b):
        la = int(offs[last][a]) if a < nodes[last] else nodes[L - 1]
        lb = int(offs[last][b]) if b < nodes[last] else nodes[L - 1]
        return cells_r[cell_start[la]:cell_start[lb]], cells_c[cell_start[la]:cell_start[lb]]

    def side_of(tl):
        side = 1 << int(tl[6])
        assert side * opts.window_batch <= max(opts.window_elems, 1)
        return side

    spans = []
    for tl in tiles:
        first, count, level = int(tl[0]), int(tl[1]), int(tl[2])
        assert count >= 1, "descent tiles are never padded"
        assert top <= level <= last
        a, b = down(level, first), down(level, first + count)
        assert b - a <= opts.tile_nodes
        spans.append((a, b))
        got = codes[int(tl[3]):int(tl[3]) + count]
        assert np.array_equal(got, all_codes[level][first:first + count])
        if tl[6] != 0xFFFFFFFF:   # a descent window (kernels accept them) is the whole quadrant
            side = side_of(tl)
            rr, cc = cells_of(a, b)
            assert np.all((rr >= tl[4]) & (rr < tl[4] + side)), "cell row outside window"
            assert np.all((cc >= tl[5]) & (cc < tl[5] + side)), "cell column outside window"
    assert spans == sorted(spans), "descent tiles must follow each other in Z order"
    pos = 0
    for a, b in sorted(spans):
        assert a == pos, "descent tiles must cover the last internal level exactly once"
        pos = b
    assert pos == nodes[last]
    for which, (ctiles, ranges) in cached.items():
        seen = []
        owners = set()
        per_band = {}
        for tl in ctiles:
            assert int(tl[3]) in (0, 1, 2, 3)
            if tl[6] != 0xFFFFFFFF:
                band = (int(tl[4]) if which == 1 else int(tl[5])) >> int(tl[6])
                per_band[band] = per_band.get(band, 0) + 1
            if int(tl[3]) & 1:   # a band's owner tile: windowed, one per band
                assert tl[6] != 0xFFFFFFFF
                assert band not in owners, "one owner tile per band"
                owners.add(band)
        if owners:   # with strays every band has an owner (up to 2^20 bands)
            log2 = int(next(tl[6] for tl in ctiles if int(tl[3]) & 1))
            n_out = (cells_r.max() if which == 1 else cells_c.max()) + 1
            assert owners >= set(range(int(n_out - 1) >> log2)), "a band without an owner tile"
        for tl in ctiles:   # bit 1: the only tile of its band
            if int(tl[3]) & 2:
                assert tl[6] != 0xFFFFFFFF
                band = (int(tl[4]) if which == 1 else int(tl[5])) >> int(tl[6])
                assert per_band[band] == 1
            elif tl[6] != 0xFFFFFFFF and owners:
                band = (int(tl[4]) if which == 1 else int(tl[5])) >> int(tl[6])
                assert per_band[band] > 1, "a band's only tile is marked"
        for tl in ctiles:
            first, count = int(tl[0]), int(tl[1])
            assert int(tl[2]) == last
            if count == 0:
                assert (opts.xcd_remap and tl[6] == 0xFFFFFFFF) or int(tl[3]) & 1
                continue
            total = 0
            for r, leaf in ranges[first:first + count]:
                lo, n = int(r) >> 32, int(r) & 0xFFFFFFFF
                assert 1 <= n <= 64
                assert int(leaf) == leaf_of(lo), "first leaf of a segment"
                seen.append((lo, n))
                total += n
                if tl[6] != 0xFFFFFFFF:   # a band window covers the output coordinate
                    side = side_of(tl)
                    rr, cc = cells_of(lo, lo + n)
                    out, base = (rr, tl[4]) if which == 1 else (cc, tl[5])
                    assert np.all((out >= base) & (out < base + side)), "output outside band"
            if tl[6] != 0xFFFFFFFF:
                assert total <= 65536
        stray = strays[which] if strays else np.zeros((0, 2), np.uint64)
        if len(stray):
            log2 = int(next(tl[6] for tl in ctiles if int(tl[3]) & 1))
        for r, leaf in stray:   # each stray's band has an owner tile
            lo, n = int(r) >> 32, int(r) & 0xFFFFFFFF
            assert 1 <= n <= 64
            assert int(leaf) == leaf_of(lo), "first leaf of a stray segment"
            seen.append((lo, n))
            for i in range(lo, lo + n):
                rr, cc = cells_of(i, i + 1)
                out = (rr if which == 1 else cc) >> log2
                assert len(out) and np.all(out == out[0]) and int(out[0]) in owners, "stray without owner"
        seen.sort()
        pos = 0
        for lo, n in seen:
            assert lo == pos, "cached ranges must cover the level exactly once"
            pos = lo + n
        assert pos == nodes[last]


@pytest.mark.parametrize("opt", [
    dict(),
    dict(xcd_remap=0),
    dict(xcd_remap=1, window_elems=0),
    dict(window_elems=8192),
    dict(tile_nodes=256, window_elems=1024, window_batch=1),
    dict(tile_nodes=4096, window_elems=16384, window_batch=1),
    dict(window_elems=0),
    dict(host_top_max=4, window_elems=8192, window_batch=64),
    dict(host_top_max=1 << 20, window_elems=2048, window_batch=2),
    dict(band_strays=0),
    dict(band_strays=0, window_elems=1024, window_batch=1),
])
def test_plan_invariants(case, opt):
    name, r, c, nr, nc, t, o = case
    opts = k2.plan_defaults(cache_last_level=1, **opt)
    top, tiles, codes = t.plan(opts, 0)
    cached = {w: t.plan(opts, w)[1:] for w in (1, 2)}
    strays = {w: t.plan(opts, w + 8)[2] for w in (1, 2)}
    assert all(len(t.plan(k2.plan_defaults(cache_last_level=0, **opt), w)[1]) == 0 for w in (1, 2))
    assert all(len(t.plan(k2.plan_defaults(cache_last_level=0, **opt), w)[2]) == 0 for w in (9, 10))
    if o.level_nodes()[o.levels - 2] == 0:
        assert len(tiles) == 0 and all(len(v[0]) == 0 for v in cached.values())
        return
    cr, cc = o.cells()
    all_codes = oracle_codes(o, o.levels - 2)
    check_plan(o, cr.astype(np.int64), cc.astype(np.int64), top, tiles, codes, cached, opts,
               all_codes, strays)
    if opts.xcd_remap:
        plain = k2.plan_defaults(cache_last_level=1, **dict(opt, xcd_remap=0))
        assert np.array_equal(tiles, t.plan(plain, 0)[1]), "XCD order leaves descent tiles alone"
        for w in (1, 2):
            ptiles = t.plan(plain, w)[1]
            check_xcd_order(cached[w][0], ptiles)


def test_scan_offsets(case):
    """With scan offsets each descent tile carries its first node's first
    child on every level it spans; they equal the oracle's child offsets
    followed down from the tile's first node."""
    name, r, c, nr, nc, t, o = case
    L = o.levels
    nodes = o.level_nodes()
    offs = [o.child_offsets(d) for d in range(L - 1)]
    for tile_nodes in (256, 4096):
        opts = k2.plan_defaults(tile_nodes=tile_nodes, offsets="scan")
        top, tiles, codes = t.plan(opts, 0)
        bases = t.plan_offsets(opts)
        used = np.zeros(bases.size, bool)
        # descent tiles, rest tiles of both directions (copies of one cut,
        # sharing its offsets), band tiles
        lists = [tiles] + [t.plan(opts, w)[1] for w in (3, 4, 7, 8)]
        for lst in lists:
            for tl in lst:
                level, first, at = int(tl[2]), int(tl[0]), int(tl[7])
                node = first
                for d in range(level, L - 1):
                    node = int(offs[d][node]) if node < nodes[d] else nodes[d + 1]
                    assert int(bases[at + d - level]) == node, (name, d)
                used[at:at + L - 1 - level] = True
        assert used.sum() <= bases.size
        dir_opts = k2.plan_defaults(tile_nodes=tile_nodes, offsets="directory")
        assert np.array_equal(t.plan(dir_opts, 0)[1][:, :7], tiles[:, :7])
        assert np.all(t.plan(dir_opts, 0)[1][:, 7] == 0)


@pytest.mark.parametrize("opt", [dict(), dict(window_elems=0), dict(window_elems=1024, window_batch=1),
                                 dict(tile_nodes=256), dict(host_top_max=4)])
def test_tree_only_plan(case, opt):
    """Tree-only products, per direction: the band groups' tiles (with their
    band window) and the rest tiles minus their skip ranges cover the last
    internal level exactly once; a band tile's outputs lie in its window and
    its subtree holds at most min(tile_nodes, 256) nodes per level and lies
    in one window quadrant (band kernels keep quadrant-relative codes); rest
    tiles come in output-block order (2^k * window_batch * 4 the largest
    power of 2 <= 16 MB) and, their skips ignored (a tile the groups cover
    whole has skip count 0xFFFFFFFF), are the whole second cut: they too
    cover the level exactly once."""
    name, r, c, nr, nc, t, o = case
    opts = k2.plan_defaults(**opt)
    L = o.levels
    last = L - 2
    nodes = o.level_nodes()
    if nodes[last] == 0:
        return
    offs = [o.child_offsets(d) for d in range(L - 1)]

    def down(d, i):
        while d < last:
            i = int(offs[d][i]) if i < nodes[d] else nodes[d + 1]
            d += 1
        return i
    cr, cc = o.cells()
    leaf_pop = np.array([bin(int(s)).count("1") for s in o.signatures(L - 1)], np.int64)
    cell_start = np.concatenate([[0], np.cumsum(leaf_pop)])

    def cells_of(a, b):
        la = int(offs[last][a]) if a < nodes[last] else nodes[L - 1]
        lb = int(offs[last][b]) if b < nodes[last] else nodes[L - 1]
        return cr[cell_start[la]:cell_start[lb]], cc[cell_start[la]:cell_start[lb]]
    all_codes = oracle_codes(o, last)
    _, _, codes = t.plan(opts, 0)
    cap = min(opts.tile_nodes, 256)
    wb = max(opts.window_batch, 1)
    kb = 0
    while kb < 30 and (2 << kb) * wb * 4 <= (16 << 20):
        kb += 1
    for w, out_is_row in ((0, True), (1, False)):
        covered = []
        groups = t.plan(opts, 5 + w)[1]
        sub = t.plan(opts, 7 + w)[1]
        assert sum(int(g[1]) for g in groups) == len(sub)
        for g in groups:
            side = 1 << int(g[6])
            base = int(g[4]) if out_is_row else int(g[5])
            for tl in sub[int(g[0]):int(g[0]) + int(g[1])]:
                first, count, level = int(tl[0]), int(tl[1]), int(tl[2])
                assert np.array_equal(codes[int(tl[3]):int(tl[3]) + count], all_codes[level][first:first + count])
                a, b = down(level, first), down(level, first + count)
                assert b - a <= cap
                rr, ccc = cells_of(a, b)
                out = rr if out_is_row else ccc
                assert np.all((out >= base) & (out < base + side)), "band output outside its window"
                assert len(np.unique(rr // side)) <= 1 and len(np.unique(ccc // side)) <= 1, "sub-tile spans quadrants"
                covered.append((a, b))
        _, rest, skips = t.plan(opts, 3 + w)
        keys, spans = [], []
        for tl in rest:
            first, count, level = int(tl[0]), int(tl[1]), int(tl[2])
            a, b = down(level, first), down(level, first + count)
            assert b - a <= cap, "a rest tile holds at most min(tile_nodes, 256) nodes per level"
            assert np.array_equal(codes[int(tl[3]):int(tl[3]) + count], all_codes[level][first:first + count])
            code = int(codes[int(tl[3])])
            coord = 0
            for k in range(level):
                coord |= ((code >> (2 * k + (1 if out_is_row else 0))) & 1) << k
            keys.append((coord << (L - level)) >> kb)
            spans.append((a, b))
            if int(tl[5]) == 0xFFFFFFFF:   # the groups cover it whole
                assert groups.size and b > a
                continue
            pos = a
            for sk in skips[int(tl[4]):int(tl[4]) + int(tl[5])]:
                lo, hi = int(sk) >> 32, int(sk) & 0xFFFFFFFF
                assert a <= lo < hi <= b and lo >= pos
                if lo > pos:
                    covered.append((pos, lo))
                pos = hi
            if pos < b:
                covered.append((pos, b))
            assert int(tl[5]) == 0 or (b - a) > sum((int(x) & 0xFFFFFFFF) - (int(x) >> 32)
                                                    for x in skips[int(tl[4]):int(tl[4]) + int(tl[5])])
        assert keys == sorted(keys)
        for items in (covered, spans):
            items.sort()
            pos = 0
            for a, b in items:
                assert a == pos, (name, w, "tree-only items must cover the level exactly once")
                pos = b
            assert pos == nodes[last]


def test_top_level(case):
    name, r, c, nr, nc, t, o = case
    nodes = o.level_nodes()
    for cap in (1, 4, 100, 1 << 16):
        top, *_ = t.plan(k2.plan_defaults(host_top_max=cap))
        want = max(d for d in range(o.levels - 1) if nodes[d] <= cap)
        assert top == want


def test_estimate_parts(case):
    name, r, c, nr, nc, t, o = case
    nodes = o.level_nodes()
    for cached, offsets in ((0, "scan"), (1, "scan"), (0, "directory"), (1, "directory")):
        opts = k2.plan_defaults(cache_last_level=cached, offsets=offsets)
        est = t.estimate(opts, semiring="plus_times", batch=3)
        top, tiles, codes = t.plan(opts, 0)
        extra = sum(32 * len(t.plan(opts, w)[1]) + 16 * len(t.plan(opts, w)[2]) for w in (1, 2))
        stray_tiles = stray_records = 0
        for w in (1, 2):   # strays: segments, band offsets and cursors; 8-byte records
            owners = [tl for tl in t.plan(opts, w)[1] if int(tl[3]) & 1]
            segs = t.plan(opts, w + 8)[2]
            if owners:
                log2 = int(owners[0][6])
                nb = ((nr if w == 1 else nc) + (1 << log2) - 1) >> log2
                stray_tiles += 16 * len(segs) + 4 * (nb + 1) + 4 * nb
                stray_records += 8 * sum(int(r) & 0xFFFFFFFF for r, _ in segs)
            else:
                assert len(segs) == 0
        L = o.levels
        assert est["tree"] == sum(8 * ((nodes[d] + 15) // 16) for d in range(top, L))
        if offsets == "directory":
            assert est["directory"] == sum(4 * ((nodes[d] + 255) // 256) for d in range(top, L - 1))
            assert t.plan_offsets(opts).size == 0
        else:
            assert est["directory"] == 4 * t.plan_offsets(opts).size
        assert est["top_codes"] == 8 * len(codes)
        # descent tiles, the tree-only lists (the rest tiles once at 16
        # bytes, per direction their order at 4 bytes and, with band groups,
        # a 16-byte entry per rest tile the groups leave), the cached tiles
        n_rest = len(t.plan(opts, 3)[1])
        tree_only = 16 * n_rest + sum(4 * n_rest + 32 * (len(t.plan(opts, 5 + w)[1]) + len(t.plan(opts, 7 + w)[1])) +
                                      8 * len(t.plan(opts, 3 + w)[2]) for w in (0, 1))
        for w in (0, 1):
            assert len(t.plan(opts, 3 + w)[1]) == n_rest
            if len(t.plan(opts, 5 + w)[1]):
                tree_only += 16 * sum(int(tl[5]) != 0xFFFFFFFF for tl in t.plan(opts, 3 + w)[1])
        # cached: plus 4 bytes of creation status
        assert est["tiles"] == 32 * len(tiles) + tree_only + (extra + stray_tiles + 4 if cached else 0)
        assert est["cached_codes"] == (12 * nodes[L - 2] + stray_records if cached else 0)
        parts = sum(est[k] for k in ("tree", "directory", "top_codes", "tiles", "cached_codes",
                                     "scratch", "alignment"))
        assert est["arena"] == parts and est["arena"] % 256 == 0
        assert est["vectors"] == (nr + nc) * 3 * 4
        assert est["total"] == est["arena"] + est["vectors"]


def test_errors():
    with pytest.raises(k2.K2Error) as e:
        k2.Tree([5], [0], 5, 5)
    assert e.value.status == k2.K2_E_INDEX_RANGE
    with pytest.raises(k2.K2Error) as e:
        k2.Tree([0], [0], 0, 5)
    assert e.value.status == k2.K2_E_INVALID_ARG
    t = k2.Tree([0, 1], [1, 0], 2, 2)
    for bad in (dict(tile_nodes=100), dict(tile_nodes=3000), dict(tile_nodes=8192),
                dict(window_elems=1 << 15)):
        with pytest.raises(k2.K2Error) as e:
            t.estimate(k2.plan_defaults(**bad))
        assert e.value.status == k2.K2_E_INVALID_ARG
    with pytest.raises(k2.K2Error):
        t.estimate(batch=0)


def test_threads_do_not_change_the_tree():
    r, c = synth.rmat(13, 60000, seed=8)
    t1 = k2.Tree(r, c, 8192, 8192, n_threads=1)
    t7 = k2.Tree(r, c, 8192, 8192, n_threads=7)
    for d in range(t1.levels):
        assert np.array_equal(t1.level_words(d), t7.level_words(d))


def test_stream_chunks(case):
    """Out-of-core plans: the chunks take the depth-first descent tiles in
    order, each fits the staging size, and every level range of a chunk's
    tiles lies inside the node words staged for that level (the leaf level
    one word beyond, for the reads of a node's next leaf dword)."""
    name, r, c, nr, nc, t, o = case
    L = o.levels
    last = L - 2
    nodes = o.level_nodes()
    if nodes[last] == 0:
        return
    offs = [o.child_offsets(d) for d in range(L - 1)]

    def down(d, i, to):
        while d < to:
            i = int(offs[d][i]) if i < nodes[d] else nodes[d + 1]
            d += 1
        return i
    opts = k2.plan_defaults(offsets="scan")
    _, tiles, _ = t.plan(opts, 0)
    for staging in (1 << 14, 1 << 16, 1 << 22):
        try:
            s = k2.Streamed(t, staging, opts)
        except k2.K2Error as e:
            assert e.status == k2.K2_E_ARENA_TOO_SMALL and staging == 1 << 14
            continue
        assert 2 * s.max_chunk_bytes <= staging and s.n_chunks >= 1
        pos = 0
        for ch in range(s.n_chunks):
            a, b, lo, nw = s.chunk(ch, L)
            assert a == pos and b > a
            pos = b
            for tl in tiles[a:b]:
                first, count, level = int(tl[0]), int(tl[1]), int(tl[2])
                for d in range(level, L):
                    x0, x1 = down(level, first, d), down(level, first + count, d)
                    if x1 == x0:
                        continue
                    w0, w1 = int(lo[d]), int(lo[d]) + int(nw[d])
                    assert w0 * 16 <= x0 and (x1 - 1) // 16 < w1, (name, staging, ch, d)
                    if d == L - 1:   # the next leaf dword of the last leaf
                        assert w1 == (nodes[d] + 15) // 16 or (x1 - 1) // 16 + 1 < w1
        assert pos == len(tiles), (name, staging)


def test_stream_arguments():
    """k2_stream_spmv refuses bad arguments before touching the device:
    a staging buffer under two chunks, an unaligned one, overlapping x and
    y, an unknown direction, semiring or flag."""
    rows, cols, n = synth.workload_edges("rmat_s12_e32k")
    t = k2.Tree(rows, cols, n, n)
    s = k2.Streamed(t, 1 << 16)
    lib = k2.lib()
    VP = ctypes.c_void_p
    x, y, stage = VP(1 << 20), VP(1 << 30), VP(1 << 34)
    need = 2 * s.max_chunk_bytes

    def call(direction=k2.K2_RIGHT, semiring=0, batch=1, flags=0, xp=x, yp=y, sp=stage, sb=need):
        return lib.k2_stream_spmv(s._h, direction, semiring, batch, flags, xp, yp, sp, sb, None)
    assert call(sb=need - 256) == k2.K2_E_INVALID_ARG
    assert call(sp=VP((1 << 34) + 64)) == k2.K2_E_INVALID_ARG
    assert call(yp=VP((1 << 20) + 64)) == k2.K2_E_INVALID_ARG
    assert call(direction=7) == k2.K2_E_INVALID_ARG
    assert call(semiring=9) == k2.K2_E_INVALID_ARG
    assert call(flags=0x2) == k2.K2_E_INVALID_ARG
    assert call(batch=0) == k2.K2_E_INVALID_ARG
    with pytest.raises(k2.K2Error):
        k2.Streamed(t, 1 << 10)


def test_spmv_refuses_host_vectors():
    """Matrix.spmv and Streamed.spmv refuse vectors that are not on the
    product's device before anything reaches the library (a host pointer
    handed to a kernel would fault the GPU instead of raising)."""
    torch = pytest.importorskip("torch")
    m = k2.Matrix.__new__(k2.Matrix)   # no device needed: the checks run first
    m.n_rows = m.n_cols = 16
    m.device = torch.device("meta")
    m._h = None
    x = torch.empty(16, device="meta")
    with pytest.raises(ValueError, match="y is not on the matrix's device"):
        m.spmv(x, torch.empty(16))
    with pytest.raises(ValueError, match="x is not on the matrix's device"):
        m.spmv(torch.empty(16), torch.empty(16, device="meta"))
    rows, cols, n = synth.workload_edges("rmat_s12_e32k")
    s = k2.Streamed(k2.Tree(rows, cols, n, n), 1 << 16)
    with pytest.raises(ValueError, match="device tensor"):
        s.spmv(torch.empty(n), torch.empty(n))


def test_band_tile_cap_splits_bands():
    """band_tile_nodes cuts a band's dense quadrants into several cached
    tiles: on a web-like 2^14 graph with 64 nodes per tile every band has
    many tiles, none of them its band's only tile (so products fill y and
    the tiles add their windows), and exactly one per band owns the band's
    strays; the default cap leaves one tile per band."""
    n = 2 ** 14
    rows, cols = synth.web(n, 16, window=1024, p_local=0.8, seed=7)
    t = k2.Tree(rows, cols, n, n)
    for which in (1, 2):
        _, tiles, _ = t.plan(k2.plan_defaults(cache_last_level=1, band_tile_nodes=64), which=which)
        win = tiles[:, 6] != 0xFFFFFFFF
        field = 4 if which == 1 else 5
        band = tiles[win, field] >> tiles[win, 6]
        _, per = np.unique(band, return_counts=True)
        assert per.size >= 16 and per.min() > 1
        assert not (tiles[:, 3] & 2).any()
        owners = band[(tiles[win, 3] & 1) != 0]
        assert np.array_equal(np.sort(owners), np.unique(band))
        _, tiles, _ = t.plan(k2.plan_defaults(cache_last_level=1), which=which)
        win = tiles[:, 6] != 0xFFFFFFFF
        assert ((tiles[win, 3] & 2) != 0).all()
    with pytest.raises(k2.K2Error):
        t.estimate(k2.plan_defaults(band_tile_nodes=63))


def _spread(v):
    v = v.astype(np.uint64)
    out = np.zeros_like(v)
    for b in range(32):
        out |= ((v >> np.uint64(b)) & np.uint64(1)) << np.uint64(2 * b)
    return out


def _compact(m):
    out = np.zeros_like(m)
    for b in range(32):
        out |= ((m >> np.uint64(2 * b)) & np.uint64(1)) << np.uint64(b)
    return out


@pytest.mark.parametrize("name", ["web14", "banded", "rmat14"])
@pytest.mark.parametrize("cap", [65536, 64])
def test_cached_segments_in_one_quadrant(name, cap):
    """The packed node words rest on the plan cutting every windowed cached
    tile's segments inside one Q x Q quadrant of the tile's band (Sec. 3.4
    tiles over a band's dense quadrants): checked against the nodes of level
    l-2 rebuilt from the edges (the distinct 4x4 blocks in Morton order)."""
    if name == "web14":
        n = 2 ** 14
        r, c = synth.web(n, 16, window=1024, p_local=0.8, seed=7)
        nr = nc = n
    else:
        r, c, nr, nc = CASES[name]()
    t = k2.Tree(r, c, nr, nc)
    blocks = np.unique((_spread(r.astype(np.uint64) >> np.uint64(2)) << np.uint64(1)) |
                       _spread(c.astype(np.uint64) >> np.uint64(2)))
    assert blocks.size == t.level_nodes()[t.levels - 2]
    row0 = (_compact(blocks >> np.uint64(1)) * 4).astype(np.int64)
    col0 = (_compact(blocks) * 4).astype(np.int64)
    opts = k2.plan_defaults(cache_last_level=1, band_tile_nodes=cap)
    checked = 0
    for which in (1, 2):
        _, tiles, segs = t.plan(opts, which=which)
        lo = (segs[:, 0] >> np.uint64(32)).astype(np.int64)
        cnt = (segs[:, 0] & np.uint64(0xFFFFFFFF)).astype(np.int64)
        for tl in tiles:
            if int(tl[6]) == 0xFFFFFFFF or int(tl[1]) == 0:
                continue
            q = 1 << int(tl[6])
            band0 = int(tl[4]) if which == 1 else int(tl[5])
            for k in range(int(tl[0]), int(tl[0]) + int(tl[1])):
                a, b = lo[k], lo[k] + cnt[k]
                qr, qc = row0[a:b] // q, col0[a:b] // q
                assert (qr == qr[0]).all() and (qc == qc[0]).all()
                assert (qr[0] if which == 1 else qc[0]) * q == band0
                checked += 1
    assert checked > 0 or name == "rmat14"
