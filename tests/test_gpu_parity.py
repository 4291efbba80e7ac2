"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Element by element on the same seeded inputs: bit-exact for the tree bits,
the Boolean and the tropical semirings; plus-times within relative 1e-5 of
the oracle's fp64 value (absolute 1e-6 below 0.1).  Covers both directions,
batches, both traversals (tiled descent and cached last level), several tile
sizes, rectangular and degenerate matrices.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from tests.helpers import (ALL_SEMIRINGS, ORC_DIR, ORC_SEMIRING, check_parity, from_device,
                           make_x, to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_graph_spmv_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


PLAN_VARIANTS = (dict(), dict(window_elems=0), dict(host_top_max=4, window_elems=4096, window_batch=4),
                 dict(xcd_remap=0, host_top_max=16), dict(offsets="directory", host_top_max=16),
                 dict(band_strays=0, window_elems=1024, window_batch=1))


def run_all(k2, rows, cols, n_rows, n_cols, dev, semirings=ALL_SEMIRINGS, batches=(1, 3),
            tiles=(256, 2048), modes=("tree", "cached"), seed=0, label="", variants=PLAN_VARIANTS):
    tree = k2.Tree(rows, cols, n_rows, n_cols)
    ref = oracle.OracleTree(rows, cols, n_rows, n_cols)
    assert tree.nnz == ref.nnz
    for d in range(tree.levels):
        assert np.array_equal(tree.level_words(d), ref.level_words(d)), f"{label} level {d}"
    rng = np.random.default_rng(seed)
    for tile, var in itertools.product(tiles, variants):
        opts = k2.plan_defaults(tile_nodes=tile, cache_last_level=1 if "cached" in modes else 0, **var)
        m = k2.Matrix(tree, opts, device=dev)
        for mode, sr, direction, B in itertools.product(modes, semirings, ("right", "left"),
                                                        batches):
            n_in = n_cols if direction == "right" else n_rows
            x = make_x(rng, sr, n_in, B)
            y = m.spmv(to_device(x, dev), direction=direction, semiring=sr, batch=B, mode=mode)
            torch.cuda.synchronize()
            want = ref.spmv(x, ORC_SEMIRING[sr], ORC_DIR[direction], B)
            check_parity(from_device(y, sr), want, sr,
                         f"{label} tile={tile} {var} {mode} {sr} {direction} B={B}")


def test_fig1(dev, fig1):
    import tree_graph_spmv_amd as k2
    pairs = [tuple(int(v) for v in p.split(",")) for p in fig1["cells"].split()]
    r = np.array([p[0] for p in pairs], np.uint32)
    c = np.array([p[1] for p in pairs], np.uint32)
    run_all(k2, r, c, 8, 8, dev, batches=(1, 3, 8), tiles=(256,), label="fig1")


@pytest.mark.parametrize("seed", range(6))
def test_small_random(dev, seed):
    import tree_graph_spmv_amd as k2
    rng = np.random.default_rng(100 + seed)
    n_rows, n_cols = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    density = [0.0, 0.002, 0.02, 0.2, 0.7, 1.0][seed]
    mask = rng.random((n_rows, n_cols)) < density
    r, c = np.nonzero(mask)
    run_all(k2, r.astype(np.uint32), c.astype(np.uint32), n_rows, n_cols, dev,
            batches=(1, 2, 5, 64, 70), seed=seed, label=f"random{seed}")


def test_degenerate(dev):
    import tree_graph_spmv_amd as k2
    # empty, single cell in a corner, identity, all-ones
    run_all(k2, np.zeros(0, np.uint32), np.zeros(0, np.uint32), 5, 7, dev, label="empty")
    run_all(k2, np.array([1000], np.uint32), np.array([3], np.uint32), 1001, 4, dev,
            label="single")
    idx = np.arange(777, dtype=np.uint32)
    run_all(k2, idx, idx, 777, 777, dev, label="identity")
    rr, cc = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    run_all(k2, rr.ravel().astype(np.uint32), cc.ravel().astype(np.uint32), 64, 64, dev,
            label="dense")


def test_rmat_s12_e32k(dev):
    """R-MAT 2^12, 32,768 distinct edges: the whole product, every variant."""
    import tree_graph_spmv_amd as k2
    rows, cols, n = synth.workload_edges("rmat_s12_e32k")
    run_all(k2, rows, cols, n, n, dev, batches=(1, 4), tiles=(256, 1024, 4096),
            label="rmat_s12_e32k")


def test_device_tree_and_cached_blocks(dev):
    """The device copy of every level equals the canonical export, and the
    cached last internal level holds each node's block origin, decoded from
    the Morton code the oracle's signatures give it."""
    import tree_graph_spmv_amd as k2
    rows, cols = synth.rmat(14, 100000, seed=9)
    n = 2 ** 14
    tree = k2.Tree(rows, cols, n, n)
    ref = oracle.OracleTree(rows, cols, n, n)
    nodes = ref.level_nodes()
    m = k2.Matrix(tree, k2.plan_defaults(cache_last_level=1, tile_nodes=512), device=dev)
    for d in range(m.top_level, tree.levels):
        assert np.array_equal(m.device_level_words(d, nodes[d]), ref.level_words(d)), d
    # codes of level l-2 by expanding the oracle's signatures in level order
    codes = np.zeros(1, np.uint64)
    for d in range(tree.levels - 2):
        sig = ref.signatures(d)
        nxt = []
        for i, s in enumerate(sig.tolist()):
            for b in range(4):
                if s >> b & 1:
                    nxt.append((int(codes[i]) << 2) | b)
        codes = np.array(nxt, np.uint64)
    got = m.cached_blocks(nodes[tree.levels - 2])
    row = np.zeros(codes.size, np.uint64)
    col = np.zeros(codes.size, np.uint64)
    for k in range(tree.levels - 2):   # bit 2k + 1 of a code is a row bit, 2k a column bit
        row |= ((codes >> np.uint64(2 * k + 1)) & np.uint64(1)) << np.uint64(k)
        col |= ((codes >> np.uint64(2 * k)) & np.uint64(1)) << np.uint64(k)
    assert np.array_equal(got, ((row * np.uint64(4)) << np.uint64(32)) | (col * np.uint64(4)))


def test_web_n20_d16(dev):
    """Web-like 2^20 (about 15M distinct edges): right and left plus-times,
    tree-only and cached, against the oracle's full product, overwriting y
    and accumulating into it; the tropical and packed Boolean semirings
    tree-only (their 79k rest tiles take several per wave)."""
    import tree_graph_spmv_amd as k2
    rows, cols, n = synth.workload_edges("web_n20_d16")
    tree = k2.Tree(rows, cols, n, n)
    ref = oracle.OracleTree(rows, cols, n, n)
    for d in range(tree.levels):
        assert np.array_equal(tree.level_words(d), ref.level_words(d)), d
    x = synth.workload_x("web_n20_d16", n)
    m = k2.Matrix(tree, k2.plan_defaults(cache_last_level=1), device=dev)
    xd = to_device(x, dev)
    for direction in ("right", "left"):
        want = ref.spmv(x, oracle.PLUS_TIMES, ORC_DIR[direction], 1, threads=16)
        for mode in ("tree", "cached"):
            y = m.spmv(xd, direction=direction, mode=mode)
            torch.cuda.synchronize()
            check_parity(from_device(y, "plus_times"), want, "plus_times",
                         f"web_n20_d16 {direction} {mode}")
            # accumulating into y0: band groups and owner tiles add their
            # windows to what y holds
            y0 = np.random.default_rng(11).random(want.shape).astype(np.float32)
            ya = to_device(y0, dev)
            m.spmv(xd, ya, direction=direction, mode=mode, accumulate=True)
            torch.cuda.synchronize()
            check_parity(from_device(ya, "plus_times"), y0.astype(np.float64) + want, "plus_times",
                         f"web_n20_d16 accumulate {direction} {mode}")
        # streamed from host memory through a 4 MB staging buffer
        st = k2.Streamed(tree, 4 << 20)
        y = st.spmv(xd, direction=direction)
        torch.cuda.synchronize()
        check_parity(from_device(y, "plus_times"), want, "plus_times", f"web_n20_d16 {direction} streamed")
        for sr in ("tropical", "boolean_u32"):
            xs = make_x(np.random.default_rng(17), sr, n, 1)
            want = ref.spmv(xs, ORC_SEMIRING[sr], ORC_DIR[direction], 1, threads=16)
            y = m.spmv(to_device(xs, dev), direction=direction, semiring=sr, mode="tree")
            torch.cuda.synchronize()
            check_parity(from_device(y, sr), want, sr, f"web_n20_d16 {sr} {direction} tree")


def test_accumulate(dev):
    """K2_SPMV_ACCUMULATE: y = y0 (+) A x, element by element against y0
    combined with the oracle's product; band tiles that own their band
    combine their window with y by plain loads and stores, the others add
    atomically."""
    import tree_graph_spmv_amd as k2
    rng = np.random.default_rng(7)
    rows, cols = synth.rmat(11, 20000, seed=3)
    n = 2 ** 11
    tree = k2.Tree(rows, cols, n, n)
    ref = oracle.OracleTree(rows, cols, n, n)
    combine = {"plus_times": lambda a, b: a.astype(np.float64) + b,
               "boolean": np.maximum, "boolean_u32": np.bitwise_or, "tropical": np.minimum}
    for var in (dict(), dict(band_strays=0), dict(window_elems=0)):
        m = k2.Matrix(tree, k2.plan_defaults(cache_last_level=1, window_batch=1, **var), device=dev)
        for mode, sr, direction, B in itertools.product(("tree", "cached"), ALL_SEMIRINGS, ("right", "left"),
                                                        (1, 3)):
            x = make_x(rng, sr, n, B)
            y0 = make_x(rng, sr, n, B)
            if sr == "boolean":   # a Boolean y holds 0 and 1
                y0 = (y0 != 0).astype(np.float32)
            y = to_device(y0, dev)
            m.spmv(to_device(x, dev), y, direction=direction, semiring=sr, batch=B, mode=mode,
                   accumulate=True)
            torch.cuda.synchronize()
            r = ref.spmv(x, ORC_SEMIRING[sr], ORC_DIR[direction], B)
            want = combine[sr](y0.reshape(r.shape), r)
            check_parity(from_device(y, sr), want, sr, f"accumulate {var} {mode} {sr} {direction} B={B}")


def test_streamed(dev):
    """Out-of-core products (k2_stream_*): the tree stays in host memory and
    goes through a small staging buffer chunk by chunk; every semiring, both
    directions, batches 1 and 3, overwriting and accumulating, against the
    oracle, and against the resident tree-only product."""
    import tree_graph_spmv_amd as k2
    rng = np.random.default_rng(17)
    rows, cols, n = synth.workload_edges("rmat_s12_e32k")
    tree = k2.Tree(rows, cols, n, n)
    ref = oracle.OracleTree(rows, cols, n, n)
    m = k2.Matrix(tree, k2.plan_defaults(), device=dev)
    combine = {"plus_times": lambda a, b: a.astype(np.float64) + b,
               "boolean": np.maximum, "boolean_u32": np.bitwise_or, "tropical": np.minimum}
    for staging in (1 << 15, 1 << 24):
        s = k2.Streamed(tree, staging)
        assert 2 * s.max_chunk_bytes <= staging
        if staging == 1 << 15:
            assert s.n_chunks > 4
        buf = s.staging(dev)
        for sr, direction, B in itertools.product(ALL_SEMIRINGS, ("right", "left"), (1, 3)):
            x = make_x(rng, sr, n, B)
            xd = to_device(x, dev)
            y = s.spmv(xd, direction=direction, semiring=sr, batch=B, staging=buf)
            torch.cuda.synchronize()
            want = ref.spmv(x, ORC_SEMIRING[sr], ORC_DIR[direction], B)
            label = f"streamed {staging} {sr} {direction} B={B}"
            check_parity(from_device(y, sr), want, sr, label)
            if sr != "plus_times":   # exact semirings: the resident product agrees bit for bit
                yr = m.spmv(xd, direction=direction, semiring=sr, batch=B, mode="tree")
                torch.cuda.synchronize()
                assert np.array_equal(from_device(y, sr), from_device(yr, sr)), label
            y0 = make_x(rng, sr, n, B)
            if sr == "boolean":
                y0 = (y0 != 0).astype(np.float32)
            ya = to_device(y0, dev)
            s.spmv(xd, ya, direction=direction, semiring=sr, batch=B, accumulate=True, staging=buf)
            torch.cuda.synchronize()
            check_parity(from_device(ya, sr), combine[sr](y0.reshape(want.shape), want), sr, "accumulate " + label)



def test_multi_tile_bands(dev):
    """Bands cut into several cached tiles (band_tile_nodes 64 and 256 on a
    web-like 2^14 graph): tiles that do not own their band add their windows
    to y with atomics after the fill, the owner tile also adds the band's
    strays.  Every semiring, both directions, batches 1, 3 and 8, overwriting
    and accumulating, whole outputs against the oracle."""
    import tree_graph_spmv_amd as k2
    rng = np.random.default_rng(23)
    n = 2 ** 14
    rows, cols = synth.web(n, 16, window=1024, p_local=0.8, seed=7)
    tree = k2.Tree(rows, cols, n, n)
    ref = oracle.OracleTree(rows, cols, n, n)
    combine = {"plus_times": lambda a, b: a.astype(np.float64) + b,
               "boolean": np.maximum, "boolean_u32": np.bitwise_or, "tropical": np.minimum}
    for cap, strays in ((64, 1), (256, 1), (64, 0)):
        opts = k2.plan_defaults(cache_last_level=1, band_tile_nodes=cap, band_strays=strays)
        m = k2.Matrix(tree, opts, device=dev)
        # with strays every cached tile has a 512-row window: the products
        # read the node words only; without, the sparse tiles need the origins
        assert m.packed_nodes == (strays == 1)
        for sr, direction, B in itertools.product(ALL_SEMIRINGS, ("right", "left"), (1, 3, 8)):
            x = make_x(rng, sr, n, B)
            xd = to_device(x, dev)
            want = ref.spmv(x, ORC_SEMIRING[sr], ORC_DIR[direction], B)
            label = f"bands cap={cap} strays={strays} {sr} {direction} B={B}"
            y = m.spmv(xd, direction=direction, semiring=sr, batch=B, mode="cached")
            torch.cuda.synchronize()
            check_parity(from_device(y, sr), want, sr, label)
            y0 = make_x(rng, sr, n, B)
            if sr == "boolean":
                y0 = (y0 != 0).astype(np.float32)
            ya = to_device(y0, dev)
            m.spmv(xd, ya, direction=direction, semiring=sr, batch=B, mode="cached", accumulate=True)
            torch.cuda.synchronize()
            check_parity(from_device(ya, sr), combine[sr](y0.reshape(want.shape), want), sr,
                         "accumulate " + label)


def test_tree_only_with_band_groups(dev):
    """Tree-only products of a web-like 2^14 graph whose plan holds band
    groups in both directions: plus-times takes the groups, then the rest
    tiles they leave with their skip ranges; the other semirings take every
    rest tile in block order and skip nothing.  Every semiring, both
    directions, batches 1, 3 and 8, scan and directory offsets, overwriting
    and accumulating, whole outputs against the oracle."""
    import tree_graph_spmv_amd as k2
    rng = np.random.default_rng(31)
    n = 2 ** 14
    rows, cols = synth.web(n, 16, window=1024, p_local=0.8, seed=11)
    tree = k2.Tree(rows, cols, n, n)
    ref = oracle.OracleTree(rows, cols, n, n)
    combine = {"plus_times": lambda a, b: a.astype(np.float64) + b,
               "boolean": np.maximum, "boolean_u32": np.bitwise_or, "tropical": np.minimum}
    for offsets in ("scan", "directory"):
        opts = k2.plan_defaults(offsets=offsets)
        for w in (0, 1):
            assert len(tree.plan(opts, 5 + w)[1]), "the plan must hold band groups"
            rest = tree.plan(opts, 3 + w)[1]
            assert (rest[:, 5] == 0xFFFFFFFF).any() and (rest[:, 5] != 0xFFFFFFFF).any(), \
                "rest tiles both inside and outside the groups"
        m = k2.Matrix(tree, opts, device=dev)
        for sr, direction, B in itertools.product(ALL_SEMIRINGS, ("right", "left"), (1, 3, 8)):
            x = make_x(rng, sr, n, B)
            xd = to_device(x, dev)
            want = ref.spmv(x, ORC_SEMIRING[sr], ORC_DIR[direction], B)
            label = f"tree with groups {offsets} {sr} {direction} B={B}"
            y = m.spmv(xd, direction=direction, semiring=sr, batch=B, mode="tree")
            torch.cuda.synchronize()
            check_parity(from_device(y, sr), want, sr, label)
            y0 = make_x(rng, sr, n, B)
            if sr == "boolean":
                y0 = (y0 != 0).astype(np.float32)
            ya = to_device(y0, dev)
            m.spmv(xd, ya, direction=direction, semiring=sr, batch=B, mode="tree", accumulate=True)
            torch.cuda.synchronize()
            check_parity(from_device(ya, sr), combine[sr](y0.reshape(want.shape), want), sr,
                         "accumulate " + label)


def test_wide_batch_windows(dev):
    """Batches 75 and 76 on a web-like 2^14 graph: a 512-row band window of
    75-76 vectors leaves no room for the band kernel's frontiers (tree-only
    plus-times products then skip the band groups and take every tile of
    the rest cut, a wave each, skipping nothing) but fits the cached
    kernel's window.
    Whole outputs against the oracle, both directions, tree-only and
    cached."""
    import tree_graph_spmv_amd as k2
    rng = np.random.default_rng(29)
    n = 2 ** 14
    rows, cols = synth.web(n, 16, window=1024, p_local=0.8, seed=11)
    tree = k2.Tree(rows, cols, n, n)
    ref = oracle.OracleTree(rows, cols, n, n)
    opts = k2.plan_defaults(cache_last_level=1)
    assert all(len(tree.plan(opts, w)[1]) for w in (5, 6)), "the plan must hold band groups to skip"
    m = k2.Matrix(tree, opts, device=dev)
    for B, direction, mode in itertools.product((75, 76), ("right", "left"), ("tree", "cached")):
        x = make_x(rng, "plus_times", n, B)
        y = m.spmv(to_device(x, dev), direction=direction, batch=B, mode=mode)
        torch.cuda.synchronize()
        want = ref.spmv(x, oracle.PLUS_TIMES, ORC_DIR[direction], B)
        check_parity(from_device(y, "plus_times"), want, "plus_times", f"wide batch {B} {direction} {mode}")


def test_ring_per_lane_count(dev):
    """Cached products size each wave's cell ring to one full pass: 512 slots
    at one lane per cell (batch 1, and every batch-1 max / or / min right
    product), 256 at two (batch 2), 128 from four.  Web-like 2^14 and R-MAT
    2^14 graphs, every semiring, both directions, batches 1 and 2, whole
    outputs against the oracle (the passes run full and drain at each tile's
    end)."""
    import tree_graph_spmv_amd as k2
    rng = np.random.default_rng(31)
    graphs = (("web14", synth.web(2 ** 14, 16, window=1024, p_local=0.8, seed=13), 2 ** 14),
              ("rmat14", synth.rmat(14, 200000, seed=14), 2 ** 14))
    for label, (rows, cols), n in graphs:
        tree = k2.Tree(rows, cols, n, n)
        ref = oracle.OracleTree(rows, cols, n, n)
        m = k2.Matrix(tree, k2.plan_defaults(cache_last_level=1), device=dev)
        for sr, direction, B in itertools.product(ALL_SEMIRINGS, ("right", "left"), (1, 2)):
            x = make_x(rng, sr, n, B)
            y = m.spmv(to_device(x, dev), direction=direction, semiring=sr, batch=B, mode="cached")
            torch.cuda.synchronize()
            want = ref.spmv(x, ORC_SEMIRING[sr], ORC_DIR[direction], B)
            check_parity(from_device(y, sr), want, sr, f"ring {label} {sr} {direction} B={B}")
