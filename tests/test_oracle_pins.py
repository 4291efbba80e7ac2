"""Pins for the CPU oracle, each against something other than the oracle.

* Figure 1 of the page (tests/golden/fig1.txt): signatures per level, child
  offsets, the S = 2 directory, leaf origins, per-thread update counts and the
  right/left products of the 8x8 example.
* Closed forms of the definition (Sec. 2.1): identity, all-ones, one cell,
  empty matrix.
* Brute force on tiny inputs: an independent construction of the level
  signatures by sorting Morton keys in Python, and dense products for all
  semirings and both directions.
* Invariants: popcount of a level = size of the next, leaf popcount = nnz,
  cells round trip, A.1 = out-degree, left(A) = right(A^T), directory = rank,
  and the tropical and Boolean special cases.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import BOOLEAN_F32, BOOLEAN_U32, LEFT, PLUS_TIMES, RIGHT, TROPICAL


# --------------------------------------------------------------- helpers

def parse_cells(text):
    pairs = [tuple(int(v) for v in p.split(",")) for p in text.split()]
    return np.array([p[0] for p in pairs], np.uint32), np.array([p[1] for p in pairs], np.uint32)


def sig_from_page(bits):
    """Page notation writes bit 0 first: '1010' has bits 0 and 2 set."""
    return sum(1 << i for i, ch in enumerate(bits) if ch == "1")


def dense(rows, cols, n_rows, n_cols):
    a = np.zeros((n_rows, n_cols), dtype=bool)
    a[np.asarray(rows, np.int64), np.asarray(cols, np.int64)] = True
    return a


def morton(r, c, bits):
    """Interleave: row bit i -> key bit 2i+1, column bit i -> key bit 2i."""
    k = 0
    for i in range(bits):
        k |= ((r >> i) & 1) << (2 * i + 1)
        k |= ((c >> i) & 1) << (2 * i)
    return k


def brute_levels(rows, cols, n_rows, n_cols):
    """Level signatures from the definition, by sorting blocks in Z-order."""
    l = max(2, math.ceil(math.log2(max(n_rows, n_cols, 1))))
    cells = sorted(set(zip((int(r) for r in rows), (int(c) for c in cols))))
    levels = []
    for d in range(l):
        shift = l - d                      # a level-d node is a 2^shift block
        sig = {}
        for r, c in cells:
            block = (r >> shift, c >> shift)
            quad = 2 * ((r >> (shift - 1)) & 1) + ((c >> (shift - 1)) & 1)
            sig[block] = sig.get(block, 0) | (1 << quad)
        if d == 0 and not sig:
            sig[(0, 0)] = 0                  # the root exists even when empty
        order = sorted(sig, key=lambda b: morton(b[0], b[1], d))
        levels.append([sig[b] for b in order])
    return levels


def brute_product(a, x, semiring, direction, batch):
    """Dense product over the semiring (the definition of Sec. 2.2)."""
    m = a if direction == RIGHT else a.T
    n_out = m.shape[0]
    x = x.reshape(m.shape[1], batch)
    if semiring == PLUS_TIMES:
        y = m.astype(np.float64) @ x.astype(np.float64)
    elif semiring == BOOLEAN_F32:
        y = ((m.astype(np.int64) @ (x != 0).astype(np.int64)) > 0).astype(np.float32)
    elif semiring == BOOLEAN_U32:
        y = np.zeros((n_out, batch), np.uint32)
        for i in range(n_out):
            for j in np.nonzero(m[i])[0]:
                y[i] |= x[j]
    else:
        y = np.full((n_out, batch), np.inf, np.float32)
        contrib = (np.float32(1.0) + x.astype(np.float32)).astype(np.float32)
        for i in range(n_out):
            js = np.nonzero(m[i])[0]
            if js.size:
                y[i] = contrib[js].min(axis=0)
    return y if batch > 1 else y.reshape(-1)


def random_x(rng, semiring, n, batch):
    if semiring == BOOLEAN_U32:
        return rng.integers(0, 2**32, size=n * batch, dtype=np.uint64).astype(np.uint32)
    if semiring == TROPICAL:
        x = rng.integers(0, 100 * 2**16, size=n * batch).astype(np.float32) / np.float32(2**16)
        x[rng.random(n * batch) < 0.4] = np.inf
        return x
    if semiring == BOOLEAN_F32:
        x = rng.integers(0, 3, size=n * batch).astype(np.float32)
        return x
    # dyadic values k * 2^-24 in [0, 1): sums stay exact in fp64
    return (rng.integers(0, 2**24, size=n * batch).astype(np.float64) / 2**24).astype(np.float32)


def assert_same(y, ref, semiring):
    if semiring in (BOOLEAN_F32, TROPICAL, BOOLEAN_U32):
        assert np.array_equal(np.asarray(y).view(np.uint32), np.asarray(ref, dtype=y.dtype).view(np.uint32))
    else:
        assert np.array_equal(y, ref)


# ------------------------------------------------------------ Figure 1

def test_fig1_signatures(fig1):
    rows, cols = parse_cells(fig1["cells"])
    t = oracle.OracleTree(rows, cols, 8, 8)
    assert t.levels == 3
    for d in range(3):
        page = [sig_from_page(s) for s in fig1[f"level{d}"].split()]
        assert t.signatures(d).tolist() == page
    assert t.level_nodes() == [1, 4, 8]
    assert t.level_words(1).tolist() == [int(fig1["words1"], 16)]
    assert t.level_words(2).tolist() == [int(fig1["words2"], 16)]
    # 24 set bits = (13 nodes - root) + 12 non-zeros
    total = sum(bin(int(s)).count("1") for d in range(3) for s in t.signatures(d))
    assert total == (13 - 1) + 12 == 24


def test_fig1_offsets_and_directory(fig1):
    rows, cols = parse_cells(fig1["cells"])
    t = oracle.OracleTree(rows, cols, 8, 8)
    fan = [bin(int(s)).count("1") for s in t.signatures(1)]
    assert fan == [int(v) for v in fig1["fanout1"].split()]
    assert t.child_offsets(1).tolist() == [int(v) for v in fig1["offsets1"].split()]
    assert sum(fan) == int(fig1["total1"]) == t.level_nodes()[2]
    assert t.directory(1, 2).tolist() == [int(v) for v in fig1["directory1_S2"].split()]
    # node 01 finds its first child at the sample 0 plus popcount(1000) = 1
    assert t.directory(1, 2)[0] + 1 == t.child_offsets(1)[1]


def test_fig1_leaves_in_level_order(fig1):
    rows, cols = parse_cells(fig1["cells"])
    t = oracle.OracleTree(rows, cols, 8, 8)
    r, c = t.cells()
    sigs2 = t.signatures(2)
    # group the enumerated cells by leaf (each leaf holds popcount(sig) cells)
    origins, k = [], 0
    for s in sigs2:
        cnt = bin(int(s)).count("1")
        origins.append((int(r[k]) & ~1, int(c[k]) & ~1))
        k += cnt
    page = [tuple(int(v) for v in p.split(",")) for p in fig1["origins2"].split()]
    assert origins == page
    # the leaf codes deinterleave to the origins: odd bits row, even bits col
    for code, (r0, c0) in zip(fig1["codes2"].split(), page):
        v = int(code, 2)
        rr = sum(((v >> (2 * i + 1)) & 1) << i for i in range(2))
        cc = sum(((v >> (2 * i)) & 1) << i for i in range(2))
        assert (2 * rr, 2 * cc) == (r0, c0)
    # per-thread updates of the last internal level
    offs = t.child_offsets(1)
    upd = []
    for i, s in enumerate(t.signatures(1)):
        f = bin(int(s)).count("1")
        upd.append(sum(bin(int(sigs2[offs[i] + j])).count("1") for j in range(f)))
    assert upd == [int(v) for v in fig1["updates1"].split()]


def _symbolic(text, x):
    out = []
    for term in text.split("|"):
        term = term.strip()
        out.append([] if term == "-" else [int(v) for v in term.split("+")])
    return out


@pytest.mark.parametrize("direction,key", [(RIGHT, "right"), (LEFT, "left")])
def test_fig1_products(fig1, direction, key):
    rows, cols = parse_cells(fig1["cells"])
    t = oracle.OracleTree(rows, cols, 8, 8)
    rng = np.random.default_rng(1)
    x = rng.integers(1, 1000, size=8).astype(np.float32)
    terms = _symbolic(fig1[key], x)
    y = t.spmv(x, PLUS_TIMES, direction)
    assert y.tolist() == [float(sum(x[j] for j in js)) for js in terms]
    # Boolean: y_i = 1 iff some x_j in the sum is non-zero
    xb = np.array([0, 1, 0, 0, 2, 0, 0, 3], np.float32)
    yb = t.spmv(xb, BOOLEAN_F32, direction)
    assert yb.tolist() == [1.0 if any(xb[j] != 0 for j in js) else 0.0 for js in terms]
    # tropical: y_i = min(1 + x_j), +inf when empty
    xt = rng.integers(0, 50, size=8).astype(np.float32)
    yt = t.spmv(xt, TROPICAL, direction)
    assert yt.tolist() == [min((1.0 + float(xt[j]) for j in js), default=math.inf) for js in terms]
    # all-ones: out-degrees (1,2,0,1,0,2,4,2) / in-degrees (0,3,2,0,1,2,2,2)
    deg = t.spmv(np.ones(8, np.float32), PLUS_TIMES, direction)
    expect = [1, 2, 0, 1, 0, 2, 4, 2] if direction == RIGHT else [0, 3, 2, 0, 1, 2, 2, 2]
    assert deg.tolist() == expect


def test_fig1_page_statements(fig1):
    rows, cols = parse_cells(fig1["cells"])
    t = oracle.OracleTree(rows, cols, 8, 8)
    # x5 reaches y3; x1 reaches y6 (single basis vectors)
    for j, i in [(5, 3), (1, 6)]:
        x = np.zeros(8, np.float32)
        x[j] = 1
        assert t.spmv(x, PLUS_TIMES, RIGHT)[i] == 1.0


# ----------------------------------------------------------- closed forms

@pytest.mark.parametrize("n", [4, 8, 64, 1024])
def test_identity(n):
    idx = np.arange(n, dtype=np.uint32)
    t = oracle.OracleTree(idx, idx, n, n)
    l = t.levels
    assert l == max(2, int(math.log2(n)))
    assert t.level_nodes() == [2 ** d for d in range(l)]
    for d in range(l):
        assert set(t.signatures(d).tolist()) == {0x9}
    x = np.arange(n, dtype=np.float32) * 0.5
    assert np.array_equal(t.spmv(x, PLUS_TIMES, RIGHT), x.astype(np.float64))
    assert np.array_equal(t.spmv(x, PLUS_TIMES, LEFT), x.astype(np.float64))


@pytest.mark.parametrize("n", [4, 8, 16])
def test_dense(n):
    r, c = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    t = oracle.OracleTree(r.ravel(), c.ravel(), n, n)
    l = t.levels
    assert t.level_nodes() == [4 ** d for d in range(l)]
    assert sum(t.level_nodes()) == (4 ** l - 1) // 3
    for d in range(l):
        assert set(t.signatures(d).tolist()) == {0xF}
    x = np.arange(n, dtype=np.float32)
    assert np.array_equal(t.spmv(x, PLUS_TIMES, RIGHT), np.full(n, x.sum(), np.float64))


@pytest.mark.parametrize("n,i,j", [(4, 0, 3), (8, 5, 2), (1000, 999, 0), (2 ** 20, 123457, 654321)])
def test_single_cell(n, i, j):
    t = oracle.OracleTree([i], [j], n, n)
    l = t.levels
    assert t.level_nodes() == [1] * l
    for d in range(l):
        bit = l - 1 - d
        b = 2 * ((i >> bit) & 1) + ((j >> bit) & 1)
        assert t.signatures(d).tolist() == [1 << b]
    x = np.zeros(n, np.float32)
    x[j] = 7.0
    y = t.spmv(x, PLUS_TIMES, RIGHT)
    assert y[i] == 7.0 and y.sum() == 7.0


def test_empty():
    t = oracle.OracleTree([], [], 10, 10)
    assert t.level_nodes()[0] == 1 and t.signatures(0).tolist() == [0]
    assert all(v == 0 for v in t.level_nodes()[1:])
    x = np.ones(10, np.float32)
    assert np.array_equal(t.spmv(x, PLUS_TIMES, RIGHT), np.zeros(10))
    assert np.all(np.isinf(t.spmv(x, TROPICAL, RIGHT)))


def test_duplicates_dropped_and_range_checked():
    t = oracle.OracleTree([1, 1, 1, 2], [2, 2, 2, 0], 4, 4)
    assert t.nnz == 2
    with pytest.raises(oracle.OracleError):
        oracle.OracleTree([4], [0], 4, 4)
    with pytest.raises(oracle.OracleError):
        oracle.OracleTree([0], [4], 4, 4)


# ------------------------------------------------------------ brute force

@st.composite
def small_matrix(draw):
    n_rows = draw(st.integers(1, 64))
    n_cols = draw(st.integers(1, 64))
    density = draw(st.floats(0.0, 1.0))
    seed = draw(st.integers(0, 2**31))
    rng = np.random.default_rng(seed)
    mask = rng.random((n_rows, n_cols)) < density
    r, c = np.nonzero(mask)
    # add duplicates in shuffled order
    if r.size:
        k = rng.integers(0, r.size, size=r.size // 3)
        r = np.concatenate([r, r[k]])
        c = np.concatenate([c, c[k]])
        p = rng.permutation(r.size)
        r, c = r[p], c[p]
    return n_rows, n_cols, r.astype(np.uint32), c.astype(np.uint32), seed


@settings(max_examples=60, deadline=None)
@given(small_matrix())
def test_brute_force_levels(m):
    n_rows, n_cols, r, c, _ = m
    t = oracle.OracleTree(r, c, n_rows, n_cols)
    ref = brute_levels(r, c, n_rows, n_cols)
    assert t.levels == len(ref)
    for d in range(t.levels):
        assert t.signatures(d).tolist() == ref[d]


@settings(max_examples=40, deadline=None)
@given(small_matrix(), st.sampled_from([PLUS_TIMES, BOOLEAN_F32, BOOLEAN_U32, TROPICAL]),
       st.sampled_from([RIGHT, LEFT]), st.sampled_from([1, 3]))
def test_brute_force_products(m, semiring, direction, batch):
    n_rows, n_cols, r, c, seed = m
    t = oracle.OracleTree(r, c, n_rows, n_cols)
    a = dense(r, c, n_rows, n_cols)
    rng = np.random.default_rng(seed + 1)
    n_in = n_cols if direction == RIGHT else n_rows
    x = random_x(rng, semiring, n_in, batch)
    y = t.spmv(x, semiring, direction, batch)
    ref = brute_product(a, x, semiring, direction, batch)
    assert_same(np.asarray(y), ref, semiring)
    y2 = oracle.spmv_edges(r, c, n_rows, n_cols, x, semiring, direction, batch)
    assert_same(np.asarray(y2), ref, semiring)


# ------------------------------------------------------------- invariants

def rmat_like(rng, scale, m):
    """Skewed random edges (recursive quadrant choice), small sizes only."""
    r = np.zeros(m, np.int64)
    c = np.zeros(m, np.int64)
    for _ in range(scale):
        u = rng.random(m)
        b1 = (u >= 0.76).astype(np.int64)            # c + d = 0.24
        b0 = (((u >= 0.57) & (u < 0.76)) | (u >= 0.95)).astype(np.int64)
        r = 2 * r + b1
        c = 2 * c + b0
    return r.astype(np.uint32), c.astype(np.uint32)


@pytest.fixture(scope="module")
def mid_tree():
    rng = np.random.default_rng(7)
    n_rows, n_cols = 3000, 2500
    r, c = rmat_like(rng, 12, 40000)
    keep = (r < n_rows) & (c < n_cols)
    r, c = r[keep], c[keep]
    return n_rows, n_cols, r, c, oracle.OracleTree(r, c, n_rows, n_cols)


def test_popcount_invariants(mid_tree):
    n_rows, n_cols, r, c, t = mid_tree
    nodes = t.level_nodes()
    for d in range(t.levels - 1):
        assert sum(bin(int(s)).count("1") for s in t.signatures(d)) == nodes[d + 1]
    assert sum(bin(int(s)).count("1") for s in t.signatures(t.levels - 1)) == t.nnz
    assert t.nnz == len(set(zip(r.tolist(), c.tolist())))
    # N_d = number of distinct (r >> (l-d), c >> (l-d))
    for d in range(t.levels):
        sh = t.levels - d
        assert nodes[d] == len(set(zip((r >> sh).tolist(), (c >> sh).tolist())))


def test_cells_round_trip(mid_tree):
    n_rows, n_cols, r, c, t = mid_tree
    cr, cc = t.cells()
    assert set(zip(cr.tolist(), cc.tolist())) == set(zip(r.tolist(), c.tolist()))
    assert len(cr) == t.nnz


def test_degrees_and_transpose(mid_tree):
    n_rows, n_cols, r, c, t = mid_tree
    a = dense(r, c, n_rows, n_cols)
    assert np.array_equal(t.spmv(np.ones(n_cols, np.float32), PLUS_TIMES, RIGHT), a.sum(1))
    assert np.array_equal(t.spmv(np.ones(n_rows, np.float32), PLUS_TIMES, LEFT), a.sum(0))
    tt = oracle.OracleTree(c, r, n_cols, n_rows)
    rng = np.random.default_rng(3)
    for semiring in (PLUS_TIMES, BOOLEAN_F32, BOOLEAN_U32, TROPICAL):
        x = random_x(rng, semiring, n_rows, 2)
        assert_same(np.asarray(t.spmv(x, semiring, LEFT, 2)),
                    np.asarray(tt.spmv(x, semiring, RIGHT, 2)), semiring)


@pytest.mark.parametrize("S", [2, 16, 256])
def test_directory_is_rank(mid_tree, S):
    *_, t = mid_tree
    for d in range(t.levels - 1):
        off = t.child_offsets(d)
        dirs = t.directory(d, S)
        assert np.array_equal(dirs, off[::S])
        # rank = popcounts of the preceding signatures (an exclusive scan)
        fan = np.array([bin(int(s)).count("1") for s in t.signatures(d)], np.uint64)
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(fan)[:-1]]).astype(np.uint64))


def test_threads_and_edges_agree(mid_tree):
    n_rows, n_cols, r, c, t = mid_tree
    rng = np.random.default_rng(11)
    for semiring in (PLUS_TIMES, BOOLEAN_F32, BOOLEAN_U32, TROPICAL):
        for direction in (RIGHT, LEFT):
            n_in = n_cols if direction == RIGHT else n_rows
            x = random_x(rng, semiring, n_in, 3)
            y1 = np.asarray(t.spmv(x, semiring, direction, 3, threads=1))
            y4 = np.asarray(t.spmv(x, semiring, direction, 3, threads=5))
            ye = np.asarray(oracle.spmv_edges(r, c, n_rows, n_cols, x, semiring, direction, 3))
            assert_same(y4, y1, semiring)
            assert_same(ye, y1, semiring)
            sample = rng.choice(y1.shape[0], size=50, replace=False).astype(np.uint32)
            ys = oracle.spmv_sample(r, c, n_rows, n_cols, x, semiring, sample, direction, 3)
            assert_same(np.asarray(ys), y1[sample], semiring)


def test_tropical_special_cases(mid_tree):
    n_rows, n_cols, r, c, t = mid_tree
    a = dense(r, c, n_rows, n_cols)
    y = t.spmv(np.zeros(n_cols, np.float32), TROPICAL, RIGHT)
    assert np.array_equal(y, np.where(a.any(1), 1.0, np.inf).astype(np.float32))
    s = int(c[0])
    x = np.full(n_cols, np.inf, np.float32)
    x[s] = 0.0
    y = t.spmv(x, TROPICAL, RIGHT)
    assert np.array_equal(y, np.where(a[:, s], 1.0, np.inf).astype(np.float32))
    s = int(r[0])
    x = np.full(n_rows, np.inf, np.float32)
    x[s] = 0.0
    y = t.spmv(x, TROPICAL, LEFT)
    assert np.array_equal(y, np.where(a[s, :], 1.0, np.inf).astype(np.float32))


def test_boolean_packed_is_32_boolean_products(mid_tree):
    n_rows, n_cols, r, c, t = mid_tree
    rng = np.random.default_rng(5)
    words = rng.integers(0, 2**32, size=n_cols, dtype=np.uint64).astype(np.uint32)
    words[rng.random(n_cols) < 0.5] = 0
    y = t.spmv(words, BOOLEAN_U32, RIGHT)
    for bit in (0, 13, 31):
        xb = ((words >> bit) & 1).astype(np.float32)
        yb = t.spmv(xb, BOOLEAN_F32, RIGHT)
        assert np.array_equal(((y >> bit) & 1).astype(np.float32), yb)


# ---- multi-source search (Sec. 5.8) -----------------------------------

def test_bfs_path_graph_closed_form():
    """Edges i -> i+1 (cells (i, i+1)): a LEFT step moves from row to column,
    so from s the distance to v >= s is v - s; a RIGHT step moves the other
    way, v <= s at s - v.  max_levels cuts both."""
    n = 40
    r = np.arange(n - 1, dtype=np.uint32)
    c = r + 1
    src = np.array([0, 7, 39], np.uint32)
    v = np.arange(n)[:, None]
    s = src[None, :].astype(np.int64)
    left = oracle.bfs(r, c, n, src, oracle.LEFT)
    right = oracle.bfs(r, c, n, src, oracle.RIGHT)
    assert np.array_equal(left, np.where(v >= s, v - s, -1))
    assert np.array_equal(right, np.where(v <= s, s - v, -1))
    cut = oracle.bfs(r, c, n, src, oracle.LEFT, max_levels=5)
    want = np.where((v >= s) & (v - s <= 5), v - s, -1)
    assert np.array_equal(cut, want)


@pytest.mark.parametrize("seed", range(4))
def test_bfs_against_scipy(seed):
    """Unweighted shortest paths of scipy.sparse.csgraph on random directed
    graphs (a cell (r, c) is the arc r -> c for LEFT steps, c -> r for
    RIGHT steps)."""
    from scipy.sparse import coo_matrix
    from scipy.sparse.csgraph import shortest_path
    rng = np.random.default_rng(50 + seed)
    n = int(rng.integers(2, 300))
    m = int(rng.integers(0, 4 * n))
    r = rng.integers(0, n, m).astype(np.uint32)
    c = rng.integers(0, n, m).astype(np.uint32)
    src = rng.integers(0, n, 7).astype(np.uint32)
    g = coo_matrix((np.ones(m), (r, c)), shape=(n, n)).tocsr()
    for direction, graph in ((oracle.LEFT, g), (oracle.RIGHT, g.T.tocsr())):
        d = shortest_path(graph, method="D", directed=True, unweighted=True, indices=src)
        want = np.where(np.isinf(d), -1, d).astype(np.int64).T
        assert np.array_equal(oracle.bfs(r, c, n, src, direction), want)


@pytest.mark.parametrize("seed", range(3))
def test_bfs_is_iterated_min_plus(seed):
    """The paper derives the search from Bellman-Ford on unit lengths: from
    x = 0 at the source and +inf elsewhere, x <- min(x, A (min,+) x) (the
    tree's tropical product, 1 + x_j per cell) converges to the hop
    distances, in either direction."""
    rng = np.random.default_rng(70 + seed)
    n = int(rng.integers(2, 200))
    m = int(rng.integers(0, 3 * n))
    r = rng.integers(0, n, m).astype(np.uint32)
    c = rng.integers(0, n, m).astype(np.uint32)
    t = oracle.OracleTree(r, c, n, n)
    src = rng.integers(0, n, 3).astype(np.uint32)
    for direction in (oracle.RIGHT, oracle.LEFT):
        want = oracle.bfs(r, c, n, src, direction)
        for j, s in enumerate(src):
            x = np.full(n, np.inf, np.float32)
            x[s] = 0
            while True:
                y = np.minimum(x, t.spmv(x, oracle.TROPICAL, direction, 1).astype(np.float32))
                if np.array_equal(y, x):
                    break
                x = y
            got = np.where(np.isinf(x), -1, x).astype(np.int64)
            assert np.array_equal(got, want[:, j])
