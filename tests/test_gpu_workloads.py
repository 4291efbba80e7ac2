"""GPU parity at the full workload sizes, in the launch configuration the
benchmark uses.

Whole outputs against the oracle where it can compute them in seconds to a
minute (oracle.spmv_edges, the product from the edge-list definition): the
R-MAT 2^22 tropical products (right and left, tree-only and cached) and the
symmetric R-MAT 2^24 packed-Boolean right product.  For the web-like 2^27
graph (1.2G edges) the oracle computes contiguous blocks of 2^20 outputs
(the first, two inner ones and the last) plus scattered outputs, one by one
from the edge-list definition (oracle.spmv_sample).  Properties that hold at
any size complete the check: left = right on a symmetric matrix, the
all-ones product = out-degrees, tree-only = cached.  Also: the library
allocates no device memory in k2_matrix_create and k2_spmv.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import ORC_DIR, ORC_SEMIRING, check_parity, from_device, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_graph_spmv_amd  # noqa: F401
    return torch.device("cuda:0")


def sample_idx(n, k, seed):
    rng = np.random.default_rng(seed)
    s = rng.choice(n, size=min(k, n), replace=False)
    # always include the first and last outputs and the R-MAT hubs near 0
    return np.unique(np.concatenate([s, [0, 1, 2, n - 1]])).astype(np.uint32)


def block_sample(n, seed, block=2 ** 20, k=3000):
    """Contiguous blocks of outputs: the first, one starting at an odd offset
    near n/4, the middle one and the last; plus k scattered outputs."""
    starts = [0, n // 4 + 12345, n // 2, n - block]
    blocks = [np.arange(s0, s0 + block, dtype=np.int64) for s0 in starts]
    return np.unique(np.concatenate(blocks + [sample_idx(n, k, seed).astype(np.int64)])).astype(np.uint32)


def log(msg):
    print(f"[workloads] {msg}", flush=True)


def test_library_allocates_nothing(dev):
    import tree_graph_spmv_amd as k2
    rows, cols = synth.rmat(16, 300000, seed=2)
    n = 2 ** 16
    tree = k2.Tree(rows, cols, n, n)
    for cached in (0, 1):
        opts = k2.plan_defaults(cache_last_level=cached)
        arena = k2.Matrix.arena_for(tree, opts, dev)
        x = torch.rand(n * 8, device=dev)
        y = torch.empty(n * 8, device=dev)
        # load the code object first
        k2.Matrix(k2.Tree([0], [0], 4, 4), device=dev).spmv(torch.zeros(4, device=dev))
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info()
        m = k2.Matrix(tree, opts, device=dev, arena=arena)
        for d in ("right", "left"):
            m.spmv(x, y, direction=d, batch=8)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        assert free0 - free1 == 0, f"library took {free0 - free1} bytes"
        est = tree.estimate(opts, batch=8)
        assert arena.numel() + x.numel() * 4 + y.numel() * 4 == est["total"]


def test_rmat_s22_e64m_tropical(dev):
    """R-MAT 2^22, 2^26 edges, min-plus with 10% finite x: right and left,
    both traversals, whole outputs bit-exact against the oracle."""
    import tree_graph_spmv_amd as k2
    rows, cols, n = synth.workload_edges("rmat_s22_e64m")
    tree = k2.Tree(rows, cols, n, n)
    assert tree.nnz == len(rows)
    x = synth.workload_x("rmat_s22_e64m", n)
    m = k2.Matrix(tree, k2.plan_defaults(cache_last_level=1), device=dev)
    xd = to_device(x, dev)
    for direction in ("right", "left"):
        want = oracle.spmv_edges(rows, cols, n, n, x, oracle.TROPICAL, ORC_DIR[direction])
        log(f"rmat_s22 oracle {direction} done")
        for mode in ("tree", "cached"):
            y = m.spmv(xd, direction=direction, semiring="tropical", mode=mode)
            torch.cuda.synchronize()
            check_parity(from_device(y, "tropical"), want, "tropical", f"rmat_s22 tropical {direction} {mode}")
            del y


def test_symrmat_s24_e256m_boolean(dev):
    """Symmetric R-MAT 2^24, 2^28 directed edges, 32 Boolean vectors per word:
    the whole right product bit-exact against the oracle, cached and
    tree-only; left = right (symmetry)."""
    import tree_graph_spmv_amd as k2
    rows, cols, n = synth.workload_edges("symrmat_s24_e256m")
    tree = k2.Tree(rows, cols, n, n)
    assert tree.nnz == len(rows) == 2 ** 28
    x = synth.workload_x("symrmat_s24_e256m", n)
    m = k2.Matrix(tree, k2.plan_defaults(cache_last_level=1), device=dev)
    xd = to_device(x, dev)
    yr = m.spmv(xd, direction="right", semiring="boolean_u32")
    yl = m.spmv(xd, direction="left", semiring="boolean_u32")
    yt = m.spmv(xd, direction="right", semiring="boolean_u32", mode="tree")
    torch.cuda.synchronize()
    assert torch.equal(yr, yl) and torch.equal(yr, yt)
    want = oracle.spmv_edges(rows, cols, n, n, x, oracle.BOOLEAN_U32, oracle.RIGHT)
    log("symrmat_s24 oracle right done")
    check_parity(from_device(yr, "boolean_u32"), want, "boolean_u32", "symrmat_s24 right")


def test_web_n27_d9_batch8(dev):
    """Web-like 2^27, ~1.2G edges, plus-times over 8 vectors, last internal
    level cached (the benchmark's configuration), tree-only and streamed
    from host memory: four contiguous blocks of 2^20 outputs (the first, the
    last and two inner ones) and 3000 scattered ones within the fp32
    tolerance, right and left; the all-ones product gives out-degrees."""
    import tree_graph_spmv_amd as k2
    rows, cols, n = synth.workload_edges("web_n27_d9")
    tree = k2.Tree(rows, cols, n, n)
    x = synth.workload_x("web_n27_d9", n)
    m = k2.Matrix(tree, k2.plan_defaults(cache_last_level=1), device=dev)
    assert m.packed_nodes   # the benchmark's products read the 4-byte node words
    xd = to_device(x, dev)
    idx = block_sample(n, 3)
    idx_t = torch.from_numpy(idx.astype(np.int64)).to(dev)
    st = k2.Streamed(tree, 256 << 20)   # the tree streamed from host memory (out of core)
    buf = st.staging(dev)
    for direction in ("right", "left"):
        want = oracle.spmv_sample(rows, cols, n, n, x, oracle.PLUS_TIMES, idx, ORC_DIR[direction], 8)
        log(f"web_n27 oracle {direction}: {idx.size} outputs")
        for mode in ("cached", "tree", "streamed"):   # tree-only: band groups, then the rest tiles
            if mode == "streamed":
                y = st.spmv(xd, direction=direction, batch=8, staging=buf)
            else:
                y = m.spmv(xd, direction=direction, batch=8, mode=mode)
            got = y.view(n, 8)[idx_t].cpu().numpy()
            check_parity(got, want, "plus_times", f"web_n27 {direction} {mode}")
            del y
    del st, buf
    ones = torch.ones(n, device=dev)
    deg = m.spmv(ones, direction="right").cpu().numpy()
    idx = sample_idx(n, 3000, 4)
    want = oracle.spmv_sample(rows, cols, n, n, np.ones(n, np.float32), oracle.PLUS_TIMES, idx)
    assert np.array_equal(deg[idx].astype(np.float64), want)
    assert deg.astype(np.float64).sum() == tree.nnz


def test_wide_offsets(dev):
    """Dimensions 2^31 x 2^31 with 4 vectors: index * batch passes 2^32, so
    the kernels keep 64-bit cell offsets.  x and y (32 GB each) live on the
    device.  The oracle computes the sampled outputs from the edges that
    reach them, over a compact copy of the x entries those edges read
    (fetched from the device), with the input indices renumbered to it."""
    import tree_graph_spmv_amd as k2
    n, B = 2 ** 31, 4
    rng = np.random.default_rng(31)
    m = 200000
    rows = rng.integers(0, n, m, dtype=np.int64)
    cols = rng.integers(0, n, m, dtype=np.int64)
    rows[:4] = [n - 1, n - 1, 0, n - 2]                  # the far corners
    cols[:4] = [n - 1, 0, n - 1, n - 1]
    rows[4:2000] = n - 1 - rng.integers(0, 64, 1996)     # a dense strip at the end
    rows, cols = rows.astype(np.uint32), cols.astype(np.uint32)
    tree = k2.Tree(rows, cols, n, n)
    x = torch.rand(n * B, device=dev)
    mat = k2.Matrix(tree, k2.plan_defaults(cache_last_level=1), device=dev)
    for direction in ("right", "left"):
        out_of, in_of = (rows, cols) if direction == "right" else (cols, rows)
        sample = np.unique(np.concatenate([out_of[:3000], rng.integers(0, n, 1000), [0, n - 1]])
                           ).astype(np.uint32)
        hit = np.isin(out_of, sample)
        need, local = np.unique(in_of[hit], return_inverse=True)
        xc = x.view(n, B)[torch.from_numpy(need.astype(np.int64)).to(dev)].cpu().numpy()
        if direction == "right":
            want = oracle.spmv_sample(out_of[hit], local.astype(np.uint32), n, need.size, xc,
                                      oracle.PLUS_TIMES, sample, oracle.RIGHT, B)
        else:
            want = oracle.spmv_sample(local.astype(np.uint32), out_of[hit], need.size, n, xc,
                                      oracle.PLUS_TIMES, sample, oracle.LEFT, B)
        for mode in ("tree", "cached"):
            y = mat.spmv(x, direction=direction, batch=B, mode=mode)
            torch.cuda.synchronize()
            got = y.view(n, B)[torch.from_numpy(sample.astype(np.int64)).to(dev)].cpu().numpy()
            check_parity(got, want, "plus_times", f"wide {direction} {mode}")
            del y
    del x
