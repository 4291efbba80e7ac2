"""GPU parity of the multi-source search (Sec. 5.8): k2_bfs through the C ABI
against the oracle's queue search, exactly (hop counts are integers).

Covers both directions, tree-only and cached matrices, 1 to 70 sources
(partial last words of the packed frontier), repeated sources, sources with
no edges, a level cap, and the per-level counts of newly reached entries."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_graph_spmv_amd  # noqa: F401
    return torch.device("cuda:0")


def run_case(k2, dev, rows, cols, n, sources, label, max_levels=1 << 16):
    tree = k2.Tree(rows, cols, n, n)
    for cached in (0, 1):
        m = k2.Matrix(tree, k2.plan_defaults(cache_last_level=cached), device=dev)
        for direction, odir in (("right", oracle.RIGHT), ("left", oracle.LEFT)):
            want = oracle.bfs(rows, cols, n, sources, odir, max_levels)
            dist, levels, reached = m.bfs(sources, direction, max_levels=max_levels)
            torch.cuda.synchronize()
            got = dist.cpu().numpy()
            bad = np.argwhere(got != want)
            assert bad.size == 0, f"{label} cached={cached} {direction}: {len(bad)} wrong, e.g. {bad[:3]}"
            assert levels == max(0, int(want.max()))
            # entries reached at each level = the oracle's distance histogram
            hist = np.bincount(want[want > 0].ravel(), minlength=levels + 1)[1:levels + 1]
            assert np.array_equal(reached[:levels], hist), label
            if levels < max_levels:
                assert reached[levels] == 0


def test_bfs_rmat_s12(dev):
    import tree_graph_spmv_amd as k2
    rows, cols, n = synth.workload_edges("rmat_s12_e32k")
    rng = np.random.default_rng(5)
    for S in (1, 31, 32, 33, 70):
        src = rng.integers(0, n, S).astype(np.uint32)
        run_case(k2, dev, rows, cols, n, src, f"rmat_s12 S={S}")


def test_bfs_edge_cases(dev):
    import tree_graph_spmv_amd as k2
    # a path, a cycle and isolated vertices; repeated sources; a source with
    # no edges; a level cap
    n = 1000
    r = np.concatenate([np.arange(0, 399), np.arange(400, 599), [599]]).astype(np.uint32)
    c = np.concatenate([np.arange(1, 400), np.arange(401, 600), [400]]).astype(np.uint32)
    src = np.array([0, 0, 399, 450, 900, 5], np.uint32)
    run_case(k2, dev, r, c, n, src, "path+cycle")
    run_case(k2, dev, r, c, n, src, "path+cycle cap 7", max_levels=7)


def test_bfs_web_n20(dev):
    import tree_graph_spmv_amd as k2
    rows, cols, n = synth.workload_edges("web_n20_d16")
    src = np.random.default_rng(6).integers(0, n, 64).astype(np.uint32)
    run_case(k2, dev, rows, cols, n, src, "web_n20")
