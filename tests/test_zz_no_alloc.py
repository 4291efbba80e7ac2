"""k2_bfs_noalloc: the multi-source search whose workspace is the library's
fixed scratch array, for callers that cannot allocate device memory.

Checked against k2_bfs with a caller-allocated workspace on the same
matrices and sources: identical distance tables, last levels and per-level
counts, on two calls in a row, the second with a smaller input (fewer
vertices and sources, the other direction, tree-only); the smaller one also
against the oracle's queue search.  The device's free memory does not move
during a call, and a search whose workspace would exceed the array is
refused before anything runs.
"""
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
    import tree_graph_spmv_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


def test_noalloc_search_matches_workspace_search(dev):
    import tree_graph_spmv_amd as k2
    rng = np.random.default_rng(5)
    rows1, cols1 = synth.rmat(16, 300000, seed=41)
    rows2, cols2 = synth.rmat(12, 20000, seed=42)
    runs = [  # (rows, cols, n, plan options, sources, direction): the second is smaller
        (rows1, cols1, 2 ** 16, dict(cache_last_level=1), 70, "right"),
        (rows2, cols2, 2 ** 12, dict(), 5, "left"),
    ]
    for rows, cols, n, opts, S, direction in runs:
        print(f"[no-alloc] n={n} sources={S} {direction} {opts}", flush=True)
        m = k2.Matrix(k2.Tree(rows, cols, n, n), k2.plan_defaults(**opts), device=dev)
        src = rng.integers(0, n, S).astype(np.uint32)
        want, want_levels, want_reached = m.bfs(src, direction)
        dist = torch.full((n, S), -7, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info()
        got, levels, reached = m.bfs_noalloc(src, dist, direction)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        assert free0 == free1, f"device memory moved by {free0 - free1} bytes"
        assert got.data_ptr() == dist.data_ptr()
        assert torch.equal(got, want)
        assert levels == want_levels and np.array_equal(reached, want_reached)
        if n <= 2 ** 12:
            ref = oracle.bfs(rows, cols, n, src, oracle.RIGHT if direction == "right" else oracle.LEFT)
            assert np.array_equal(got.cpu().numpy(), ref)


def test_noalloc_search_refuses_oversize(dev):
    import tree_graph_spmv_amd as k2
    n = 2 ** 20
    rows, cols = synth.rmat(20, 5000, seed=43)
    m = k2.Matrix(k2.Tree(rows, cols, n, n), device=dev)
    S = 64   # two words per vertex: about 75 MB of workspace, over the 64 MiB array
    dist = torch.full((n, S), -7, dtype=torch.int32, device=dev)
    with pytest.raises(k2.K2Error) as e:
        m.bfs_noalloc(np.arange(S, dtype=np.uint32), dist)
    assert e.value.status == k2.K2_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert int((dist != -7).sum()) == 0
