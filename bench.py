"""Benchmark: k^2-tree SpMV on one MI355X.

Default workload: web-like graph, 2^27 vertices, ~1.2G distinct edges (mean
out-degree 9, 85% of targets within +-4096 of the source), last internal level
cached, plus-times over a batch of 8 fp32 vectors; one step = one right and one
left product (fill + cached-level leaf kernel each).  Inputs are resident in
HBM before the timed region starts.

Prints one JSON line: edges/s over the step (both products), the dominant
kernel's roofline (algorithmic bytes per launch over its HIP-event duration),
device bytes (estimate vs measured) and the CPU oracle's rate on a bounded
sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, published


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="web_n27_d9")
    p.add_argument("--mode", default=None, help="tree or cached (default: the workload's)")
    p.add_argument("--tile-nodes", type=int, default=1024)
    p.add_argument("--batch", type=int, default=None, help="vectors per product (default: the workload's)")
    p.add_argument("--window-elems", type=int, default=None, help="plan option (default: the library's)")
    p.add_argument("--window-batch", type=int, default=None, help="plan option (default: the library's)")
    p.add_argument("--offsets", default=None, choices=("auto", "directory", "scan"),
                   help="plan option (default: the library's)")
    p.add_argument("--xcd-remap", type=int, default=None, help="plan option (default: the library's)")
    p.add_argument("--band-strays", type=int, default=None, help="plan option (default: the library's)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-stride", type=int, default=8,
                   help="oracle sample: the edges whose source is a multiple of this")
    p.add_argument("--bfs", type=int, default=0,
                   help="time multi-source searches from this many seeded sources instead of products")
    p.add_argument("--stream-mb", type=int, default=0,
                   help="time out-of-core products streamed through a staging buffer of this many MB")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a 1 GiB device copy (counter calibration) and exit")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the sources that decide the main kernel's memory traffic: the
    device code and the tile planner (tile order changes what the caches
    catch)."""
    h = hashlib.sha256()
    for name in ("k2_device.hip", "k2_plan.cpp"):
        with open(os.path.join(ROOT, "tree_graph_spmv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(nodes, top, n_in, n_out, batch, mode, elem=4):
    """Bytes a product's main kernel must move: matrix structure read once,
    x read once, y read and written once (the atomics' read-modify-write)."""
    L = len(nodes)
    vec = elem * n_in * batch + 2 * elem * n_out * batch
    if mode == "cached":
        n2, n1 = nodes[L - 2], nodes[L - 1]
        struct = 8 * n2 + 8 * ((n2 + 15) // 16) + 4 * ((n2 + 255) // 256) + 8 * ((n1 + 15) // 16)
    else:
        struct = sum(8 * ((nodes[d] + 15) // 16) for d in range(top, L))
        struct += sum(4 * ((nodes[d] + 255) // 256) for d in range(top, L - 1))
        struct += 8 * nodes[top]
    return struct + vec, struct, vec


def copy_probe():
    import torch
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": a.numel() * 4, "copy_probe_bytes_written":
                      a.numel() * 4, "launches": 5}))


ORACLE_SEMIRING = {"plus_times": 0, "boolean": 1, "boolean_u32": 2, "tropical": 3}


def cpu_baseline(rows, cols, n, x_by_dir, batch, directions, stride, semiring):
    """The oracle, as it is, on the edges whose source is a multiple of
    'stride' (same dimensions, same x): one product per direction."""
    import numpy as np

    import oracle
    sel = (rows % stride) == 0
    r, c = rows[sel], cols[sel]
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(int(threads), 64))
    t0 = time.perf_counter()
    tree = oracle.OracleTree(r, c, n, n)
    build_s = time.perf_counter() - t0
    total_s = 0.0
    for d in directions:
        t0 = time.perf_counter()
        tree.spmv(x_by_dir[d], ORACLE_SEMIRING[semiring], oracle.RIGHT if d == "right" else oracle.LEFT,
                  batch, threads=threads)
        total_s += time.perf_counter() - t0
    products = len(directions)
    return {"value": tree.nnz * products / total_s, "unit": "edges/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"edges with source % {stride} == 0 ({tree.nnz} distinct of the workload's), "
                       f"same 2^{int(np.log2(n))} dimensions and x; one {' and one '.join(directions)}"
                       f" product, batch {batch}; oracle build {build_s:.1f} s "
                       f"not counted"),
            "seconds": total_s}


def search_bench(args, k2, tree, opts, n, mode, dev):
    """Multi-source search (k2_bfs) from args.bfs seeded sources, right and
    left: mean wall time of a whole search (every level, with its host read
    of the level's count) over args.steps searches after args.warmup
    two-level ones."""
    import numpy as np
    import torch
    src = np.random.default_rng(9).integers(0, n, args.bfs).astype(np.uint32)
    m = k2.Matrix(tree, opts, device=dev)
    per = {}
    for d in ("right", "left"):
        for _ in range(max(args.warmup, 1)):
            m.bfs(src, d, max_levels=2)
        torch.cuda.synchronize()
        times = []
        for _ in range(max(args.steps, 1)):
            t0 = time.perf_counter()
            dist, levels, reached = m.bfs(src, d, max_levels=1 << 16)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
            del dist
        per[d] = {"levels": levels, "search_s": sum(times) / len(times), "min_s": min(times),
                  "reached": int(reached.sum()) if reached is not None else None}
        log(f"search {d}: {levels} levels, {per[d]['search_s']:.4f} s")
    print(json.dumps({"metric": "multi_source_search_s", "unit": "s", "higher_is_better": False,
                      "workload": args.workload, "mode": mode, "sources": args.bfs, "steps": args.steps,
                      "warmup": args.warmup, "data": "synthetic", "per_direction": per,
                      "kernel_source": kernel_source_hash()}))


def stream_bench(args, k2, tree, opts, n, semiring, batch, directions, dev):
    """Out-of-core products (k2_stream_*): the tree stays in host memory and
    each product streams it through a staging buffer of args.stream_mb MB.
    Reports each direction's mean wall time over args.steps products after
    args.warmup, the bytes one product copies and the rate they imply."""
    import numpy as np
    import torch
    import synth
    t0 = time.perf_counter()
    s = k2.Streamed(tree, args.stream_mb << 20, opts)
    plan_s = time.perf_counter() - t0
    buf = s.staging(dev)
    xh = synth.workload_x(args.workload, n, batch=batch)
    x = torch.from_numpy(xh.view(np.int32) if xh.dtype == np.uint32 else xh).to(dev)
    y = torch.empty(n * batch, dtype=x.dtype, device=dev)
    per = {}
    for d in directions:
        for _ in range(max(args.warmup, 1)):
            s.spmv(x, y, direction=d, semiring=semiring, batch=batch, staging=buf)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(max(args.steps, 1)):
            s.spmv(x, y, direction=d, semiring=semiring, batch=batch, staging=buf)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / max(args.steps, 1)
        per[d] = {"product_s": sec, "edges_per_s": tree.nnz / sec,
                  "staged_gb_per_s": s.staged_bytes / sec / 1e9}
        log(f"streamed {d}: {sec * 1e3:.1f} ms per product")
    print(json.dumps({"metric": "streamed_product_edges_per_s", "unit": "edges/s", "higher_is_better": True,
                      "workload": args.workload, "semiring": semiring, "batch": batch,
                      "staging_mb": args.stream_mb, "chunks": s.n_chunks, "max_chunk_bytes": s.max_chunk_bytes,
                      "staged_bytes_per_product": s.staged_bytes, "plan_s": plan_s, "steps": args.steps,
                      "warmup": args.warmup, "data": "synthetic", "per_direction": per,
                      "kernel_source": kernel_source_hash()}))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return

    import numpy as np
    import torch

    import synth
    import tree_graph_spmv_amd as k2

    w = synth.WORKLOADS[args.workload]
    mode = args.mode or ("cached" if w["cached"] else "tree")
    batch = args.batch or w["batch"]
    semiring = w["semiring"]
    directions = list(w["directions"])
    dev = torch.device("cuda:0")

    t0 = time.perf_counter()
    rows, cols, n = synth.workload_edges(args.workload)
    gen_s = time.perf_counter() - t0
    log(f"generated {len(rows)} edges in {gen_s:.1f}s")
    t0 = time.perf_counter()
    tree = k2.Tree(rows, cols, n, n)
    build_s = time.perf_counter() - t0
    nodes = tree.level_nodes()
    log(f"built: nnz={tree.nnz} nodes={tree.nodes} levels={tree.levels} in {build_s:.1f}s")

    extra = {k: v for k, v in (("window_elems", args.window_elems), ("window_batch", args.window_batch),
                               ("offsets", args.offsets), ("xcd_remap", args.xcd_remap),
                               ("band_strays", args.band_strays)) if v is not None}
    opts = k2.plan_defaults(tile_nodes=args.tile_nodes, cache_last_level=int(mode == "cached"), **extra)
    if args.bfs:
        search_bench(args, k2, tree, opts, n, mode, dev)
        return
    if args.stream_mb:
        stream_bench(args, k2, tree, opts, n, semiring, batch, directions, dev)
        return
    est = tree.estimate(opts, semiring=semiring, batch=batch)
    # run the same kernels once on a tiny matrix first (the runtime loads a
    # kernel's code on its first launch), so that the memory measured below
    # is the matrix's and the vectors' alone
    tiny = k2.Tree([0], [0], 4, 4)
    tm = k2.Matrix(tiny, opts, device=dev)
    tx = torch.zeros(4 * batch, dtype=torch.int32 if semiring == "boolean_u32" else torch.float32,
                     device=dev)
    for d in directions:
        tm.spmv(tx, direction=d, semiring=semiring, batch=batch, mode=mode)
    torch.cuda.synchronize()
    del tm, tx
    xh = synth.workload_x(args.workload, n, batch=batch)   # one x and one y serve both directions
    x = torch.from_numpy(xh.view(np.int32) if xh.dtype == np.uint32 else xh).to(dev)
    y = torch.empty(n * batch, dtype=x.dtype, device=dev)
    del xh
    arena = k2.Matrix.arena_for(tree, opts, dev)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    t0 = time.perf_counter()
    m = k2.Matrix(tree, opts, device=dev, arena=arena)
    torch.cuda.synchronize()
    create_s = time.perf_counter() - t0
    for d in directions:
        m.spmv(x, y, direction=d, semiring=semiring, batch=batch, mode=mode)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    lib_alloc = free0 - free1   # device memory the library took during create + products
    used = arena.numel() + x.numel() * 4 + y.numel() * 4 + lib_alloc
    log(f"matrix created in {create_s:.1f}s; device bytes estimate {est['total']} used {used} "
        f"(library allocations {lib_alloc})")
    xs = {d: x for d in directions}
    ys = {d: y for d in directions}

    def step():
        for d in directions:
            m.spmv(xs[d], ys[d], direction=d, semiring=semiring, batch=batch, mode=mode)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region.  HIP events on the product stream bracket the fill and the
    # main kernel of every product; reading them waits for that product, which
    # adds a host round trip per product to ms_per_step (tens of microseconds).
    m.set_timing(True)
    fills = {d: [] for d in directions}
    mains = {d: [] for d in directions}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for d in directions:
            m.spmv(xs[d], ys[d], direction=d, semiring=semiring, batch=batch, mode=mode)
            f_ms, k_ms = m.last_timing()
            fills[d].append(f_ms)
            mains[d].append(k_ms)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    m.set_timing(False)
    ms_per_step = 1000.0 * elapsed / args.steps
    log(f"{args.steps} steps in {elapsed:.3f}s")

    per_dir = {}
    for d in directions:
        alg, struct, vec = algorithmic_bytes(nodes, m.top_level, n, n, batch, mode)
        k_ms = statistics.mean(mains[d])
        f_ms = statistics.mean(fills[d])
        per_dir[d] = {"kernel_ms": k_ms, "kernel_ms_median": statistics.median(mains[d]),
                      "fill_ms": f_ms,
                      "edges_per_s": tree.nnz / ((k_ms + f_ms) / 1000.0),
                      "edges_per_s_per_vector": tree.nnz * batch / ((k_ms + f_ms) / 1000.0),
                      "alg_bytes": alg, "alg_struct_bytes": struct, "alg_vector_bytes": vec,
                      "alg_gbs": alg / (k_ms / 1000.0) / 1e9}

    dom = "right" if "right" in per_dir else directions[0]
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            tj = json.load(f)
        key = f"{args.workload}:{mode}:{dom}"
        if tj.get("kernel_source") == kernel_source_hash() and key in tj.get("per_launch_bytes", {}):
            traffic = tj["per_launch_bytes"][key]
    achieved = per_dir[dom]["alg_gbs"]
    result = {
        "metric": "edges/sec and achieved HBM GB/s (% of peak) per SpMV, right & left, 1 GPU",
        "value": tree.nnz * len(directions) / (ms_per_step / 1000.0),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if semiring != "boolean_u32" else "u32",
        "data": "synthetic",
        "config": {"workload": args.workload, "vertices": n, "edges": tree.nnz,
                   "tree_nodes": tree.nodes, "levels": tree.levels, "batch": batch,
                   "semiring": semiring, "mode": mode, "directions": directions,
                   "tile_nodes": args.tile_nodes, **extra},
        "roofline": {"kernel": f"{'cached_kernel' if mode == 'cached' else 'descent_kernel'} "
                               f"({dom} product)",
                     "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic},
        "per_direction": per_dir,
        "device_bytes": {"estimate": est["total"], "estimate_arena": est["arena"],
                         "used": int(used), "library_allocated": int(lib_alloc),
                         "within_estimate": bool(used <= est["total"])},
        "setup_s": {"generate": gen_s, "build": build_s, "create": create_s},
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a sample)")
        xh = {d: xs[d].cpu().numpy() for d in directions}
        xh = {d: (v.view(np.uint32) if v.dtype == np.int32 else v) for d, v in xh.items()}
        result["cpu_baseline"] = cpu_baseline(rows, cols, n, xh, batch, directions,
                                              args.cpu_sample_stride, semiring)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
