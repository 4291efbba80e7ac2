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
    p.add_argument("--cpu-one-core-stride", type=int, default=256,
                   help="one-core oracle sample: the edges whose source is a multiple of this")
    p.add_argument("--no-per-config", action="store_true",
                   help="skip the other workloads (per_config in the JSON line)")
    p.add_argument("--bfs", type=int, default=0,
                   help="time multi-source searches from this many seeded sources instead of products")
    p.add_argument("--stream-mb", type=int, default=0,
                   help="time out-of-core products streamed through a staging buffer of this many MB")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a 1 GiB device copy (counter calibration) and exit")
    p.add_argument("--probe", default=None,
                   choices=("copy", "read", "write", "update", "gather", "scatter", "lds", "all"),
                   help="ceiling microbenchmarks (k2_probe_run): one JSON line per measurement, then exit")
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


def probe_bench(which, reps=5):
    """Ceiling microbenchmarks in the style of the paper's Sec. 5.6 / Table 4
    (copy bandwidth, consecutive and scattered y_o += x_i update rates) plus
    the operations the kernels use: random gathers and atomic scatters of
    batch rows (R = 8 floats, 32 bytes, as a batch-8 row of x or y) over a
    2^27-row vector, and LDS window updates.  Each line reports the median
    of 'reps' launches timed with HIP events."""
    import torch

    import tree_graph_spmv_amd as k2
    dev = torch.device("cuda:0")

    def run(name, kind, a, b, idx=None, n=0, row_elems=1, r=0, per_launch=None, unit=None, note=""):
        k2.probe(kind, a, b, idx, n, row_elems, r)   # warm-up
        times = sorted(k2.probe(kind, a, b, idx, n, row_elems, r) for _ in range(reps))
        ms = times[len(times) // 2]
        rate = per_launch / (ms / 1000.0)
        print(json.dumps({"probe": name, "kind": kind, "value": rate / 1e9, "unit": unit, "ms": ms,
                          "launches": reps, "per_launch": per_launch, "note": note}), flush=True)

    want = (lambda k: which in (k, "all"))
    N = 1 << 28   # 1 GiB of floats
    if want("copy") or want("read") or want("write") or want("update"):
        a = torch.rand(N, device=dev)
        b = torch.zeros(N, device=dev)
        if want("copy"):
            run("copy", "copy", a, b, n=N, per_launch=8 * N, unit="GB/s", note="1 GiB read + 1 GiB written")
        if want("read"):
            run("read", "read", a, b, n=N, per_launch=4 * N, unit="GB/s", note="1 GiB read")
        if want("write"):
            run("write", "write", None, b, n=N, per_launch=4 * N, unit="GB/s", note="1 GiB written")
        if want("update"):
            run("update_seq_atomic", "update_seq_atomic", a, b, n=N, per_launch=N, unit="G updates/s",
                note="y[i] += x[i], device-scope atomic add, 2^28 consecutive entries")
            run("update_seq_store", "update_seq_store", a, b, n=N, per_launch=N, unit="G updates/s",
                note="y[i] = y[i] + x[i], plain load and store, 2^28 consecutive entries")
        del a, b
    rows = 1 << 27
    if want("gather") or want("scatter"):
        for R in (8, 1):
            x = torch.rand(rows * R, device=dev)
            n_idx = rows
            idx = torch.randint(0, rows, (n_idx,), device=dev, dtype=torch.int32)
            if want("gather"):
                out = torch.zeros(1 << 24, device=dev)
                for kind, how in (("gather_rows", "plain loads"), ("gather_rows_nt", "non-temporal loads"),
                                  ("gather_rows_buf_nt", "buffer loads, sc0 nt"),
                                  ("gather_rows_buf_sys", "buffer loads, sc0 sc1")):
                    run(f"{kind}_R{R}", kind, x, out, idx, n=n_idx, row_elems=R, r=rows,
                        per_launch=n_idx, unit="G rows/s",
                        note=f"2^27 rows of {4 * R} bytes gathered at uniform random rows of a "
                             f"{4 * R}x2^27-byte x, {how}")
                if R == 8:
                    # the same gathers from an x that the caches hold: 1 MB
                    # (inside every XCD's 4 MB L2) and 128 MB (inside the
                    # 256 MB MALL, not the L2s)
                    for lg, where in ((15, "L2"), (22, "MALL")):
                        xs = x[: (1 << lg) * R]
                        ids = torch.randint(0, 1 << lg, (n_idx,), device=dev, dtype=torch.int32)
                        run(f"gather_rows_R{R}_{where}", "gather_rows", xs, out, ids, n=n_idx, row_elems=R,
                            r=1 << lg, per_launch=n_idx, unit="G rows/s",
                            note=f"2^27 rows of {4 * R} bytes gathered at uniform random rows of a "
                                 f"{4 * R}x2^{lg}-byte x (resident in the {where}), plain loads")
                        del ids
            if want("scatter"):
                y = torch.zeros(rows * R, device=dev)
                src = torch.rand(n_idx * R, device=dev)
                run(f"scatter_rows_atomic_R{R}", "scatter_rows_atomic", src, y, idx, n=n_idx, row_elems=R,
                    per_launch=n_idx, unit="G rows/s",
                    note=f"2^27 rows of {4 * R} bytes atomically added at uniform random rows of y")
                del y, src
            del x, idx
    if want("lds"):
        wgs = 256 * 8 * 4
        out = torch.zeros(wgs * 256, device=dev)
        per = wgs * 256 * 256
        for kind in ("lds_add_f32", "lds_cas_f32", "lds_add_u32"):
            run(kind, kind, None, out, n=wgs, row_elems=8, r=256, per_launch=per, unit="G updates/s",
                note="8192 workgroups x 256 lanes x 256 updates at random rows (8 floats) of a 16 KB window")


ORACLE_SEMIRING = {"plus_times": 0, "boolean": 1, "boolean_u32": 2, "tropical": 3}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_threads():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(int(n), 64))


def time_oracle(tree, x_by_dir, batch, directions, semiring, threads, runs=3):
    """The oracle's products timed as the paper's protocol asks (one
    warm-up, then the median of 'runs'), per direction, in seconds."""
    import oracle
    out = {}
    for d in directions:
        how = oracle.RIGHT if d == "right" else oracle.LEFT
        tree.spmv(x_by_dir[d], ORACLE_SEMIRING[semiring], how, batch, threads=threads)   # warm-up
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            tree.spmv(x_by_dir[d], ORACLE_SEMIRING[semiring], how, batch, threads=threads)
            ts.append(time.perf_counter() - t0)
        out[d] = statistics.median(ts)
    return out


def cpu_baseline(rows, cols, n, x_by_dir, batch, directions, semiring, stride, stride_one):
    """The oracle, as it is, on the edges whose source is a multiple of
    'stride' (same dimensions, same x), on every host core: one warm-up
    product per direction, then the median of three.  The same on one core,
    on the smaller sample of sources divisible by 'stride_one' (a product of
    the larger sample takes about 40 s on one core).  The oracle's builds
    (single-threaded) are reported, not counted."""
    import oracle
    threads = host_threads()
    sel = (rows % stride) == 0
    t0 = time.perf_counter()
    tree = oracle.OracleTree(rows[sel], cols[sel], n, n)
    build_s = time.perf_counter() - t0
    per = time_oracle(tree, x_by_dir, batch, directions, semiring, threads)
    nnz = tree.nnz
    del tree
    sel1 = (rows % stride_one) == 0
    t0 = time.perf_counter()
    tree1 = oracle.OracleTree(rows[sel1], cols[sel1], n, n)
    build1_s = time.perf_counter() - t0
    per1 = time_oracle(tree1, x_by_dir, batch, directions, semiring, 1)
    nnz1 = tree1.nnz
    del tree1
    products = len(directions)
    return {"value": nnz * products / sum(per.values()), "unit": "edges/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"edges with source % {stride} == 0 ({nnz} distinct of the workload's), "
                       f"same 2^{int(round(__import__('math').log2(n)))} dimensions and x; per direction "
                       f"({' and '.join(directions)}, batch {batch}) the median of 3 products after one "
                       f"warm-up, on {threads} threads; oracle build {build_s:.1f} s (one core) not counted"),
            "cpu_model": cpu_model(), "runs": 3, "warmup": 1,
            "seconds_per_product": per, "build_s": build_s,
            "one_core": {"value": nnz1 * products / sum(per1.values()), "unit": "edges/s", "cores": 1,
                         "sample": f"edges with source % {stride_one} == 0 ({nnz1} distinct); median of 3 "
                                   f"after one warm-up per direction",
                         "seconds_per_product": per1, "build_s": build1_s}}


# The other workloads of the benchmark set, each at its stated semiring,
# batch and directions, measured after the headline one.
PER_CONFIG = ("rmat_s12_e32k", "web_n20_d16", "rmat_s22_e64m", "symrmat_s24_e256m")
# full-size oracle timings: all cores for these, one core only where a
# product takes seconds (rmat_s22_e64m: about 45 s a product on one core)
CPU_FULL = {"rmat_s12_e32k": (True, True), "web_n20_d16": (True, True), "rmat_s22_e64m": (True, False)}


def warm_kernels(k2, opts, semiring, batch, directions, mode, dev):
    """Launch the product's kernels once on a 4x4 matrix: the runtime loads
    a kernel's code on its first launch, which would otherwise count as
    memory the library took."""
    import torch
    tm = k2.Matrix(k2.Tree([0], [0], 4, 4), opts, device=dev)
    tx = torch.zeros(4 * batch, dtype=torch.int32 if semiring == "boolean_u32" else torch.float32, device=dev)
    for d in directions:
        tm.spmv(tx, direction=d, semiring=semiring, batch=batch, mode=mode)
    torch.cuda.synchronize()


def measure_products(k2, tree, nodes, n, semiring, batch, directions, mode, x, dev, steps, warmup):
    """Mean kernel and fill times (HIP events) of 'steps' products per
    direction after 'warmup', with the device bytes against the estimate."""
    import torch
    opts = k2.plan_defaults(cache_last_level=int(mode == "cached"))
    est = tree.estimate(opts, semiring=semiring, batch=batch)
    warm_kernels(k2, opts, semiring, batch, directions, mode, dev)
    y = torch.empty(n * batch, dtype=x.dtype, device=dev)
    arena = k2.Matrix.arena_for(tree, opts, dev)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    m = k2.Matrix(tree, opts, device=dev, arena=arena)
    for d in directions:
        m.spmv(x, y, direction=d, semiring=semiring, batch=batch, mode=mode)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    lib_alloc = free0 - free1
    for _ in range(warmup):
        for d in directions:
            m.spmv(x, y, direction=d, semiring=semiring, batch=batch, mode=mode)
    torch.cuda.synchronize()
    m.set_timing(True)
    per = {}
    for d in directions:
        ks, fs = [], []
        for _ in range(steps):
            m.spmv(x, y, direction=d, semiring=semiring, batch=batch, mode=mode)
            f_ms, k_ms = m.last_timing()
            ks.append(k_ms)
            fs.append(f_ms)
        k_ms, f_ms = statistics.mean(ks), statistics.mean(fs)
        alg, struct, vec = algorithmic_bytes(nodes, m.top_level, n, n, batch, mode)
        gbs = alg / (k_ms / 1000.0) / 1e9
        per[d] = {"kernel_ms": k_ms, "fill_ms": f_ms, "edges_per_s": tree.nnz / ((k_ms + f_ms) / 1000.0),
                  "alg_bytes": alg, "alg_gbs": gbs, "frac": gbs / PEAK_HBM_GBS}
    m.set_timing(False)
    used = arena.numel() + x.numel() * 4 + y.numel() * 4 + lib_alloc
    mem = {"estimate": est, "used": int(used), "library_allocated": int(lib_alloc),
           "within_estimate": bool(used <= est["total"])}
    del m, arena, y
    torch.cuda.empty_cache()
    return per, mem


def per_config_bench(k2, dev, steps, warmup, cpu):
    """Every other workload of the set: tree-only and cached products in its
    directions (GPU), and, for the three smaller ones, the oracle on the
    full input (all cores; one core on the two smallest)."""
    import numpy as np
    import torch

    import synth
    out = {}
    for name in PER_CONFIG:
        w = synth.WORKLOADS[name]
        t0 = time.perf_counter()
        rows, cols, n = synth.workload_edges(name)
        tree = k2.Tree(rows, cols, n, n)
        nodes = tree.level_nodes()
        xh = synth.workload_x(name, n)
        x = torch.from_numpy(xh.view(np.int32) if xh.dtype == np.uint32 else xh).to(dev)
        rec = {"vertices": n, "edges": tree.nnz, "tree_nodes": tree.nodes, "semiring": w["semiring"],
               "batch": w["batch"], "directions": list(w["directions"]),
               "setup_s": round(time.perf_counter() - t0, 2)}
        for mode in ("tree", "cached"):
            per, mem = measure_products(k2, tree, nodes, n, w["semiring"], w["batch"], w["directions"], mode,
                                        x, dev, steps, warmup)
            rec[mode] = {"per_direction": per, "device_bytes": mem}
        log(f"per-config {name}: " + ", ".join(
            f"{mode} {d} {rec[mode]['per_direction'][d]['kernel_ms']:.3f} ms" for mode in ("tree", "cached")
            for d in w["directions"]))
        del x
        if cpu and name in CPU_FULL:
            import oracle
            all_core, one_core = CPU_FULL[name]
            t0 = time.perf_counter()
            ot = oracle.OracleTree(rows, cols, n, n)
            build_s = time.perf_counter() - t0
            xs = {d: xh for d in w["directions"]}
            c = {"kind": "oracle", "unit": "edges/s", "sample": "the whole workload", "build_s": build_s,
                 "runs": 3, "warmup": 1}
            if all_core:
                per = time_oracle(ot, xs, w["batch"], w["directions"], w["semiring"], host_threads())
                c["all_cores"] = {"value": ot.nnz * len(per) / sum(per.values()), "cores": host_threads(),
                                  "seconds_per_product": per}
            if one_core:
                per = time_oracle(ot, xs, w["batch"], w["directions"], w["semiring"], 1)
                c["one_core"] = {"value": ot.nnz * len(per) / sum(per.values()), "cores": 1,
                                 "seconds_per_product": per}
            rec["cpu_baseline"] = c
            del ot
        out[name] = rec
        del tree, rows, cols, xh
    return out


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
        print(json.dumps({"error": "the benchmark runs the product on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.probe:
        probe_bench(args.probe)
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
                         "within_estimate": bool(used <= est["total"]),
                         "breakdown": est,
                         # 8 bytes (block origin) and 4 (node word) per node of the
                         # last internal level; the rest of cached_codes is the stray
                         # records (8 bytes per stray and direction)
                         "cached_level": 8 * nodes[-2] if mode == "cached" else 0,
                         "node_words": 4 * nodes[-2] if mode == "cached" else 0,
                         "stray_records": (est["cached_codes"] - 12 * nodes[-2]) if mode == "cached" else 0,
                         "arena_without_strays": tree.estimate(k2.plan_defaults(
                             tile_nodes=args.tile_nodes, cache_last_level=int(mode == "cached"),
                             **{**extra, "band_strays": 0}), semiring=semiring, batch=batch)["arena"],
                         "tree_only": tree.estimate(k2.plan_defaults(tile_nodes=args.tile_nodes),
                                                    semiring=semiring, batch=batch)},
        "setup_s": {"generate": gen_s, "build": build_s, "create": create_s},
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_per_config:
        del m, arena
        torch.cuda.empty_cache()
        result["per_config"] = per_config_bench(k2, dev, steps=10, warmup=2, cpu=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a sample)")
        xh = {d: xs[d].cpu().numpy() for d in directions}
        xh = {d: (v.view(np.uint32) if v.dtype == np.int32 else v) for d, v in xh.items()}
        result["cpu_baseline"] = cpu_baseline(rows, cols, n, xh, batch, directions, semiring,
                                              args.cpu_sample_stride, args.cpu_one_core_stride)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
