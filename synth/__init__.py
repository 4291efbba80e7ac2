"""Seeded synthetic inputs shared by the tests and the benchmark.

Input generation only (no tree, no product): R-MAT and web-like edge lists and
the dense vectors of the five workloads.  The C code (``synth.c``) is built
with gcc and wrapped with ctypes; all randomness is counter-based, so arrays
do not depend on the thread count.

Workloads (stand-ins for the pages' Wikidata, Software Heritage and web-crawl
graphs, which are not available here):

=====================  =========================================================
rmat_s12_e32k          R-MAT, 2^12 vertices, exactly 32,768 distinct edges
                       (a,b,c,d = .57,.19,.19,.05); plus-times right product.
web_n20_d16            web-like, 2^20 vertices, out-degree power law (density
                       exponent 2.1, mean 16 before deduplication, cap 4096),
                       80% of targets within +-1024 of the source; plus-times.
rmat_s22_e64m          R-MAT, 2^22 vertices, exactly 2^26 distinct edges;
                       tropical x: 10% uniform [0,100), else +inf.
symrmat_s24_e256m      symmetric R-MAT, 2^24 vertices, 2^28 distinct directed
                       edges, no self-loops; 32 Boolean vectors per uint32,
                       each bit set with probability 0.01.
web_n27_d9             web-like, 2^27 vertices, mean out-degree 9, 85% of
                       targets within +-4096; plus-times, batch of 8.
=====================  =========================================================
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def default_threads():
    """Host threads to use: the process's CPU share, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def build_library():
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build_library()
    lib = ctypes.CDLL(_LIB)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    f32p = ctypes.POINTER(ctypes.c_float)
    lib.synth_rmat.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_double, ctypes.c_double,
                               ctypes.c_double, ctypes.c_uint64, ctypes.c_int, u32p, u32p,
                               ctypes.c_int]
    lib.synth_rmat.restype = ctypes.c_int
    lib.synth_pareto_scale.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_uint32]
    lib.synth_pareto_scale.restype = ctypes.c_double
    lib.synth_web_degrees.argtypes = [ctypes.c_uint64, ctypes.c_double, ctypes.c_double,
                                      ctypes.c_uint32, ctypes.c_uint64, u32p, ctypes.c_int]
    lib.synth_web_degrees.restype = ctypes.c_uint64
    lib.synth_web_edges.argtypes = [ctypes.c_uint64, u32p, ctypes.c_double, ctypes.c_uint32,
                                    ctypes.c_uint64, u32p, u32p, ctypes.c_int]
    lib.synth_web_edges.restype = ctypes.c_int
    lib.synth_uniform01.argtypes = [ctypes.c_uint64, ctypes.c_uint64, f32p, ctypes.c_int]
    lib.synth_tropical.argtypes = [ctypes.c_uint64, ctypes.c_double, ctypes.c_double,
                                   ctypes.c_uint64, f32p, ctypes.c_int]
    lib.synth_bitmask.argtypes = [ctypes.c_uint64, ctypes.c_double, ctypes.c_uint64, u32p,
                                  ctypes.c_int]
    _lib = lib
    return lib


def _p32(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))


def rmat(scale, n_edges, a=0.57, b=0.19, c=0.19, seed=1, symmetric=False, threads=None):
    """Exactly n_edges distinct directed R-MAT edges on 2^scale vertices."""
    lib = _load()
    rows = np.empty(n_edges, np.uint32)
    cols = np.empty(n_edges, np.uint32)
    rc = lib.synth_rmat(scale, n_edges, a, b, c, seed, int(bool(symmetric)), _p32(rows), _p32(cols),
                        threads or default_threads())
    if rc != 0:
        raise ValueError("R-MAT parameters rejected (too dense, odd symmetric count, or no memory)")
    return rows, cols


def pareto_scale(mean, alpha, cap):
    return _load().synth_pareto_scale(mean, alpha, cap)


def web(n, mean, exponent=2.1, cap=4096, p_local=0.8, window=1024, seed=1, threads=None):
    """Web-like edge list (sources ascending, duplicates kept).

    Out-degrees follow a power law whose density decays as k^-exponent, i.e.
    floor of a Pareto variable of tail index exponent-1, capped, with the
    Pareto scale solved so that the capped mean equals ``mean``.
    """
    lib = _load()
    th = threads or default_threads()
    deg = np.empty(n, np.uint32)
    total = lib.synth_web_degrees(n, mean, exponent - 1.0, cap, seed, _p32(deg), th)
    rows = np.empty(total, np.uint32)
    cols = np.empty(total, np.uint32)
    if lib.synth_web_edges(n, _p32(deg), p_local, window, seed, _p32(rows), _p32(cols), th) != 0:
        raise MemoryError("web-like generator ran out of memory")
    return rows, cols


def uniform01(count, seed, threads=None):
    out = np.empty(count, np.float32)
    _load().synth_uniform01(count, seed, out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                            threads or default_threads())
    return out


def tropical(count, seed, p_finite=0.1, hi=100.0, threads=None):
    out = np.empty(count, np.float32)
    _load().synth_tropical(count, p_finite, hi, seed,
                           out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                           threads or default_threads())
    return out


def bitmask(count, seed, p=0.01, threads=None):
    out = np.empty(count, np.uint32)
    _load().synth_bitmask(count, p, seed, _p32(out), threads or default_threads())
    return out


# ------------------------------------------------------------ workloads

WORKLOADS = {
    "rmat_s12_e32k": dict(kind="rmat", scale=12, n_edges=32768, symmetric=False, seed=12,
                          semiring="plus_times", directions=("right",), batch=1, cached=False),
    "web_n20_d16": dict(kind="web", n=2 ** 20, mean=16, p_local=0.8, window=1024, seed=20,
                        semiring="plus_times", directions=("right", "left"), batch=1,
                        cached=False),
    "rmat_s22_e64m": dict(kind="rmat", scale=22, n_edges=2 ** 26, symmetric=False, seed=22,
                          semiring="tropical", directions=("right", "left"), batch=1,
                          cached=False),
    "symrmat_s24_e256m": dict(kind="rmat", scale=24, n_edges=2 ** 28, symmetric=True, seed=24,
                              semiring="boolean_u32", directions=("right",), batch=1,
                              cached=False),
    "web_n27_d9": dict(kind="web", n=2 ** 27, mean=9, p_local=0.85, window=4096, seed=27,
                       semiring="plus_times", directions=("right", "left"), batch=8,
                       cached=True),
}


def workload_edges(name, threads=None):
    """(rows, cols, n) of a named workload."""
    w = WORKLOADS[name]
    if w["kind"] == "rmat":
        r, c = rmat(w["scale"], w["n_edges"], seed=w["seed"], symmetric=w["symmetric"],
                    threads=threads)
        return r, c, 2 ** w["scale"]
    r, c = web(w["n"], w["mean"], p_local=w["p_local"], window=w["window"], seed=w["seed"],
               threads=threads)
    return r, c, w["n"]


def workload_x(name, n, seed_offset=0, threads=None, batch=None):
    """The input vector(s) of a named workload, row-major (n, batch) flattened
    (batch: the workload's unless given)."""
    w = WORKLOADS[name]
    seed = 1000 + w["seed"] + seed_offset
    count = n * (w["batch"] if batch is None else batch)
    if w["semiring"] == "tropical":
        return tropical(count, seed, threads=threads)
    if w["semiring"] == "boolean_u32":
        return bitmask(count, seed, threads=threads)
    return uniform01(count, seed, threads=threads)
