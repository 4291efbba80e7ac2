"""CPU oracle for k^2-tree SpMV -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library under
``tree_graph_spmv_amd`` never imports, links or calls it, and the two share no
code: the oracle is plain C (``k2_oracle.c``) built with gcc, wrapped here
with ctypes over numpy arrays.

Everything it computes follows Tosoni & Mencagli, "A GPU Engine for Sparse
Matrix-Vector Products on k^2-Tree-Compressed Graphs": the tree of Sec. 2.1,
the semiring product of Sec. 2.2 / Table 1, and the sampled directory of
Sec. 3.2.  The readings taken where the pages are silent are listed at the
top of ``k2_oracle.c``.

Parity pins for every function here live in ``tests/test_oracle_pins.py``;
fp32 plus-times results on the GPU side are pinned only by tolerance, since
the order in which atomics land is free.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "k2_oracle.c")
_LIB = os.path.join(_HERE, "libk2oracle.so")

PLUS_TIMES, BOOLEAN_F32, BOOLEAN_U32, TROPICAL = 0, 1, 2, 3
RIGHT, LEFT = 0, 1

_lib = None


def build_library():
    """Compile the oracle with gcc (plain -O2, OpenMP for the band split)."""
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
    u64p = ctypes.POINTER(ctypes.c_uint64)
    vp = ctypes.c_void_p
    lib.orc_build.argtypes = [u32p, u32p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                              ctypes.POINTER(vp)]
    lib.orc_build.restype = ctypes.c_int
    lib.orc_free.argtypes = [vp]
    lib.orc_levels.argtypes = [vp]
    lib.orc_levels.restype = ctypes.c_int
    lib.orc_nnz.argtypes = [vp]
    lib.orc_nnz.restype = ctypes.c_uint64
    lib.orc_level_nodes.argtypes = [vp, ctypes.c_int]
    lib.orc_level_nodes.restype = ctypes.c_uint64
    lib.orc_level_nwords.argtypes = [vp, ctypes.c_int]
    lib.orc_level_nwords.restype = ctypes.c_uint64
    lib.orc_level_words.argtypes = [vp, ctypes.c_int, u64p]
    lib.orc_child_offsets.argtypes = [vp, ctypes.c_int, u64p]
    lib.orc_directory.argtypes = [vp, ctypes.c_int, ctypes.c_uint64, u64p]
    lib.orc_cells.argtypes = [vp, u32p, u32p]
    lib.orc_cells.restype = ctypes.c_uint64
    lib.orc_spmv.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, vp, vp, ctypes.c_int]
    lib.orc_spmv.restype = ctypes.c_int
    lib.orc_spmv_edges.argtypes = [u32p, u32p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_uint32, vp, vp]
    lib.orc_spmv_edges.restype = ctypes.c_int
    lib.orc_spmv_sample.argtypes = [u32p, u32p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_uint32, vp, u32p,
                                    ctypes.c_uint64, vp]
    lib.orc_spmv_sample.restype = ctypes.c_int
    lib.orc_bfs.argtypes = [u32p, u32p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, u32p,
                            ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    lib.orc_bfs.restype = ctypes.c_int
    _lib = lib
    return lib


def _u32(a):
    a = np.ascontiguousarray(a, dtype=np.uint32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))


def _out_dtype(semiring):
    return {PLUS_TIMES: np.float64, BOOLEAN_F32: np.float32,
            BOOLEAN_U32: np.uint32, TROPICAL: np.float32}[semiring]


def _in_dtype(semiring):
    return np.uint32 if semiring == BOOLEAN_U32 else np.float32


class OracleError(RuntimeError):
    pass


def _check(rc):
    if rc != 0:
        raise OracleError({-1: "invalid argument", -2: "index out of range",
                           -3: "out of memory"}.get(rc, f"error {rc}"))


class OracleTree:
    """The k^2-tree built by plain recursive quadrant splitting."""

    def __init__(self, rows, cols, n_rows, n_cols):
        lib = _load()
        r, rp = _u32(rows)
        c, cp = _u32(cols)
        if r.shape != c.shape:
            raise ValueError("rows and cols differ in length")
        h = ctypes.c_void_p()
        _check(lib.orc_build(rp, cp, r.size, int(n_rows), int(n_cols), ctypes.byref(h)))
        self._h = h
        self._lib = lib   # kept for __del__, which may run after module teardown
        self.n_rows, self.n_cols = int(n_rows), int(n_cols)
        self.levels = lib.orc_levels(h)
        self.nnz = int(lib.orc_nnz(h))

    def __del__(self):
        h = getattr(self, "_h", None)
        lib = getattr(self, "_lib", None)
        if h is not None and h.value and lib is not None:
            lib.orc_free(h)
            self._h = None

    def level_nodes(self):
        lib = _load()
        return [int(lib.orc_level_nodes(self._h, d)) for d in range(self.levels)]

    def level_words(self, d):
        """Canonical export: node i's nibble at bits 4(i%16) of word i//16."""
        lib = _load()
        nw = int(lib.orc_level_nwords(self._h, d))
        out = np.zeros(nw, dtype=np.uint64)
        lib.orc_level_words(self._h, d, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)))
        return out

    def signatures(self, d):
        """Level d's signatures as small ints (node order)."""
        words = self.level_words(d)
        n = self.level_nodes()[d]
        idx = np.arange(n, dtype=np.uint64)
        return ((words[idx // 16] >> ((idx % 16) * 4)) & 0xF).astype(np.uint8)

    def child_offsets(self, d):
        lib = _load()
        n = self.level_nodes()[d]
        out = np.zeros(n, dtype=np.uint64)
        lib.orc_child_offsets(self._h, d, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)))
        return out

    def directory(self, d, S):
        lib = _load()
        n = self.level_nodes()[d]
        out = np.zeros((n + S - 1) // S, dtype=np.uint64)
        lib.orc_directory(self._h, d, S, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)))
        return out

    def cells(self):
        lib = _load()
        r = np.zeros(max(self.nnz, 1), dtype=np.uint32)
        c = np.zeros(max(self.nnz, 1), dtype=np.uint32)
        k = lib.orc_cells(self._h, r.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                          c.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)))
        return r[:k], c[:k]

    def spmv(self, x, semiring, direction=RIGHT, batch=1, threads=1):
        """y = A x (RIGHT) or x^T A (LEFT); x, y row-major (n, batch)."""
        lib = _load()
        n_in = self.n_cols if direction == RIGHT else self.n_rows
        n_out = self.n_rows if direction == RIGHT else self.n_cols
        x = np.ascontiguousarray(x, dtype=_in_dtype(semiring)).reshape(-1)
        if x.size != n_in * batch:
            raise ValueError(f"x has {x.size} entries, expected {n_in * batch}")
        y = np.zeros(n_out * batch, dtype=_out_dtype(semiring))
        _check(lib.orc_spmv(self._h, direction, semiring, batch, x.ctypes.data, y.ctypes.data,
                            int(threads)))
        return y if batch == 1 else y.reshape(n_out, batch)


def spmv_edges(rows, cols, n_rows, n_cols, x, semiring, direction=RIGHT, batch=1):
    """The product straight from the definition over the deduplicated edges."""
    lib = _load()
    r, rp = _u32(rows)
    c, cp = _u32(cols)
    n_in = n_cols if direction == RIGHT else n_rows
    n_out = n_rows if direction == RIGHT else n_cols
    x = np.ascontiguousarray(x, dtype=_in_dtype(semiring)).reshape(-1)
    if x.size != n_in * batch:
        raise ValueError("x has the wrong length")
    y = np.zeros(n_out * batch, dtype=_out_dtype(semiring))
    _check(lib.orc_spmv_edges(rp, cp, r.size, n_rows, n_cols, direction, semiring, batch,
                              x.ctypes.data, y.ctypes.data))
    return y if batch == 1 else y.reshape(n_out, batch)


def spmv_sample(rows, cols, n_rows, n_cols, x, semiring, sample, direction=RIGHT, batch=1):
    """Outputs sample[k] of the product, from the definition (distinct sample)."""
    lib = _load()
    r, rp = _u32(rows)
    c, cp = _u32(cols)
    s, sp = _u32(sample)
    n_in = n_cols if direction == RIGHT else n_rows
    x = np.ascontiguousarray(x, dtype=_in_dtype(semiring)).reshape(-1)
    if x.size != n_in * batch:
        raise ValueError("x has the wrong length")
    y = np.zeros(s.size * batch, dtype=_out_dtype(semiring))
    _check(lib.orc_spmv_sample(rp, cp, r.size, n_rows, n_cols, direction, semiring, batch,
                               x.ctypes.data, sp, s.size, y.ctypes.data))
    return y if batch == 1 else y.reshape(s.size, batch)


def bfs(rows, cols, n, sources, direction=RIGHT, max_levels=2 ** 31 - 1):
    """Hop distances (n, len(sources)) int32 from each source of the square
    n x n matrix, -1 where unreached within max_levels (Sec. 5.8).  A RIGHT
    step reaches row r from column c for a cell (r, c); LEFT the reverse."""
    lib = _load()
    r, rp = _u32(rows)
    c, cp = _u32(cols)
    s, sp = _u32(sources)
    dist = np.empty((n, s.size), np.int32)
    _check(lib.orc_bfs(rp, cp, r.size, n, direction, sp, s.size, max_levels, dist.ctypes.data))
    return dist
