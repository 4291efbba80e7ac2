"""k^2-tree SpMV on AMD Instinct MI355X: Python binding of libk2spmv.so.

Argument marshalling only: every step of a product runs in the library's HIP
kernels.  torch supplies device memory (the arena and the vectors) and
streams.  The C functions keep their names (``k2_build``, ``k2_spmv``, ...);
the classes ``Tree`` and ``Matrix`` wrap the handles.

The library must have been built (``python -m tree_graph_spmv_amd._build`` or
``__graft_entry__.build()``); importing this package raises if it is missing,
and there is no fallback of any kind.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libk2spmv.so")

K2_OK, K2_E_INVALID_ARG, K2_E_INDEX_RANGE, K2_E_ARENA_TOO_SMALL, K2_E_HOST_OOM, K2_E_HIP, \
    K2_E_UNSUPPORTED = range(7)
K2_PLUS_TIMES_F32, K2_BOOLEAN_F32, K2_BOOLEAN_U32X32, K2_TROPICAL_F32 = range(4)
K2_RIGHT, K2_LEFT = 0, 1
K2_MODE_AUTO, K2_MODE_TREE_ONLY, K2_MODE_CACHED = 0, 1, 2
K2_SPMV_ACCUMULATE = 0x100
K2_OFFSETS_AUTO, K2_OFFSETS_DIRECTORY, K2_OFFSETS_SCAN = 0, 1, 2
OFFSETS = {"auto": K2_OFFSETS_AUTO, "directory": K2_OFFSETS_DIRECTORY, "scan": K2_OFFSETS_SCAN}

SEMIRINGS = {"plus_times": K2_PLUS_TIMES_F32, "boolean": K2_BOOLEAN_F32,
             "boolean_u32": K2_BOOLEAN_U32X32, "tropical": K2_TROPICAL_F32}
DIRECTIONS = {"right": K2_RIGHT, "left": K2_LEFT}
MODES = {"auto": K2_MODE_AUTO, "tree": K2_MODE_TREE_ONLY, "cached": K2_MODE_CACHED}


class PlanOpts(ctypes.Structure):
    _fields_ = [("tile_nodes", ctypes.c_uint32), ("host_top_max", ctypes.c_uint32),
                ("cache_last_level", ctypes.c_int32), ("xcd_remap", ctypes.c_int32),
                ("window_elems", ctypes.c_uint32), ("window_batch", ctypes.c_uint32),
                ("offsets", ctypes.c_int32), ("band_strays", ctypes.c_int32),
                ("band_tile_nodes", ctypes.c_uint32)]


class MemBreakdown(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("tree", "directory", "top_codes", "tiles", "cached_codes", "scratch",
                 "alignment", "arena", "vectors", "total")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class TreeInfo(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_uint32), ("n_cols", ctypes.c_uint32),
                ("levels", ctypes.c_uint32), ("top_level", ctypes.c_uint32),
                ("nnz", ctypes.c_uint64), ("nodes", ctypes.c_uint64)]


class K2Error(RuntimeError):
    def __init__(self, status, where):
        msg = lib().k2_status_string(status).decode()
        if status == K2_E_HIP:
            msg += " (" + lib().k2_last_hip_error().decode() + ")"
        super().__init__(f"{where}: {msg}")
        self.status = status


_lib = None

# name -> (restype, argtypes)
_VP = ctypes.c_void_p
_U32P = ctypes.POINTER(ctypes.c_uint32)
_U64P = ctypes.POINTER(ctypes.c_uint64)
_SIGS = {
    "k2_plan_defaults": (ctypes.c_int, [ctypes.POINTER(PlanOpts)]),
    "k2_build": (ctypes.c_int, [_U32P, _U32P, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                ctypes.c_uint32, ctypes.POINTER(_VP)]),
    "k2_tree_free": (None, [_VP]),
    "k2_tree_info": (ctypes.c_int, [_VP, ctypes.POINTER(TreeInfo)]),
    "k2_tree_level_nodes": (ctypes.c_int, [_VP, _U64P]),
    "k2_tree_level_words": (ctypes.c_int, [_VP, ctypes.c_uint32, _U64P, ctypes.c_uint64]),
    "k2_tree_directory": (ctypes.c_int, [_VP, ctypes.c_uint32, _U32P, ctypes.c_uint64]),
    "k2_estimate_device_bytes": (ctypes.c_int, [_VP, ctypes.POINTER(PlanOpts), ctypes.c_int,
                                                ctypes.c_uint32, ctypes.POINTER(MemBreakdown)]),
    "k2_plan_info": (ctypes.c_int, [_VP, ctypes.POINTER(PlanOpts), ctypes.c_int32, _U32P, _U64P,
                                    _U64P]),
    "k2_plan_tiles": (ctypes.c_int, [_VP, ctypes.POINTER(PlanOpts), ctypes.c_int32, _U32P,
                                     ctypes.c_uint64, _U64P, ctypes.c_uint64]),
    "k2_matrix_create": (ctypes.c_int, [_VP, ctypes.POINTER(PlanOpts), _VP, ctypes.c_uint64, _VP,
                                        ctypes.POINTER(_VP)]),
    "k2_spmv": (ctypes.c_int, [_VP, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_int32,
                               _VP, _VP, _VP]),
    "k2_matrix_destroy": (ctypes.c_int, [_VP]),
    "k2_matrix_info": (ctypes.c_int, [_VP, _U32P, _U64P, ctypes.POINTER(ctypes.c_int32)]),
    "k2_matrix_level_words": (ctypes.c_int, [_VP, ctypes.c_uint32, _U64P, ctypes.c_uint64, _VP]),
    "k2_plan_offsets": (ctypes.c_int, [_VP, _VP, _U32P, ctypes.c_uint64, _U64P]),
    "k2_bfs_workspace_bytes": (ctypes.c_int, [_VP, ctypes.c_uint32, _U64P]),
    "k2_bfs": (ctypes.c_int, [_VP, ctypes.c_int, _U32P, ctypes.c_uint32, ctypes.c_uint32, _VP, _VP,
                              ctypes.c_uint64, _VP, _U32P, _U64P]),
    "k2_bfs_noalloc": (ctypes.c_int, [_VP, ctypes.c_int, _U32P, ctypes.c_uint32, ctypes.c_uint32, _VP, _VP,
                                      _U32P, _U64P]),
    "k2_matrix_cached_blocks": (ctypes.c_int, [_VP, _U64P, ctypes.c_uint64, _VP]),
    "k2_matrix_set_timing": (ctypes.c_int, [_VP, ctypes.c_int32]),
    "k2_matrix_last_timing": (ctypes.c_int, [_VP, ctypes.POINTER(ctypes.c_float),
                                             ctypes.POINTER(ctypes.c_float)]),
    "k2_stream_create": (ctypes.c_int, [_VP, ctypes.POINTER(PlanOpts), ctypes.c_uint64, ctypes.POINTER(_VP)]),
    "k2_stream_info": (ctypes.c_int, [_VP, _U64P, _U64P, _U64P]),
    "k2_stream_chunk": (ctypes.c_int, [_VP, ctypes.c_uint64, _U64P, _U64P, _U64P, _U64P, ctypes.c_uint32]),
    "k2_stream_spmv": (ctypes.c_int, [_VP, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_int32, _VP, _VP,
                                      _VP, ctypes.c_uint64, _VP]),
    "k2_stream_destroy": (None, [_VP]),
    "k2_probe_run": (ctypes.c_int, [ctypes.c_int32, _VP, _VP, _VP, ctypes.c_uint64, ctypes.c_uint64,
                                    ctypes.c_uint32, ctypes.c_uint32, _VP, ctypes.POINTER(ctypes.c_float)]),
    "k2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "k2_last_hip_error": (ctypes.c_char_p, []),
}


def lib():
    """The loaded libk2spmv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m tree_graph_spmv_amd._build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def _check(status, where):
    if status != K2_OK:
        raise K2Error(status, where)


def _u32(a):
    a = np.ascontiguousarray(a, dtype=np.uint32)
    return a, a.ctypes.data_as(_U32P)


def plan_defaults(**kw):
    o = PlanOpts()
    _check(lib().k2_plan_defaults(ctypes.byref(o)), "k2_plan_defaults")
    for k, v in kw.items():
        if k == "offsets" and isinstance(v, str):
            v = OFFSETS[v]
        setattr(o, k, int(v))
    return o


class Tree:
    """Host k^2-tree (k2_build)."""

    def __init__(self, rows, cols, n_rows, n_cols, n_threads=0):
        r, rp = _u32(rows)
        c, cp = _u32(cols)
        if r.shape != c.shape:
            raise ValueError("rows and cols differ in length")
        h = _VP()
        _check(lib().k2_build(rp, cp, r.size, int(n_rows), int(n_cols), int(n_threads),
                              ctypes.byref(h)), "k2_build")
        self._h = h
        info = TreeInfo()
        _check(lib().k2_tree_info(h, ctypes.byref(info)), "k2_tree_info")
        self.n_rows, self.n_cols = int(info.n_rows), int(info.n_cols)
        self.levels, self.nnz, self.nodes = int(info.levels), int(info.nnz), int(info.nodes)

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.k2_tree_free(h)
            self._h = None

    def level_nodes(self):
        out = np.zeros(self.levels, np.uint64)
        _check(lib().k2_tree_level_nodes(self._h, out.ctypes.data_as(_U64P)), "k2_tree_level_nodes")
        return [int(v) for v in out]

    def level_words(self, level):
        n = self.level_nodes()[level]
        out = np.zeros((n + 15) // 16, np.uint64)
        _check(lib().k2_tree_level_words(self._h, level, out.ctypes.data_as(_U64P), out.size),
               "k2_tree_level_words")
        return out

    def directory(self, level):
        n = self.level_nodes()[level]
        out = np.zeros((n + 255) // 256, np.uint32)
        _check(lib().k2_tree_directory(self._h, level, out.ctypes.data_as(_U32P), out.size),
               "k2_tree_directory")
        return out

    def estimate(self, opts=None, semiring="plus_times", batch=1):
        opts = opts or plan_defaults()
        m = MemBreakdown()
        _check(lib().k2_estimate_device_bytes(self._h, ctypes.byref(opts), SEMIRINGS[semiring],
                                              int(batch), ctypes.byref(m)),
               "k2_estimate_device_bytes")
        return m.as_dict()

    def plan_offsets(self, opts=None):
        """The descent tiles' scan offsets (k2_plan_offsets), uint32."""
        opts = opts or plan_defaults()
        n = ctypes.c_uint64()
        _check(lib().k2_plan_offsets(self._h, ctypes.byref(opts), None, 0, ctypes.byref(n)),
               "k2_plan_offsets")
        out = np.zeros(max(n.value, 1), np.uint32)
        _check(lib().k2_plan_offsets(self._h, ctypes.byref(opts), out.ctypes.data_as(_U32P), n.value,
                                     ctypes.byref(n)), "k2_plan_offsets")
        return out[:n.value]

    def plan(self, opts=None, which=0):
        """(top_level, tiles (n,8) uint32, aux uint64) of one tile plan:
        which = 0 descent tiles (aux = start codes); 1 / 2 cached-level
        tiles of right / left products (aux = (n_segments, 2): (first node
        << 32) | count, and the first node's first leaf); 3-8 the tree-only
        lists; 9 / 10 the stray segments of right / left products (no tiles,
        aux as for 1 / 2)."""
        opts = opts or plan_defaults()
        top = ctypes.c_uint32()
        nt = ctypes.c_uint64()
        na = ctypes.c_uint64()
        _check(lib().k2_plan_info(self._h, ctypes.byref(opts), int(which), ctypes.byref(top),
                                  ctypes.byref(nt), ctypes.byref(na)), "k2_plan_info")
        tiles = np.zeros((max(nt.value, 1), 8), np.uint32)
        aux = np.zeros(max(na.value, 1), np.uint64)
        _check(lib().k2_plan_tiles(self._h, ctypes.byref(opts), int(which),
                                   tiles.ctypes.data_as(_U32P), nt.value, aux.ctypes.data_as(_U64P),
                                   na.value), "k2_plan_tiles")
        aux = aux[:na.value]
        return int(top.value), tiles[:nt.value], aux.reshape(-1, 2) if which in (1, 2, 9, 10) else aux


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return _VP(stream.cuda_stream)


class Matrix:
    """A tree resident in a device arena allocated through torch."""

    @staticmethod
    def arena_for(tree, opts=None, device="cuda"):
        """A torch uint8 device tensor of exactly the estimated arena size."""
        import torch
        est = tree.estimate(opts or plan_defaults())
        return torch.empty(max(est["arena"], 256), dtype=torch.uint8, device=device)

    def __init__(self, tree, opts=None, device="cuda", stream=None, arena=None):
        """Upload 'tree'.  'arena' (optional) is a caller-allocated uint8
        device tensor of at least the estimated arena size, 256-byte aligned;
        by default one is allocated here."""
        self.opts = opts or plan_defaults()
        est = tree.estimate(self.opts)
        self.arena_bytes = est["arena"]
        if arena is None:
            arena = Matrix.arena_for(tree, self.opts, device)
        if arena.numel() < self.arena_bytes or arena.data_ptr() % 256:
            raise ValueError("arena too small or not 256-byte aligned")
        self._raw = arena
        self.arena_ptr = arena.data_ptr()
        self.device = arena.device
        self.n_rows, self.n_cols, self.levels = tree.n_rows, tree.n_cols, tree.levels
        h = _VP()
        _check(lib().k2_matrix_create(tree.handle, ctypes.byref(self.opts), _VP(self.arena_ptr),
                                      self.arena_bytes, _stream_handle(stream), ctypes.byref(h)),
               "k2_matrix_create")
        self._h = h
        top = ctypes.c_uint32()
        nt = ctypes.c_uint64()
        cached = ctypes.c_int32()
        _check(lib().k2_matrix_info(h, ctypes.byref(top), ctypes.byref(nt), ctypes.byref(cached)),
               "k2_matrix_info")
        self.top_level, self.n_tiles, self.cached = int(top.value), int(nt.value), bool(cached.value)
        # the cached level's products read only its 4-byte node words
        self.packed_nodes = cached.value == 2

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.k2_matrix_destroy(h)
            self._h = None

    def set_timing(self, enable=True):
        _check(lib().k2_matrix_set_timing(self._h, int(bool(enable))), "k2_matrix_set_timing")

    def last_timing(self):
        """(fill ms, main kernel ms) of the last product (waits for it)."""
        a = ctypes.c_float()
        b = ctypes.c_float()
        _check(lib().k2_matrix_last_timing(self._h, ctypes.byref(a), ctypes.byref(b)),
               "k2_matrix_last_timing")
        return float(a.value), float(b.value)

    def spmv(self, x, y=None, direction="right", semiring="plus_times", batch=1, mode="auto",
             accumulate=False, stream=None):
        """y = A x ('right') or x^T A ('left'); x, y torch device tensors.
        accumulate=True: y is not filled first, the product is or-ed/added/
        min-ed into it (y must then be given)."""
        import torch
        d = DIRECTIONS[direction]
        n_in = self.n_cols if d == K2_RIGHT else self.n_rows
        n_out = self.n_rows if d == K2_RIGHT else self.n_cols
        dtype = torch.int32 if semiring == "boolean_u32" else torch.float32
        if x.dtype != dtype or x.numel() != n_in * batch or not x.is_contiguous():
            raise ValueError(f"x must be a contiguous {dtype} tensor of {n_in * batch} elements")
        if x.device != self.device:
            raise ValueError("x is not on the matrix's device")
        if y is None:
            if accumulate:
                raise ValueError("accumulate needs y")
            y = torch.empty(n_out * batch, dtype=dtype, device=self.device)
        elif y.dtype != dtype or y.numel() != n_out * batch or not y.is_contiguous():
            raise ValueError(f"y must be a contiguous {dtype} tensor of {n_out * batch} elements")
        if y.device != self.device:
            raise ValueError("y is not on the matrix's device")
        flags = MODES[mode] | (K2_SPMV_ACCUMULATE if accumulate else 0)
        _check(lib().k2_spmv(self._h, d, SEMIRINGS[semiring], int(batch), flags,
                             _VP(x.data_ptr()), _VP(y.data_ptr()), _stream_handle(stream)),
               "k2_spmv")
        return y

    def bfs(self, sources, direction="right", max_levels=2 ** 31 - 1, dist=None, workspace=None,
            stream=None):
        """Multi-source search to the fixed point (k2_bfs): returns (dist, levels,
        reached) with dist an (n, len(sources)) int32 device tensor of hop
        counts (-1 unreached), levels the last level that reached something
        new, reached the entries each level run reached."""
        import torch
        src, sp = _u32(sources)
        n = self.n_rows
        nb = ctypes.c_uint64()
        _check(lib().k2_bfs_workspace_bytes(self._h, src.size, ctypes.byref(nb)), "k2_bfs_workspace_bytes")
        if dist is None:
            dist = torch.empty((n, src.size), dtype=torch.int32, device=self.device)
        if workspace is None:
            workspace = torch.empty(nb.value, dtype=torch.uint8, device=self.device)
        if dist.numel() != n * src.size or dist.dtype != torch.int32 or not dist.is_contiguous():
            raise ValueError("dist must be a contiguous int32 tensor of n x len(sources)")
        levels = ctypes.c_uint32()
        max_levels = int(min(max_levels, 2 ** 31 - 1))
        # per-level counts are kept for searches of at most 2^16 levels
        reached = np.zeros(max(max_levels, 1), np.uint64) if max_levels <= (1 << 16) else None
        _check(lib().k2_bfs(self._h, DIRECTIONS[direction], sp, src.size, max_levels, _VP(dist.data_ptr()),
                            _VP(workspace.data_ptr()), workspace.numel(), _stream_handle(stream),
                            ctypes.byref(levels),
                            reached.ctypes.data_as(_U64P) if reached is not None else None), "k2_bfs")
        if reached is not None:
            reached = reached[:min(levels.value + 1, max_levels)]
        return dist, levels.value, reached

    def bfs_noalloc(self, sources, dist, direction="right", max_levels=2 ** 31 - 1, stream=None):
        """The search of bfs() through k2_bfs_noalloc, whose workspace is the
        library's fixed scratch array: the caller passes the (n,
        len(sources)) int32 device tensor dist, and nothing is allocated on
        the device.  Returns (dist, levels, reached) like bfs()."""
        src, sp = _u32(sources)
        n = self.n_rows
        if dist.numel() != n * src.size or str(dist.dtype) != "torch.int32" or not dist.is_contiguous():
            raise ValueError("dist must be a contiguous int32 tensor of n x len(sources)")
        if dist.device != self.device:
            raise ValueError("dist is not on the matrix's device")
        levels = ctypes.c_uint32()
        max_levels = int(min(max_levels, 2 ** 31 - 1))
        reached = np.zeros(max(max_levels, 1), np.uint64) if max_levels <= (1 << 16) else None
        _check(lib().k2_bfs_noalloc(self._h, DIRECTIONS[direction], sp, src.size, max_levels,
                                    _VP(dist.data_ptr()), _stream_handle(stream), ctypes.byref(levels),
                                    reached.ctypes.data_as(_U64P) if reached is not None else None),
               "k2_bfs_noalloc")
        if reached is not None:
            reached = reached[:min(levels.value + 1, max_levels)]
        return dist, levels.value, reached

    def device_level_words(self, level, n_nodes, stream=None):
        out = np.zeros((n_nodes + 15) // 16, np.uint64)
        _check(lib().k2_matrix_level_words(self._h, level, out.ctypes.data_as(_U64P), out.size,
                                           _stream_handle(stream)), "k2_matrix_level_words")
        return out

    def cached_blocks(self, n_nodes, stream=None):
        """(first row << 32) | first column of each cached node's 4x4 block."""
        out = np.zeros(max(n_nodes, 1), np.uint64)
        _check(lib().k2_matrix_cached_blocks(self._h, out.ctypes.data_as(_U64P), n_nodes,
                                             _stream_handle(stream)), "k2_matrix_cached_blocks")
        return out[:n_nodes]


class Streamed:
    """Out-of-core products (k2_stream_*): the tree stays in host memory and
    each product copies it chunk by chunk into a device staging buffer of at
    most staging_bytes.  Creating one plans the chunks (host only); the
    tree must stay alive."""

    def __init__(self, tree, staging_bytes, opts=None):
        h = _VP()
        o = opts if opts is not None else plan_defaults()
        _check(lib().k2_stream_create(tree._h, ctypes.byref(o), int(staging_bytes), ctypes.byref(h)),
               "k2_stream_create")
        self._h = h
        self._tree = tree
        self._default_staging = {}
        self.n_rows, self.n_cols = tree.n_rows, tree.n_cols
        nc, mb, sb = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
        _check(lib().k2_stream_info(h, ctypes.byref(nc), ctypes.byref(mb), ctypes.byref(sb)), "k2_stream_info")
        self.n_chunks, self.max_chunk_bytes, self.staged_bytes = nc.value, mb.value, sb.value

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.k2_stream_destroy(h)
            self._h = None

    def chunk(self, k, levels):
        """(first tile, end tile, first staged word per level, staged words per level)."""
        a, b = ctypes.c_uint64(), ctypes.c_uint64()
        lo = np.zeros(levels, np.uint64)
        nw = np.zeros(levels, np.uint64)
        _check(lib().k2_stream_chunk(self._h, int(k), ctypes.byref(a), ctypes.byref(b),
                                     lo.ctypes.data_as(_U64P), nw.ctypes.data_as(_U64P), int(levels)),
               "k2_stream_chunk")
        return a.value, b.value, lo, nw

    def staging(self, device="cuda"):
        """A device staging buffer for products: two halves of the largest chunk."""
        import torch
        return torch.empty(max(2 * self.max_chunk_bytes, 256), dtype=torch.uint8, device=device)

    def spmv(self, x, y=None, direction="right", semiring="plus_times", batch=1, accumulate=False,
             staging=None, stream=None):
        """As Matrix.spmv in tree mode, with the tree streamed from host memory."""
        import torch
        d = DIRECTIONS[direction]
        n_in = self.n_cols if d == K2_RIGHT else self.n_rows
        n_out = self.n_rows if d == K2_RIGHT else self.n_cols
        dtype = torch.int32 if semiring == "boolean_u32" else torch.float32
        if x.dtype != dtype or x.numel() != n_in * batch or not x.is_contiguous():
            raise ValueError(f"x must be a contiguous {dtype} tensor of {n_in * batch} elements")
        if x.device.type != "cuda":
            raise ValueError("x must be a device tensor")
        if y is None:
            if accumulate:
                raise ValueError("accumulate needs y")
            y = torch.empty(n_out * batch, dtype=dtype, device=x.device)
        elif y.dtype != dtype or y.numel() != n_out * batch or not y.is_contiguous():
            raise ValueError(f"y must be a contiguous {dtype} tensor of {n_out * batch} elements")
        if y.device != x.device:
            raise ValueError("y is not on x's device")
        if staging is None:
            # one buffer per Streamed and device, kept across products: the
            # copies and kernels of a product still read it after this call
            # returns, so it must not go back to torch's allocator here
            staging = self._default_staging.get(x.device)
            if staging is None:
                staging = self.staging(x.device)
                self._default_staging[x.device] = staging
        if staging.device != x.device:
            raise ValueError("the staging buffer is not on x's device")
        _check(lib().k2_stream_spmv(self._h, d, SEMIRINGS[semiring], int(batch),
                                    K2_SPMV_ACCUMULATE if accumulate else 0, _VP(x.data_ptr()),
                                    _VP(y.data_ptr()), _VP(staging.data_ptr()), staging.numel(),
                                    _stream_handle(stream)), "k2_stream_spmv")
        return y


PROBES = {"copy": 0, "read": 1, "write": 2, "update_seq_atomic": 3, "update_seq_store": 4,
          "gather_rows": 5, "scatter_rows_atomic": 6, "lds_add_f32": 7, "lds_cas_f32": 8,
          "lds_add_u32": 9, "gather_rows_nt": 10, "gather_rows_buf_nt": 11, "gather_rows_buf_sys": 12}


def probe(kind, a, b, idx=None, n=0, row_elems=1, reps=0, stream=None):
    """One timed launch of a ceiling microbenchmark (k2_probe_run): a, b
    torch device tensors (a may be None where unused), idx a uint32 (as
    int32) device tensor of row indexes or None; returns milliseconds."""
    ms = ctypes.c_float()
    _check(lib().k2_probe_run(PROBES[kind], _VP(a.data_ptr()) if a is not None else None,
                              _VP(b.data_ptr()), _VP(idx.data_ptr()) if idx is not None else None,
                              int(n), b.numel(), int(row_elems), int(reps), _stream_handle(stream),
                              ctypes.byref(ms)), "k2_probe_run")
    return float(ms.value)
