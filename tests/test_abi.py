"""The C-ABI library loads and exports every function include/k2spmv.h
declares (no compute call: this runs without a GPU)."""
import ctypes
import os
import re

import tree_graph_spmv_amd as k2

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "k2spmv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(k2_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("k2_build", "k2_estimate_device_bytes", "k2_matrix_create", "k2_spmv",
                 "k2_matrix_destroy", "k2_tree_free", "k2_status_string"):
        assert must in names
    assert len(names) >= 15


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(k2.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_binding_covers_every_declared_function():
    assert set(declared_functions()) <= set(k2._SIGS)


def test_status_strings():
    for st in range(7):
        assert k2.lib().k2_status_string(st)
