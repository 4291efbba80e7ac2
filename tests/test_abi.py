"""The C-ABI library loads and exports every function include/*.h declares
(no compute call: this runs without a GPU)."""
import ctypes
import glob
import os
import re

import tree_graph_spmv_amd as k2

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "k2spmv.h")
HEADERS = sorted(glob.glob(os.path.join(INCLUDE, "*.h")))


def declared_functions():
    names = []
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(k2_[a-z0-9_]+)\s*\(",
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


CITES = re.compile(r"Sec\. [0-9]|Table [0-9]|Algorithm [0-9]|Fig(?:ure|\.) [0-9]")
# the one entry point the pages do not define: it serves callers that cannot
# allocate device memory, and its comment says so instead of citing a passage
NO_PASSAGE_NEEDS = re.compile(r"cannot allocate")


def declarations_with_comments():
    """(name, comment) for every function the header declares: the comment
    block right above its declaration, or above the run of declarations it
    belongs to."""
    out = []
    for h in HEADERS:
        out += _declarations_with_comments(open(h).read())
    return out


def _declarations_with_comments(text):
    # comments blanked (same length), so that names inside them do not match
    code = re.sub(r"/\*.*?\*/", lambda c: re.sub(r"[^\n]", " ", c.group(0)), text, flags=re.S)
    out = []
    pat = re.compile(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(k2_[a-z0-9_]+)\s*\(", re.M)
    for m in pat.finditer(code):
        line = text.rfind("\n", 0, m.start(1)) + 1   # the declaration's first line
        end = text.rfind("*/", 0, line)
        start = text.rfind("/*", 0, end)
        between = text[end + 2:line]
        # only declarations may sit between the comment and this one
        stripped = re.sub(r"[^;]*\([^;]*\)\s*;", "", between).strip()
        out.append((m.group(1), text[start:end + 2] if not stripped else ""))
    return out


def test_every_declaration_cites_its_passage():
    """Each call of the boundary states the passage of the pages that defines
    the operation (section, table, algorithm or figure)."""
    missing = [n for n, c in declarations_with_comments()
               if not (CITES.search(c) or NO_PASSAGE_NEEDS.search(c))]
    assert not missing, f"no passage cited for: {missing}"


def test_status_strings():
    for st in range(7):
        assert k2.lib().k2_status_string(st)
