"""The C-ABI library loads, exports every entry point include/qgemv.h declares, and its
host-only helpers behave as declared. No call here touches device memory (no GPU needed)."""

import ctypes
import os
import re

import pytest

import block_quantized_weight_act_amd as qg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")

# HIP's hipGraphNodeType values (hip_runtime_api.h): kernel 0, memcpy 1, memset 2, empty 5
KERNEL, MEMCPY, MEMSET, EMPTY = 0, 1, 2, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qgemv_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(qg.library_path)
    names = declared_functions()
    assert len(names) >= 14
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_function():
    names = set(declared_functions()) - {"qgemv_last_error"}
    assert names <= set(qg.__all__), names - set(qg.__all__)


def test_graph_record_check_refuses_memset_nodes():
    """qgemv_graph_end's check of a record, on node types alone: kernels and other nodes are
    counted, a memset node anywhere refuses the record (a memset is never recorded on a GPU
    to test this)."""
    assert qg.qgemv_graph_classify([]) == (0, 0)
    assert qg.qgemv_graph_classify([KERNEL] * 5) == (5, 0)
    assert qg.qgemv_graph_classify([KERNEL, MEMCPY, KERNEL, EMPTY]) == (2, 2)
    for types in ([MEMSET], [KERNEL, KERNEL, MEMSET], [MEMSET, KERNEL], [EMPTY, MEMSET, MEMCPY]):
        with pytest.raises(qg.QgemvError) as e:
            qg.qgemv_graph_classify(types)
        assert e.value.status == 1
        assert b"memset" in qg._load().qgemv_last_error()
    lib = qg._load()
    k, o = ctypes.c_int64(), ctypes.c_int64()
    arr = (ctypes.c_int32 * 1)(KERNEL)
    assert lib.qgemv_graph_classify(None, 1, ctypes.byref(k), ctypes.byref(o)) == 1
    assert lib.qgemv_graph_classify(arr, -1, ctypes.byref(k), ctypes.byref(o)) == 1
    assert lib.qgemv_graph_classify(arr, 1, None, ctypes.byref(o)) == 1
