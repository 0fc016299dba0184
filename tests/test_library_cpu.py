"""CPU-only checks of the C ABI library: it builds, loads, exports every
function include/fedavg.h declares, and rejects bad arguments on the host
before touching a device.  No kernel is launched here."""

import ctypes
import glob
import os
import re

import pytest

import weighted_model_update_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"(?m)^(?!typedef|#)\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text):
            names.add(m.group(1))
    return names


def test_header_declares_what_the_binding_exports():
    assert declared_functions() == set(fa.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = fa.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    # plain dynamic-symbol check, independent of ctypes
    out = os.popen(f"nm -D --defined-only {fa.library_path()}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_abi_version():
    assert fa.fedavg_abi_version() == 1


def _lib():
    return fa.load()


def test_host_side_argument_errors_need_no_device():
    lib = _lib()
    P = ctypes.c_void_p
    # K outside [1, 64]
    assert lib.fedavg_aggregate(0, None, 0, None, 10, 0, None, 0, None, 0, 0, None, None, None) == -3
    assert b"K=0" in lib.fedavg_last_error()
    x = (P * 1)(1 << 20)
    n = (ctypes.c_int64 * 1)(-5)
    assert lib.fedavg_aggregate(1, x, 0, n, 10, 0, None, 0, P(1 << 21), 0, 0, None, None, None) == -3
    n[0] = 5
    assert lib.fedavg_aggregate(1, x, 7, n, 10, 0, None, 0, P(1 << 21), 0, 0, None, None, None) == -2
    assert lib.fedavg_aggregate(1, x, 0, n, 10, 1, None, 0, P(1 << 21), 0, 0, None, None, None) == -1
    # sparse: workspace too small
    assert lib.sparse_masked_accumulate(1, (P * 1)(1 << 20), (P * 1)(1 << 20), (ctypes.c_int64 * 1)(4),
                                        (ctypes.c_int64 * 1)(1), 100, 1, P(1 << 22), P(1 << 23), None, 0,
                                        None, P(1 << 24), 8, None, None) == -8
    assert lib.fedavg_set_option(99, 1) == -1
    assert lib.fedavg_set_option(fa.FA_OPT_SPARSE_BLOCKS, 70000) == -3
    assert lib.fedavg_checksum(None, 10, 0, None, None) == -1


def test_workspace_sizes_do_not_depend_on_the_number_of_clients():
    acc, ws, cnt, stag = fa.fedavg_workspace_size(10 ** 6, 0, 64 << 20, 2)
    assert acc == 4 * 10 ** 6 and ws == 0 and cnt == 0
    assert stag >= 2 * (64 << 20)
    acc, ws, cnt, stag2 = fa.fedavg_workspace_size(10 ** 6, 1, 64 << 20, 2)
    assert ws == 4 * 10 ** 6 and cnt == 10 ** 6 and stag2 > stag
    with pytest.raises(fa.FedAvgError):
        fa.fedavg_workspace_size(10, 0, 0, 2)
    assert fa.sparse_workspace_size(20, 10 ** 9) < 16 << 20
    assert fa.sparse_workspace_size(20, 4096) < 1024


def test_streaming_null_handle_and_state():
    lib = _lib()
    assert lib.fedavg_accumulate(None, 0, 1, None, 0, 0, 0, None, None) == -1
    assert lib.fedavg_finalize(None, None, 0, None, 0) == -1
    assert lib.fedavg_destroy(None) == 0
