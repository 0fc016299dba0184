"""CPU-only checks of the C ABI library: it builds, loads, exports every
function include/fedavg.h declares, and rejects bad arguments on the host
before touching a device.  No kernel is launched here."""

import ctypes
import glob
import os
import re

import pytest
import torch

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


@pytest.mark.parametrize("nbytes", [0, 1, 4096, (2 << 20) - 1, 2 << 20, (2 << 20) + 16, 3_843_756_032])
@pytest.mark.parametrize("count", [1, 2, 17, 33, 65])
def test_arena_layout_staggers_disjoint_buffers(count, nbytes):
    """Buffer j lies 32 KiB further into its 2 MiB page than buffer j - 1
    (modulo 2 MiB), buffers never overlap, every offset is 16-byte aligned
    and the total ends with the last buffer."""
    offs, total = fa.arena_layout(count, nbytes)
    page, step = 2 << 20, 32 << 10
    assert offs[0] == 0 and total == offs[-1] + nbytes
    for j in range(1, count):
        assert offs[j] >= offs[j - 1] + nbytes
        assert offs[j] % 16 == 0
        assert offs[j] % page == (j * step) % page
        assert offs[j] - offs[j - 1] < nbytes + page + step


def test_arena_layout_argument_errors():
    lib = _lib()
    offs = (ctypes.c_int64 * 4)()
    total = ctypes.c_int64()
    assert lib.fedavg_arena_layout(0, 10, offs, ctypes.byref(total)) == -1
    assert lib.fedavg_arena_layout(4097, 10, offs, ctypes.byref(total)) == -1
    assert lib.fedavg_arena_layout(4, -1, offs, ctypes.byref(total)) == -1
    assert lib.fedavg_arena_layout(4, 10, None, ctypes.byref(total)) == -1
    assert lib.fedavg_arena_layout(4, 10, offs, None) == -1
    assert lib.fedavg_arena_layout(4, 1 << 61, offs, ctypes.byref(total)) == -3
    assert lib.fedavg_arena_layout(4, (1 << 62) - (4 << 20), offs, ctypes.byref(total)) == -3
    assert lib.fedavg_arena_layout(1, (1 << 62) - (4 << 20), offs, ctypes.byref(total)) == 0
    assert total.value == (1 << 62) - (4 << 20)


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
    assert lib.fedavg_set_option(fa.FA_OPT_SPARSE_BLOCKS, (1 << 19) + 1) == -3
    assert lib.fedavg_set_option(fa.FA_OPT_TOPK_SAMPLED, 2) == -3
    assert lib.fedavg_set_option(fa.FA_OPT_INDEX_TILES, 3) == -3
    assert lib.fedavg_set_option(fa.FA_OPT_INDEX_TILES, -1) == -3
    assert lib.fedavg_set_option(fa.FA_OPT_INDEX_TILES, 0) == 0
    # residency: -1 (by client count, the default), 0 (no cap) .. 32
    assert lib.fedavg_set_option(fa.FA_OPT_RESIDENT_PER_CU, -2) == -3
    assert lib.fedavg_set_option(fa.FA_OPT_RESIDENT_PER_CU, 33) == -3
    assert lib.fedavg_set_option(fa.FA_OPT_RESIDENT_PER_CU, 32) == 0
    assert lib.fedavg_set_option(fa.FA_OPT_RESIDENT_PER_CU, -1) == 0
    b = ctypes.c_size_t(0)
    assert lib.topk_workspace_size(0, 100, 101, ctypes.byref(b)) == -3   # k > N
    assert lib.topk_workspace_size(7, 100, 10, ctypes.byref(b)) == -2    # unknown dtype
    assert lib.topk_workspace_size(0, 100, 10, None) == -1
    assert lib.topk_workspace_size(0, (1 << 36) + 1, 10, ctypes.byref(b)) == -3   # one tile per workgroup
    assert lib.topk_workspace_size(0, 1 << 36, 10, ctypes.byref(b)) == 0
    assert lib.topk_select(P(1 << 20), 0, (1 << 36) + 1, 10, P(1 << 21), P(1 << 22), P(1 << 23), 1 << 40,
                           None) == -3
    assert lib.fedavg_checksum(None, 10, 0, None, None) == -1
    d = ctypes.c_void_p
    assert lib.fedavg_checksum_sum(d(1 << 20), 10, 0, None, None, None, 0, None) == -1   # no sum
    assert lib.fedavg_checksum_sum(d(1 << 20), 10, 5, None, d(1 << 22), d(1 << 23), 8, None) == -2
    assert lib.fedavg_checksum_sum(d(1 << 20), 10, 0, None, d(1 << 22), None, 0, None) == -8
    assert lib.fedavg_checksum_sum(d(1 << 20), 10, 0, None, d(1 << 22), d(1 << 23), 7, None) == -8
    assert lib.fedavg_checksum_sum(d(1 << 20), 10, 0, None, d(1 << 22), d((1 << 23) + 4), 8, None) == -1
    assert lib.fedavg_checksum_sum(d(1 << 20), 10, 0, None, d((1 << 20) + 8), d(1 << 23), 8, None) == -1
    assert lib.fedavg_checksum_sum(d(1 << 20), 10, 0, d(1 << 23), d(1 << 22), d(1 << 23), 8, None) == -1


def test_topk_workspace_holds_a_staging_copy_only_while_it_pays():
    """While 3k < N for fp32 (4k < N for bf16) the workspace grows by 6 (4)
    bytes per kept entry for the staging copy; beyond that it does not grow."""
    N = 10 ** 6
    kf, kb = (N - 1) // 3, (N - 1) // 4          # the largest k that still stages
    f = [fa.topk_workspace_size(N, k, torch.float32) for k in (1, 1001, kf, kf + 1, N)]
    assert abs((f[1] - f[0]) - 6 * 1000) <= 6 * 256     # staging is carved in 256 regions
    assert f[3] < f[2] and f[3] == f[4]
    h = [fa.topk_workspace_size(N, k, torch.bfloat16) for k in (1, 1001, kb, kb + 1)]
    assert abs((h[1] - h[0]) - 4 * 1000) <= 4 * 256
    assert h[3] < h[2] and h[3] == f[4]


def test_workspace_sizes_do_not_depend_on_the_number_of_clients():
    acc, ws, cnt, stag = fa.fedavg_workspace_size(10 ** 6, 0, 64 << 20, 2)
    assert acc == 4 * 10 ** 6 and ws == 0 and cnt == 0
    assert stag >= 2 * (64 << 20)
    acc, ws, cnt, stag2 = fa.fedavg_workspace_size(10 ** 6, 1, 64 << 20, 2)
    assert ws == 4 * 10 ** 6 and cnt == 10 ** 6 and stag2 > stag
    with pytest.raises(fa.FedAvgError):
        fa.fedavg_workspace_size(10, 0, 0, 2)
    # one list offset per client and range boundary, at most 2^19 ranges
    assert fa.sparse_workspace_size(20, 10 ** 9) <= 256 + 20 * ((1 << 19) + 1) * 8
    assert fa.sparse_workspace_size(20, 4096) < 2048
    # the value sum keeps one fp64 per tile of 8192 elements
    assert [fa.fedavg_sum_workspace_size(n) for n in (0, 1, 8192, 8193, 10 ** 9)] == \
        [0, 8, 8, 16, 8 * 122071]


def test_sizes_beyond_the_parameter_cap_are_range_errors():
    """At most 2^40 parameters (and chunk_bytes at most 2^40), so that no
    byte count the library forms can overflow 64 bits."""
    lib = fa.load()
    z = ctypes.c_size_t(0)
    M = fa.FA_MAX_N
    assert lib.fedavg_workspace_size(M, 1, 1 << 20, 2, None, None, None, ctypes.byref(z)) == 0
    assert lib.fedavg_workspace_size(M + 1, 1, 1 << 20, 2, None, None, None, ctypes.byref(z)) == -3
    assert lib.fedavg_workspace_size(10, 1, M + 1, 2, None, None, None, ctypes.byref(z)) == -3
    assert lib.fedavg_workspace_size(10, 1, (1 << 63) - 1, 64, None, None, None, ctypes.byref(z)) == -3
    assert lib.fedavg_workspace_size(10, 1, 4096, 65, None, None, None, ctypes.byref(z)) == -3
    assert lib.sparse_workspace_size(4, M + 1, ctypes.byref(z)) == -3
    assert lib.sparse_workspace_size(4, M, ctypes.byref(z)) == 0
    x = (ctypes.c_void_p * 1)(1 << 20)
    n = (ctypes.c_int64 * 1)(5)
    P = ctypes.c_void_p
    assert lib.fedavg_aggregate(1, x, 0, n, M + 1, 0, None, 0, P(1 << 21), 0, 0, None, None, None) == -3
    assert lib.fedavg_checksum(P(1 << 20), M + 1, 0, P(1 << 21), None) == -3
    assert lib.fedavg_sum_workspace_size(M + 1, ctypes.byref(z)) == -3
    assert b"2^40" in lib.fedavg_last_error()


def test_streaming_null_handle_and_state():
    lib = _lib()
    assert lib.fedavg_accumulate(None, 0, 1, None, 0, 0, 0, None, None) == -1
    assert lib.fedavg_finalize(None, None, 0, None, 0) == -1
    assert lib.fedavg_accumulate_partial(None, 0, 1, 1, None, None, None, 0, 0) == -1
    assert lib.fedavg_partial_info(None, None, None) == -1
    assert lib.fedavg_destroy(None) == 0


def _no_gpu_here():
    # these checks pass fake device pointers and rely on the first HIP launch
    # failing; they must never run where a GPU could execute that launch
    if os.path.exists("/dev/kfd"):
        return False
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_gpu_here(), reason="host-only check; needs a machine without a GPU")
@pytest.mark.parametrize("tile", [512, 1024, 2048, 4096, 8192])
@pytest.mark.parametrize("blocks", [0, 1, 7, 65536])
def test_sparse_workspace_covers_every_range_plan(tile, blocks):
    """With exactly sparse_workspace_size bytes, the library's range plan
    always fits: the call gets past argument and workspace checks and fails
    only at its first HIP launch (no device here), never with
    FA_ERR_WORKSPACE.  One byte less is refused before any launch."""
    lib = _lib()
    P = ctypes.c_void_p
    assert lib.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, tile) == 0
    assert lib.fedavg_set_option(fa.FA_OPT_SPARSE_BLOCKS, blocks) == 0
    try:
        for K in (1, 20, 33, 64):
            for N in (1, 255, 256, 257, 4096, 300_007, 1_000_003, 10 ** 9):
                need = fa.sparse_workspace_size(K, N)
                fake = (P * K)(*([1 << 40] * K))
                nnz = (ctypes.c_int64 * K)(*([1] * K))
                n = (ctypes.c_int64 * K)(*([1] * K))
                args = (K, fake, fake, nnz, n, N, 1, P(1 << 41), P(1 << 42), None, 0, None, P(1 << 43))
                rc = lib.sparse_masked_accumulate(*args, need, None, None)
                assert rc == -9, (K, N, rc, lib.fedavg_last_error())
                rc = lib.sparse_masked_accumulate(*args, need - 1, None, None)
                assert rc == -8, (K, N, rc)
    finally:
        lib.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, 2048)
        lib.fedavg_set_option(fa.FA_OPT_SPARSE_BLOCKS, 0)


# ---------------------------------------------------------------- spill/resume

def _fnv1a64(b):
    h = 0xcbf29ce484222325
    for c in b:
        h ^= c
        h = (h * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    return h


def _state(N=1000, mode=0, partial=0, has_count=0, finalized=0, clients=((0, 1, 5, 1000),),
           magic=0x54534146, version=1, corrupt=False):
    """An exported-state record built from the layout include/fedavg.h
    documents."""
    import struct
    body = struct.pack("<IIqiiiiII", magic, version, N, mode, partial, has_count, finalized,
                       len(clients), 0)
    for cid, members, w, covered in clients:
        body += struct.pack("<iiqq", cid, members, w, covered)
    h = _fnv1a64(body) ^ (1 if corrupt else 0)
    return body + struct.pack("<Q", h)


def _resume(state, N=1000, mode=0, partial=0, count=None, staging_bytes=1 << 30):
    lib = _lib()
    P = ctypes.c_void_p
    h = P(0)
    buf = ctypes.create_string_buffer(state, len(state))
    return lib.fedavg_resume(ctypes.byref(h), buf, len(state), N, mode, partial, P(1 << 40),
                             P(1 << 41) if partial else None, count, P(1 << 42), staging_bytes,
                             4096, 2, None, None)


def test_resume_rejects_bad_state_records():
    P = ctypes.c_void_p
    assert _resume(_state(magic=0x12345678)) == -1
    assert _resume(_state(version=2)) == -1
    assert _resume(_state(corrupt=True)) == -1
    assert b"checksum" in _lib().fedavg_last_error()
    assert _resume(_state()[:-1]) == -1                                   # truncated
    assert _resume(_state(), N=999) == -1                                 # other N
    assert _resume(_state(), mode=1) == -1                                # other mode
    assert _resume(_state(partial=1, has_count=1), partial=1) == -1       # counts saved, none given
    assert _resume(_state(partial=1), partial=1, count=P(1 << 43)) == -1  # no counts saved
    assert _resume(_state(has_count=1)) == -1                             # counts without partial
    assert _resume(_state(clients=((0, 1, 5, 1000), (0, 1, 7, 1000)))) == -1   # repeated id
    assert _resume(_state(clients=((-1, 1, 5, 1000),))) == -1
    assert _resume(_state(clients=((0, 0, 5, 1000),))) == -1             # no members
    assert _resume(_state(clients=((0, 1, 5, 1001),))) == -1             # covered beyond N
    assert _resume(_state(clients=((0, 1, 1 << 31, 1000), (1, 1, 1 << 31, 1000)))) == -1  # S >= 2^32
    many = tuple((i, 1, 1, 0) for i in range(256))
    assert _resume(_state(partial=1, clients=many), partial=1) == -1     # 256 clients behind counts
    lib = _lib()
    assert lib.fedavg_state_size(None, None) == -1
    assert lib.fedavg_export_state(None, None, 0) == -1


@pytest.mark.skipif(not _no_gpu_here(), reason="host-only check; needs a machine without a GPU")
def test_resume_accepts_a_good_record_up_to_the_first_hip_call():
    # validation passes; the first HIP call (stream creation) fails here
    assert _resume(_state(clients=((3, 1, 5, 400), (9, 4, 70000, 1000)))) == -9
    assert _resume(_state(partial=1, has_count=1, clients=((0, 255, 7, 10),)), partial=1,
                   count=ctypes.c_void_p(1 << 43)) == -9


@pytest.mark.skipif(not _no_gpu_here(), reason="host-only check; needs a machine without a GPU")
def test_resume_survives_any_record():
    """Random records -- mutated bytes of a good record, truncations,
    extensions, and well-formed records with random fields and a correct
    checksum -- are either refused with an error status or pass validation
    up to the first HIP call; none crashes the parser or reads past the
    buffer it is given."""
    from hypothesis import given, settings, strategies as st, HealthCheck

    good = _state(partial=1, has_count=1, clients=((3, 2, 5, 400), (9, 4, 70000, 1000)))

    @settings(max_examples=400, derandomize=True, deadline=None,
              suppress_health_check=[HealthCheck.too_slow])
    @given(st.data())
    def run(data):
        kind = data.draw(st.sampled_from(["flip", "cut", "grow", "fields"]))
        if kind == "flip":
            b = bytearray(good)
            for _ in range(data.draw(st.integers(1, 8))):
                b[data.draw(st.integers(0, len(b) - 1))] = data.draw(st.integers(0, 255))
            rec = bytes(b)
        elif kind == "cut":
            rec = good[:data.draw(st.integers(0, len(good) - 1))]
        elif kind == "grow":
            rec = good + bytes(data.draw(st.binary(min_size=1, max_size=64)))
        else:
            nc = data.draw(st.integers(0, 6))
            clients = tuple((data.draw(st.integers(-2, 5)), data.draw(st.integers(-1, 300)),
                             data.draw(st.integers(-1, 1 << 33)), data.draw(st.integers(-5, 1100)))
                            for _ in range(nc))
            rec = _state(N=data.draw(st.sampled_from([1000, 0, -1, 1 << 41])),
                         partial=data.draw(st.integers(0, 2)), has_count=data.draw(st.integers(0, 1)),
                         finalized=data.draw(st.integers(-1, 2)), clients=clients)
        rc = _resume(rec, partial=1, count=ctypes.c_void_p(1 << 43))
        assert rc in (-1, -3, -9), rc

    run()


def test_missing_library_fails_loudly():
    """Without libfedavg.so (and no way to build it) every entry point raises;
    nothing falls back to a CPU path.  Run in a fresh interpreter so the
    library this session loaded stays untouched."""
    import subprocess
    import sys
    code = r"""
import torch
import weighted_model_update_amd as fa
import weighted_model_update_amd.build as b
b.LIB_PATH = "/nonexistent/libfedavg.so"
def no_build(*a, **k):
    raise RuntimeError("no toolchain")
b.build = no_build
for call in (lambda: fa.load(build_if_missing=False),
             lambda: fa.fedavg_aggregate([torch.zeros(8)], [1], torch.zeros(8)),
             lambda: fa.fedavg_checksum(torch.zeros(8))):
    try:
        call()
    except RuntimeError as e:
        print("raised", "libfedavg" in str(e) or "toolchain" in str(e))
    else:
        print("returned")
"""
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    lines = [l for l in r.stdout.splitlines() if l.startswith(("raised", "returned"))]
    assert lines == ["raised True"] * 3, r.stdout + r.stderr


def test_binding_refuses_host_tensors_where_the_device_is_required():
    """A host pointer handed to a kernel would fault the device: the binding
    refuses CPU tensors for device-only arguments, and client lists whose
    length differs from the weights, before any library call."""
    x = torch.zeros(16)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fedavg_aggregate([x, x], [1, 2], torch.zeros(16))
    with pytest.raises(ValueError, match="entries for 2 clients"):
        fa.fedavg_aggregate([x, x], [1], torch.zeros(16))
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.sparse_masked_accumulate([torch.zeros(2, dtype=torch.int64)], [torch.zeros(2)], [1], 16,
                                    torch.zeros(16), torch.zeros(16))
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.topk_select(x, 4)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fedavg_checksum(x)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fedavg_checksum_sum(x)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fedavg_begin(16, "weights", False, torch.zeros(16), None, None,
                        torch.zeros(4096, dtype=torch.uint8), 64, 2)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fedavg_finalize(None, None, torch.zeros(16))
