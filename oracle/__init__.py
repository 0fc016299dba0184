"""CPU oracle for FedAvg aggregation -- TEST INFRASTRUCTURE ONLY.

Plain fp64 loops in C (``fedavg_oracle.c``) behind ctypes, plus an exact
rational brute force (``exact.py``) for tiny inputs.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package; the HIP library never does, and the two share no code.

Passages followed (cited per function in the C source):
  * "NVIDIA Clara implements federated learning" (epnc.co.kr): plain or
    contribution-weighted averaging of client models; partial weight sharing.
  * "Building Federated Multimodal AI Workflows with NVIDIA FLARE"
    (ai-thai.com): the client update contract (component-level updates) and
    the adapter-only FedUMM example.
  * "NVFP4 training with JAX and MaxText" (ai-thai.com): round-to-nearest-even
    for weights, fp32 master weights.
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fedavg_oracle.c")
_LIB = os.path.join(_HERE, "libfedavg_oracle.so")

F32, BF16 = 0, 1
WEIGHTS, DELTAS, DELTAS_ZERO_FILL = 0, 1, 2

_lib = None


def build():
    """Compile the C oracle with gcc (IEEE arithmetic: no fast-math, no FMA
    contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-mfma", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.orc_weighted_average.argtypes = [ctypes.c_int, P, ctypes.c_int, P, P, i64, ctypes.c_int,
                                         P, ctypes.c_int, P, P, P, P]
    lib.orc_weighted_average.restype = ctypes.c_int
    lib.orc_sparse_average.argtypes = [ctypes.c_int, P, P, P, P, i64, ctypes.c_int, P, P, P, P, P]
    lib.orc_sparse_average.restype = ctypes.c_int
    lib.orc_sparse_average_at.argtypes = [ctypes.c_int, P, P, P, P, i64, ctypes.c_int, P, i64, P,
                                          P, P, P, P]
    lib.orc_sparse_average_at.restype = ctypes.c_int
    lib.orc_round_to_bf16.argtypes = [P, P, i64]
    lib.orc_round_to_bf16.restype = None
    lib.orc_checksum.argtypes = [P, i64, ctypes.c_int, i64]
    lib.orc_checksum.restype = ctypes.c_uint64
    lib.orc_mirror_f32.argtypes = [ctypes.c_int, P, ctypes.c_int, P, P, i64, ctypes.c_int, P,
                                   ctypes.c_int, ctypes.c_int, P]
    lib.orc_mirror_f32.restype = ctypes.c_int
    lib.orc_sum.argtypes = [P, i64, ctypes.c_int]
    lib.orc_sum.restype = ctypes.c_double
    lib.orc_sum_set_carry_period.argtypes = [i64]
    lib.orc_sum_set_carry_period.restype = None
    lib.orc_topk.argtypes = [P, ctypes.c_int, i64, i64, P, P]
    lib.orc_topk.restype = ctypes.c_int
    lib.orc_sparse_mirror_f32.argtypes = [ctypes.c_int, P, P, P, P, i64, i64, ctypes.c_int, P, P,
                                          P, P]
    lib.orc_sparse_mirror_f32.restype = ctypes.c_int
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = ctypes.c_int
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _ptr_array(arrays):
    arr = (ctypes.c_void_p * len(arrays))()
    for k, a in enumerate(arrays):
        arr[k] = a.ctypes.data if a is not None else None
    return arr


def _raw(a, dtype):
    """Contiguous raw buffer of an fp32 array or a uint16 bf16-bits array."""
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == BF16:
        return np.ascontiguousarray(a, dtype=np.uint16)
    raise ValueError("dtype must be F32 or BF16")


def weighted_average(xs, n, mode=WEIGHTS, base=None, x_dtype=F32, base_dtype=F32, sent=None):
    """Per-parameter weighted average of the clients' values.

    xs: K arrays of N values (float32, or uint16 bf16 bits when x_dtype=BF16).
    n: K sample counts.  sent: None or K arrays of N flags (client k sent i).
    Returns (ref32, mag, count, wsum): the fp32-rounded exact result, the error
    scale M_i, the number of contributing clients and their weight sum."""
    lib = _load()
    K = len(xs)
    xs = [_raw(x, x_dtype) for x in xs]
    N = int(xs[0].shape[0]) if K else 0
    n = np.ascontiguousarray(n, dtype=np.int64)
    assert n.shape == (K,)
    if base is not None:
        base = _raw(base, base_dtype)
        assert base.shape == (N,)
    sent_arrs = None
    if sent is not None:
        sent = [np.ascontiguousarray(s, dtype=np.uint8) for s in sent]
        sent_arrs = _ptr_array(sent)
    ref32 = np.empty(N, np.float32)
    mag = np.empty(N, np.float64)
    count = np.empty(N, np.uint32)
    wsum = np.empty(N, np.uint64)
    rc = lib.orc_weighted_average(K, _ptr_array(xs), x_dtype, _ptr(n), sent_arrs, N, mode,
                                  _ptr(base), base_dtype, _ptr(ref32), _ptr(mag), _ptr(count),
                                  _ptr(wsum))
    if rc != 0:
        raise OracleError(f"orc_weighted_average failed: {rc}")
    return ref32, mag, count, wsum


def sparse_average(idx, val, n, N, mode=DELTAS, base=None):
    """Weighted average over sparse (sorted index, value) client lists."""
    lib = _load()
    K = len(idx)
    idx = [np.ascontiguousarray(a, dtype=np.int64) for a in idx]
    val = [np.ascontiguousarray(a, dtype=np.float32) for a in val]
    nnz = np.array([len(a) for a in idx], dtype=np.int64)
    n = np.ascontiguousarray(n, dtype=np.int64)
    if base is not None:
        base = np.ascontiguousarray(base, dtype=np.float32)
    ref32 = np.empty(N, np.float32)
    mag = np.empty(N, np.float64)
    count = np.empty(N, np.uint32)
    wsum = np.empty(N, np.uint64)
    rc = lib.orc_sparse_average(K, _ptr_array(idx), _ptr_array(val), _ptr(nnz), _ptr(n), N, mode,
                                _ptr(base), _ptr(ref32), _ptr(mag), _ptr(count), _ptr(wsum))
    if rc != 0:
        raise OracleError(f"orc_sparse_average failed: {rc}")
    return ref32, mag, count, wsum


def sparse_average_at(idx, val, n, N, at, mode=DELTAS, base=None):
    """The sparse definition evaluated at the parameters listed in `at` only."""
    lib = _load()
    K = len(idx)
    idx = [np.ascontiguousarray(a, dtype=np.int64) for a in idx]
    val = [np.ascontiguousarray(a, dtype=np.float32) for a in val]
    nnz = np.array([len(a) for a in idx], dtype=np.int64)
    n = np.ascontiguousarray(n, dtype=np.int64)
    at = np.ascontiguousarray(at, dtype=np.int64)
    if base is not None:
        base = np.ascontiguousarray(base, dtype=np.float32)
    S = at.shape[0]
    ref32 = np.empty(S, np.float32)
    mag = np.empty(S, np.float64)
    count = np.empty(S, np.uint32)
    wsum = np.empty(S, np.uint64)
    rc = lib.orc_sparse_average_at(K, _ptr_array(idx), _ptr_array(val), _ptr(nnz), _ptr(n), N,
                                   mode, _ptr(base), S, _ptr(at), _ptr(ref32), _ptr(mag),
                                   _ptr(count), _ptr(wsum))
    if rc != 0:
        raise OracleError(f"orc_sparse_average_at failed: {rc}")
    return ref32, mag, count, wsum


def round_to_bf16(a):
    """uint16 bf16 bits of float32 values, round to nearest even."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    lib.orc_round_to_bf16(_ptr(a), _ptr(out), a.size)
    return out


def checksum(a, dtype, first=0):
    """Order-independent 64-bit checksum of a raw fp32 or bf16-bits array whose
    first element has index `first` in the whole buffer."""
    lib = _load()
    a = _raw(a, dtype)
    return int(lib.orc_checksum(_ptr(a), a.size, dtype, first))


def mirror_f32(xs, n, mode=WEIGHTS, base=None, x_dtype=F32, base_dtype=F32, out_dtype=F32, sent=None):
    """The library's stated fp32 rounding order, for bit-for-bit checks: per
    parameter, fused multiply-adds of fp32(n_k) * x in client order from +0,
    one fp32 division by fp32(W) (fp32(S) in zero-fill mode), the base added
    in fp32 in delta modes, rounded to nearest-even into out_dtype.  Returns
    float32 values, or uint16 bf16 bits."""
    lib = _load()
    K = len(xs)
    xs = [_raw(x, x_dtype) for x in xs]
    N = int(xs[0].shape[0]) if K else 0
    n = np.ascontiguousarray(n, dtype=np.int64)
    if base is not None:
        base = _raw(base, base_dtype)
    sent_arrs = None
    if sent is not None:
        sent = [np.ascontiguousarray(s_, dtype=np.uint8) for s_ in sent]
        sent_arrs = _ptr_array(sent)
    out = np.empty(N, np.float32 if out_dtype == F32 else np.uint16)
    rc = lib.orc_mirror_f32(K, _ptr_array(xs), x_dtype, _ptr(n), sent_arrs, N, mode, _ptr(base),
                            base_dtype, out_dtype, _ptr(out))
    if rc != 0:
        raise OracleError(f"orc_mirror_f32 failed: {rc}")
    return out


def sparse_mirror_f32(idx, val, n, first, length, mode=DELTAS, base=None):
    """The library's fp32 rounding order for sparse lists over the window
    [first, first + length): client by client in order, fused multiply-adds
    of fp32(n_k) * v into each parameter's sum from +0, one fp32 division by
    fp32(W_i) (fp32(S) in zero-fill mode), the base added in fp32 in delta
    modes; a parameter nobody sent keeps base.  idx[k], val[k]: client k's
    entries inside the window (global indices).  base: the window's float32
    values.  Returns (out float32, count uint32, wsum uint64)."""
    lib = _load()
    K = len(idx)
    idx = [np.ascontiguousarray(i, dtype=np.int64) for i in idx]
    val = [np.ascontiguousarray(v, dtype=np.float32) for v in val]
    nnz = np.array([i.size for i in idx], dtype=np.int64)
    n = np.ascontiguousarray(n, dtype=np.int64)
    base = np.ascontiguousarray(base, dtype=np.float32)
    assert base.shape == (length,)
    out = np.empty(length, np.float32)
    cnt = np.empty(length, np.uint32)
    ws = np.empty(length, np.uint64)
    rc = lib.orc_sparse_mirror_f32(K, _ptr_array(idx), _ptr_array(val), _ptr(nnz), _ptr(n), int(first),
                                   int(length), mode, _ptr(base), _ptr(out), _ptr(cnt), _ptr(ws))
    if rc != 0:
        raise OracleError(f"orc_sparse_mirror_f32 failed: {rc}")
    return out, cnt, ws


def set_threads(t=0):
    """Threads of the oracle's per-parameter loops (t <= 0: leave as is);
    returns the count in use."""
    return int(_load().orc_set_threads(int(t)))


def value_sum(a, dtype):
    """The exact sum of a raw fp32 or bf16-bits array's values, rounded once
    to the nearest fp64 (ties to even); NaN or +-infinity as IEEE addition
    gives them; a zero sum is +0."""
    lib = _load()
    a = _raw(a, dtype)
    return float(lib.orc_sum(_ptr(a), a.size, dtype))


def set_sum_carry_period(p):
    """Test hook: run the sum's carry pass every p additions (0: the default)."""
    _load().orc_sum_set_carry_period(int(p))


def topk(x, dtype, k):
    """The k entries of largest magnitude of a client's update (ties to the
    lower index; NaNs above infinity), as increasing int64 indices and their
    float32 values.  x: float32 array, or uint16 bf16 bits."""
    lib = _load()
    x = _raw(x, dtype)
    N = x.size
    idx = np.empty(k, np.int64)
    val = np.empty(k, np.float32)
    rc = lib.orc_topk(_ptr(x), dtype, N, k, _ptr(idx), _ptr(val))
    if rc != 0:
        raise OracleError(f"orc_topk failed: {rc}")
    return idx, val
