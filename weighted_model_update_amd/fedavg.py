"""Python binding of libfedavg.so (include/fedavg.h) over torch tensors.

Argument marshalling only: every step of the aggregation runs in the HIP
kernels of the library.  Torch provides device memory, pinned host memory and
streams.  The names follow the C ABI.  There is no fallback path: if the
library cannot be loaded, every call raises.
"""

import ctypes
import os

import torch

from . import build as _build

FA_OK = 0
FA_F32, FA_BF16 = 0, 1
FA_WEIGHTS, FA_DELTAS, FA_DELTAS_ZERO_FILL = 0, 1, 2
FA_COUNT_U8, FA_COUNT_U32 = 0, 1
FA_OPT_BLOCKS_PER_CU, FA_OPT_MASK_VECTORS_PER_BLOCK, FA_OPT_SPARSE_BLOCKS, FA_OPT_RESIDENT_PER_CU = 1, 2, 3, 4
FA_OPT_SPARSE_TILE = 5
FA_OPT_TOPK_SAMPLED = 6
FA_OPT_INDEX_TILES = 7
FA_MAX_CLIENTS = 64
FA_MAX_N = 1 << 40

STATUS_NAMES = {
    0: "FA_OK", -1: "FA_ERR_ARG", -2: "FA_ERR_DTYPE", -3: "FA_ERR_RANGE",
    -4: "FA_ERR_ZERO_WEIGHT", -5: "FA_ERR_STATE", -6: "FA_ERR_INCOMPLETE",
    -7: "FA_ERR_INDEX", -8: "FA_ERR_WORKSPACE", -9: "FA_ERR_HIP",
}

# every symbol include/fedavg.h declares
EXPORTS = [
    "fedavg_abi_version", "fedavg_last_error", "fedavg_aggregate", "fedavg_workspace_size",
    "fedavg_begin", "fedavg_accumulate", "fedavg_finalize", "fedavg_sync", "fedavg_destroy",
    "fedavg_accumulate_partial", "fedavg_partial_info", "fedavg_state_size", "fedavg_export_state",
    "fedavg_resume", "topk_workspace_size", "topk_select", "fedavg_controller_step",
    "sparse_workspace_size", "sparse_masked_accumulate", "fedavg_checksum", "fedavg_set_option",
    "fedavg_sum_workspace_size", "fedavg_checksum_sum", "sparse_masked_accumulate_noalloc",
    "fedavg_arena_layout",
]


class FedAvgError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


_lib = None


def library_path():
    return _build.LIB_PATH


def load(build_if_missing=True):
    """Load libfedavg.so (building it first if it does not exist).  torch is
    imported before the library so both share torch's HIP runtime."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB_PATH):
        if not build_if_missing:
            raise RuntimeError(f"{_build.LIB_PATH} is not built")
        _build.build()
    lib = ctypes.CDLL(_build.LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "fedavg_abi_version": ([], i32),
        "fedavg_last_error": ([], ctypes.c_char_p),
        "fedavg_aggregate": ([i32, P, i32, P, i64, i32, P, i32, P, i32, i32, P, P, P], i32),
        "fedavg_workspace_size": ([i64, i32, i64, i32, P, P, P, P], i32),
        "fedavg_begin": ([P, i64, i32, i32, P, P, P, P, sz, i64, i32, P, P], i32),
        "fedavg_accumulate": ([P, i32, i64, P, i32, i64, i64, P, P], i32),
        "fedavg_accumulate_partial": ([P, i32, i64, i32, P, P, P, i64, i64], i32),
        "fedavg_partial_info": ([P, P, P], i32),
        "fedavg_state_size": ([P, P], i32),
        "fedavg_export_state": ([P, P, sz], i32),
        "fedavg_resume": ([P, P, sz, i64, i32, i32, P, P, P, P, sz, i64, i32, P, P], i32),
        "fedavg_finalize": ([P, P, i32, P, i32], i32),
        "fedavg_sync": ([P], i32),
        "fedavg_destroy": ([P], i32),
        "sparse_workspace_size": ([i32, i64, P], i32),
        "sparse_masked_accumulate": ([i32, P, P, P, P, i64, i32, P, P, P, i32, P, P, sz, P, P], i32),
        "sparse_masked_accumulate_noalloc": ([i32, P, P, P, P, i64, i32, P, P, P, i32, P, P, P], i32),
        "fedavg_checksum": ([P, i64, i32, P, P], i32),
        "fedavg_sum_workspace_size": ([i64, P], i32),
        "fedavg_checksum_sum": ([P, i64, i32, P, P, P, sz, P], i32),
        "topk_workspace_size": ([i32, i64, i64, P], i32),
        "fedavg_controller_step": ([i32, P, P, P, i64, P, P, P, i32, P], i32),
        "topk_select": ([P, i32, i64, i64, P, P, P, sz, P], i32),
        "fedavg_set_option": ([i32, i64], i32),
        "fedavg_arena_layout": ([i32, i64, P, P], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(rc):
    if rc != FA_OK:
        msg = load().fedavg_last_error()
        raise FedAvgError(rc, msg.decode() if msg else "")


def _dtype_code(dt):
    if dt == torch.float32:
        return FA_F32
    if dt == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {dt}; use float32 or bfloat16")


def _dtype(t):
    return _dtype_code(t.dtype)


def _mode(mode):
    if mode in ("weights", FA_WEIGHTS):
        return FA_WEIGHTS
    if mode in ("deltas", FA_DELTAS):
        return FA_DELTAS
    if mode in ("deltas_zero_fill", FA_DELTAS_ZERO_FILL):
        return FA_DELTAS_ZERO_FILL
    raise ValueError(f"mode must be 'weights', 'deltas' or 'deltas_zero_fill', got {mode!r}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _contig(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_gpu(t, name):
    # device-only arguments: a host pointer would reach a kernel
    if t is not None and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _i64_array(vals):
    vals = [int(v) for v in vals]
    return (ctypes.c_int64 * len(vals))(*vals)


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))()
    for k, t in enumerate(tensors):
        arr[k] = t.data_ptr() if t is not None else None
    return arr


def fedavg_abi_version():
    return load().fedavg_abi_version()


def fedavg_set_option(option, value):
    _check(load().fedavg_set_option(int(option), int(value)))


# ------------------------------------------------------------------ resident

def fedavg_aggregate(xs, n, out, mode="weights", base=None, seg_bounds=None, present=None,
                     stream=None):
    """out <- weighted average of the K client tensors `xs` with weights `n`
    (see fedavg_aggregate in include/fedavg.h).  seg_bounds (int64 [T+1]) and
    present (uint8 [K, T]) select per-segment masks; both live on the GPU."""
    lib = load()
    K = len(xs)
    if K == 0:
        raise ValueError("need at least one client")
    if len(n) != K:
        raise ValueError(f"n has {len(n)} entries for {K} clients")
    N = out.numel()
    xdt = None
    for k, x in enumerate(xs):
        if x is None:
            continue
        _contig(x, f"xs[{k}]")
        _on_gpu(x, f"xs[{k}]")
        if x.numel() != N:
            raise ValueError(f"xs[{k}] has {x.numel()} elements, out has {N}")
        d = _dtype(x)
        if xdt is not None and d != xdt:
            raise TypeError("all clients must share one dtype")
        xdt = d
    _on_gpu(_contig(out, "out"), "out")
    _on_gpu(_contig(base, "base"), "base")
    if base is not None and base.numel() != N:
        raise ValueError("base must have as many elements as out")
    T = 0
    if seg_bounds is not None or present is not None:
        if seg_bounds is None or present is None:
            raise ValueError("seg_bounds and present go together")
        _on_gpu(_contig(seg_bounds, "seg_bounds"), "seg_bounds")
        _on_gpu(_contig(present, "present"), "present")
        if seg_bounds.dtype != torch.int64 or present.dtype != torch.uint8:
            raise TypeError("seg_bounds must be int64 and present uint8")
        T = seg_bounds.numel() - 1
        if T < 1 or present.numel() != K * T:
            raise ValueError("present must hold K*T flags for T = len(seg_bounds) - 1")
    rc = lib.fedavg_aggregate(K, _ptr_array(xs), xdt if xdt is not None else FA_F32, _i64_array(n), N,
                              _mode(mode), _ptr(base), _dtype(base) if base is not None else FA_F32,
                              _ptr(out), _dtype(out), T, _ptr(seg_bounds), _ptr(present),
                              _stream_handle(stream))
    _check(rc)


def arena_layout(count, nbytes):
    """(offsets, total_bytes): byte offsets of `count` buffers of `nbytes`
    bytes inside one allocation of total_bytes, each 32 KiB further into its
    2 MiB page than the one before (fedavg_arena_layout in include/fedavg.h)."""
    offs = (ctypes.c_int64 * int(count))()
    total = ctypes.c_int64(0)
    _check(load().fedavg_arena_layout(int(count), int(nbytes), offs, ctypes.byref(total)))
    return list(offs), total.value


def client_arena(count, numel, dtype=torch.bfloat16, device="cuda"):
    """One device allocation holding `count` tensors of `numel` elements of
    `dtype`, placed by arena_layout (for example the K clients and the output
    of a resident aggregation).  Returns (arena, [tensor, ...]); the tensors
    are views of the arena, which must outlive them."""
    esize = torch.empty(0, dtype=dtype).element_size()
    offs, total = arena_layout(count, int(numel) * esize)
    arena = torch.empty(total, dtype=torch.uint8, device=device)
    views = [arena[o:o + int(numel) * esize].view(dtype) for o in offs]
    return arena, views


# ------------------------------------------------------------------ streaming

def fedavg_workspace_size(N, partial, chunk_bytes, n_slots):
    """(acc_bytes, wsum_bytes, count_bytes, staging_bytes)."""
    out = [ctypes.c_size_t(0) for _ in range(4)]
    _check(load().fedavg_workspace_size(int(N), int(bool(partial)), int(chunk_bytes), int(n_slots),
                                        *[ctypes.byref(o) for o in out]))
    return tuple(o.value for o in out)


def fedavg_begin(N, mode, partial, acc, wsum, count, staging, chunk_bytes, n_slots,
                 compute_stream=None, copy_stream=None):
    """Returns an opaque handle (ctypes pointer)."""
    for t, name in ((acc, "acc"), (wsum, "wsum"), (count, "count"), (staging, "staging")):
        _on_gpu(t, name)
    h = ctypes.c_void_p(0)
    rc = load().fedavg_begin(ctypes.byref(h), int(N), _mode(mode), int(bool(partial)), _ptr(acc),
                             _ptr(wsum), _ptr(count), _ptr(staging),
                             staging.numel() * staging.element_size(), int(chunk_bytes),
                             int(n_slots), _stream_handle(compute_stream),
                             None if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream))
    _check(rc)
    return h


def fedavg_accumulate(h, client_id, n_k, chunk, offset=0, mask=None, indices=None):
    _contig(chunk, "chunk")
    _contig(mask, "mask")
    _contig(indices, "indices")
    if mask is not None and mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError("mask must be uint8 or bool")
    if indices is not None and indices.dtype != torch.int64:
        raise TypeError("indices must be int64")
    rc = load().fedavg_accumulate(h, int(client_id), int(n_k), _ptr(chunk), _dtype(chunk),
                                  int(offset), chunk.numel(), _ptr(mask), _ptr(indices))
    _check(rc)


def fedavg_accumulate_partial(h, client_id, W, n_clients, acc_src, wsum_src=None, count_src=None,
                              offset=0):
    """Add a lower-level aggregation's partial sums (fp32 acc_src over
    [offset, offset+len), with its uint32 weight sums and uint8 counts in
    partial mode) as one pseudo-client of weight W standing for n_clients
    clients."""
    _contig(acc_src, "acc_src")
    _contig(wsum_src, "wsum_src")
    _contig(count_src, "count_src")
    if acc_src.dtype != torch.float32:
        raise TypeError("acc_src must be float32")
    n = acc_src.numel()
    if wsum_src is not None and (wsum_src.numel() != n or wsum_src.dtype != torch.int32):
        raise ValueError("wsum_src must be int32 (holding uint32) with one entry per element of acc_src")
    if count_src is not None and (count_src.numel() != n or count_src.dtype != torch.uint8):
        raise ValueError("count_src must hold one uint8 count per element of acc_src")
    rc = load().fedavg_accumulate_partial(h, int(client_id), int(W), int(n_clients), _ptr(acc_src),
                                          _ptr(wsum_src), _ptr(count_src), int(offset), n)
    _check(rc)


def fedavg_partial_info(h):
    """(total weight, number of clients) accumulated so far in h."""
    W = ctypes.c_int64(0)
    m = ctypes.c_int(0)
    _check(load().fedavg_partial_info(h, ctypes.byref(W), ctypes.byref(m)))
    return W.value, m.value


def fedavg_export_state(h):
    """The handle's host-side record as bytes (waits for its work first)."""
    lib = load()
    n = ctypes.c_size_t(0)
    _check(lib.fedavg_state_size(h, ctypes.byref(n)))
    buf = ctypes.create_string_buffer(n.value)
    _check(lib.fedavg_export_state(h, buf, n.value))
    return buf.raw


def fedavg_resume(state, N, mode, partial, acc, wsum, count, staging, chunk_bytes, n_slots,
                  compute_stream=None, copy_stream=None):
    """Open a handle over restored acc/wsum/count tensors and an exported
    record (bytes).  Returns the handle."""
    for t, name in ((acc, "acc"), (wsum, "wsum"), (count, "count"), (staging, "staging")):
        _on_gpu(t, name)
    h = ctypes.c_void_p(0)
    rc = load().fedavg_resume(ctypes.byref(h), state, len(state), int(N), _mode(mode),
                              int(bool(partial)), _ptr(acc), _ptr(wsum), _ptr(count),
                              _ptr(staging), staging.numel() * staging.element_size(), int(chunk_bytes),
                              int(n_slots), _stream_handle(compute_stream),
                              None if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream))
    _check(rc)
    return h


def fedavg_finalize(h, base, out):
    _on_gpu(_contig(base, "base"), "base")
    _on_gpu(_contig(out, "out"), "out")
    rc = load().fedavg_finalize(h, _ptr(base), _dtype(base) if base is not None else FA_F32,
                                _ptr(out), _dtype(out))
    _check(rc)


def fedavg_sync(h):
    _check(load().fedavg_sync(h))


def fedavg_destroy(h):
    _check(load().fedavg_destroy(h))


class StreamingAccumulator:
    """begin/accumulate/finalize over a caller-held set of workspace tensors.

    Allocates the accumulator (N fp32), in partial mode the per-parameter
    weight sums (uint32 stored as int32) and client counts (uint8), and the
    staging slots, then calls fedavg_begin.  Use as a context manager or call
    close()."""

    def __init__(self, N, mode="weights", partial=False, chunk_bytes=64 << 20, n_slots=2,
                 counts=True, device="cuda", compute_stream=None, copy_stream=None, _resume=None):
        acc_b, wsum_b, count_b, stag_b = fedavg_workspace_size(N, partial, chunk_bytes, n_slots)
        self.N = N
        self.acc = torch.empty(max(acc_b // 4, 1), dtype=torch.float32, device=device)
        self.wsum = torch.empty(max(wsum_b // 4, 1), dtype=torch.int32, device=device) if partial else None
        self.count = (torch.empty(max(count_b, 1), dtype=torch.uint8, device=device)
                      if partial and counts else None)
        self.staging = torch.empty(stag_b, dtype=torch.uint8, device=device)
        if _resume is None:
            self.handle = fedavg_begin(N, mode, partial, self.acc, self.wsum, self.count, self.staging,
                                       chunk_bytes, n_slots, compute_stream, copy_stream)
        else:
            # the library checks the record against N, mode and partial first;
            # the buffers are filled before anything can be accumulated
            state, restore = _resume
            self.handle = fedavg_resume(state, N, mode, partial, self.acc, self.wsum, self.count,
                                        self.staging, chunk_bytes, n_slots, compute_stream,
                                        copy_stream)
            try:
                restore(self)
            except BaseException:
                self.close()
                raise

    # spill to / resume from a directory: state.bin (the handle's record) and
    # the raw acc.f32, wsum.u32, count.u8 buffers, copied through a pinned
    # bounce buffer piece by piece
    _SPILL_PIECE = 64 << 20

    def save(self, path):
        """Write the running aggregate to directory `path` (created if needed).
        The accumulator stays usable."""
        import os
        import numpy as np
        state = fedavg_export_state(self.handle)
        os.makedirs(path, exist_ok=True)
        with open(os.path.join(path, "state.bin"), "wb") as f:
            f.write(state)
        for name, t in (("acc.f32", self.acc), ("wsum.u32", self.wsum), ("count.u8", self.count)):
            if t is None:
                continue
            flat = t[:self.N].view(torch.uint8) if self.N > 0 else t[:0].view(torch.uint8)
            total = flat.numel()
            mm = np.memmap(os.path.join(path, name), dtype=np.uint8, mode="w+", shape=(max(total, 1),))
            bounce = torch.empty(min(self._SPILL_PIECE, max(total, 1)), dtype=torch.uint8, pin_memory=True)
            for off in range(0, total, bounce.numel()):
                n = min(bounce.numel(), total - off)
                bounce[:n].copy_(flat[off:off + n])
                mm[off:off + n] = bounce[:n].numpy()
            mm.flush()
            del mm

    @classmethod
    def load(cls, path, N, mode="weights", partial=False, chunk_bytes=64 << 20, n_slots=2,
             device="cuda", compute_stream=None, copy_stream=None):
        """Resume an aggregate written by save().  N, mode and partial must be
        the saved ones (the library checks N, mode and partial against the
        saved record)."""
        import os
        import numpy as np
        with open(os.path.join(path, "state.bin"), "rb") as f:
            state = f.read()
        counts = os.path.exists(os.path.join(path, "count.u8"))

        def restore(self):
            for name, t in (("acc.f32", self.acc), ("wsum.u32", self.wsum), ("count.u8", self.count)):
                if t is None:
                    continue
                flat = t[:N].view(torch.uint8)
                total = flat.numel()
                if total == 0:
                    continue
                mm = np.memmap(os.path.join(path, name), dtype=np.uint8, mode="r")
                if mm.shape[0] != total:
                    raise ValueError(f"{name} holds {mm.shape[0]} bytes, expected {total}")
                bounce = torch.empty(min(self._SPILL_PIECE, total), dtype=torch.uint8, pin_memory=True)
                for off in range(0, total, bounce.numel()):
                    n = min(bounce.numel(), total - off)
                    bounce[:n].numpy()[:] = mm[off:off + n]
                    flat[off:off + n].copy_(bounce[:n])
                torch.cuda.synchronize()
                del mm

        return cls(N, mode=mode, partial=partial, chunk_bytes=chunk_bytes, n_slots=n_slots,
                   counts=counts, device=device, compute_stream=compute_stream,
                   copy_stream=copy_stream, _resume=(state, restore))

    def accumulate(self, client_id, n_k, chunk, offset=0, mask=None, indices=None):
        fedavg_accumulate(self.handle, client_id, n_k, chunk, offset, mask, indices)

    def accumulate_partial(self, client_id, W, n_clients, acc_src, wsum_src=None, count_src=None,
                           offset=0):
        fedavg_accumulate_partial(self.handle, client_id, W, n_clients, acc_src, wsum_src, count_src,
                                  offset)

    def add_silo(self, client_id, silo):
        """Feed another StreamingAccumulator's whole partial (after its work
        is done) as one pseudo-client of this one."""
        silo.sync()
        W, members = fedavg_partial_info(silo.handle)
        N = self.N
        fedavg_accumulate_partial(self.handle, client_id, W, members, silo.acc[:N],
                                  None if silo.wsum is None else silo.wsum[:N],
                                  None if silo.count is None else silo.count[:N], 0)

    def info(self):
        """(total weight, number of clients) accumulated so far."""
        return fedavg_partial_info(self.handle)

    def finalize(self, base, out):
        fedavg_finalize(self.handle, base, out)

    def sync(self):
        fedavg_sync(self.handle)

    def close(self):
        if self.handle is not None:
            h, self.handle = self.handle, None
            fedavg_destroy(h)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------ sparse

def sparse_workspace_size(K, N):
    b = ctypes.c_size_t(0)
    _check(load().sparse_workspace_size(int(K), int(N), ctypes.byref(b)))
    return b.value


def _sparse_args(idx, val, n, N, base, out, counts, wsum, err_flag):
    """Checks the sparse merge's tensors; returns the counts dtype code."""
    K = len(idx)
    if len(val) != K or len(n) != K:
        raise ValueError("idx, val and n must have one entry per client")
    for k in range(K):
        _on_gpu(_contig(idx[k], f"idx[{k}]"), f"idx[{k}]")
        _on_gpu(_contig(val[k], f"val[{k}]"), f"val[{k}]")
        if idx[k].dtype != torch.int64 or val[k].dtype != torch.float32:
            raise TypeError("indices must be int64 and values float32")
        if idx[k].numel() != val[k].numel():
            raise ValueError(f"idx[{k}] and val[{k}] differ in length")
    for t, name in ((base, "base"), (out, "out")):
        _on_gpu(_contig(t, name), name)
        if t.dtype != torch.float32 or t.numel() != N:
            raise ValueError(f"{name} must be float32 with N elements")
    cdt = FA_COUNT_U8
    if counts is not None:
        _on_gpu(_contig(counts, "counts"), "counts")
        if counts.numel() != N or counts.dtype not in (torch.uint8, torch.int32):
            raise ValueError("counts must be uint8 or int32 with N elements")
        cdt = FA_COUNT_U8 if counts.dtype == torch.uint8 else FA_COUNT_U32
    if wsum is not None:
        _on_gpu(_contig(wsum, "wsum"), "wsum")
        if wsum.numel() != N or wsum.dtype != torch.int32:
            raise ValueError("wsum must be int32 (holding uint32) with N elements")
    if err_flag is not None and (err_flag.numel() < 1 or err_flag.dtype != torch.int32):
        raise ValueError("err_flag must be an int32 tensor of at least one element")
    _on_gpu(err_flag, "err_flag")
    return cdt


def sparse_masked_accumulate(idx, val, n, N, base, out, mode="deltas", counts=None, wsum=None,
                             workspace=None, err_flag=None, stream=None):
    """One-pass merge of K sorted sparse client lists (see include/fedavg.h).
    counts: uint8 or int32 tensor of N (nullable); wsum: int32 tensor of N
    holding the uint32 weight sums (nullable); err_flag: int32 tensor of 1."""
    lib = load()
    K = len(idx)
    cdt = _sparse_args(idx, val, n, N, base, out, counts, wsum, err_flag)
    if workspace is None and N > 0:      # an empty model needs none
        workspace = torch.empty(sparse_workspace_size(K, N), dtype=torch.uint8, device=out.device)
    _on_gpu(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.sparse_masked_accumulate(K, _ptr_array(idx), _ptr_array(val),
                                      _i64_array([t.numel() for t in idx]), _i64_array(n), int(N),
                                      _mode(mode), _ptr(base), _ptr(out), _ptr(counts), cdt,
                                      _ptr(wsum), _ptr(workspace), ws_bytes, _ptr(err_flag),
                                      _stream_handle(stream))
    _check(rc)
    return workspace


def sparse_masked_accumulate_noalloc(idx, val, n, N, base, out, mode="deltas", counts=None, wsum=None,
                                     err_flag=None, stream=None):
    """The same merge without a workspace: the library keeps the list
    offsets in a static per-GPU scratch array and allocates nothing (for
    callers that cannot allocate, e.g. under graph capture).  Calls that
    overlap in time on one GPU share that array and must be serialized."""
    lib = load()
    K = len(idx)
    cdt = _sparse_args(idx, val, n, N, base, out, counts, wsum, err_flag)
    rc = lib.sparse_masked_accumulate_noalloc(K, _ptr_array(idx), _ptr_array(val),
                                              _i64_array([t.numel() for t in idx]), _i64_array(n),
                                              int(N), _mode(mode), _ptr(base), _ptr(out), _ptr(counts),
                                              cdt, _ptr(wsum), _ptr(err_flag), _stream_handle(stream))
    _check(rc)


# ------------------------------------------------------------------ windows

def stream_windows(N, clients, base, out, window=None, mode="weights", partial=False,
                   chunk_bytes=64 << 20, n_slots=2, counts=True, device="cuda"):
    """Streaming aggregation of an N-parameter model one window of the
    parameter space at a time, for models whose accumulator (4 B per
    parameter, 9 B in partial mode) does not fit in device memory beside the
    rest.  A parameter's result depends only on its own clients' values in
    client order, so the windows give the same bits as one handle over all N.

    clients: a sequence of (client_id, n_k, chunks), where chunks() returns,
    each time it is called, the client's chunks as (offset, values) or
    (offset, values, mask), in ascending offset; values live on the device
    or in pinned host memory.  chunks() is called once per window, and only
    the part of each chunk inside the window is accumulated (a view, no
    copy); a chunk wholly outside it is passed as an empty chunk, so every
    chunk is one library call and a host buffer may be reused n_slots chunks
    later, as with fedavg_accumulate.  Every client is entered in every window, also where
    it sent nothing inside it, so zero-fill mode divides by the same S.
    base, out: N elements each, on the device or on the host (then copied a
    window at a time); base may be None in dense weights mode.
    window: parameters per window (default N).  The window's accumulator,
    weight sums, counts and staging are allocated once and reused.
    Returns the number of windows."""
    N = int(N)
    window = max(N, 1) if window is None else int(window)
    if window < 1:
        raise ValueError("window must be >= 1")
    window = max(1, min(window, N))
    acc_b, wsum_b, count_b, stag_b = fedavg_workspace_size(window, partial, chunk_bytes, n_slots)
    acc = torch.empty(max(acc_b // 4, 1), dtype=torch.float32, device=device)
    wsum = torch.empty(max(wsum_b // 4, 1), dtype=torch.int32, device=device) if partial else None
    count = (torch.empty(max(count_b, 1), dtype=torch.uint8, device=device)
             if partial and counts else None)
    staging = torch.empty(stag_b, dtype=torch.uint8, device=device)
    empty = torch.empty(0, dtype=torch.float32, device=device)
    windows = 0
    for w0 in range(0, N, window):
        w1 = min(w0 + window, N)
        h = fedavg_begin(w1 - w0, mode, partial, acc, wsum, count, staging, chunk_bytes, n_slots)
        try:
            for cid, n_k, chunks in clients:
                fedavg_accumulate(h, cid, n_k, empty, 0)
                for item in chunks():
                    off, vals = int(item[0]), item[1]
                    mask = item[2] if len(item) > 2 else None
                    lo, hi = max(off, w0), min(off + vals.numel(), w1)
                    if lo >= hi:
                        # nothing inside the window; still one call, which
                        # keeps the host-buffer reuse count of the chunks
                        fedavg_accumulate(h, cid, n_k, empty, 0)
                        continue
                    fedavg_accumulate(h, cid, n_k, vals[lo - off:hi - off], lo - w0,
                                      None if mask is None else mask[lo - off:hi - off])
            bw = None if base is None else base[w0:w1]
            if bw is not None and not bw.is_cuda:
                bw = bw.to(device)
            ow = out[w0:w1] if out.is_cuda else torch.empty(w1 - w0, dtype=out.dtype, device=device)
            fedavg_finalize(h, bw, ow)
            fedavg_sync(h)
            if not out.is_cuda:
                out[w0:w1].copy_(ow)
        finally:
            fedavg_destroy(h)
        windows += 1
    return windows


# ------------------------------------------------------------------ checksum

def fedavg_checksum(t, stream=None, hash_out=None):
    """Order-independent 64-bit checksum of a contiguous float32/bfloat16 GPU
    tensor.  Returns the value as a Python int (synchronizes the stream)
    unless hash_out (an int64 tensor of one element) is given."""
    lib = load()
    _on_gpu(_contig(t, "tensor"), "tensor")
    if hash_out is not None and (hash_out.numel() < 1 or hash_out.element_size() != 8):
        raise ValueError("hash_out must be a 64-bit tensor of at least one element")
    _on_gpu(hash_out, "hash_out")
    own = hash_out is None
    if own:
        hash_out = torch.empty(1, dtype=torch.int64, device=t.device)
    _check(lib.fedavg_checksum(_ptr(t), t.numel(), _dtype(t), _ptr(hash_out),
                                  _stream_handle(stream)))
    if own:
        return int(hash_out.item()) & 0xFFFFFFFFFFFFFFFF
    return None


def fedavg_sum_workspace_size(count):
    """Bytes of workspace fedavg_checksum_sum needs for `count` elements."""
    b = ctypes.c_size_t(0)
    _check(load().fedavg_sum_workspace_size(int(count), ctypes.byref(b)))
    return b.value


def fedavg_checksum_sum(t, stream=None, workspace=None, hash_out=None, sum_out=None, with_hash=True):
    """In one read of a contiguous float32/bfloat16 GPU tensor, its checksum
    and a deterministic fp64 sum of its values (fixed order of additions).
    Returns (hash or None, sum) as Python values (synchronizing the stream)
    unless sum_out (a float64 tensor of one element) is given; then the
    results stay on the device (hash_out: an int64 tensor of one element, or
    None for no hash)."""
    lib = load()
    _on_gpu(_contig(t, "tensor"), "tensor")
    if workspace is None:
        workspace = torch.empty(max(fedavg_sum_workspace_size(t.numel()), 8), dtype=torch.uint8,
                                device=t.device)
    for o, name in ((hash_out, "hash_out"), (sum_out, "sum_out")):
        if o is not None and (o.numel() < 1 or o.element_size() != 8):
            raise ValueError(f"{name} must be a 64-bit tensor of at least one element")
        _on_gpu(o, name)
    _on_gpu(workspace, "workspace")
    own = sum_out is None
    if own:
        sum_out = torch.empty(1, dtype=torch.float64, device=t.device)
        if with_hash:
            hash_out = torch.empty(1, dtype=torch.int64, device=t.device)
    _check(lib.fedavg_checksum_sum(_ptr(t), t.numel(), _dtype(t), _ptr(hash_out), _ptr(sum_out),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream_handle(stream)))
    if own:
        h = int(hash_out.item()) & 0xFFFFFFFFFFFFFFFF if hash_out is not None else None
        return h, float(sum_out.item())
    return None


# ------------------------------------------------------------------ top-k

def topk_workspace_size(N, k, dtype=torch.float32):
    """Device workspace bytes topk_select needs to keep k of N values."""
    b = ctypes.c_size_t(0)
    _check(load().topk_workspace_size(_dtype_code(dtype), int(N), int(k), ctypes.byref(b)))
    return b.value


def topk_select(x, k, idx_out=None, val_out=None, workspace=None, stream=None):
    """The k entries of largest magnitude of the 1-D update x (ties to the
    lower index), as (int64 indices in increasing order, float32 values)."""
    lib = load()
    _on_gpu(_contig(x, "x"), "x")
    N = x.numel()
    k = int(k)
    dev = x.device
    if idx_out is None:
        idx_out = torch.empty(k, dtype=torch.int64, device=dev)
    if val_out is None:
        val_out = torch.empty(k, dtype=torch.float32, device=dev)
    if idx_out.numel() < k or val_out.numel() < k or idx_out.dtype != torch.int64 \
            or val_out.dtype != torch.float32:
        raise ValueError("idx_out must be int64 and val_out float32, each with room for k entries")
    _on_gpu(_contig(idx_out, "idx_out"), "idx_out")
    _on_gpu(_contig(val_out, "val_out"), "val_out")
    if workspace is None:
        workspace = torch.empty(max(topk_workspace_size(N, k, x.dtype), 1), dtype=torch.uint8, device=dev)
    _on_gpu(workspace, "workspace")
    rc = lib.topk_select(_ptr(x), _dtype(x), N, k, _ptr(idx_out), _ptr(val_out), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _check(rc)
    return idx_out[:k], val_out[:k]


def topk_count(N, frac):
    """k = floor(frac * N), with frac read as the decimal it is written as."""
    from fractions import Fraction
    import math
    return int(math.floor(Fraction(str(frac)) * int(N)))


# ------------------------------------------------------------------ sample allocation

class _Controller(ctypes.Structure):
    _fields_ = [("w_time", ctypes.c_double), ("w_energy", ctypes.c_double),
                ("ema", ctypes.c_double), ("deadband", ctypes.c_double)]


class SampleController:
    """Next-round sample counts n_k (the FedAvg weights) from each
    participant's measured time and energy (fedavg_controller_step)."""

    def __init__(self, P, w_time=1.0, w_energy=0.0, ema=0.5, deadband=0.05):
        self.P = int(P)
        self.params = _Controller(float(w_time), float(w_energy), float(ema), float(deadband))
        self.tau = (ctypes.c_double * self.P)()
        self.eps = (ctypes.c_double * self.P)()
        self.first = True

    def step(self, t, e, n, total):
        P = self.P
        if not (len(t) == len(e) == len(n) == P):
            raise ValueError(f"need {P} times, energies and counts")
        out = (ctypes.c_int64 * P)()
        rc = load().fedavg_controller_step(P, (ctypes.c_double * P)(*map(float, t)),
                                           (ctypes.c_double * P)(*map(float, e)), _i64_array(n),
                                           int(total), ctypes.byref(self.params), self.tau, self.eps,
                                           int(self.first), out)
        _check(rc)
        self.first = False
        return [int(v) for v in out]

    def state(self):
        return list(self.tau), list(self.eps)
