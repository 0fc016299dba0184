"""GPU results equal the fp32 mirror of the stated rounding order bit for
bit: fused multiply-adds of fp32(n_k) * x in client order from +0, one
IEEE division by fp32(W) (fp32(S) in zero-fill mode), the base added in fp32,
nearest-even rounding into the output type.  Every aggregation path promises
this order: resident dense, per-segment masks (both kernels and the
element-wise path), the sparse merge and streaming (dense, masked and
indexed chunks)."""

import numpy as np
import pytest
import torch

import oracle
import synth
import weighted_model_update_amd as fa
from gpu_util import dev_of, dev_f32, host_of, empty

pytestmark = pytest.mark.gpu

OD = {"f32": oracle.F32, "bf16": oracle.BF16}
MODES = {"weights": oracle.WEIGHTS, "deltas": oracle.DELTAS, "deltas_zero_fill": oracle.DELTAS_ZERO_FILL}


def same_bits(got, want):
    g = np.asarray(got)
    w = np.asarray(want)
    assert g.dtype == w.dtype and g.shape == w.shape
    bad = np.nonzero(g.view(np.uint32 if g.dtype == np.float32 else np.uint16) !=
                     w.view(np.uint32 if w.dtype == np.float32 else np.uint16))[0]
    assert bad.size == 0, (bad.size, bad[:5], g[bad[:5]], w[bad[:5]])


def clients(seed, K, N, xdt, scale=1e-2):
    r = np.random.default_rng(seed)
    x32 = [(r.standard_normal(N) * scale * 10.0 ** r.integers(-1, 2)).astype(np.float32) for _ in range(K)]
    return [synth.bf16_bits_from_f32(x) for x in x32] if xdt == "bf16" else x32


def base_of(seed, N, bdt):
    b = (np.random.default_rng(seed + 7).standard_normal(N) * 0.02).astype(np.float32)
    return synth.bf16_bits_from_f32(b) if bdt == "bf16" else b


def test_bf16_output_every_fp32_pattern():
    # One client with n = 1 passes each fp32 value through fma(1, x, +0) and a
    # division by 1 (only -0 and NaN payloads change) to the bf16 rounding of
    # the output stage, so the 2^32 bit patterns, in 16 pieces, cover every
    # rounding case of that stage: ties, carries into the exponent, overflow
    # to infinity, subnormals and NaNs.
    piece = 1 << 28
    out = empty(piece, "bf16")
    for p in range(16):
        x = np.arange(p * piece, (p + 1) * piece, dtype=np.uint64).astype(np.uint32).view(np.float32)
        xd = dev_f32(x)
        fa.fedavg_aggregate([xd], [1], out)
        torch.cuda.synchronize()
        want = oracle.mirror_f32([x], np.array([1]), x_dtype=oracle.F32, out_dtype=oracle.BF16)
        got = host_of(out)
        # NaN matches NaN: the payload after the fused product is the FMA unit's
        nan = ((got & 0x7fff) > 0x7f80) & ((want & 0x7fff) > 0x7f80)
        bad = np.nonzero((got != want) & ~nan)[0]
        assert bad.size == 0, (p, bad.size, bad[:5], got[bad[:5]], want[bad[:5]])
        assert np.array_equal((got & 0x7fff) > 0x7f80, (want & 0x7fff) > 0x7f80)
        del xd


@pytest.mark.parametrize("K", [1, 3, 5, 8, 16, 17, 20, 64])
@pytest.mark.parametrize("xdt,odt,mode", [("f32", "f32", "weights"), ("bf16", "bf16", "deltas"),
                                          ("bf16", "f32", "deltas"), ("f32", "bf16", "weights")])
def test_dense(K, xdt, odt, mode):
    N = 100_003
    xs = clients(K, K, N, xdt)
    n = synth.sample_counts(K, K, 1, 100_000)
    base = base_of(K, N, xdt) if mode != "weights" else None
    out = empty(N, odt)
    fa.fedavg_aggregate([dev_of(x, xdt) for x in xs], n.tolist(), out, mode=mode,
                        base=None if base is None else dev_of(base, xdt))
    torch.cuda.synchronize()
    want = oracle.mirror_f32(xs, n, mode=MODES[mode], base=base, x_dtype=OD[xdt], base_dtype=OD[xdt],
                             out_dtype=OD[odt])
    same_bits(host_of(out), want)


@pytest.mark.parametrize("K", [2, 4, 12, 20])
def test_dense_residency_caps_give_the_same_bits(K):
    """The resident-workgroup cap (by default chosen from the number of
    contributing clients) changes only how many workgroups share a CU:
    every cap gives the oracle mirror's bits."""
    N = 300_007
    xs = clients(100 + K, K, N, "bf16")
    n = synth.sample_counts(K, K, 1, 100_000)
    base = base_of(K, N, "bf16")
    want = oracle.mirror_f32(xs, n, mode=oracle.DELTAS, base=base, x_dtype=oracle.BF16,
                             base_dtype=oracle.BF16, out_dtype=oracle.BF16)
    try:
        for cap in (-1, 0, 1, 3, 6, 8):
            fa.fedavg_set_option(fa.FA_OPT_RESIDENT_PER_CU, cap)
            out = empty(N, "bf16")
            fa.fedavg_aggregate([dev_of(x, "bf16") for x in xs], n.tolist(), out, mode="deltas",
                                base=dev_of(base, "bf16"))
            torch.cuda.synchronize()
            same_bits(host_of(out), want)
    finally:
        fa.fedavg_set_option(fa.FA_OPT_RESIDENT_PER_CU, -1)


def test_dense_unaligned_view():
    N, K = 50_001, 4
    xs = clients(2, K, N + 1, "bf16")
    n = [3, 500, 70001, 12]
    out = torch.empty(N + 1, dtype=torch.bfloat16, device="cuda")
    fa.fedavg_aggregate([dev_of(x, "bf16")[1:] for x in xs], n, out[1:])
    torch.cuda.synchronize()
    same_bits(host_of(out)[1:], oracle.mirror_f32([x[1:] for x in xs], n, x_dtype=oracle.BF16,
                                                  out_dtype=oracle.BF16))


@pytest.mark.parametrize("T", [300, 900])
@pytest.mark.parametrize("mode", ["weights", "deltas", "deltas_zero_fill"])
@pytest.mark.parametrize("xdt,odt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")])
def test_masked(T, mode, xdt, odt):
    # T = 300: the whole-table kernel; 900: the windowed one.  An fp32
    # output takes two 4-parameter quads per lane, 1 KiB apart, and falls
    # back to elements where they lie in different segments.
    r = np.random.default_rng(T)
    sizes = r.integers(0, 600, size=T)
    sizes[::7] = r.integers(2000, 9000, size=len(sizes[::7]))  # segments longer than a run of quads
    bounds = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    N, K = int(bounds[-1]), 8
    present = (r.random((K, T)) < 0.6).astype(np.uint8)
    xs = clients(T + 1, K, N, xdt)
    base = base_of(T, N, xdt)
    n = synth.sample_counts(T, K, 500, 5000)
    out = empty(N, odt)
    fa.fedavg_aggregate([dev_of(x, xdt) for x in xs], n.tolist(), out, mode=mode,
                        base=dev_of(base, xdt),
                        seg_bounds=torch.tensor(bounds, dtype=torch.int64, device="cuda"),
                        present=torch.from_numpy(present).cuda())
    torch.cuda.synchronize()
    seg_of = np.repeat(np.arange(T), np.diff(bounds))
    sent = [present[k][seg_of] for k in range(K)]
    want = oracle.mirror_f32(xs, n, mode=MODES[mode], base=base, x_dtype=OD[xdt],
                             base_dtype=OD[xdt], out_dtype=OD[odt], sent=sent)
    same_bits(host_of(out), want)


def _lists_as_dense(idx, val, N):
    xs, sent = [], []
    for i, v in zip(idx, val):
        x = np.zeros(N, np.float32)
        s = np.zeros(N, np.uint8)
        x[i] = v
        s[i] = 1
        xs.append(x)
        sent.append(s)
    return xs, sent


def _sparse_bits(mode, K, tile):
    N = 200_003
    idx, val = zip(*[synth.topk_sparse_deltas(11, k, N, 0.1, 1e-3) for k in range(K)])
    base = synth.normal_f32(11, synth.ROLE_BASE, 0, N, 0.02)
    n = synth.sample_counts(11, K, 100, 1000)
    out = torch.empty(N, device="cuda")
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, tile)
    try:
        fa.sparse_masked_accumulate([torch.from_numpy(np.asarray(i, np.int64)).cuda() for i in idx],
                                    [dev_f32(v) for v in val], n.tolist(), N, dev_f32(base), out,
                                    mode=mode)
        torch.cuda.synchronize()
    finally:
        fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, 2048)
    xs, sent = _lists_as_dense(idx, val, N)
    same_bits(host_of(out), oracle.mirror_f32(xs, n, mode=MODES[mode], base=base, sent=sent))


@pytest.mark.parametrize("mode", ["weights", "deltas", "deltas_zero_fill"])
@pytest.mark.parametrize("K", [6, 40])
def test_sparse(mode, K):
    _sparse_bits(mode, K, 2048)


@pytest.mark.parametrize("tile", [512, 1024, 4096, 8192])
def test_sparse_two_mask_words_every_tile(tile):
    # K > 32 takes the kernels with two client-mask words; the 8192 tile is
    # the largest LDS footprint (about 98 KB with 1024 threads)
    _sparse_bits("deltas", 40, tile)


@pytest.mark.parametrize("kind", ["dense", "masks", "indices"])
def test_streaming(kind):
    N, K, chunk = 120_007, 5, 8192
    xs = clients(40, K, N, "bf16")
    base = base_of(40, N, "bf16")
    n = synth.sample_counts(40, K, 100, 10_000)
    r = np.random.default_rng(41)
    sent = [(r.random(N) < 0.5).astype(np.uint8) for _ in range(K)] if kind != "dense" else None
    out = empty(N, "bf16")
    with fa.StreamingAccumulator(N, mode="deltas", partial=kind != "dense", chunk_bytes=16 * chunk) as acc:
        for k in range(K):
            d = dev_of(xs[k], "bf16")
            for off in range(0, N, chunk):
                ln = min(chunk, N - off)
                if kind == "dense":
                    acc.accumulate(k, int(n[k]), d[off:off + ln], offset=off)
                elif kind == "masks":
                    acc.accumulate(k, int(n[k]), d[off:off + ln], offset=off,
                                   mask=torch.from_numpy(sent[k][off:off + ln]).cuda())
                else:
                    rel = np.nonzero(sent[k][off:off + ln])[0].astype(np.int64)
                    if rel.size:
                        acc.accumulate(k, int(n[k]), d[off:off + ln][torch.from_numpy(rel).cuda()].contiguous(),
                                       offset=off, indices=torch.from_numpy(rel).cuda())
        acc.finalize(dev_of(base, "bf16"), out)
        acc.sync()
    want = oracle.mirror_f32(xs, n, mode=oracle.DELTAS, base=base, x_dtype=oracle.BF16,
                             base_dtype=oracle.BF16, out_dtype=oracle.BF16, sent=sent)
    same_bits(host_of(out), want)


def test_subnormal_results_are_not_flushed():
    """Tiny values whose weighted sums and quotients are fp32 subnormals:
    the GPU keeps them as IEEE fp32 arithmetic does (no flush to zero)."""
    N, K = 4096, 3
    r = np.random.default_rng(12)
    xs = [(r.standard_normal(N) * 1e-39).astype(np.float32) for _ in range(K)]
    n = [3, 7, 11]
    out = empty(N, "f32")
    fa.fedavg_aggregate([dev_f32(x) for x in xs], n, out)
    torch.cuda.synchronize()
    want = oracle.mirror_f32(xs, n)
    assert (np.abs(want) < np.float32(1.17549435e-38)).sum() > N // 2
    same_bits(host_of(out), want)
