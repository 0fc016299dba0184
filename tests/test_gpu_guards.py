"""GPU: every entry point writes only its outputs.  Each output sits inside a
larger buffer whose neighbouring words hold a sentinel, at aligned and
unaligned starts; after the call the sentinels are intact and the outputs
match the oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
import weighted_model_update_amd as fa
from parity import check
from gpu_util import dev_f32, host_of

pytestmark = pytest.mark.gpu

G = 64


def guarded(n, dtype, shift, fill):
    whole = torch.full((G + shift + n + G,), fill, dtype=dtype, device="cuda")
    return whole, whole[G + shift:G + shift + n]


def intact(whole, n, shift, fill):
    return bool((whole[:G + shift] == fill).all()) and bool((whole[G + shift + n:] == fill).all())


@pytest.mark.parametrize("shift", [0, 1])
def test_sparse_writes_only_out_counts_and_wsum(shift):
    N, K = 100_003, 6
    idx, val = zip(*[synth.topk_sparse_deltas(8, k, N, 0.1, 1e-3) for k in range(K)])
    base = synth.normal_f32(8, synth.ROLE_BASE, 0, N, 0.02)
    n = synth.sample_counts(8, K, 100, 1000)
    wo, out = guarded(N, torch.float32, shift, -3.5)
    wc, cnt = guarded(N, torch.uint8, shift, 201)
    ww, ws = guarded(N, torch.int32, shift, -77)
    fa.sparse_masked_accumulate([torch.from_numpy(np.asarray(i, np.int64)).cuda() for i in idx],
                                [dev_f32(v) for v in val], n.tolist(), N, dev_f32(base), out,
                                counts=cnt, wsum=ws)
    torch.cuda.synchronize()
    assert intact(wo, N, shift, -3.5) and intact(wc, N, shift, 201) and intact(ww, N, shift, -77)
    ref, mag, rcnt, rws = oracle.sparse_average(list(idx), list(val), n, N, base=base)
    assert np.array_equal(cnt.cpu().numpy(), rcnt.astype(np.uint8))
    check(host_of(out), ref, mag, "f32", copied=rcnt == 0, copy_expect=base)


@pytest.mark.parametrize("shift", [0, 1])
def test_topk_writes_only_its_k_entries(shift):
    N, k = 300_007, 30_001
    x = np.random.default_rng(9).laplace(0.0, 1e-3, N).astype(np.float32)
    wi, idx = guarded(k, torch.int64, shift, -5)
    wv, val = guarded(k, torch.float32, shift, 9.75)
    fa.topk_select(dev_f32(x), k, idx_out=idx, val_out=val)
    torch.cuda.synchronize()
    assert intact(wi, k, shift, -5) and intact(wv, k, shift, 9.75)
    oi, ov = oracle.topk(x, oracle.F32, k)
    assert np.array_equal(idx.cpu().numpy(), oi)
    assert np.array_equal(val.cpu().numpy().view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("shift", [0, 1])
def test_streaming_finalize_writes_only_out(shift):
    N, K = 50_001, 3
    r = np.random.default_rng(10)
    xs = [(r.standard_normal(N) * 1e-3).astype(np.float32) for _ in range(K)]
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    n = [5, 9, 2]
    wo, out = guarded(N, torch.float32, shift, 1234.5)
    with fa.StreamingAccumulator(N, mode="deltas", chunk_bytes=4 * 8192) as acc:
        for k in range(K):
            d = dev_f32(xs[k])
            for off in range(0, N, 8192):
                acc.accumulate(k, n[k], d[off:off + 8192], offset=off)
        acc.finalize(dev_f32(base), out)
        acc.sync()
    assert intact(wo, N, shift, 1234.5)
    ref, mag, _, _ = oracle.weighted_average(xs, n, mode=oracle.DELTAS, base=base)
    check(host_of(out), ref, mag, "f32")


@pytest.mark.parametrize("N", [1001, 1002, 1003, 1004])
def test_begin_clears_exactly_the_buffers_it_is_given(N):
    """fedavg_begin zeroes N accumulator words, N weight sums and N count
    bytes, and nothing past them (N not a multiple of 4 leaves a count tail
    shorter than a word)."""
    acc_b, wsum_b, count_b, stag_b = fa.fedavg_workspace_size(N, True, 4096, 2)
    assert (acc_b, wsum_b, count_b) == (4 * N, 4 * N, N)
    wa, acc = guarded(N, torch.float32, 0, -2.5)
    ww, ws = guarded(N, torch.int32, 0, -77)
    wc, cnt = guarded(N, torch.uint8, 0, 201)
    staging = torch.empty(stag_b, dtype=torch.uint8, device="cuda")
    h = fa.fedavg_begin(N, "weights", True, acc, ws, cnt, staging, 4096, 2)
    try:
        fa.fedavg_sync(h)
    finally:
        fa.fedavg_destroy(h)
    torch.cuda.synchronize()
    assert intact(wa, N, 0, -2.5) and intact(ww, N, 0, -77) and intact(wc, N, 0, 201)
    assert int(torch.count_nonzero(acc)) == 0 and int(torch.count_nonzero(ws)) == 0
    assert int(torch.count_nonzero(cnt)) == 0
