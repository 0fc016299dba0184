"""GPU parity for the averaging-rule variants: the zero-fill reading of
partial sharing (a parameter a client did not send counts as a zero delta,
so the divisor is the total weight of all clients), and the unweighted mean
(every n_k = 1)."""

import numpy as np
import pytest
import torch

import oracle
import synth
import weighted_model_update_amd as fa
from parity import check, base_copy_expect
from gpu_util import dev_of, host_of, empty

pytestmark = pytest.mark.gpu

ODT = {"f32": oracle.F32, "bf16": oracle.BF16}


def segments(T, max_size, seed):
    r = np.random.default_rng(seed)
    sizes = r.integers(0, max_size, size=T)
    sizes[::13] = 0
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


@pytest.mark.parametrize("T,max_size", [(150, 3000), (1500, 300)])
@pytest.mark.parametrize("xdt,bdt,odt", [("f32", "f32", "f32"), ("bf16", "bf16", "bf16"), ("bf16", "f32", "f32")])
def test_masked_zero_fill_matches_oracle(T, max_size, xdt, bdt, odt):
    r = np.random.default_rng(T)
    bounds = segments(T, max_size, T + 1)
    N = int(bounds[-1])
    K = 6
    present = (r.random((K, T)) < 0.5).astype(np.uint8)
    present[:, 2] = 0
    n = synth.sample_counts(21, K, 1, 5000)
    n[3] = 0
    xs32 = [(r.standard_normal(N) * 1e-3).astype(np.float32) for _ in range(K)]
    xs = [synth.bf16_bits_from_f32(x) for x in xs32] if xdt == "bf16" else xs32
    b32 = (r.standard_normal(N) * 0.02).astype(np.float32)
    base = synth.bf16_bits_from_f32(b32) if bdt == "bf16" else b32
    out = empty(N, odt)
    fa.fedavg_aggregate([dev_of(x, xdt) for x in xs], n.tolist(), out, mode="deltas_zero_fill",
                        base=dev_of(base, bdt), seg_bounds=torch.from_numpy(bounds).cuda(),
                        present=torch.from_numpy(present).cuda())
    torch.cuda.synchronize()
    seg_of = np.repeat(np.arange(T), np.diff(bounds))
    sent = [present[k][seg_of] for k in range(K)]
    ref, mag, cnt, _ = oracle.weighted_average(xs, n, mode=oracle.DELTAS_ZERO_FILL, base=base,
                                               x_dtype=ODT[xdt], base_dtype=ODT[bdt], sent=sent)
    check(host_of(out), ref, mag, odt, copied=cnt == 0, copy_expect=base_copy_expect(base, bdt, odt))


def test_zero_fill_with_full_support_is_plain_deltas_bit_for_bit():
    K, N = 5, 100_003
    r = np.random.default_rng(22)
    xs = [(r.standard_normal(N) * 1e-3).astype(np.float32) for _ in range(K)]
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    n = [3, 1, 4, 1, 5]
    bounds = torch.tensor([0, 50_000, N], dtype=torch.int64, device="cuda")
    present = torch.ones(2 * K, dtype=torch.uint8, device="cuda")
    outs = []
    for mode in ("deltas", "deltas_zero_fill"):
        for masks in (False, True):
            o = empty(N, "f32")
            fa.fedavg_aggregate([dev_of(x, "f32") for x in xs], n, o, mode=mode, base=dev_of(base, "f32"),
                                seg_bounds=bounds if masks else None, present=present if masks else None)
            outs.append(o)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


@pytest.mark.parametrize("tile", [2048, 4096])
def test_sparse_zero_fill_matches_oracle(tile):
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, tile)
    try:
        N, K = 300_007, 8
        idx, val = zip(*[synth.topk_sparse_deltas(31, k, N, 0.1, 1e-3) for k in range(K)])
        idx, val = list(idx), list(val)
        idx[2] = np.array([], np.int64)            # a client that sent nothing still counts in S
        val[2] = np.array([], np.float32)
        n = synth.sample_counts(32, K, 100, 1000)
        base = synth.normal_f32(33, synth.ROLE_BASE, 0, N, 0.02)
        out = torch.empty(N, dtype=torch.float32, device="cuda")
        counts = torch.empty(N, dtype=torch.uint8, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        fa.sparse_masked_accumulate([torch.from_numpy(i).cuda() for i in idx], [dev_of(v, "f32") for v in val],
                                    n.tolist(), N, dev_of(base, "f32"), out, mode="deltas_zero_fill",
                                    counts=counts, err_flag=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        ref, mag, rcnt, _ = oracle.sparse_average(idx, val, n, N, mode=oracle.DELTAS_ZERO_FILL, base=base)
        assert np.array_equal(counts.cpu().numpy(), rcnt.astype(np.uint8))
        check(host_of(out), ref, mag, "f32", copied=rcnt == 0, copy_expect=base)
    finally:
        fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, 2048)


def test_streaming_partial_zero_fill_matches_oracle():
    K, N = 5, 60_001
    r = np.random.default_rng(41)
    xs = [synth.bf16_bits_from_f32((r.standard_normal(N) * 1e-3).astype(np.float32)) for _ in range(K)]
    masks = [(r.random(N) < 0.3).astype(np.uint8) for _ in range(K)]
    n = synth.sample_counts(42, K, 100, 1000)
    base = synth.bf16_bits_from_f32((r.standard_normal(N) * 0.02).astype(np.float32))
    out = empty(N, "bf16")
    with fa.StreamingAccumulator(N, mode="deltas_zero_fill", partial=True, chunk_bytes=2 * N) as acc:
        for k in range(K):
            x = dev_of(xs[k], "bf16")
            if k % 2 == 0:
                m = torch.from_numpy(masks[k]).cuda()
                for off in range(0, N, 7000):
                    acc.accumulate(k, int(n[k]), x[off:off + 7000], offset=off, mask=m[off:off + 7000])
            else:
                ii = torch.from_numpy(np.nonzero(masks[k])[0].astype(np.int64)).cuda()
                acc.accumulate(k, int(n[k]), x[ii].contiguous(), indices=ii)
        acc.finalize(dev_of(base, "bf16"), out)
        acc.sync()
    ref, mag, cnt, _ = oracle.weighted_average(xs, n, mode=oracle.DELTAS_ZERO_FILL, base=base,
                                               x_dtype=oracle.BF16, base_dtype=oracle.BF16, sent=masks)
    check(host_of(out), ref, mag, "bf16", copied=cnt == 0, copy_expect=base)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_unweighted_mean(dt):
    """The plain average is the weighted one with every n_k = 1; it matches
    numpy's fp64 mean rounded once to fp32."""
    K, N = 7, 123_457
    r = np.random.default_rng(51)
    xs32 = [(r.standard_normal(N) * 0.02).astype(np.float32) for _ in range(K)]
    xs = [synth.bf16_bits_from_f32(x) for x in xs32] if dt == "bf16" else xs32
    vals = [synth.f32_from_bf16_bits(x) for x in xs] if dt == "bf16" else xs32
    out = empty(N, "f32")
    fa.fedavg_aggregate([dev_of(x, dt) for x in xs], [1] * K, out)
    torch.cuda.synchronize()
    ref, mag, _, _ = oracle.weighted_average(xs, [1] * K, x_dtype=ODT[dt])
    check(host_of(out), ref, mag, "f32")
    npmean = np.mean(np.stack(vals).astype(np.float64), axis=0).astype(np.float32)
    check(host_of(out), npmean, mag, "f32", label="numpy mean")
