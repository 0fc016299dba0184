"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (library defaults).  Inputs come from the same seeded device
generators as bench.py; the oracle checks sampled outputs one by one (its
inputs gathered at those parameters), and whole-buffer properties that hold
at any size are checked exactly."""

import gc
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import synth.device as sd
import weighted_model_update_amd as fa
from parity import check
from gpu_util import host_of


def same_bits(got, want):
    """Equal bit patterns (the stated fp32 rounding order, checked against
    the oracle's fp32 mirror of it)."""
    g, w = np.asarray(got), np.asarray(want)
    assert g.dtype == w.dtype and g.shape == w.shape
    v = np.uint32 if g.dtype == np.float32 else np.uint16
    assert np.array_equal(g.view(v), w.view(v)), int((g.view(v) != w.view(v)).sum())

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sample_positions(N, S, seed):
    r = np.random.default_rng(seed)
    at = np.concatenate([np.arange(min(N, 2048)), np.arange(max(0, N - 2048), N),
                         r.integers(0, N, S)])
    return np.unique(at).astype(np.int64)


def gather_bits(t, at_dev):
    """Values of t at the positions at_dev, as float32 or uint16 bf16 bits."""
    return host_of(t.index_select(0, at_dev))


def test_dense_2b_k16_bf16_sampled():
    n, xs = sd.dense_2b()
    N = xs[0].numel()
    assert N == 1_921_878_016 and len(xs) == 16
    out = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    fa.fedavg_aggregate(xs, n.tolist(), out)
    h1 = fa.fedavg_checksum(out)
    fa.fedavg_aggregate(xs, n.tolist(), out)
    assert fa.fedavg_checksum(out) == h1          # bit-identical rerun
    at = sample_positions(N, 200_000, 3)
    at_dev = torch.from_numpy(at).cuda()
    got = gather_bits(out, at_dev)
    xk = [gather_bits(x, at_dev) for x in xs]
    ref, mag, _, _ = oracle.weighted_average(xk, n, x_dtype=oracle.BF16)
    check(got, ref, mag, "bf16", label="dense 2B sampled")
    same_bits(got, oracle.mirror_f32(xk, n, x_dtype=oracle.BF16, out_dtype=oracle.BF16))
    # the bf16 output's checksum and value sum against the oracle's, over the
    # whole 1.92-billion-element buffer
    h, vs = fa.fedavg_checksum_sum(out)
    assert h == h1
    bits = host_of(out)
    assert h == oracle.checksum(bits, oracle.BF16)
    want = oracle.value_sum(bits, oracle.BF16)
    absum = oracle.value_sum(bits & np.uint16(0x7FFF), oracle.BF16)
    T = -(-N // 8192)
    hh = 48 + -(-T // 1024)
    u = 2.0 ** -53
    assert abs(vs - want) <= hh * u / (1 - hh * u) * absum * (1 + 4 * u), (vs, want)


def test_adapter_k8_full_compare():
    n, xs, base, bounds, present = sd.adapter()
    N = xs[0].numel()
    out = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    fa.fedavg_aggregate(xs, n.tolist(), out, base=base,
                        seg_bounds=torch.from_numpy(bounds).cuda(),
                        present=torch.from_numpy(np.ascontiguousarray(present, np.uint8)).cuda())
    torch.cuda.synchronize()
    seg_of = np.repeat(np.arange(len(bounds) - 1), np.diff(bounds))
    sent = [present[k][seg_of].astype(np.uint8) for k in range(len(xs))]
    hb = host_of(base)
    ref, mag, cnt, _ = oracle.weighted_average([host_of(x) for x in xs], n, x_dtype=oracle.BF16,
                                               base=hb, base_dtype=oracle.BF16, sent=sent)
    check(host_of(out), ref, mag, "bf16", copied=cnt == 0, copy_expect=hb, label="adapter full")
    same_bits(host_of(out), oracle.mirror_f32([host_of(x) for x in xs], n, x_dtype=oracle.BF16, base=hb,
                                              base_dtype=oracle.BF16, out_dtype=oracle.BF16, sent=sent))


def test_sparse_1b_k20_sampled():
    n, idx, val, base = sd.sparse_1b()
    N = base.numel()
    K = len(idx)
    assert all(i.numel() == N // 10 for i in idx)
    out = torch.empty(N, dtype=torch.float32, device="cuda")
    counts = torch.empty(N, dtype=torch.uint8, device="cuda")
    wsum = torch.empty(N, dtype=torch.int32, device="cuda")
    err = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    fa.sparse_masked_accumulate(idx, val, n.tolist(), N, base, out, counts=counts, wsum=wsum,
                                err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # every sent pair is counted exactly once
    assert int(counts.sum(dtype=torch.int64).item()) == sum(i.numel() for i in idx)
    assert int(wsum.view(torch.int32).to(torch.int64).sum().item()) == \
        sum(int(n[k]) * idx[k].numel() for k in range(K))
    at = sample_positions(N, 200_000, 5)
    at_dev = torch.from_numpy(at).cuda()
    sent, vals = [], []
    for k in range(K):
        pos = torch.searchsorted(idx[k], at_dev)
        pos_c = pos.clamp(max=idx[k].numel() - 1)
        found = (idx[k].index_select(0, pos_c) == at_dev)
        sent.append(found.cpu().numpy().astype(np.uint8))
        vals.append(torch.where(found, val[k].index_select(0, pos_c), torch.zeros_like(at_dev, dtype=torch.float32))
                    .cpu().numpy())
    hb = gather_bits(base, at_dev)
    ref, mag, rcnt, rws = oracle.weighted_average(vals, n, mode=oracle.DELTAS, base=hb, sent=sent)
    assert np.array_equal(gather_bits(counts, at_dev), rcnt.astype(np.uint8))
    assert np.array_equal(wsum.index_select(0, at_dev).cpu().numpy().view(np.uint32), rws.astype(np.uint32))
    check(gather_bits(out, at_dev), ref, mag, "f32", copied=rcnt == 0, copy_expect=hb,
          label="sparse 1B sampled")
    same_bits(gather_bits(out, at_dev), oracle.mirror_f32(vals, n, mode=oracle.DELTAS, base=hb, sent=sent))


def test_client_at_a_time_sparse_1b_k20_equals_the_one_pass_merge():
    """The 20 top-10% lists of the 10^9-parameter sparse workload, scattered
    one client at a time into the partial-mode streaming accumulator, give
    the one-pass merge's output bit for bit over the whole buffer (both take
    each parameter's clients in order with one fused multiply-add each, then
    one division and the base), the same client counts and weight sums, and
    agree with the oracle at sampled parameters."""
    n, idx, val, base = sd.sparse_1b()
    N = base.numel()
    K = len(idx)
    out1 = torch.empty(N, dtype=torch.float32, device="cuda")
    counts1 = torch.empty(N, dtype=torch.uint8, device="cuda")
    wsum1 = torch.empty(N, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fa.sparse_masked_accumulate(idx, val, n.tolist(), N, base, out1, counts=counts1, wsum=wsum1,
                                err_flag=err)
    out2 = torch.empty(N, dtype=torch.float32, device="cuda")
    with fa.StreamingAccumulator(N, mode="deltas", partial=True, chunk_bytes=1 << 20, n_slots=2) as acc:
        for k in range(K):
            acc.accumulate(k, int(n[k]), val[k], indices=idx[k])
        acc.finalize(base, out2)
        acc.sync()
        assert torch.equal(acc.count[:N], counts1)
        assert torch.equal(acc.wsum[:N].view(torch.int32), wsum1)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32))
    del out1, counts1, wsum1
    at = sample_positions(N, 100_000, 11)
    at_dev = torch.from_numpy(at).cuda()
    sent, vals = [], []
    for k in range(K):
        pos = torch.searchsorted(idx[k], at_dev)
        pos_c = pos.clamp(max=idx[k].numel() - 1)
        found = (idx[k].index_select(0, pos_c) == at_dev)
        sent.append(found.cpu().numpy().astype(np.uint8))
        vals.append(torch.where(found, val[k].index_select(0, pos_c), torch.zeros_like(at_dev, dtype=torch.float32))
                    .cpu().numpy())
    hb = gather_bits(base, at_dev)
    ref, mag, rcnt, _ = oracle.weighted_average(vals, n, mode=oracle.DELTAS, base=hb, sent=sent)
    check(gather_bits(out2, at_dev), ref, mag, "f32", copied=rcnt == 0, copy_expect=hb,
          label="client-at-a-time sparse 1B sampled")


def test_streaming_8b_k32_sampled():
    per = synth.CHUNK_BYTES_8B // 2
    pool = sd.stream_8b_pool()
    P = pool.shape[0]
    base = sd.stream_8b_base()
    N = base.numel()
    assert N == 8_030_261_248
    n = sd.stream_8b_counts(32)
    cpc = (N + per - 1) // per
    at = sample_positions(N, 100_000, 7)
    at_dev = torch.from_numpy(at).cuda()
    base_before = gather_bits(base, at_dev)
    with fa.StreamingAccumulator(N, mode="deltas", chunk_bytes=synth.CHUNK_BYTES_8B, n_slots=3) as acc:
        for k in range(32):
            for c in range(cpc):
                off = c * per
                ln = min(per, N - off)
                acc.accumulate(k, int(n[k]), pool[sd.pool_index(k, c, cpc, P)][:ln], offset=off)
        acc.finalize(base, base)
        acc.sync()
    got = gather_bits(base, at_dev)
    pool_bits = pool.view(torch.int16).numpy().view(np.uint16)
    c_of = at // per
    e_of = at - c_of * per
    deltas = [pool_bits[[sd.pool_index(k, int(c), cpc, P) for c in c_of], e_of] for k in range(32)]
    ref, mag, _, _ = oracle.weighted_average(deltas, n, mode=oracle.DELTAS, base=base_before,
                                             x_dtype=oracle.BF16, base_dtype=oracle.BF16)
    check(got, ref, mag, "bf16", label="streaming 8B sampled")
    same_bits(got, oracle.mirror_f32(deltas, n, mode=oracle.DELTAS, base=base_before, x_dtype=oracle.BF16,
                                     base_dtype=oracle.BF16, out_dtype=oracle.BF16))


def test_two_level_8b_three_silos_sampled():
    """Two-level aggregation at the 8B size, through the call the benchmark
    times: each of three silos is one client with n = W_g (its partial is
    W_g * x_g, one fp32 rounding, as a silo accumulator forms it), the
    partials enter the top-level accumulator as pseudo-clients in deltas
    mode, and finalize writes bf16.  In exact arithmetic this is the flat
    weighted average of the silos' clients: the flat oracle checks sampled
    outputs."""
    N = synth.numel_of(synth.stream_8b_tensor_shapes())
    assert N == 8_030_261_248
    W = [int(w) for w in synth.sample_counts(synth.CFG_STREAM_8B, 3, 1000, 80000)]
    at = sample_positions(N, 100_000, 11)
    at_dev = torch.from_numpy(at).cuda()
    acc_b, _, _, stag_b = fa.fedavg_workspace_size(N, 0, 1 << 20, 1)
    acc = torch.empty(acc_b // 4, dtype=torch.float32, device="cuda")
    staging = torch.empty(stag_b, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda")
    xs = []
    h = fa.fedavg_begin(N, "deltas", False, acc, None, None, staging, 1 << 20, 1)
    try:
        for k in range(3):
            g.manual_seed(9100 + k)
            x = torch.empty(N, dtype=torch.bfloat16, device="cuda")
            x.normal_(0.0, 1e-3, generator=g)
            xs.append(gather_bits(x, at_dev))
            part = x.float()
            del x
            part.mul_(float(W[k]))
            fa.fedavg_accumulate_partial(h, k, W[k], 1, part, offset=0)
            torch.cuda.synchronize()
            del part
        g.manual_seed(9200)
        base = torch.empty(N, dtype=torch.bfloat16, device="cuda")
        base.normal_(0.0, 0.02, generator=g)
        base_at = gather_bits(base, at_dev)
        out = torch.empty(N, dtype=torch.bfloat16, device="cuda")
        fa.fedavg_finalize(h, base, out)
        fa.fedavg_sync(h)
    finally:
        fa.fedavg_destroy(h)
    got = gather_bits(out, at_dev)
    ref, mag, _, _ = oracle.weighted_average(xs, np.array(W, np.int64), mode=oracle.DELTAS, base=base_at,
                                             x_dtype=oracle.BF16, base_dtype=oracle.BF16)
    check(got, ref, mag, "bf16", label="two-level 8B sampled")
    # the stated order, in numpy's IEEE float32: each partial one rounded
    # product, the partials added in call order, one division, the base added
    x32 = [(xb.astype(np.uint32) << 16).view(np.float32) for xb in xs]
    acc32 = np.zeros(len(at), np.float32)
    for k in range(3):
        acc32 = (acc32 + (np.float32(W[k]) * x32[k]).astype(np.float32)).astype(np.float32)
    q = (acc32 / np.float32(sum(W))).astype(np.float32)
    r = ((base_at.astype(np.uint32) << 16).view(np.float32) + q).astype(np.float32)
    same_bits(got, oracle.round_to_bf16(r))


def test_topk_1b_client_update_properties():
    """Top-10% of a 10^9-parameter fp32 client update.  The kept set is
    unique, and these properties pin it at any size: k entries, strictly
    increasing indices, the values read at those indices, every kept key at
    least every dropped key, and among keys equal to the threshold the kept
    ones all lie below the dropped ones.  The sampled and the three-pass
    paths agree bit for bit."""
    N = 10 ** 9
    x = sd.client_delta_1b(0, N)
    k = fa.topk_count(N, 0.1)
    idx, val = fa.topk_select(x, k)
    torch.cuda.synchronize()
    assert idx.numel() == k
    assert bool((idx[1:] > idx[:-1]).all()) and int(idx[0]) >= 0 and int(idx[-1]) < N
    assert torch.equal(val.view(torch.int32), x[idx].view(torch.int32))
    key = x.view(torch.int32) & 0x7FFFFFFF
    kept = torch.zeros(N, dtype=torch.bool, device="cuda")
    kept[idx] = True
    T = int(key[idx].min())
    dropped_max = int(key.masked_fill(kept, -1).max())
    assert dropped_max <= T
    if dropped_max == T:
        tie = key == T
        kept_ties = torch.nonzero(tie & kept).flatten()
        dropped_ties = torch.nonzero(tie & ~kept).flatten()
        assert int(kept_ties.max()) < int(dropped_ties.min())
    # the threshold sits where the distribution says: b*ln(10) for Laplace(0, b)
    t = float(torch.tensor(T, dtype=torch.int32).view(torch.float32))
    assert abs(t / (1e-3 * math.log(10)) - 1) < 0.01
    # the three-pass path (no sample) keeps exactly the same entries
    fa.fedavg_set_option(fa.FA_OPT_TOPK_SAMPLED, 0)
    try:
        i3, v3 = fa.topk_select(x, k)
        torch.cuda.synchronize()
    finally:
        fa.fedavg_set_option(fa.FA_OPT_TOPK_SAMPLED, 1)
    assert torch.equal(i3, idx) and torch.equal(v3.view(torch.int32), val.view(torch.int32))
    del i3, v3
    # and the oracle agrees on a window of the update (its own top-k of the
    # window, compared with the GPU's on the same window)
    w = x[:2_000_000].cpu().numpy()
    kw = 200_000
    wi, wv = fa.topk_select(x[:2_000_000], kw)
    oi, ov = oracle.topk(w, oracle.F32, kw)
    assert np.array_equal(wi.cpu().numpy(), oi) and np.array_equal(wv.cpu().numpy().view(np.uint32),
                                                                   ov.view(np.uint32))


def test_value_sum_1b_fp32_against_the_exact_sum():
    """The fused checksum and fp64 value sum of a 10^9-parameter fp32 client
    update: the hash equals the oracle's bit for bit, the sum lies within the
    rounding bound of the exact sum (h = 48 + ceil(T / 1024) additions on the
    longest chain, T tiles of 8192), and other launch shapes give the same
    bits."""
    N = 10 ** 9
    x = sd.client_delta_1b(0, N)
    h, s = fa.fedavg_checksum_sum(x)
    fa.fedavg_set_option(fa.FA_OPT_BLOCKS_PER_CU, 2)
    try:
        _, s2 = fa.fedavg_checksum_sum(x, with_hash=False)
    finally:
        fa.fedavg_set_option(fa.FA_OPT_BLOCKS_PER_CU, 0)
    assert s2.hex() == s.hex()
    a = x.cpu().numpy()
    del x
    assert np.isfinite(a).all()          # the Laplace generator yields no infinities
    assert h == oracle.checksum(a, oracle.F32)
    want = oracle.value_sum(a, oracle.F32)
    absum = oracle.value_sum((a.view(np.uint32) & np.uint32(0x7FFFFFFF)).view(np.float32), oracle.F32)
    T = -(-N // 8192)
    hh = 48 + -(-T // 1024)
    u = 2.0 ** -53
    assert abs(s - want) <= hh * u / (1 - hh * u) * absum * (1 + 4 * u), (s, want, absum)


def test_past_2_35_parameters_the_grid_stride_covers_every_vector():
    """Two bf16 clients of 2^35 + 8003 parameters: one 8-parameter vector
    per lane would take more than the 2^32 - 1 work-items a launch holds, so
    the grid stops at that and the dense kernel walks the rest grid-stride.
    Sampled outputs, among them the last vectors and the ragged tail, match
    the oracle."""
    N = (1 << 35) + 8003

    def normal_bf16(g, piece=1 << 30):
        # drawn in fp32 pieces so that no full-size fp32 copy is ever held
        x = torch.empty(N, dtype=torch.bfloat16, device="cuda")
        tmp = torch.empty(piece, dtype=torch.float32, device="cuda")
        for o in range(0, N, piece):
            m = min(piece, N - o)
            tmp[:m].normal_(0.0, 0.02, generator=g)
            x[o:o + m].copy_(tmp[:m])
        return x

    xs = [normal_bf16(sd.generator(synth.CFG_DENSE_2B, synth.ROLE_VALUES, 900 + c)) for c in range(2)]
    n = np.array([300, 700], dtype=np.int64)
    out = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    fa.fedavg_aggregate(xs, n.tolist(), out)
    torch.cuda.synchronize()
    r = np.random.default_rng(35)
    at = np.unique(np.concatenate([np.arange(N - 20_000, N), (1 << 35) - 8 + np.arange(16),
                                   r.integers(0, N, 200_000)])).astype(np.int64)
    at_dev = torch.from_numpy(at).cuda()
    got = gather_bits(out, at_dev)
    xk = [gather_bits(x, at_dev) for x in xs]
    ref, mag, _, _ = oracle.weighted_average(xk, n, x_dtype=oracle.BF16)
    check(got, ref, mag, "bf16", label="2^35 + 8003 dense")
    same_bits(got, oracle.mirror_f32(xk, n, x_dtype=oracle.BF16, out_dtype=oracle.BF16))


def test_topk_1b_bf16_client_update_properties():
    """Top-10% of a 10^9-parameter bf16 update (the fp32 Laplace update
    rounded to bf16, so many magnitudes tie): k entries, strictly increasing
    indices, values read at those indices and widened to fp32, every kept
    key at least every dropped key, the kept ties below the dropped ones;
    the sampled and three-pass paths agree bit for bit; the oracle agrees on
    a window."""
    N = 10 ** 9
    x = sd.client_delta_1b(0, N).to(torch.bfloat16)
    k = fa.topk_count(N, 0.1)
    idx, val = fa.topk_select(x, k)
    torch.cuda.synchronize()
    assert idx.numel() == k
    assert bool((idx[1:] > idx[:-1]).all()) and int(idx[0]) >= 0 and int(idx[-1]) < N
    assert torch.equal(val, x[idx].float())
    key = x.view(torch.int16).to(torch.int32) & 0x7FFF
    kept = torch.zeros(N, dtype=torch.bool, device="cuda")
    kept[idx] = True
    T = int(key[idx].min())
    dropped_max = int(key.masked_fill(kept, -1).max())
    assert dropped_max <= T
    if dropped_max == T:
        tie = key == T
        assert int(torch.nonzero(tie & kept).flatten().max()) < int(torch.nonzero(tie & ~kept).flatten().min())
    del key, kept
    fa.fedavg_set_option(fa.FA_OPT_TOPK_SAMPLED, 0)
    try:
        i3, v3 = fa.topk_select(x, k)
        torch.cuda.synchronize()
    finally:
        fa.fedavg_set_option(fa.FA_OPT_TOPK_SAMPLED, 1)
    assert torch.equal(i3, idx) and torch.equal(v3.view(torch.int32), val.view(torch.int32))
    del i3, v3
    w = host_of(x[:2_000_000])
    kw = 200_000
    wi, wv = fa.topk_select(x[:2_000_000], kw)
    oi, ov = oracle.topk(w, oracle.BF16, kw)
    assert np.array_equal(wi.cpu().numpy(), oi) and np.array_equal(wv.cpu().numpy().view(np.uint32),
                                                                   ov.view(np.uint32))
