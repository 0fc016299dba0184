"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (library defaults).  Inputs come from the same seeded device
generators as bench.py.  The dense 2B, sparse 1B and streaming 8B outputs are
checked whole: window by window, every output element against the oracle's
fp32 mirror bit for bit (its inputs copied to the host), the mirror's
checksum summed over the windows against the library's checksum of the whole
buffer, client counts and weight sums exactly, and one window in eight
against the fp64 definition within the stated tolerance (one in 24 for
streaming).  The other workloads are checked at sampled outputs (the
oracle's inputs gathered at those parameters) and through properties that
hold at any size."""

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


class HostWindows:
    """Pinned host buffers that device windows are copied into, reused from
    window to window."""

    def __init__(self):
        self.bufs = {}

    def get(self, t, name):
        """Host numpy copy of the contiguous device tensor t (float32, uint8,
        int32/uint32 views kept; bfloat16 as uint16 bits)."""
        n = t.numel()
        b = self.bufs.get(name)
        if b is None or b.numel() < n or b.dtype != t.dtype:
            b = torch.empty(max(n, 1), dtype=t.dtype, pin_memory=True)
            self.bufs[name] = b
        b[:n].copy_(t, non_blocking=True)
        return b[:n]

    @staticmethod
    def numpy(h):
        if h.dtype == torch.bfloat16:
            return h.view(torch.int16).numpy().view(np.uint16)
        return h.numpy()


def windows(N, W):
    return [(w0, min(w0 + W, N)) for w0 in range(0, N, W)]


def o1_window(i):
    """Windows checked against the fp64 definition as well: one in eight."""
    return i % 8 == 3


def test_dense_2b_k16_bf16_whole_output():
    # the clients and the output laid out as the benchmark's headline has them
    N = synth.numel_of(synth.dense_2b_tensor_shapes())
    arena, views = fa.client_arena(17, N, torch.bfloat16)
    n, xs = sd.dense_2b(N=N, dest=views[:16])
    out = views[16]
    assert N == 1_921_878_016 and len(xs) == 16
    fa.fedavg_aggregate(xs, n.tolist(), out)
    h1 = fa.fedavg_checksum(out)
    fa.fedavg_aggregate(xs, n.tolist(), out)
    assert fa.fedavg_checksum(out) == h1          # bit-identical rerun
    # the same clients in separate allocations give the same bits
    sep = [x.clone() for x in xs]
    out_sep = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    fa.fedavg_aggregate(sep, n.tolist(), out_sep)
    assert fa.fedavg_checksum(out_sep) == h1
    del sep, out_sep
    hw = HostWindows()
    want_hash = 0
    o1_elems = 0
    for i, (w0, w1) in enumerate(windows(N, 1 << 24)):
        hx = [hw.get(x[w0:w1], f"x{k}") for k, x in enumerate(xs)]
        ho = hw.get(out[w0:w1], "out")
        torch.cuda.synchronize()
        xk = [HostWindows.numpy(h) for h in hx]
        got = HostWindows.numpy(ho)
        mirror = oracle.mirror_f32(xk, n, x_dtype=oracle.BF16, out_dtype=oracle.BF16)
        same_bits(got, mirror)
        want_hash = (want_hash + oracle.checksum(mirror, oracle.BF16, first=w0)) % (1 << 64)
        if o1_window(i):
            ref, mag, _, _ = oracle.weighted_average(xk, n, x_dtype=oracle.BF16)
            check(got, ref, mag, "bf16", label=f"dense 2B window {w0}")
            o1_elems += w1 - w0
    assert h1 == want_hash
    assert o1_elems >= N // 10
    # the bf16 output's fixed-order value sum against the exact sum, over
    # the whole 1.92-billion-element buffer
    h, vs = fa.fedavg_checksum_sum(out)
    assert h == h1
    bits = host_of(out)
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


def test_sparse_1b_k20_whole_output():
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
    h_out, h_cnt = fa.fedavg_checksum(out), fa.fedavg_checksum(wsum.view(torch.float32))
    # the lists on the host, whole (24 GB)
    hidx = [i.cpu().numpy() for i in idx]
    hval = [v.cpu().numpy() for v in val]
    del idx, val
    hw = HostWindows()
    want_hash = want_wsum_hash = 0
    o1_elems = 0
    for i, (w0, w1) in enumerate(windows(N, 1 << 26)):
        hb = hw.get(base[w0:w1], "base")
        ho = hw.get(out[w0:w1], "out")
        hc = hw.get(counts[w0:w1], "counts")
        hws = hw.get(wsum[w0:w1], "wsum")
        cuts = [np.searchsorted(ix, [w0, w1]) for ix in hidx]
        wi = [ix[c0:c1] for ix, (c0, c1) in zip(hidx, cuts)]
        wv = [v[c0:c1] for v, (c0, c1) in zip(hval, cuts)]
        torch.cuda.synchronize()
        hb_, got = hb.numpy(), ho.numpy()
        mirror, mcnt, mws = oracle.sparse_mirror_f32(wi, wv, n, w0, w1 - w0, mode=oracle.DELTAS, base=hb_)
        same_bits(got, mirror)
        assert np.array_equal(hc.numpy(), mcnt.astype(np.uint8))
        assert np.array_equal(hws.numpy().view(np.uint32), mws.astype(np.uint32))
        want_hash = (want_hash + oracle.checksum(mirror, oracle.F32, first=w0)) % (1 << 64)
        want_wsum_hash = (want_wsum_hash +
                          oracle.checksum(mws.astype(np.uint32).view(np.float32), oracle.F32, first=w0)) % (1 << 64)
        if o1_window(i):
            ref, mag, rcnt, rws = oracle.sparse_average([x - w0 for x in wi], wv, n, w1 - w0,
                                                        mode=oracle.DELTAS, base=hb_)
            check(got, ref, mag, "f32", copied=rcnt == 0, copy_expect=hb_, label=f"sparse 1B window {w0}")
            assert np.array_equal(hc.numpy(), rcnt.astype(np.uint8))
            o1_elems += w1 - w0
    assert h_out == want_hash and h_cnt == want_wsum_hash
    assert o1_elems >= N // 10
    # every sent pair is counted exactly once
    assert int(counts.sum(dtype=torch.int64).item()) == sum(x.size for x in hidx)
    assert int(wsum.view(torch.int32).to(torch.int64).sum().item()) == \
        sum(int(n[k]) * hidx[k].size for k in range(K))


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


@pytest.fixture(scope="module")
def streamed_8b():
    """The 8B streaming workload run once: 32 clients, 240 chunks each from
    the pinned pool; the output is kept beside an untouched base."""
    per = synth.CHUNK_BYTES_8B // 2
    pool = sd.stream_8b_pool()
    P = pool.shape[0]
    base = sd.stream_8b_base()
    N = base.numel()
    assert N == 8_030_261_248
    n = sd.stream_8b_counts(32)
    cpc = (N + per - 1) // per
    out = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    with fa.StreamingAccumulator(N, mode="deltas", chunk_bytes=synth.CHUNK_BYTES_8B, n_slots=3) as acc:
        for k in range(32):
            for c in range(cpc):
                off = c * per
                ln = min(per, N - off)
                acc.accumulate(k, int(n[k]), pool[sd.pool_index(k, c, cpc, P)][:ln], offset=off)
        acc.finalize(base, out)
        acc.sync()
    torch.cuda.synchronize()
    state = {"pool": pool, "base": base, "out": out, "n": n, "per": per, "cpc": cpc, "N": N,
             "hash": fa.fedavg_checksum(out), "mirror_hash": {}}
    yield state
    del state["pool"], state["base"], state["out"]
    gc.collect()
    torch.cuda.empty_cache()


STREAM_PARTS = 4


@pytest.mark.parametrize("part", range(STREAM_PARTS))
def test_streaming_8b_k32_whole_output(streamed_8b, part):
    """The streamed output, one 64 MiB chunk window at a time (every
    STREAM_PARTS-th window in each part): bit for bit against the mirror of
    the same 32 pool chunks in arrival order, the fp64 definition on one
    window in 24 (10 windows), and, once every part has run, the summed mirror
    checksums against the library's checksum of the whole output."""
    st = streamed_8b
    pool, base, out, n, per, cpc, N = (st[k] for k in ("pool", "base", "out", "n", "per", "cpc", "N"))
    P = pool.shape[0]
    pool_bits = pool.view(torch.int16).numpy().view(np.uint16)
    hw = HostWindows()
    for c in range(part, cpc, STREAM_PARTS):
        w0, w1 = c * per, min((c + 1) * per, N)
        hb = hw.get(base[w0:w1], "base")
        ho = hw.get(out[w0:w1], "out")
        torch.cuda.synchronize()
        deltas = [pool_bits[sd.pool_index(k, c, cpc, P)][:w1 - w0] for k in range(32)]
        hb_, got = HostWindows.numpy(hb), HostWindows.numpy(ho)
        mirror = oracle.mirror_f32(deltas, n, mode=oracle.DELTAS, base=hb_, x_dtype=oracle.BF16,
                                   base_dtype=oracle.BF16, out_dtype=oracle.BF16)
        same_bits(got, mirror)
        st["mirror_hash"][c] = oracle.checksum(mirror, oracle.BF16, first=w0)
        if c % 24 == 5:
            ref, mag, _, _ = oracle.weighted_average(deltas, n, mode=oracle.DELTAS, base=hb_,
                                                     x_dtype=oracle.BF16, base_dtype=oracle.BF16)
            check(got, ref, mag, "bf16", label=f"streaming 8B window {c}")
    if len(st["mirror_hash"]) == cpc:
        assert sum(st["mirror_hash"].values()) % (1 << 64) == st["hash"]
