"""GPU parity: the client-at-a-time sparse accumulate (fedavg_accumulate with
indices) over dense tiles.  The tiled path must leave the fp32 sums, weight
sums and counts bit for bit as the scatter path does, give the oracle
mirror's finalized bits, and hand lists it cannot take (unsorted, duplicate
or out-of-range entries) to the scatter path, which reports and skips the bad
entries."""

import numpy as np
import pytest
import torch

import oracle
import weighted_model_update_amd as fa
from gpu_util import dev_of, host_of, empty

pytestmark = pytest.mark.gpu

SCATTER, TILES = 1, 2
BF16 = {"f32": oracle.F32, "bf16": oracle.BF16}


@pytest.fixture(autouse=True)
def _default_path():
    yield
    fa.fedavg_set_option(fa.FA_OPT_INDEX_TILES, 0)


def _lists(case, N, K, seed):
    """K clients' (offset, sorted relative indices) for one test case."""
    r = np.random.default_rng(seed)
    out = []
    for k in range(K):
        if case == "dense10":
            off, rel = 0, np.nonzero(r.random(N) < 0.1)[0]
        elif case == "full":            # every parameter: 2048 entries per tile
            off, rel = 0, np.arange(N)
        elif case == "sub_range":       # a client covering part of the model
            off = 1000 + 8 * k
            rel = np.nonzero(r.random(6000) < 0.4)[0] + 2000
        elif case == "ends":            # the first and last parameters
            off, rel = 0, np.array([0, 1, 2047, 2048, 4093, N - 2, N - 1])
        elif case == "single":
            off, rel = 7, np.array([N - 8 - 3 * k])
        elif case == "clustered":       # bursts with long gaps between them
            starts = np.sort(r.choice(N // 512, 6, replace=False)) * 512
            rel = np.unique(np.concatenate([s + r.choice(400, 300, replace=False) for s in starts]))
            off = 0
        else:
            raise ValueError(case)
        out.append((off, np.ascontiguousarray(rel, np.int64)))
    return out


def _run(path, N, lists, vals, n, dt, counts, base):
    fa.fedavg_set_option(fa.FA_OPT_INDEX_TILES, path)
    out = empty(N, "f32")
    with fa.StreamingAccumulator(N, mode="deltas", partial=True, counts=counts,
                                 chunk_bytes=4 * N, n_slots=2) as acc:
        for k, (off, rel) in enumerate(lists):
            acc.accumulate(k, int(n[k]), dev_of(vals[k][off + rel], dt), offset=off,
                           indices=torch.from_numpy(rel).cuda())
        acc.sync()
        state = (acc.acc[:N].clone(), acc.wsum[:N].clone(),
                 acc.count[:N].clone() if counts else None)
        acc.finalize(dev_of(base, "f32"), out)
        acc.sync()
    return state, host_of(out)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("counts", [True, False])
@pytest.mark.parametrize("case", ["dense10", "full", "sub_range", "ends", "single", "clustered"])
def test_tiles_equal_scatter_and_oracle(case, counts, dt):
    N = 5 * 2048 + 516                  # ragged last tile (N % 4 == 0)
    K = 3
    lists = _lists(case, N, K, 5)
    r = np.random.default_rng(6)
    if dt == "f32":
        vals = [(r.standard_normal(N) * 1e-3).astype(np.float32) for _ in range(K)]
    else:
        vals = [(r.standard_normal(N) * 1e-3).astype(np.float32).view(np.uint32) >> 16 for _ in range(K)]
        vals = [v.astype(np.uint16) for v in vals]
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    n = [300, 7, 4096]
    (a1, w1, c1), o1 = _run(SCATTER, N, lists, vals, n, dt, counts, base)
    (a2, w2, c2), o2 = _run(TILES, N, lists, vals, n, dt, counts, base)
    assert torch.equal(a1.view(torch.int32), a2.view(torch.int32))
    assert torch.equal(w1, w2)
    if counts:
        assert torch.equal(c1, c2)
    sent = []
    for off, rel in lists:
        s = np.zeros(N, np.uint8)
        s[off + rel] = 1
        sent.append(s)
    full = [v.astype(np.float32) if dt == "f32" else v for v in vals]
    want = oracle.mirror_f32(full, n, mode=oracle.DELTAS, base=base, x_dtype=BF16[dt], sent=sent)
    assert np.array_equal(o1.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(o2.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("path", [0, TILES])
def test_many_tiles_and_workgroups(path):
    """About 490 tiles over several hundred workgroups, each workgroup but
    the first finding its first entry by search; one client covers a
    30% list, another a sub-range from an offset; the default rule (path 0)
    takes the tiles at these densities."""
    N = 1_000_004
    r = np.random.default_rng(9)
    lists = [(0, np.nonzero(r.random(N) < 0.3)[0].astype(np.int64)),
             (123_456, (np.nonzero(r.random(500_000) < 0.5)[0] + 7).astype(np.int64))]
    vals = [(r.standard_normal(N) * 1e-3).astype(np.float32) for _ in range(2)]
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    n = [11, 12]
    (a1, w1, c1), o1 = _run(SCATTER, N, lists, vals, n, "f32", True, base)
    (a2, w2, c2), o2 = _run(path, N, lists, vals, n, "f32", True, base)
    assert torch.equal(a1.view(torch.int32), a2.view(torch.int32))
    assert torch.equal(w1, w2) and torch.equal(c1, c2)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


@pytest.mark.parametrize("bad", ["unsorted", "duplicate", "negative", "past_end", "wraps"])
def test_tiles_hand_bad_lists_to_the_scatter_path(bad):
    """Forced tiles: a list the check refuses is scattered instead, so the
    call reports FA_ERR_INDEX at sync, skips the bad entries and applies
    the good ones, exactly as the scatter path alone does."""
    N = 4096
    offset = 16
    rel = {"unsorted": [1, 5, 3, 9, 40],
           "duplicate": [1, 5, 5, 9, 40],
           "negative": [-4, -2, 3, 9, 40],
           "past_end": [1, 5, 9, N - offset, N + 100],
           "wraps": [1, 5, 9, (1 << 63) - 8, (1 << 63) - 2]}[bad]
    got = []
    for path in (SCATTER, TILES):
        fa.fedavg_set_option(fa.FA_OPT_INDEX_TILES, path)
        with fa.StreamingAccumulator(N, mode="weights", partial=True, chunk_bytes=4 * N) as acc:
            acc.accumulate(0, 3, torch.arange(1, len(rel) + 1, dtype=torch.float32, device="cuda"),
                           offset=offset, indices=torch.tensor(rel, dtype=torch.int64, device="cuda"))
            with pytest.raises(fa.FedAvgError) as e:
                acc.sync()
            assert e.value.code == -7
            got.append((acc.acc[:N].clone(), acc.wsum[:N].clone(), acc.count[:N].clone()))
    for x, y in zip(*got):
        assert torch.equal(x, y)
    assert int(torch.count_nonzero(got[1][0])) >= 3


def test_tiles_after_a_refused_list_take_the_next_list():
    """The check's verdict is per call: a bad list followed by a good one on
    the same handle -- the good one is tiled and lands whole."""
    N = 8192
    fa.fedavg_set_option(fa.FA_OPT_INDEX_TILES, TILES)
    good = np.arange(0, N, 3, dtype=np.int64)
    with fa.StreamingAccumulator(N, mode="weights", partial=True, chunk_bytes=4 * N) as acc:
        acc.accumulate(0, 2, torch.ones(3, device="cuda"), offset=0,
                       indices=torch.tensor([9, 4, 10], dtype=torch.int64, device="cuda"))
        acc.accumulate(1, 5, torch.full((good.size,), 2.0, device="cuda"), offset=0,
                       indices=torch.from_numpy(good).cuda())
        with pytest.raises(fa.FedAvgError):
            acc.sync()
        cnt = acc.count[:N].cpu().numpy()
        s = acc.acc[:N].cpu().numpy()
    want = np.zeros(N, np.float32)
    want[good] += 10.0
    want[[9, 10]] += 2.0
    assert np.array_equal(s, want)
    assert int(cnt[good].min()) >= 1 and int(cnt[4]) == 0


def test_unaligned_or_ragged_accumulators_scatter():
    """N % 4 != 0: forced tiles fall back to the scatter path (whole
    16-byte quads are the tiles' unit); results are those of the scatter."""
    N = 10_001
    r = np.random.default_rng(2)
    rel = np.nonzero(r.random(N) < 0.2)[0].astype(np.int64)
    v = (r.standard_normal(rel.size) * 1e-3).astype(np.float32)
    res = []
    for path in (SCATTER, TILES):
        fa.fedavg_set_option(fa.FA_OPT_INDEX_TILES, path)
        with fa.StreamingAccumulator(N, mode="weights", partial=True, chunk_bytes=4 * N) as acc:
            acc.accumulate(0, 9, torch.from_numpy(v).cuda(), offset=0, indices=torch.from_numpy(rel).cuda())
            acc.sync()
            res.append(acc.acc[:N].clone())
    assert torch.equal(res[0].view(torch.int32), res[1].view(torch.int32))


@pytest.mark.parametrize("flaw", [1, 2, 64, 127, 128, 129, 256])
def test_the_check_finds_a_single_flaw_anywhere(flaw):
    """A 257-entry list (an odd length) whose only flaw is one entry equal to
    the one before it: inside a pair, between pairs, between two waves' runs
    of 128 entries and in the unpaired last entry.  Forced tiles refuse the
    list and the scatter path reports it and lands the rest, as alone."""
    N = 4096
    rel = np.arange(0, 3 * 257, 3, dtype=np.int64)
    rel[flaw] = rel[flaw - 1]
    vals = torch.arange(1, 258, dtype=torch.float32, device="cuda")
    got = []
    for path in (SCATTER, TILES):
        fa.fedavg_set_option(fa.FA_OPT_INDEX_TILES, path)
        with fa.StreamingAccumulator(N, mode="weights", partial=True, chunk_bytes=4 * N) as acc:
            acc.accumulate(0, 3, vals, offset=0, indices=torch.from_numpy(rel).cuda())
            with pytest.raises(fa.FedAvgError) as e:
                acc.sync()
            assert e.value.code == -7
            got.append((acc.acc[:N].clone(), acc.wsum[:N].clone(), acc.count[:N].clone()))
    for x, y in zip(*got):
        assert torch.equal(x, y)
    assert int(torch.count_nonzero(got[1][2])) == 256
