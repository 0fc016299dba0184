"""GPU parity: one-pass sparse partial-sharing merge (sparse_masked_accumulate)
against the oracle: values to tolerance, client counts, weight sums and the
set of touched parameters bit-exact."""

import numpy as np
import pytest
import torch

import oracle
import synth
import weighted_model_update_amd as fa
from parity import check
from gpu_util import dev_f32, host_of

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore_options():
    yield
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_BLOCKS, 0)
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, DEFAULT_TILE)


DEFAULT_TILE = 2048
TILES = [512, 1024, 2048, 4096, 8192]


def run_sparse(idx, val, n, N, base, mode="deltas", counts_dtype=torch.uint8, want_wsum=True,
               out_is_base=False):
    d_idx = [torch.from_numpy(np.ascontiguousarray(i, np.int64)).cuda() for i in idx]
    d_val = [dev_f32(v) for v in val]
    d_base = dev_f32(base)
    out = d_base if out_is_base else torch.empty(N, dtype=torch.float32, device="cuda")
    counts = torch.empty(N, dtype=counts_dtype, device="cuda")
    wsum = torch.empty(N, dtype=torch.int32, device="cuda") if want_wsum else None
    err = torch.full((1,), 123, dtype=torch.int32, device="cuda")
    fa.sparse_masked_accumulate(d_idx, d_val, list(n), N, d_base, out, mode=mode, counts=counts,
                                wsum=wsum, err_flag=err)
    torch.cuda.synchronize()
    return (host_of(out), counts.cpu().numpy(), None if wsum is None else wsum.cpu().numpy().view(np.uint32),
            int(err.item()))


def topk_case(N, K, frac, seed):
    idx, val = zip(*[synth.topk_sparse_deltas(seed, k, N, frac, 1e-3) for k in range(K)])
    base = synth.normal_f32(seed, synth.ROLE_BASE, 0, N, 0.02)
    n = synth.sample_counts(seed, K, 100, 1000)
    return list(idx), list(val), n, base


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("blocks", [0, 3, 64])
def test_topk_partial_sharing_matches_oracle(blocks, tile):
    # K=20 clients each sending its top-10% |delta|: many tiles per block
    # (3 blocks), a few (64), and the default (one or two per block)
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, tile)
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_BLOCKS, blocks)
    N, K = 300_007, 20
    idx, val, n, base = topk_case(N, K, 0.1, synth.CFG_SPARSE_1B)
    got, cnt, ws, err = run_sparse(idx, val, n, N, base)
    assert err == 0
    ref, mag, rcnt, rws = oracle.sparse_average(idx, val, n, N, base=base)
    assert np.array_equal(cnt, rcnt.astype(np.uint8))
    assert np.array_equal(ws, rws.astype(np.uint32))
    check(got, ref, mag, "f32", copied=rcnt == 0, copy_expect=base, label=f"blocks={blocks}")


@pytest.mark.parametrize("blocks", [0, 5, 997])
def test_skewed_supports_place_every_range_boundary(blocks):
    """Index lists far from uniform -- a dense cluster with a far outlier,
    quadratically spaced indices, one narrow band, huge gaps, a single
    entry -- so that estimating a range boundary's list position from the
    index values misses by far; the positions (and so the merge) must still
    be exact."""
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_BLOCKS, blocks)
    N = 1_000_003
    r = np.random.default_rng(41)
    lists = [
        np.concatenate([np.arange(0, N // 100), [N - 1]]),
        np.unique((np.arange(1000, dtype=np.int64) ** 2) % N),
        np.arange(N // 2, N // 2 + 3000),
        np.array([0, 1, 2, N - 3, N - 2, N - 1]),
        np.array([N // 3]),
        np.sort(r.choice(N, 50_000, replace=False)),
        np.unique(np.minimum((r.pareto(0.5, 40_000) * 10).astype(np.int64), N - 1)),
    ]
    idx = [np.asarray(l, np.int64) for l in lists]
    val = [r.laplace(0.0, 1e-3, len(i)).astype(np.float32) for i in idx]
    n = synth.sample_counts(17, len(idx), 100, 1000)
    base = synth.normal_f32(17, synth.ROLE_BASE, 0, N, 0.02)
    got, cnt, ws, err = run_sparse(idx, val, n, N, base)
    assert err == 0
    ref, mag, rcnt, rws = oracle.sparse_average(idx, val, n, N, base=base)
    assert np.array_equal(cnt, rcnt.astype(np.uint8))
    assert np.array_equal(ws, rws.astype(np.uint32))
    check(got, ref, mag, "f32", copied=rcnt == 0, copy_expect=base, label=f"skewed blocks={blocks}")


@pytest.mark.parametrize("tile", TILES)
def test_dense_support_overflows_batches(tile):
    # 60% density: several batches of each client per tile
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, tile)
    N, K = 50_001, 6
    idx, val, n, base = topk_case(N, K, 0.6, 77)
    got, cnt, ws, err = run_sparse(idx, val, n, N, base, counts_dtype=torch.int32)
    assert err == 0
    ref, mag, rcnt, rws = oracle.sparse_average(idx, val, n, N, base=base)
    assert np.array_equal(cnt, rcnt.astype(np.int32))
    assert np.array_equal(ws, rws.astype(np.uint32))
    check(got, ref, mag, "f32", copied=rcnt == 0, copy_expect=base)


@pytest.mark.parametrize("tile", [2048, 4096])
def test_full_support_equals_dense_delta_aggregate(tile):
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, tile)
    N, K = 20_000, 4
    r = np.random.default_rng(1)
    vals = [(r.standard_normal(N) * 1e-3).astype(np.float32) for _ in range(K)]
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    n = [11, 22, 33, 44]
    got, cnt, ws, err = run_sparse([np.arange(N)] * K, vals, n, N, base)
    dense = torch.empty(N, dtype=torch.float32, device="cuda")
    fa.fedavg_aggregate([dev_f32(v) for v in vals], n, dense, mode="deltas", base=dev_f32(base))
    torch.cuda.synchronize()
    assert err == 0 and (cnt == K).all()
    assert np.array_equal(got.view(np.uint32), host_of(dense).view(np.uint32))


@pytest.mark.parametrize("tile", [2048, 8192])
def test_weights_mode_empty_and_zero_weight_clients_in_place(tile):
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, tile)
    N = 70_000
    r = np.random.default_rng(2)
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    idx = [np.sort(r.choice(N, 5000, replace=False)), np.array([], np.int64),
           np.sort(r.choice(N, 9000, replace=False)), np.sort(r.choice(N, 100, replace=False))]
    val = [r.standard_normal(len(i)).astype(np.float32) for i in idx]
    n = [5, 7, 0, 13]
    got, cnt, ws, err = run_sparse(idx, val, n, N, base, mode="weights", out_is_base=True)
    assert err == 0
    ref, mag, rcnt, rws = oracle.sparse_average(idx, val, n, N, mode=oracle.WEIGHTS, base=base)
    assert np.array_equal(cnt, rcnt.astype(np.uint8))
    check(got, ref, mag, "f32", copied=rcnt == 0, copy_expect=base)


@pytest.mark.parametrize("tile", [2048, 4096])
@pytest.mark.parametrize("bad", ["unsorted", "duplicate", "too_large", "negative", "unsorted_far"])
def test_bad_index_lists_are_flagged(bad, tile):
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, tile)
    N = 10_000
    base = np.zeros(N, np.float32)
    good = np.arange(0, N, 7, dtype=np.int64)
    broken = good.copy()
    if bad == "unsorted":
        broken[100], broken[101] = broken[101], broken[100]
    elif bad == "duplicate":
        broken[200] = broken[199]
    elif bad == "too_large":
        broken[-1] = N + 5
    elif bad == "unsorted_far":
        broken[300] = 5    # far below its neighbours, inside another range
    else:
        broken[0] = -3
    val = np.ones(len(good), np.float32)
    _, _, _, err = run_sparse([good, broken], [val, val], [1, 1], N, base)
    assert err == -7
    _, _, _, err = run_sparse([good, good], [val, val], [1, 1], N, base)
    assert err == 0


@pytest.mark.parametrize("tile", [512, 2048, 4096])
@pytest.mark.parametrize("blocks", [0, 7])
def test_order_violations_at_every_kind_of_edge(tile, blocks):
    """Each entry is checked against its predecessor, which the merge finds in
    different places: the lane below, the last lane of the wave before, the
    last entry of the batch before (full support: every batch lies inside the
    tile), or the entry before a range's first one.  A swapped or repeated
    pair at each of those edges must be flagged; the intact list must not."""
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, tile)
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_BLOCKS, blocks)
    N = 50_000
    tiles = -(-N // tile)
    # the library's range count: the option, else ranges of 4 tiles but at
    # least 4096 ranges while there are that many tiles
    nb = min(tiles, blocks if blocks > 0 else max(-(-tiles // 4), min(tiles, 4096)))
    R = -(-tiles // nb) * tile                     # parameters per range
    base = np.zeros(N, np.float32)
    good = np.arange(N, dtype=np.int64)
    val = np.ones(N, np.float32)
    edges = {0, 62, 63, 64, 127, 255, 256, 511, 512, tile - 1, tile, R - 2, R - 1, R, 2 * R - 1}
    for p in sorted(e for e in edges if 0 <= e < N - 1):
        for kind in ("swap", "repeat"):
            broken = good.copy()
            if kind == "swap":
                broken[p], broken[p + 1] = broken[p + 1], broken[p]
            else:
                broken[p + 1] = broken[p]
            _, _, _, err = run_sparse([good, broken], [val, val], [1, 1], N, base)
            assert err == -7, (kind, p)
    _, cnt, _, err = run_sparse([good, good], [val, val], [1, 1], N, base)
    assert err == 0 and (cnt == 2).all()


@pytest.mark.parametrize("tile", TILES)
def test_tiny_and_ragged_sizes(tile):
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, tile)
    for N in (1, 7, 255, 257, 4095, 4097, 8193):
        r = np.random.default_rng(N)
        K = 3
        idx = [np.sort(r.choice(N, max(1, N // 3), replace=False)) for _ in range(K)]
        val = [r.standard_normal(len(i)).astype(np.float32) for i in idx]
        base = r.standard_normal(N).astype(np.float32)
        n = [1, 2, 3]
        got, cnt, ws, err = run_sparse(idx, val, n, N, base)
        assert err == 0
        ref, mag, rcnt, rws = oracle.sparse_average(idx, val, n, N, base=base)
        assert np.array_equal(cnt, rcnt.astype(np.uint8))
        check(got, ref, mag, "f32", copied=rcnt == 0, copy_expect=base, label=f"N={N}")


def test_sparse_argument_errors():
    N = 100
    b = torch.zeros(N, device="cuda")
    i = torch.arange(10, device="cuda")
    v = torch.ones(10, device="cuda")
    with pytest.raises(fa.FedAvgError) as e:
        fa.sparse_masked_accumulate([i], [v], [1], N, b, b, workspace=torch.empty(8, dtype=torch.uint8,
                                                                                   device="cuda"))
    assert e.value.code == -8
    with pytest.raises(fa.FedAvgError) as e:
        fa.sparse_masked_accumulate([i], [v], [-1], N, b, b)
    assert e.value.code == -3


@pytest.mark.parametrize("tile", [2048, 4096])
@pytest.mark.parametrize("K", [1, 9, 17, 25, 33, 64])
def test_client_counts_across_kernel_variants(K, tile):
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_TILE, tile)
    # client counts below and above one group of batches, and the two-word
    # client masks of K > 32
    N = 40_000
    idx, val, n, base = topk_case(N, K, 0.15, 100 + K)
    got, cnt, ws, err = run_sparse(idx, val, n, N, base)
    assert err == 0
    ref, mag, rcnt, rws = oracle.sparse_average(idx, val, n, N, base=base)
    assert np.array_equal(cnt, rcnt.astype(np.uint8))
    assert np.array_equal(ws, rws.astype(np.uint32))
    check(got, ref, mag, "f32", copied=rcnt == 0, copy_expect=base, label=f"K={K}")
