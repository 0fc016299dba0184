"""GPU parity: client-side top-k selection (topk_select) against the oracle.
The selection is unique (magnitude order, ties to the lower index), so the
kept indices and their values must match bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import synth
import weighted_model_update_amd as fa
from parity import check
from gpu_util import dev_of

pytestmark = pytest.mark.gpu

DT = {"f32": oracle.F32, "bf16": oracle.BF16}


@pytest.fixture(params=[1, 0], ids=["sampled", "three_pass"])
def path(request):
    """Run a test on the sampled path (the default: the threshold bounded
    from a sample, one read of the update) and on the three-pass path."""
    fa.fedavg_set_option(fa.FA_OPT_TOPK_SAMPLED, request.param)
    yield request.param
    fa.fedavg_set_option(fa.FA_OPT_TOPK_SAMPLED, 1)


def run_topk(x, dt, k, misalign=False):
    """x: float32 array or uint16 bf16 bits.  misalign: place the input one
    element past a 16-byte boundary (the unvectorised path)."""
    d = dev_of(x, dt)
    if misalign:
        buf = torch.empty(d.numel() + 1, dtype=d.dtype, device="cuda")
        buf[1:].copy_(d)
        d = buf[1:]
    idx, val = fa.topk_select(d, k)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def expect(x, dt, k):
    return oracle.topk(x, DT[dt], k)


def laplace(seed, N, dt, scale=1e-3):
    x = np.random.default_rng(seed).laplace(0.0, scale, N).astype(np.float32)
    return synth.bf16_bits_from_f32(x) if dt == "bf16" else x


def same(got, want):
    gi, gv = got
    wi, wv = want
    assert np.array_equal(gi, wi), (len(gi), len(wi), np.nonzero(gi[:min(len(gi), len(wi))] !=
                                                                    wi[:min(len(gi), len(wi))])[0][:5])
    assert np.array_equal(gv.view(np.uint32), wv.view(np.uint32))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 7, 4095, 8192, 8193, 100_003, 1_000_000])
def test_topk_matches_oracle(dt, N, path):
    x = laplace(N, N, dt)
    for k in sorted({0, 1, N // 10, N // 2, N - 1, N}):
        same(run_topk(x, dt, k), expect(x, dt, k))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_threshold_inside_a_tie_group(dt, path):
    # few distinct magnitudes: the k-th key sits inside a large group of
    # equal keys spread over many tiles, so the kept ties are the lowest
    # indices across tiles
    r = np.random.default_rng(3)
    N = 300_000
    x = (r.integers(-4, 5, N) * 0.25).astype(np.float32)
    x = synth.bf16_bits_from_f32(x) if dt == "bf16" else x
    for k in (1, 37_000, 100_001, 150_000, 299_999):
        same(run_topk(x, dt, k), expect(x, dt, k))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_candidate_overflow_falls_back_to_the_whole_input(dt, path):
    # three magnitudes: the threshold bin holds about a third of the input,
    # more than the candidate buffer (N/16 + 65536 entries) takes
    r = np.random.default_rng(8)
    N = 2_000_003
    x = (r.integers(-2, 3, N)).astype(np.float32)
    x = synth.bf16_bits_from_f32(x) if dt == "bf16" else x
    for k in (500_000, 1_000_001, 1_700_000):
        same(run_topk(x, dt, k), expect(x, dt, k))


def test_special_values_and_signed_zeros(path):
    r = np.random.default_rng(4)
    N = 50_000
    x = r.standard_normal(N).astype(np.float32)
    x[r.choice(N, 50, replace=False)] = np.inf
    x[r.choice(N, 50, replace=False)] = -np.inf
    x[r.choice(N, 30, replace=False)] = np.nan
    x[r.choice(N, 30, replace=False)] = -np.nan
    x[r.choice(N, 2000, replace=False)] = 0.0
    x[r.choice(N, 2000, replace=False)] = -0.0
    x[r.choice(N, 100, replace=False)] = 1e-42          # subnormal
    for k in (10, 60, 110, 130, 20_000, 49_000):
        same(run_topk(x, "f32", k), expect(x, "f32", k))


def test_special_values_bf16(path):
    """The same specials in bf16: NaNs above infinity, -0 tied with +0,
    subnormals (bf16 keeps fp32's exponent range)."""
    r = np.random.default_rng(5)
    N = 50_000
    x = r.standard_normal(N).astype(np.float32)
    x[r.choice(N, 50, replace=False)] = np.inf
    x[r.choice(N, 50, replace=False)] = -np.inf
    x[r.choice(N, 30, replace=False)] = np.nan
    x[r.choice(N, 2000, replace=False)] = 0.0
    x[r.choice(N, 2000, replace=False)] = -0.0
    x[r.choice(N, 100, replace=False)] = 1e-39          # subnormal, kept by bf16
    xb = synth.bf16_bits_from_f32(x)
    xb[r.choice(N, 30, replace=False)] = 0xFFC1        # negative NaN with payload
    for k in (10, 60, 110, 130, 20_000, 49_000):
        same(run_topk(xb, "bf16", k), expect(xb, "bf16", k))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("k", [1, 37, 5000])
def test_small_k_on_a_large_update(dt, k, path):
    """k far below the sample's resolution: the sample gives no upper bound,
    the candidates are every key at or above its floor, and their absolute
    digits decide the threshold."""
    N = 3_000_017
    x = laplace(81 + k, N, dt)
    same(run_topk(x, dt, k), expect(x, dt, k))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_unaligned_input(dt, path):
    N = 40_001
    x = laplace(7, N, dt)
    for k in (1, 4000, 40_000):
        same(run_topk(x, dt, k, misalign=True), expect(x, dt, k))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("sampled_small", [True, False])
def test_a_misleading_sample_falls_back_to_the_full_path(dt, sampled_small):
    """The sample takes every stride-th 16-byte vector of the update (2^20
    keys in all).  Give exactly those vectors magnitudes unlike the rest's:
    the sampled range then misses the threshold (far too many keys above it,
    or too few at or above its floor), the check fails and the call finishes
    on the three-pass path -- with the same result."""
    N = 1 << 22
    V = 4 if dt == "f32" else 8
    stride = (N // V) // ((1 << 20) // V)
    r = np.random.default_rng(12 + sampled_small)
    in_sample = (np.arange(N) // V) % stride == 0
    small = r.laplace(0.0, 1e-6, N).astype(np.float32)
    large = r.laplace(0.0, 1.0, N).astype(np.float32)
    x = np.where(in_sample == sampled_small, small, large)
    x = synth.bf16_bits_from_f32(x) if dt == "bf16" else x
    for k in (N // 10, N // 40 + 3):
        same(run_topk(x, dt, k), expect(x, dt, k))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_threshold_in_a_gap_between_clusters(dt, path):
    """Half the magnitudes near 1e-6, half near 1: at k = N/2 the sampled
    range reaches across the gap, many octaves wide, too wide for two
    digits counted from its floor, so the candidates' absolute digits are
    counted instead.  At k = N/2 +- 1000 the threshold sits inside a
    cluster."""
    r = np.random.default_rng(71)
    N = 1 << 21
    big = r.random(N) < 0.5
    x = np.where(big, r.laplace(0.0, 1.0, N), r.laplace(0.0, 1e-6, N)).astype(np.float32)
    x = synth.bf16_bits_from_f32(x) if dt == "bf16" else x
    nbig = int(big.sum())
    for k in (nbig, nbig - 1000, nbig + 1000):
        same(run_topk(x, dt, k), expect(x, dt, k))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_layered_update(dt, path):
    """An update made of layers of very different scales and sizes (a few
    small layers dominate the top entries): the kept set crosses layers."""
    r = np.random.default_rng(61)
    sizes = r.integers(1, 200_000, 40)
    scales = 10.0 ** r.uniform(-6, 0, 40)
    x = np.concatenate([r.laplace(0.0, s, n) for s, n in zip(scales, sizes)]).astype(np.float32)
    x = synth.bf16_bits_from_f32(x) if dt == "bf16" else x
    N = x.shape[0]
    for k in (N // 100, N // 20, N // 5):
        same(run_topk(x, dt, k), expect(x, dt, k))


def test_topk_feeds_the_sparse_merge():
    """Clients select their top-10% on the GPU; the server merges the lists.
    The result matches the oracle merging the oracle's own selections."""
    N, K = 200_003, 6
    n = synth.sample_counts(91, K, 100, 1000)
    xs = [laplace(100 + k, N, "f32") for k in range(K)]
    base = synth.normal_f32(92, synth.ROLE_BASE, 0, N, 0.02)
    k_sel = fa.topk_count(N, 0.1)
    lists = [fa.topk_select(dev_of(x, "f32"), k_sel) for x in xs]
    out = torch.empty(N, dtype=torch.float32, device="cuda")
    counts = torch.empty(N, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fa.sparse_masked_accumulate([i for i, _ in lists], [v for _, v in lists], n.tolist(), N,
                                dev_of(base, "f32"), out, counts=counts, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    sel = [oracle.topk(x, oracle.F32, k_sel) for x in xs]
    ref, mag, rcnt, _ = oracle.sparse_average([i for i, _ in sel], [v for _, v in sel], n, N, base=base)
    assert np.array_equal(counts.cpu().numpy(), rcnt.astype(np.uint8))
    check(out.cpu().numpy(), ref, mag, "f32", copied=rcnt == 0, copy_expect=base)


def test_topk_count_reads_the_fraction_as_written():
    assert fa.topk_count(10 ** 9, 0.1) == 10 ** 8
    assert fa.topk_count(1000, 0.3) == 300          # 0.3 * 1000 is 300.00000000000006 in binary
    assert fa.topk_count(7, 0.5) == 3


def test_topk_argument_errors():
    x = torch.zeros(100, device="cuda")
    with pytest.raises(fa.FedAvgError) as e:
        fa.topk_select(x, 101)
    assert e.value.code == -3
    with pytest.raises(fa.FedAvgError) as e:
        fa.topk_select(x, 10, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.code == -8
    with pytest.raises(fa.FedAvgError) as e:
        fa.topk_select(x, 10, val_out=x[:10])          # output overlaps the input
    assert e.value.code == -1
    idx, val = fa.topk_select(x, 0)
    assert idx.numel() == 0 and val.numel() == 0
