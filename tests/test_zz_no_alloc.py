"""GPU: the allocation-free sparse merge (sparse_masked_accumulate_noalloc),
called through the C ABI, gives the bits of sparse_masked_accumulate with a
caller workspace -- values, client counts, weight sums and the error flag --
on two calls in a row, the second smaller than the first (the static scratch
keeps the first call's contents, which must not leak into the second)."""

import numpy as np
import pytest
import torch

import synth
import weighted_model_update_amd as fa
from gpu_util import dev_f32, host_of

pytestmark = pytest.mark.gpu


def case(N, K, frac, seed):
    idx, val = zip(*[synth.topk_sparse_deltas(seed, k, N, frac, 1e-3) for k in range(K)])
    base = synth.normal_f32(seed, synth.ROLE_BASE, 0, N, 0.02)
    n = synth.sample_counts(seed, K, 100, 1000)
    d_idx = [torch.from_numpy(np.ascontiguousarray(i, np.int64)).cuda() for i in idx]
    d_val = [dev_f32(v) for v in val]
    return d_idx, d_val, [int(x) for x in n], dev_f32(base)


def run(fn, d_idx, d_val, n, N, base, mode, with_flag, **kw):
    out = torch.empty(N, dtype=torch.float32, device="cuda")
    counts = torch.empty(N, dtype=torch.uint8, device="cuda")
    wsum = torch.empty(N, dtype=torch.int32, device="cuda")
    err = torch.full((1,), 77, dtype=torch.int32, device="cuda") if with_flag else None
    fn(d_idx, d_val, n, N, base, out, mode=mode, counts=counts, wsum=wsum, err_flag=err, **kw)
    torch.cuda.synchronize()
    return (host_of(out).view(np.uint32), counts.cpu().numpy(), wsum.cpu().numpy(),
            None if err is None else int(err.item()))


@pytest.mark.parametrize("mode", ["deltas", "weights", "deltas_zero_fill"])
def test_noalloc_equals_the_workspace_call_on_two_calls_in_a_row(mode):
    # first a large call (K=20 top-10% lists over 3.1M parameters: many
    # ranges of offsets in the scratch), then a smaller one (K=6, 50,021
    # parameters, a ragged last tile)
    for N, K, seed in ((3_100_013, 20, 601), (50_021, 6, 602)):
        d_idx, d_val, n, base = case(N, K, 0.1, seed)
        want = run(fa.sparse_masked_accumulate, d_idx, d_val, n, N, base, mode, True)
        got = run(fa.sparse_masked_accumulate_noalloc, d_idx, d_val, n, N, base, mode, True)
        assert want[3] == 0 and got[3] == 0
        for g, w in zip(got[:3], want[:3]):
            assert np.array_equal(g, w)
        # without a caller flag the call keeps it in the scratch
        got2 = run(fa.sparse_masked_accumulate_noalloc, d_idx, d_val, n, N, base, mode, False)
        for g, w in zip(got2[:3], want[:3]):
            assert np.array_equal(g, w)


def test_noalloc_reports_a_bad_list_then_recovers():
    N, K = 200_003, 5
    d_idx, d_val, n, base = case(N, K, 0.1, 611)
    bad = d_idx[2].clone()
    bad[1000], bad[1001] = bad[1001].item(), bad[1000].item()      # out of order
    got = run(fa.sparse_masked_accumulate_noalloc, d_idx[:2] + [bad] + d_idx[3:], d_val, n, N, base,
              "deltas", True)
    assert got[3] == -7                         # FA_ERR_INDEX
    # the next call resets the flag and gives the workspace call's bits
    want = run(fa.sparse_masked_accumulate, d_idx, d_val, n, N, base, "deltas", True)
    got = run(fa.sparse_masked_accumulate_noalloc, d_idx, d_val, n, N, base, "deltas", True)
    assert got[3] == 0 and all(np.array_equal(g, w) for g, w in zip(got[:3], want[:3]))


def test_noalloc_rejects_offsets_beyond_the_scratch():
    # 40 contributing clients over the 131,072 ranges of 2^30 parameters need
    # 40 * 131,073 * 8 bytes of offsets, more than the 32 MiB scratch:
    # refused before any device work
    N, K = 1 << 30, 40
    base = torch.zeros(N, dtype=torch.float32, device="cuda")
    out = torch.empty_like(base)
    d_idx = [torch.tensor([k], dtype=torch.int64, device="cuda") for k in range(K)]
    d_val = [torch.ones(1, dtype=torch.float32, device="cuda") for _ in range(K)]
    with pytest.raises(fa.FedAvgError) as e:
        fa.sparse_masked_accumulate_noalloc(d_idx, d_val, [1] * K, N, base, out)
    assert e.value.code == -3 and "allocation-free" in str(e.value)
    # the same clients with fewer ranges fit
    fa.fedavg_set_option(fa.FA_OPT_SPARSE_BLOCKS, 1024)
    try:
        fa.sparse_masked_accumulate_noalloc(d_idx, d_val, [1] * K, N, base, out, mode="deltas")
        torch.cuda.synchronize()
    finally:
        fa.fedavg_set_option(fa.FA_OPT_SPARSE_BLOCKS, 0)
    got = out[:K + 1].cpu().numpy()
    assert np.array_equal(got, np.r_[np.full(K, 1.0, np.float32), np.float32(0.0)])
