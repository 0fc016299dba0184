"""GPU: an empty model (N = 0) is a no-op for every entry point.  The empty
tensors' data pointers are NULL, which the library accepts for N = 0."""

import pytest
import torch

import weighted_model_update_amd as fa

pytestmark = pytest.mark.gpu


def empty(dtype=torch.float32):
    return torch.empty(0, dtype=dtype, device="cuda")


@pytest.mark.parametrize("mode", ["weights", "deltas", "deltas_zero_fill"])
def test_aggregate_of_an_empty_model(mode):
    e = empty()
    assert e.data_ptr() == 0
    fa.fedavg_aggregate([e, e], [1, 2], e, mode=mode, base=e)
    fa.fedavg_aggregate([e, e], [0, 0], e, mode=mode, base=e)        # no weight, nothing to do
    bounds = torch.zeros(2, dtype=torch.int64, device="cuda")
    present = torch.ones(2, dtype=torch.uint8, device="cuda")
    fa.fedavg_aggregate([e, e], [1, 2], e, mode=mode, base=e, seg_bounds=bounds, present=present)
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", ["weights", "deltas"])
def test_sparse_merge_of_an_empty_model(mode):
    e = empty()
    err = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    fa.sparse_masked_accumulate([empty(torch.int64)] * 2, [e, e], [3, 4], 0, e, e, mode=mode,
                                counts=empty(torch.uint8), wsum=empty(torch.int32), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0


@pytest.mark.parametrize("partial", [False, True])
def test_streaming_of_an_empty_model(partial):
    e = empty()
    with fa.StreamingAccumulator(0, mode="deltas", partial=partial, chunk_bytes=4096) as acc:
        acc.accumulate(0, 3, e, offset=0)
        acc.accumulate(1, 4, empty(torch.bfloat16), offset=0)
        assert acc.info() == (7, 2)
        acc.finalize(e, e)
        acc.sync()


def test_checksum_and_sum_of_an_empty_buffer():
    # a sum over no elements: 0 for the hash (mod 2^64) and for the values
    assert fa.fedavg_checksum(empty()) == 0
    assert fa.fedavg_checksum_sum(empty(torch.bfloat16)) == (0, 0.0)
    assert fa.fedavg_checksum_sum(empty(), with_hash=False) == (None, 0.0)
