"""GPU parity: the order-independent checksum equals the oracle's, bit for
bit, and tells apart buffers that differ in one element."""

import numpy as np
import pytest
import torch

import oracle
import synth
import weighted_model_update_amd as fa
from gpu_util import dev_f32, dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [0, 1, 63, 1000, 1_000_003, 20_000_001])
def test_checksum_matches_oracle(N):
    r = np.random.default_rng(N)
    a = r.standard_normal(N).astype(np.float32)
    assert fa.fedavg_checksum(dev_f32(a)) == oracle.checksum(a, oracle.F32)
    b = synth.bf16_bits_from_f32(a)
    assert fa.fedavg_checksum(dev_bf16(b)) == oracle.checksum(b, oracle.BF16)


def test_checksum_sees_one_changed_bit():
    a = np.random.default_rng(1).standard_normal(100_000).astype(np.float32)
    t = dev_f32(a)
    h = fa.fedavg_checksum(t)
    t[54_321] = torch.nextafter(t[54_321], torch.tensor(np.inf, device="cuda"))
    assert fa.fedavg_checksum(t) != h


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_checksum_of_an_unaligned_view(dt):
    """A view that starts one element past a 16-byte boundary takes the
    element loop; the hash indexes the view's own elements."""
    r = np.random.default_rng(9)
    a = r.standard_normal(300_001).astype(np.float32)
    if dt == "bf16":
        b = synth.bf16_bits_from_f32(a)
        t = dev_bf16(b)
        assert fa.fedavg_checksum(t[1:]) == oracle.checksum(b[1:], oracle.BF16)
    else:
        t = dev_f32(a)
        assert fa.fedavg_checksum(t[1:]) == oracle.checksum(a[1:], oracle.F32)
