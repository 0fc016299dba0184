"""GPU parity: the order-independent checksum equals the oracle's, bit for
bit, and tells apart buffers that differ in one element; the fixed-order
fp64 value sum lies within its rounding bound of the oracle's exact sum and
is the same bits for every launch shape."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import weighted_model_update_amd as fa
from gpu_util import dev_f32, dev_bf16, dev_of

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


# ---------------------------------------------------------------- value sum

U = 2.0 ** -53


def _abs_bits(a, dt):
    return (np.asarray(a).view(np.uint32) & np.uint32(0x7FFFFFFF)).view(np.float32) if dt == "f32" \
        else np.asarray(a, np.uint16) & np.uint16(0x7FFF)


def check_sum(got, a, dt):
    """The GPU's fixed-order fp64 sum against the oracle's correctly rounded
    exact sum: NaN and infinities alike; otherwise within the rounding bound
    of a fixed order whose longest chain of roundings is h additions,
    h = 48 + ceil(T / 1024) for T tiles of 8192 elements."""
    code = oracle.F32 if dt == "f32" else oracle.BF16
    want = oracle.value_sum(a, code)
    if math.isnan(want) or math.isinf(want):
        assert (math.isnan(got) and math.isnan(want)) or got == want, (got, want)
        return
    n = len(a)
    T = -(-n // 8192)
    h = 48 + -(-T // 1024)
    bound = h * U / (1 - h * U) * oracle.value_sum(_abs_bits(a, dt), code) * (1 + 4 * U)
    assert abs(got - want) <= bound, (got, want, bound)
    if want == 0.0 and bound == 0.0:
        assert got == 0.0 and math.copysign(1.0, got) == 1.0


def host_bits(a, dt):
    return synth.bf16_bits_from_f32(a) if dt == "bf16" else a


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [0, 1, 63, 8191, 8192, 8193, 1_000_003, 20_000_001])
def test_value_sum_and_hash_match_oracle(N, dt):
    """The fused pass: its hash equals the oracle's bit for bit, its sum lies
    within the bound of the exact sum.  The values mix a few scales and
    cancel in part, so a dropped, doubled or sign-flipped element shows."""
    r = np.random.default_rng(100 + N)
    a = (r.standard_normal(N) * np.exp2(r.integers(-20, 20, N))).astype(np.float32)
    a = host_bits(a, dt)
    h, s = fa.fedavg_checksum_sum(dev_of(a, dt))
    assert h == oracle.checksum(a, oracle.F32 if dt == "f32" else oracle.BF16)
    check_sum(s, a, dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_value_sum_is_the_same_bits_for_every_launch_shape(dt):
    """The order of the additions depends on the count alone: repeated calls,
    other grid sizes, the pass without the hash, and an unaligned copy of the
    same elements give the same bits."""
    r = np.random.default_rng(77)
    N = 3_000_017
    a = host_bits((r.standard_normal(N) * np.exp2(r.integers(-30, 30, N))).astype(np.float32), dt)
    t = dev_of(a, dt)
    _, s0 = fa.fedavg_checksum_sum(t)
    check_sum(s0, a, dt)
    seen = {s0.hex()}
    for bpc in (1, 3, 0):
        fa.fedavg_set_option(fa.FA_OPT_BLOCKS_PER_CU, bpc)
        try:
            seen.add(fa.fedavg_checksum_sum(t)[1].hex())
            seen.add(fa.fedavg_checksum_sum(t, with_hash=False)[1].hex())
        finally:
            fa.fedavg_set_option(fa.FA_OPT_BLOCKS_PER_CU, 0)
    buf = torch.empty(N + 1, dtype=t.dtype, device="cuda")
    buf[1:].copy_(t)
    seen.add(fa.fedavg_checksum_sum(buf[1:])[1].hex())
    assert seen == {s0.hex()}


def test_value_sum_special_values():
    r = np.random.default_rng(8)
    a = r.standard_normal(50_000).astype(np.float32)
    cases = []
    b = a.copy(); b[40_000] = np.nan; cases.append(b)
    b = a.copy(); b[3] = np.inf; b[49_999] = -np.inf; cases.append(b)
    b = a.copy(); b[12_345] = -np.inf; cases.append(b)
    cases.append(np.full(20_000, -0.0, np.float32))
    cases.append(np.concatenate([a, -a]))
    for c in cases:
        for dt in ("f32", "bf16"):
            cb = host_bits(c, dt)
            h, s = fa.fedavg_checksum_sum(dev_of(cb, dt))
            check_sum(s, cb, dt)
    h, s = fa.fedavg_checksum_sum(dev_f32(np.full(20_000, -0.0, np.float32)))
    assert s == 0.0 and math.copysign(1.0, s) == 1.0


def test_value_sum_argument_errors():
    t = dev_f32(np.ones(100_000, np.float32))
    need = fa.fedavg_sum_workspace_size(100_000)
    assert need == 8 * 13
    out = torch.empty(1, dtype=torch.float64, device="cuda")
    with pytest.raises(fa.FedAvgError) as e:
        fa.fedavg_checksum_sum(t, workspace=torch.empty(need - 8, dtype=torch.uint8, device="cuda"),
                               sum_out=out)
    assert e.value.code == -8
    with pytest.raises(fa.FedAvgError) as e:        # tile sums inside the buffer
        fa.fedavg_checksum_sum(t, workspace=t[:need // 4].view(torch.uint8), sum_out=out)
    assert e.value.code == -1
    with pytest.raises(fa.FedAvgError) as e:        # result inside the buffer
        fa.fedavg_checksum_sum(t, sum_out=t[8:10].view(torch.float64))
    assert e.value.code == -1
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    fa.fedavg_checksum_sum(t, workspace=ws, sum_out=out)
    assert float(out.item()) == 100_000.0
