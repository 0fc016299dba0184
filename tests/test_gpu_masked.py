"""GPU parity: per-segment (per-tensor) masked aggregation, e.g. adapter-only
updates where each client sends only some adapters, against the oracle."""

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


@pytest.fixture(autouse=True)
def _restore_options():
    yield
    fa.fedavg_set_option(fa.FA_OPT_MASK_VECTORS_PER_BLOCK, 1024)


def sent_from_segments(bounds, present):
    K, T = present.shape
    N = bounds[-1]
    seg_of = np.repeat(np.arange(T), np.diff(bounds))
    return [present[k][seg_of].astype(np.uint8) for k in range(K)]


def run_masked(xs, n, bounds, present, base, xdt, bdt, odt, mode):
    N = int(bounds[-1])
    out = empty(N, odt)
    fa.fedavg_aggregate([dev_of(x, xdt) for x in xs], list(n), out, mode=mode,
                        base=dev_of(base, bdt),
                        seg_bounds=torch.tensor(bounds, dtype=torch.int64, device="cuda"),
                        present=torch.from_numpy(np.ascontiguousarray(present, dtype=np.uint8)).cuda())
    torch.cuda.synchronize()
    return host_of(out)


def oracle_masked(xs, n, bounds, present, base, xdt, bdt, mode):
    sent = sent_from_segments(np.asarray(bounds), np.asarray(present))
    return oracle.weighted_average(xs, n, mode=oracle.DELTAS if mode == "deltas" else oracle.WEIGHTS,
                                   base=base, x_dtype=ODT[xdt], base_dtype=ODT[bdt], sent=sent)


def lora_case(layers, hidden, rank, K, p, seed):
    """Shrunken adapter layout: q,k,v,o LoRA A/B pairs per layer; presence per
    (client, module), shared by the module's A and B segments."""
    bounds, module_of = synth.adapter_segments(layers=layers, hidden=hidden, rank=rank)
    n_mod = max(module_of) + 1
    pres_mod = synth.adapter_presence(seed, K, n_mod, p)
    present = pres_mod[:, module_of]
    return np.asarray(bounds, np.int64), present


@pytest.mark.parametrize("vpb", [1024, 16, 1 << 20])
def test_adapter_masks_match_oracle(vpb):
    fa.fedavg_set_option(fa.FA_OPT_MASK_VECTORS_PER_BLOCK, vpb)
    K = 8
    bounds, present = lora_case(layers=6, hidden=512, rank=8, K=K, p=0.6, seed=2)
    N = int(bounds[-1])
    n = synth.sample_counts(synth.CFG_ADAPTER, K, 500, 5000)
    r = np.random.default_rng(3)
    xs = [synth.bf16_bits_from_f32((r.standard_normal(N) * 0.01).astype(np.float32)) for _ in range(K)]
    base = synth.bf16_bits_from_f32((r.standard_normal(N) * 0.01).astype(np.float32))
    got = run_masked(xs, n, bounds, present, base, "bf16", "bf16", "bf16", "weights")
    ref, mag, cnt, _ = oracle_masked(xs, n, bounds, present, base, "bf16", "bf16", "weights")
    check(got, ref, mag, "bf16", copied=cnt == 0, copy_expect=base, label=f"vpb={vpb}")


@pytest.mark.parametrize("xdt,bdt,odt,mode", [("f32", "f32", "f32", "weights"),
                                              ("bf16", "f32", "bf16", "deltas"),
                                              ("f32", "bf16", "f32", "deltas"),
                                              ("bf16", "bf16", "f32", "weights")])
@pytest.mark.parametrize("vpb", [8, 1024])
@pytest.mark.parametrize("T,max_size", [(150, 3000), (1500, 300)])
def test_ragged_segments_match_oracle(xdt, bdt, odt, mode, vpb, T, max_size):
    # segment sizes from 0 to max_size, most not a multiple of 8; 150
    # segments fit the whole-table LDS kernel, 1500 take the windowed one
    fa.fedavg_set_option(fa.FA_OPT_MASK_VECTORS_PER_BLOCK, vpb)
    r = np.random.default_rng(11 + T)
    sizes = r.integers(0, max_size, size=T)
    sizes[::17] = 0
    sizes[5] = 1
    bounds = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    N = int(bounds[-1])
    K = 5
    present = (r.random((K, T)) < 0.5).astype(np.uint8)
    present[:, 3] = 0           # nobody sent segment 3
    present[:, 4] = 1           # everybody sent segment 4
    n = synth.sample_counts(9, K, 1, 10000)
    n[2] = 0                    # a zero-weight client
    sig = 1e-3 if mode == "deltas" else 0.02
    xs32 = [(r.standard_normal(N) * sig).astype(np.float32) for _ in range(K)]
    xs = [synth.bf16_bits_from_f32(x) for x in xs32] if xdt == "bf16" else xs32
    b32 = (r.standard_normal(N) * 0.02).astype(np.float32)
    base = synth.bf16_bits_from_f32(b32) if bdt == "bf16" else b32
    got = run_masked(xs, n, bounds, present, base, xdt, bdt, odt, mode)
    ref, mag, cnt, _ = oracle_masked(xs, n, bounds, present, base, xdt, bdt, mode)
    check(got, ref, mag, odt, copied=cnt == 0, copy_expect=base_copy_expect(base, bdt, odt))


@pytest.mark.parametrize("T", [511, 512, 513])
def test_table_size_boundary(T):
    """Tables of 512 segments are staged whole in LDS, 513 are windowed;
    both sides of the switch agree with the oracle, with a zero-length last
    segment and segments that end mid-vector."""
    r = np.random.default_rng(100 + T)
    sizes = r.integers(1, 200, size=T)
    sizes[-1] = 0
    sizes[T // 2] = 8 * 257 + 3
    bounds = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    N = int(bounds[-1])
    K = 3
    present = (r.random((K, T)) < 0.7).astype(np.uint8)
    n = [4, 9, 2]
    xs = [(r.standard_normal(N) * 0.05).astype(np.float32) for _ in range(K)]
    base = (r.standard_normal(N) * 0.05).astype(np.float32)
    got = run_masked(xs, n, bounds, present, base, "f32", "f32", "f32", "deltas")
    ref, mag, cnt, _ = oracle_masked(xs, n, bounds, present, base, "f32", "f32", "deltas")
    check(got, ref, mag, "f32", copied=cnt == 0, copy_expect=base, label=f"T={T}")


def test_all_present_equals_dense_bit_for_bit():
    K, N = 6, 200_000
    r = np.random.default_rng(5)
    xs = [synth.bf16_bits_from_f32((r.standard_normal(N) * 0.02).astype(np.float32)) for _ in range(K)]
    base = synth.bf16_bits_from_f32(np.zeros(N, np.float32))
    n = synth.sample_counts(5, K, 100, 1000)
    bounds = np.array([0, 1000, 1000, 70_001, N], np.int64)
    present = np.ones((K, 4), np.uint8)
    got = run_masked(xs, n, bounds, present, base, "bf16", "bf16", "bf16", "weights")
    out = empty(N, "bf16")
    fa.fedavg_aggregate([dev_of(x, "bf16") for x in xs], n.tolist(), out)
    torch.cuda.synchronize()
    assert np.array_equal(got, host_of(out))


def test_nobody_present_copies_base():
    K, N = 3, 10_007
    r = np.random.default_rng(6)
    xs = [np.full(N, np.nan, np.float32) for _ in range(K)]   # never read
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    bounds = np.array([0, 5000, N], np.int64)
    got = run_masked(xs, [1, 2, 3], bounds, np.zeros((K, 2), np.uint8), base, "f32", "f32", "bf16",
                     "weights")
    assert np.array_equal(got, oracle.round_to_bf16(base))


def test_single_segment_table():
    K, N = 4, 33
    r = np.random.default_rng(7)
    xs = [(r.standard_normal(N)).astype(np.float32) for _ in range(K)]
    base = np.zeros(N, np.float32)
    bounds = np.array([0, N], np.int64)
    present = np.array([[1], [0], [1], [1]], np.uint8)
    n = [3, 5, 7, 11]
    got = run_masked(xs, n, bounds, present, base, "f32", "f32", "f32", "weights")
    ref, mag, _, _ = oracle_masked(xs, n, bounds, present, base, "f32", "f32", "weights")
    check(got, ref, mag, "f32")


def test_masked_argument_errors():
    x = torch.zeros(16, device="cuda")
    with pytest.raises(fa.FedAvgError):
        fa.fedavg_aggregate([x], [1], torch.zeros(16, device="cuda"),
                            seg_bounds=torch.tensor([0, 16], device="cuda"),
                            present=torch.ones(1, dtype=torch.uint8, device="cuda"))  # no base


@pytest.mark.parametrize("K", [33, 64])
@pytest.mark.parametrize("T", [40, 700])
def test_many_clients_use_every_mask_bit(K, T):
    """Up to 64 clients: the per-segment client masks and weight sums use
    all 64 bits, in the whole-table kernel (40 segments) and the windowed
    one (700).  Clients above 32 alone send some segments, so a mask cut to
    32 bits would drop them."""
    r = np.random.default_rng(300 + K + T)
    sizes = r.integers(1, 400, size=T)
    bounds = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    N = int(bounds[-1])
    present = (r.random((K, T)) < 0.3).astype(np.uint8)
    present[:, 0] = 0
    present[K - 1, 0] = 1              # only the last client sent segment 0
    present[:, 1] = 0
    present[32:, 1] = 1                # only clients 32.. sent segment 1
    present[:, 2] = 0                  # nobody sent segment 2
    n = synth.sample_counts(21, K, 1, 1000)
    xs = [(r.standard_normal(N) * 1e-3).astype(np.float32) for _ in range(K)]
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    for mode in ("weights", "deltas"):
        got = run_masked(xs, n, bounds, present, base, "f32", "f32", "f32", mode)
        ref, mag, cnt, _ = oracle_masked(xs, n, bounds, present, base, "f32", "f32", mode)
        check(got, ref, mag, "f32", copied=cnt == 0, copy_expect=base, label=f"K={K} T={T} {mode}")


@pytest.mark.parametrize("T,misalign", [(300, False), (900, False), (300, True)])
def test_absent_segments_are_never_read_and_nothing_outside_out_is_written(T, misalign):
    """Every client's absent segments hold NaN: none may reach the output
    (a read times a zero weight would still give NaN).  The output sits
    inside a larger buffer whose neighbouring words must stay untouched.
    The whole-table kernel (300 segments), the windowed kernel (900) and the
    element-wise path (an unaligned output) are all checked."""
    r = np.random.default_rng(500 + T + misalign)
    sizes = r.integers(0, 700, size=T)
    bounds = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    N, K = int(bounds[-1]), 5
    present = (r.random((K, T)) < 0.5).astype(np.uint8)
    sent = sent_from_segments(bounds, present)
    xs = []
    for k in range(K):
        x = (r.standard_normal(N) * 1e-3).astype(np.float32)
        x[sent[k] == 0] = np.nan
        xs.append(x)
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    n = synth.sample_counts(31, K, 1, 1000)
    G = 64 + (1 if misalign else 0)
    whole = torch.full((G + N + 64,), -7.25, dtype=torch.float32, device="cuda")
    out = whole[G:G + N]
    fa.fedavg_aggregate([dev_of(x, "f32") for x in xs], list(n), out, mode="deltas",
                        base=dev_of(base, "f32"),
                        seg_bounds=torch.tensor(bounds, dtype=torch.int64, device="cuda"),
                        present=torch.from_numpy(present).cuda())
    torch.cuda.synchronize()
    got = host_of(out)
    assert not np.isnan(got).any()
    ref, mag, cnt, _ = oracle.weighted_average(xs, n, mode=oracle.DELTAS, base=base, sent=sent)
    check(got, ref, mag, "f32", copied=cnt == 0, copy_expect=base, label=f"T={T}")
    guard = torch.cat([whole[:G], whole[G + N:]])
    assert bool((guard == -7.25).all())
