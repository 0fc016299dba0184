"""GPU: spill the running aggregate to disk and resume it (export / resume).
An aggregation interrupted at any point -- between clients or inside one
client's chunk sequence -- saved, its device buffers thrown away, restored
and continued, ends with exactly the bits of the uninterrupted run."""

import numpy as np
import pytest
import torch

import oracle
import synth
import weighted_model_update_amd as fa
from parity import check
from gpu_util import dev_of, host_of, empty

pytestmark = pytest.mark.gpu

_KEEP = []


@pytest.fixture(autouse=True)
def _release_host_buffers():
    yield
    torch.cuda.synchronize()
    _KEEP.clear()


def pinned_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)
    t = t.pin_memory()
    _KEEP.append(t)
    return t


def dense_steps(xs, n, chunk):
    """The accumulate calls of a dense run, in order: (client, n_k, offset)."""
    N = len(xs[0])
    return [(k, int(n[k]), off) for k in range(len(xs)) for off in range(0, N, chunk)]


@pytest.mark.parametrize("cut", [0.0, 0.37, 0.5, 1.0])
def test_dense_resume_is_bit_identical(tmp_path, cut):
    K, N, chunk = 5, 70_001, 8192
    n = synth.sample_counts(71, K, 100, 1000)
    r = np.random.default_rng(72)
    xs = [synth.bf16_bits_from_f32((r.standard_normal(N) * 1e-3).astype(np.float32)) for _ in range(K)]
    base = synth.bf16_bits_from_f32((r.standard_normal(N) * 0.02).astype(np.float32))
    srcs = [pinned_bf16(x) for x in xs]
    steps = dense_steps(xs, n, chunk)
    cb = chunk * 2

    def feed(acc, part):
        for k, nk, off in part:
            acc.accumulate(k, nk, srcs[k][off:off + chunk], offset=off)

    ref_out = empty(N, "bf16")
    with fa.StreamingAccumulator(N, mode="deltas", chunk_bytes=cb) as acc:
        feed(acc, steps)
        acc.finalize(dev_of(base, "bf16"), ref_out)
        acc.sync()

    at = int(len(steps) * cut)          # 0.37 stops inside a client's chunks
    with fa.StreamingAccumulator(N, mode="deltas", chunk_bytes=cb) as acc:
        feed(acc, steps[:at])
        acc.save(str(tmp_path / "spill"))
    torch.cuda.empty_cache()
    out = empty(N, "bf16")
    with fa.StreamingAccumulator.load(str(tmp_path / "spill"), N, mode="deltas", chunk_bytes=cb,
                                      n_slots=3) as acc:
        feed(acc, steps[at:])
        acc.finalize(dev_of(base, "bf16"), out)
        acc.sync()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    ref, mag, _, _ = oracle.weighted_average(xs, n, mode=oracle.DELTAS, base=base, x_dtype=oracle.BF16,
                                             base_dtype=oracle.BF16)
    check(host_of(out), ref, mag, "bf16")


def test_partial_resume_with_masks_indices_and_counts(tmp_path):
    K, N = 6, 40_003
    n = synth.sample_counts(81, K, 100, 1000)
    r = np.random.default_rng(82)
    xs = [(r.standard_normal(N) * 0.02).astype(np.float32) for _ in range(K)]
    masks = [(r.random(N) < 0.4).astype(np.uint8) for _ in range(K)]
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    # clients 0-2 send masked ranges, clients 3-5 index lists
    calls = []
    for k in range(K):
        if k < 3:
            for off in range(0, N, 10_000):
                calls.append(("mask", k, off, min(10_000, N - off)))
        else:
            calls.append(("idx", k, 0, N))
    dx = [dev_of(x, "f32") for x in xs]
    dm = [torch.from_numpy(m).cuda() for m in masks]
    di = [torch.from_numpy(np.nonzero(m)[0].astype(np.int64)).cuda() for m in masks]

    def feed(acc, part):
        for kind, k, off, ln in part:
            if kind == "mask":
                acc.accumulate(k, int(n[k]), dx[k][off:off + ln], offset=off, mask=dm[k][off:off + ln])
            else:
                acc.accumulate(k, int(n[k]), dx[k][di[k]].contiguous(), offset=0, indices=di[k])

    def run(split, path=None):
        out = empty(N, "f32")
        kw = dict(mode="weights", partial=True, chunk_bytes=4 * N)
        if split is None:
            acc = fa.StreamingAccumulator(N, **kw)
        else:
            with fa.StreamingAccumulator(N, **kw) as a0:
                feed(a0, calls[:split])
                a0.save(path)
            acc = fa.StreamingAccumulator.load(path, N, **kw)
        with acc:
            feed(acc, calls[split or 0:] if split is not None else calls)
            acc.finalize(dev_of(base, "f32"), out)
            acc.sync()
            return host_of(out), acc.wsum[:N].cpu().numpy(), acc.count[:N].cpu().numpy()

    ref = run(None)
    for split in (2, 7, 16):
        got = run(split, str(tmp_path / f"s{split}"))
        for a, b in zip(ref, got):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), split
    want, mag, rcnt, rws = oracle.weighted_average(xs, n, base=base, sent=masks)
    assert np.array_equal(ref[2], rcnt.astype(np.uint8))
    check(ref[0], want, mag, "f32", copied=rcnt == 0, copy_expect=base)


def test_resume_keeps_finalized_state_and_partials(tmp_path):
    N = 4096
    x = torch.ones(N, device="cuda")
    base = torch.zeros(N, device="cuda")
    with fa.StreamingAccumulator(N, chunk_bytes=4 * N) as acc:
        acc.accumulate(0, 3, x)
        acc.accumulate_partial(5, 40, 4, x * 40)            # a silo of 4 clients, weight 40
        out1 = torch.empty(N, device="cuda")
        acc.finalize(base, out1)
        acc.save(str(tmp_path / "f"))
    with fa.StreamingAccumulator.load(str(tmp_path / "f"), N, chunk_bytes=4 * N) as acc:
        assert acc.info() == (43, 5)
        with pytest.raises(fa.FedAvgError) as e:
            acc.accumulate(1, 2, x)
        assert e.value.code == -5                           # finalized before the spill
        out2 = torch.empty(N, device="cuda")
        acc.finalize(base, out2)
        acc.sync()
    assert torch.equal(out1, out2) and torch.all(out1 == 1.0)
    with pytest.raises(fa.FedAvgError) as e:
        fa.StreamingAccumulator.load(str(tmp_path / "f"), N + 8, chunk_bytes=4 * N)
    assert e.value.code == -1


def test_export_reports_deferred_index_errors():
    N = 1000
    with fa.StreamingAccumulator(N, partial=True, chunk_bytes=4 * N) as acc:
        vals = torch.ones(3, device="cuda")
        acc.accumulate(0, 1, vals, indices=torch.tensor([5, 5, 9], device="cuda"))
        with pytest.raises(fa.FedAvgError) as e:
            fa.fedavg_export_state(acc.handle)
        assert e.value.code == -7
