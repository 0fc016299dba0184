"""GPU: pinned host buffers recycled as soon as the streaming contract allows.

A host buffer handed to one accumulate call may be refilled once n_slots
further calls on the handle have returned, whatever those calls were: device
chunks, empty chunks, zero-weight clients, refused calls.  These tests refill
a small pool of pinned buffers at exactly that distance, with every other
kind of call in between, and check the bits against the same aggregation fed
from buffers that are never reused (chunks arriving from disk through a ring
of pinned buffers is the use this serves: FLARE page, Tensor Downloader and
"Offload Aggregation to Disk")."""

import numpy as np
import pytest
import torch

import synth
import weighted_model_update_amd as fa
from gpu_util import dev_of, host_of, empty

pytestmark = pytest.mark.gpu


class Pool:
    """Pinned buffers of one size, each handed out again once more than
    n_slots calls have passed since its last use (call numbers from the
    caller)."""

    def __init__(self, n_slots, numel, dtype):
        self.n_slots, self.numel, self.dtype = n_slots, numel, dtype
        self.bufs = []          # [tensor, call of last use]
        self.reused = 0

    def take(self, call):
        for b in self.bufs:
            if call - b[1] > self.n_slots:
                b[1] = call
                self.reused += 1
                return b[0]
        t = torch.empty(self.numel, dtype=self.dtype, pin_memory=True)
        self.bufs.append([t, call])
        return t


def test_pool_distance_rule():
    p = Pool(2, 4, torch.float32)
    a = p.take(0)
    b = p.take(1)
    c = p.take(2)
    assert p.take(3) is a and p.reused == 1       # calls 1 and 2 returned since a's use
    assert p.take(4) is b and p.take(5) is c
    assert len(p.bufs) == 3


@pytest.mark.parametrize("n_slots", [1, 2, 3])
def test_recycled_pinned_chunks_between_other_calls(n_slots):
    K, chunk = 4, 1 << 20
    N = 3 * chunk + 12_345
    r = np.random.default_rng(90 + n_slots)
    xs = [(r.standard_normal(N) * 1e-3).astype(np.float32) for _ in range(K)]
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    n = synth.sample_counts(91, K, 100, 10000)
    base_dev = dev_of(base, "f32")
    dev_x = [dev_of(x, "f32") for x in xs]

    # reference: every host chunk in a buffer of its own, kept until the end
    keep = []
    ref = empty(N, "f32")
    with fa.StreamingAccumulator(N, mode="deltas", chunk_bytes=4 * chunk, n_slots=n_slots) as acc:
        for k in range(K):
            for off in range(0, N, chunk):
                t = torch.from_numpy(xs[k][off:off + chunk].copy()).pin_memory()
                keep.append(t)
                acc.accumulate(k, int(n[k]), t, offset=off)
        acc.finalize(base_dev, ref)
        acc.sync()

    pool = Pool(n_slots, chunk, torch.float32)
    out = empty(N, "f32")
    nothing = torch.empty(0, dtype=torch.float32, device="cuda")
    call = 0
    with fa.StreamingAccumulator(N, mode="deltas", chunk_bytes=4 * chunk, n_slots=n_slots) as acc:
        for k in range(K):
            for c, off in enumerate(range(0, N, chunk)):
                ln = min(chunk, N - off)
                kind = (3 * k + c) % 4
                if kind == 1:                       # a device chunk in between
                    acc.accumulate(k, int(n[k]), dev_x[k][off:off + ln], offset=off)
                    call += 1
                    continue
                if kind == 2:                       # an empty chunk and a zero-weight client
                    acc.accumulate(k, int(n[k]), nothing, offset=0)
                    acc.accumulate(100 + k, 0, nothing, offset=0)
                    call += 2
                if kind == 3:                       # a refused call (range past N)
                    with pytest.raises(fa.FedAvgError):
                        acc.accumulate(k, int(n[k]), dev_x[k][:chunk], offset=N - 1)
                    call += 1
                buf = pool.take(call)[:ln]
                buf.numpy()[:] = xs[k][off:off + ln]      # refill the recycled buffer
                acc.accumulate(k, int(n[k]), buf, offset=off)
                call += 1
        acc.finalize(base_dev, out)
        acc.sync()
    assert pool.reused > 0
    assert np.array_equal(host_of(out).view(np.uint32), host_of(ref).view(np.uint32))


@pytest.mark.parametrize("n_slots", [1, 2])
def test_recycled_pinned_chunks_through_windows(n_slots):
    """stream_windows skips chunks outside each window by passing them as
    empty chunks, so a pool recycled every n_slots + 1 chunks stays safe."""
    K, chunk, N = 3, 131_072, 600_011
    window = 250_000
    r = np.random.default_rng(95 + n_slots)
    xs = [synth.bf16_bits_from_f32((r.standard_normal(N) * 1e-3).astype(np.float32))
          for _ in range(K)]
    base = synth.bf16_bits_from_f32((r.standard_normal(N) * 0.02).astype(np.float32))
    n = synth.sample_counts(96, K, 100, 1000)
    base_dev = dev_of(base, "bf16")
    pool = Pool(n_slots, chunk, torch.int16)
    yields = [0]

    def chunks_of(k):
        def gen():
            for off in range(0, N, chunk):
                end = min(off + chunk, N)
                buf = pool.take(yields[0])[:end - off]
                buf.numpy()[:] = xs[k][off:end].view(np.int16)
                yields[0] += 1
                yield off, buf.view(torch.bfloat16)
        return gen

    out = empty(N, "bf16")
    fa.stream_windows(N, [(k, int(n[k]), chunks_of(k)) for k in range(K)], base_dev, out,
                      window=window, mode="deltas", chunk_bytes=2 * chunk, n_slots=n_slots)
    torch.cuda.synchronize()
    assert pool.reused > 0

    ref = empty(N, "bf16")
    keep = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).pin_memory() for x in xs]
    with fa.StreamingAccumulator(N, mode="deltas", chunk_bytes=2 * chunk, n_slots=n_slots) as acc:
        for k in range(K):
            for off in range(0, N, chunk):
                acc.accumulate(k, int(n[k]), keep[k][off:off + chunk], offset=off)
        acc.finalize(base_dev, ref)
        acc.sync()
    assert np.array_equal(host_of(out), host_of(ref))
