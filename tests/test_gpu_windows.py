"""GPU parity: streaming aggregation one window of the parameter space at a
time (stream_windows, for models whose accumulator does not fit in device
memory) gives the bits of one handle over the whole model, and matches the
oracle."""

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


def pinned(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if dt == "bf16" else np.float32))
    t = t.view(torch.bfloat16) if dt == "bf16" else t
    return t.pin_memory()


def chunked(t, chunk, masks=None, start=0, stop=None):
    """chunks() for one client: consecutive pieces of `chunk` elements of t
    over [start, stop), with the matching mask pieces."""
    stop = t.numel() if stop is None else stop

    def gen():
        for off in range(start, stop, chunk):
            end = min(off + chunk, stop)
            if masks is None:
                yield off, t[off:end]
            else:
                yield off, t[off:end], masks[off:end]
    return gen


def untiled(N, clients, base, out, mode, partial):
    with fa.StreamingAccumulator(N, mode=mode, partial=partial, chunk_bytes=1 << 20, n_slots=2) as acc:
        for cid, n_k, chunks in clients:
            for item in chunks():
                acc.accumulate(cid, n_k, item[1], offset=item[0], mask=item[2] if len(item) > 2 else None)
        acc.finalize(base, out)
        acc.sync()


@pytest.mark.parametrize("window", [300_007, 131_072, 2_000_000])
def test_dense_windows_give_the_bits_of_one_handle(window):
    """bf16 deltas from pinned host memory in 131,072-element chunks that
    straddle the window edges; a ragged last window; a window larger than
    the model (one window)."""
    N, K, dt = 1_000_003, 5, "bf16"
    r = np.random.default_rng(5)
    xs = [synth.bf16_bits_from_f32((r.standard_normal(N) * 1e-3).astype(np.float32)) for _ in range(K)]
    base = synth.bf16_bits_from_f32((r.standard_normal(N) * 0.02).astype(np.float32))
    n = synth.sample_counts(6, K, 100, 1000)
    hx = [pinned(x, dt) for x in xs]
    clients = [(k, int(n[k]), chunked(hx[k], 131_072)) for k in range(K)]
    d_base = dev_of(base, dt)
    want = empty(N, dt)
    untiled(N, clients, d_base, want, "deltas", False)
    got = empty(N, dt)
    nw = fa.stream_windows(N, clients, d_base, got, window=window, mode="deltas", chunk_bytes=1 << 20)
    assert nw == -(-N // min(window, N))
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    ref, mag, _, _ = oracle.weighted_average(xs, n, mode=oracle.DELTAS, base=base, x_dtype=oracle.BF16,
                                             base_dtype=oracle.BF16)
    check(host_of(got), ref, mag, "bf16", label=f"window={window}")


@pytest.mark.parametrize("mode", ["deltas", "deltas_zero_fill"])
def test_partial_windows_with_a_client_absent_from_some_windows(mode):
    """Masked fp32 chunks in partial mode; client 3 sends only the first
    third of the model, so it has no chunk in the later windows and must
    still count in the zero-fill divisor there.  Host base and output."""
    N, K, dt = 600_011, 4, "f32"
    r = np.random.default_rng(9)
    xs = [(r.standard_normal(N) * 1e-3).astype(np.float32) for _ in range(K)]
    sent = [(r.random(N) < p).astype(np.uint8) for p in (0.3, 0.6, 0.9, 0.5)]
    sent[3][N // 3:] = 0
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    n = synth.sample_counts(10, K, 1, 500)
    hx = [pinned(x, dt) for x in xs]
    hm = [torch.from_numpy(s).pin_memory() for s in sent]
    clients = [(k, int(n[k]), chunked(hx[k], 65_536, hm[k], stop=N if k != 3 else N // 3)) for k in range(K)]
    want = empty(N, dt)
    untiled(N, clients, dev_of(base, dt), want, mode, True)
    host_base = pinned(base, dt)
    host_out = torch.empty(N, dtype=torch.float32).pin_memory()
    nw = fa.stream_windows(N, clients, host_base, host_out, window=150_001, mode=mode, partial=True,
                           chunk_bytes=1 << 20)
    assert nw == 5                     # the last window holds 7 parameters
    assert torch.equal(host_out.view(torch.int32), want.cpu().view(torch.int32))
    om = oracle.DELTAS if mode == "deltas" else oracle.DELTAS_ZERO_FILL
    ref, mag, cnt, _ = oracle.weighted_average(xs, n, mode=om, base=base, sent=sent)
    check(host_out.numpy(), ref, mag, "f32", copied=cnt == 0, copy_expect=base, label=mode)


def test_windows_of_an_empty_model_and_bad_window():
    assert fa.stream_windows(0, [], None, torch.empty(0, device="cuda")) == 0
    with pytest.raises(ValueError):
        fa.stream_windows(10, [], None, torch.empty(10, device="cuda"), window=0)
