"""GPU parity: two-level (hierarchical) aggregation.  Silos aggregate their own
clients with the streaming accumulator; their unnormalised partial sums then
enter a top-level accumulator as pseudo-clients (fedavg_accumulate_partial).
In exact arithmetic this is the flat weighted average over every silo's
clients, so the flat oracle is the reference."""

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


def silo_values(seed, K, N, dt, sig=0.02):
    r = np.random.default_rng(seed)
    xs32 = [(r.standard_normal(N) * sig).astype(np.float32) for _ in range(K)]
    return [synth.bf16_bits_from_f32(x) for x in xs32] if dt == "bf16" else xs32


def run_silo(xs, n, dt, chunk, partial=False, masks=None, first_id=0):
    """A silo's streaming accumulator over its clients (device chunks);
    returns the open accumulator (caller closes)."""
    N = len(xs[0])
    esize = 2 if dt == "bf16" else 4
    acc = fa.StreamingAccumulator(N, mode="weights", partial=partial, chunk_bytes=chunk * esize,
                                  n_slots=2)
    for k, x in enumerate(xs):
        src = dev_of(x, dt)
        m = None if masks is None else torch.from_numpy(masks[k]).cuda()
        for off in range(0, N, chunk):
            acc.accumulate(first_id + k, int(n[k]), src[off:off + chunk], offset=off,
                           mask=None if m is None else m[off:off + chunk])
    acc.sync()
    return acc


@pytest.mark.parametrize("dt,odt,mode", [("bf16", "bf16", "weights"), ("f32", "f32", "deltas"),
                                         ("bf16", "f32", "deltas")])
def test_silos_match_flat_oracle(dt, odt, mode):
    N = 100_003                       # not a multiple of 8: ragged tail
    sizes = [2, 3, 4]
    n_all = synth.sample_counts(31, sum(sizes), 100, 1000)
    xs_all = silo_values(32, sum(sizes), N, dt)
    r = np.random.default_rng(33)
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    silos, at = [], 0
    for g, K in enumerate(sizes):
        silos.append(run_silo(xs_all[at:at + K], n_all[at:at + K], dt, chunk=8192 + 8 * g))
        at += K
    out = empty(N, odt)
    with fa.StreamingAccumulator(N, mode=mode, chunk_bytes=1 << 20) as top:
        for g, s in enumerate(silos):
            top.add_silo(g, s)
        W, members = top.info()
        assert W == int(np.sum(n_all)) and members == sum(sizes)
        top.finalize(dev_of(base, "f32"), out)
        top.sync()
    for s in silos:
        s.close()
    ref, mag, _, _ = oracle.weighted_average(xs_all, n_all, mode=oracle.DELTAS if mode == "deltas"
                                             else oracle.WEIGHTS, base=base, x_dtype=ODT[dt])
    check(host_of(out), ref, mag, odt, label="two-level vs flat")


def test_one_silo_is_the_silo_itself_bit_for_bit():
    """0 + acc is exact, so a top level holding one silo finalizes to exactly
    what the silo itself finalizes to."""
    N = 65_536 + 5
    n = [120, 340, 999]
    xs = silo_values(41, 3, N, "bf16")
    silo = run_silo(xs, n, "bf16", chunk=4096)
    base = torch.zeros(N, dtype=torch.float32, device="cuda")
    own = empty(N, "bf16")
    silo.finalize(base, own)
    silo.sync()
    out = empty(N, "bf16")
    with fa.StreamingAccumulator(N, mode="weights", chunk_bytes=1 << 20) as top:
        top.add_silo(7, silo)
        top.finalize(base, out)
        top.sync()
    silo.close()
    assert torch.equal(own.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("piece", [4096, 1001])
def test_pinned_host_partials_equal_device_partials(piece):
    """Partials arriving in pinned host memory (e.g. sent by a remote silo
    server), staged in pieces, give the same bits as device partials."""
    N = 50_000
    sizes = [2, 2]
    n_all = [100, 200, 300, 400]
    xs_all = silo_values(51, 4, N, "f32")
    silos = [run_silo(xs_all[0:2], n_all[0:2], "f32", chunk=5000),
             run_silo(xs_all[2:4], n_all[2:4], "f32", chunk=7000)]
    base = torch.zeros(N, dtype=torch.float32, device="cuda")
    outs = []
    keep = []
    for where in ("device", "pinned"):
        out = empty(N, "f32")
        with fa.StreamingAccumulator(N, mode="weights", chunk_bytes=4 * 4096, n_slots=3) as top:
            for g, s in enumerate(silos):
                W, m = s.info()
                src = s.acc[:N] if where == "device" else s.acc[:N].cpu().pin_memory()
                keep.append(src)
                for off in range(0, N, piece):
                    top.accumulate_partial(g, W, m, src[off:off + piece], offset=off)
            top.finalize(base, out)
            top.sync()
        outs.append(out)
    for s in silos:
        s.close()
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    ref, mag, _, _ = oracle.weighted_average(xs_all, n_all)
    check(host_of(outs[0]), ref, mag, "f32")


@pytest.mark.parametrize("where", ["device", "pinned"])
def test_partial_mode_silos_counts_and_weight_sums(where):
    """Masked (partial) silos: per-parameter weight sums and client counts add
    exactly; values match the flat oracle over the senders."""
    N = 30_011
    sizes = [3, 2, 4]
    K = sum(sizes)
    r = np.random.default_rng(61)
    n_all = synth.sample_counts(62, K, 100, 1000)
    xs_all = silo_values(63, K, N, "bf16")
    masks = [(r.random(N) < 0.5).astype(np.uint8) for _ in range(K)]
    masks[0][:100] = 0
    for m in masks:
        m[200:300] = 0                # nobody sent these: keep base
    base = synth.bf16_bits_from_f32((r.standard_normal(N) * 0.02).astype(np.float32))
    silos, at = [], 0
    for g, Kg in enumerate(sizes):
        silos.append(run_silo(xs_all[at:at + Kg], n_all[at:at + Kg], "bf16", chunk=4096, partial=True,
                              masks=masks[at:at + Kg]))
        at += Kg
    out = empty(N, "bf16")
    keep = []
    with fa.StreamingAccumulator(N, mode="weights", partial=True, chunk_bytes=4 * N) as top:
        for g, s in enumerate(silos):
            if where == "device":
                top.add_silo(g, s)
            else:
                W, m = s.info()
                srcs = [t[:N].cpu().pin_memory() for t in (s.acc, s.wsum, s.count)]
                keep.extend(srcs)
                top.accumulate_partial(g, W, m, *srcs)
        top.finalize(dev_of(base, "bf16"), out)
        top.sync()
        cnt = top.count[:N].cpu().numpy()
        ws = top.wsum[:N].cpu().numpy().view(np.uint32)
    for s in silos:
        s.close()
    ref, mag, rcnt, rws = oracle.weighted_average(xs_all, n_all, base=base, x_dtype=oracle.BF16,
                                                  base_dtype=oracle.BF16, sent=masks)
    assert np.array_equal(cnt, rcnt.astype(np.uint8))
    assert np.array_equal(ws, rws.astype(np.uint32))
    check(host_of(out), ref, mag, "bf16", copied=rcnt == 0, copy_expect=base_copy_expect(base, "bf16", "bf16"))


def test_partial_argument_errors():
    N = 1024
    acc_src = torch.zeros(N, device="cuda")
    with fa.StreamingAccumulator(N, mode="weights", partial=True, chunk_bytes=4 * N) as top:
        ws = torch.zeros(N, dtype=torch.int32, device="cuda")
        cn = torch.zeros(N, dtype=torch.uint8, device="cuda")
        with pytest.raises(fa.FedAvgError) as e:
            top.accumulate_partial(0, 10, 1, acc_src)          # wsum missing in partial mode
        assert e.value.code == -1
        with pytest.raises(fa.FedAvgError) as e:
            top.accumulate_partial(0, 1 << 32, 1, acc_src, ws, cn)
        assert e.value.code == -3
        top.accumulate_partial(0, 10, 200, acc_src, ws, cn)
        with pytest.raises(fa.FedAvgError) as e:
            top.accumulate_partial(1, 10, 56, acc_src, ws, cn)  # 256 clients behind the counts
        assert e.value.code == -3
        with pytest.raises(fa.FedAvgError) as e:
            top.accumulate_partial(0, 11, 200, acc_src, ws, cn, offset=0)  # weight changed
        assert e.value.code == -1
        top.accumulate_partial(2, 0, 1, acc_src, ws, cn)        # zero weight: no work
        assert top.info() == (10, 200)
    with fa.StreamingAccumulator(N, mode="weights", chunk_bytes=4 * N) as top:
        top.accumulate_partial(0, 10, 1, acc_src[:512])
        with pytest.raises(fa.FedAvgError) as e:
            top.finalize(None, torch.empty(N, device="cuda"))
        assert e.value.code == -6                                # [512, N) never covered
