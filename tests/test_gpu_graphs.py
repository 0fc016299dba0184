"""GPU: the resident entry points enqueue kernels only -- no allocation, no
memset, no host wait -- so a caller can capture them in a HIP graph.  Each
case captures one call, then changes its inputs with eager work between
replays; every replay gives the bits of the same call run eagerly on the
changed inputs."""

import numpy as np
import pytest
import torch

import synth
import weighted_model_update_amd as fa
from gpu_util import dev_f32

pytestmark = pytest.mark.gpu


def replays_match_eager(call, outs, eager, mutate, rounds=3):
    """call(): the captured call writing `outs`; eager(): the same call into
    fresh outputs, returned; mutate(r): eager work that changes the inputs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(rounds):
        mutate(r)
        want = eager()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o.view(torch.uint8), w.view(torch.uint8)), f"replay {r}"


def test_dense_call_in_a_graph():
    N = 1_000_000
    r = np.random.default_rng(3)
    xs = [dev_f32((r.standard_normal(N) * 0.02).astype(np.float32)) for _ in range(3)]
    n = [300, 500, 900]
    out = torch.empty(N, device="cuda")

    def eager():
        o = torch.empty(N, device="cuda")
        fa.fedavg_aggregate(xs, n, o)
        return [o]

    def mutate(k):
        xs[k % 3].mul_(0.75).add_(1e-3 * (k + 1))

    replays_match_eager(lambda: fa.fedavg_aggregate(xs, n, out), [out], eager, mutate)


def test_masked_call_in_a_graph():
    r = np.random.default_rng(4)
    sizes = r.integers(1, 5000, 300)
    bounds = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int64, device="cuda")
    N, K, T = int(sizes.sum()), 6, 300
    xs = [torch.from_numpy((r.standard_normal(N) * 0.01).astype(np.float32)).to(torch.bfloat16).cuda()
          for _ in range(K)]
    base = torch.from_numpy((r.standard_normal(N) * 0.01).astype(np.float32)).to(torch.bfloat16).cuda()
    present = torch.from_numpy((r.random((K, T)) < 0.6).astype(np.uint8)).cuda()
    n = synth.sample_counts(4, K, 500, 5000).tolist()
    out = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    kw = dict(base=base, seg_bounds=bounds, present=present)

    def eager():
        o = torch.empty(N, dtype=torch.bfloat16, device="cuda")
        fa.fedavg_aggregate(xs, n, o, **kw)
        return [o]

    alt = [torch.from_numpy((r.random((K, T)) < p).astype(np.uint8)).cuda() for p in (0.2, 0.9, 0.5)]

    def mutate(k):
        present.copy_(alt[k])           # the replay reads the new presence table
        xs[k].mul_(-1.0)

    replays_match_eager(lambda: fa.fedavg_aggregate(xs, n, out, **kw), [out], eager, mutate)


def test_sparse_call_in_a_graph():
    N, K = 300_007, 8
    idx, val = [], []
    for k in range(K):
        i, v = synth.topk_sparse_deltas(5, k, N, 0.1, 1e-3)
        idx.append(torch.from_numpy(np.ascontiguousarray(i, np.int64)).cuda())
        val.append(dev_f32(v))
    base = dev_f32(synth.normal_f32(5, synth.ROLE_BASE, 0, N, 0.02))
    n = synth.sample_counts(5, K, 100, 1000).tolist()
    ws = torch.empty(fa.sparse_workspace_size(K, N), dtype=torch.uint8, device="cuda")
    out = torch.empty(N, device="cuda")
    counts = torch.empty(N, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call():
        fa.sparse_masked_accumulate(idx, val, n, N, base, out, counts=counts, workspace=ws, err_flag=err)

    def eager():
        o = torch.empty(N, device="cuda")
        c = torch.empty(N, dtype=torch.uint8, device="cuda")
        e = torch.ones(1, dtype=torch.int32, device="cuda")
        fa.sparse_masked_accumulate(idx, val, n, N, base, o, counts=c, err_flag=e)
        return [o, c, e]

    def mutate(k):
        val[k].mul_(2.0)
        base.add_(1e-4)

    replays_match_eager(call, [out, counts, err], eager, mutate)
    assert int(err.item()) == 0


def test_topk_call_in_a_graph():
    """Top-k decides between its sampled and its three-pass path on the
    device, so one captured call serves whichever the data asks for: the
    changes rescale the update, give every 16th vector another scale than
    the rest, and make it tie-heavy."""
    N, k = 2_000_003, 200_000
    r = np.random.default_rng(6)
    x = dev_f32(r.laplace(0.0, 1e-3, N).astype(np.float32))
    ws = torch.empty(fa.topk_workspace_size(N, k), dtype=torch.uint8, device="cuda")
    idx = torch.empty(k, dtype=torch.int64, device="cuda")
    val = torch.empty(k, dtype=torch.float32, device="cuda")
    alts = [r.laplace(0.0, 1.0, N).astype(np.float32),
            np.where((np.arange(N) // 4) % 16 == 0, r.laplace(0.0, 1e-6, N), r.laplace(0.0, 1.0, N))
            .astype(np.float32),
            (r.integers(-2, 3, N)).astype(np.float32)]

    def eager():
        i, v = fa.topk_select(x, k)
        return [i, v]

    def mutate(j):
        x.copy_(dev_f32(alts[j]))

    replays_match_eager(lambda: fa.topk_select(x, k, idx_out=idx, val_out=val, workspace=ws),
                        [idx, val], eager, mutate)


def test_checksum_and_sum_in_a_graph():
    N = 3_000_017
    x = dev_f32(np.random.default_rng(7).standard_normal(N).astype(np.float32))
    ws = torch.empty(fa.fedavg_sum_workspace_size(N), dtype=torch.uint8, device="cuda")
    h = torch.empty(1, dtype=torch.int64, device="cuda")
    s = torch.empty(1, dtype=torch.float64, device="cuda")

    def eager():
        h2 = torch.empty(1, dtype=torch.int64, device="cuda")
        s2 = torch.empty(1, dtype=torch.float64, device="cuda")
        fa.fedavg_checksum_sum(x, workspace=torch.empty_like(ws), hash_out=h2, sum_out=s2)
        return [h2, s2]

    def mutate(j):
        x[j * 1000 + 17] += 1.0

    replays_match_eager(lambda: fa.fedavg_checksum_sum(x, workspace=ws, hash_out=h, sum_out=s),
                        [h, s], eager, mutate)
