"""Device-side (torch, seeded) generators for the full-size workloads.

Random draws and layout only, no aggregation arithmetic.  Each stream is a
torch.Generator seeded from SeedSequence([2026, cfg, role, client]), so a run
regenerates the same inputs on the same hardware.  Sample counts n_k come from
the host generators (numpy), identical to the small cases.
"""

import math

import numpy as np
import torch

from .configs import (ROLE_BASE, ROLE_VALUES, ROLE_SUPPORT, CFG_DENSE_2B, CFG_STREAM_8B,
                      CFG_SPARSE_1B, CFG_ADAPTER, CFG_DENSE_SMALL, dense_2b_tensor_shapes,
                      stream_8b_tensor_shapes, adapter_segments, numel_of, CHUNK_BYTES_8B)
from .host import sample_counts, adapter_presence


def generator(cfg, role, client=0, device="cuda"):
    seed = int(np.random.SeedSequence([2026, int(cfg), int(role), int(client)])
               .generate_state(1, dtype=np.uint64)[0] >> 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(N, sigma, g, dtype=torch.float32, device="cuda"):
    t = torch.empty(N, dtype=torch.float32, device=device)
    t.normal_(0.0, sigma, generator=g)
    return t if dtype == torch.float32 else t.to(dtype)


def dense_small(device="cuda"):
    """K=3 fp32 clients of 1,000,000 parameters ~N(0,0.02), n_k in [100,1000]."""
    K, N = 3, 1_000_000
    n = sample_counts(CFG_DENSE_SMALL, K, 100, 1000)
    xs = [normal(N, 0.02, generator(CFG_DENSE_SMALL, ROLE_VALUES, k, device), device=device)
          for k in range(K)]
    return n, xs


def adapter(device="cuda", K=8, p=0.6):
    """LoRA rank-16 A/B adapters of q,k,v,o on 32 layers at hidden 4096 (bf16,
    ~N(0,0.01)); client k sent module m iff present[k, m] (Bernoulli(p))."""
    bounds, module_of = adapter_segments()
    N = bounds[-1]
    n = sample_counts(CFG_ADAPTER, K, 500, 5000)
    pres_mod = adapter_presence(CFG_ADAPTER, K, max(module_of) + 1, p)
    present = pres_mod[:, module_of]
    xs = [normal(N, 0.01, generator(CFG_ADAPTER, ROLE_VALUES, k, device), torch.bfloat16, device)
          for k in range(K)]
    base = normal(N, 0.01, generator(CFG_ADAPTER, ROLE_BASE, 0, device), torch.bfloat16, device)
    return n, xs, base, np.asarray(bounds, np.int64), present


def dense_2b(device="cuda", K=16, N=None, dest=None):
    """K bf16 clients of the 2.0B-parameter tensor list: base ~N(0,0.02) in
    fp32, client k = bf16(base + N(0,1e-3)); n_k in [100,1000].  dest: K bf16
    tensors of N elements to write the clients into (else new tensors)."""
    if N is None:
        N = numel_of(dense_2b_tensor_shapes())
    n = sample_counts(CFG_DENSE_2B, K, 100, 1000)
    base = normal(N, 0.02, generator(CFG_DENSE_2B, ROLE_BASE, 0, device), device=device)
    xs = []
    for k in range(K):
        pert = normal(N, 1e-3, generator(CFG_DENSE_2B, ROLE_VALUES, k, device), device=device)
        pert.add_(base)
        if dest is None:
            xs.append(pert.to(torch.bfloat16))
        else:
            dest[k].copy_(pert)          # the same round-to-nearest-even conversion
            xs.append(dest[k])
        del pert
    del base
    return n, xs


def stream_8b_pool(device="cuda", pool_chunks=64, chunk_bytes=CHUNK_BYTES_8B):
    """Pinned host pool of `pool_chunks` distinct 64 MiB bf16 chunks of deltas
    ~N(0,1e-3).  Client k's chunk c is pool[(k*chunks_per_client + c)*37 % P]."""
    per = chunk_bytes // 2
    pool = torch.empty((pool_chunks, per), dtype=torch.bfloat16).pin_memory()
    g = generator(CFG_STREAM_8B, ROLE_VALUES, 0, device)
    for i in range(pool_chunks):
        pool[i].copy_(normal(per, 1e-3, g, torch.bfloat16, device))
    return pool


def stream_8b_counts(K=32):
    return sample_counts(CFG_STREAM_8B, K, 100, 10000)


def stream_8b_base(N=None, device="cuda"):
    if N is None:
        N = numel_of(stream_8b_tensor_shapes())
    return normal(N, 0.02, generator(CFG_STREAM_8B, ROLE_BASE, 0, device), torch.bfloat16, device)


def pool_index(k, c, chunks_per_client, pool_chunks):
    return ((k * chunks_per_client + c) * 37) % pool_chunks


def uniform_support(N, k, g, device="cuda"):
    """Sorted indices of a uniformly random k-subset of [0, N): a Bernoulli
    draw slightly above k/N, then a uniformly random surplus removed."""
    sd = math.sqrt(N * (k / N) * (1 - k / N))
    p = min(1.0, (k + 8 * sd + 16) / N)
    while True:
        u = torch.rand(N, generator=g, device=device)
        idx = torch.nonzero(u < p).squeeze(1)
        del u
        c = idx.numel()
        if c >= k:
            break
        p = min(1.0, p * 1.01 + 1.0 / N)
    if c > k:
        drop = torch.randperm(c, generator=g, device=device)[: c - k]
        keep = torch.ones(c, dtype=torch.bool, device=device)
        keep[drop] = False
        idx = idx[keep]
    return idx.contiguous()


def laplace_tail(k, scale, frac, g, device="cuda"):
    """Values of the top-frac |x| entries of Laplace(0, scale) samples: random
    sign, magnitude scale*ln(1/frac) + Exp(scale)."""
    mag = torch.empty(k, dtype=torch.float32, device=device)
    mag.exponential_(1.0 / scale, generator=g)
    mag.add_(scale * math.log(1.0 / frac))
    sign = torch.rand(k, generator=g, device=device) < 0.5
    return torch.where(sign, -mag, mag).contiguous()


def sparse_1b(device="cuda", K=20, N=10 ** 9, frac=0.1, scale=1e-3):
    """K clients each sending exactly floor(frac*N) sorted (index, value)
    pairs; base ~N(0,0.02) fp32; n_k in [100,1000]."""
    n = sample_counts(CFG_SPARSE_1B, K, 100, 1000)
    k = int(math.floor(frac * N))
    idx, val = [], []
    for c in range(K):
        idx.append(uniform_support(N, k, generator(CFG_SPARSE_1B, ROLE_SUPPORT, c, device), device))
        val.append(laplace_tail(k, scale, frac, generator(CFG_SPARSE_1B, ROLE_VALUES, c, device), device))
    base = normal(N, 0.02, generator(CFG_SPARSE_1B, ROLE_BASE, 0, device), device=device)
    return n, idx, val, base


def laplace(N, scale, g, device="cuda"):
    """N i.i.d. Laplace(0, scale) draws (scale = b, the Laplace scale) as
    float32, by inverting the CDF of uniform draws in (-1/2, 1/2)."""
    u = torch.empty(N, dtype=torch.float32, device=device)
    u.uniform_(-0.5, 0.5, generator=g)
    # x = -b * sign(u) * ln(1 - 2|u|).  uniform_ draws from [-0.5, 0.5), so
    # u = -0.5 does occur (about once in 2^24 draws) and would give an
    # infinity: |u| is held to the largest float below 0.5, the tail's next
    # draw, 0.5 - 2^-25
    a = u.abs()
    a.clamp_(max=0.5 - 2.0 ** -25)
    a.mul_(-2.0).add_(1.0).log_().mul_(-scale)
    return a.copysign_(u)


def client_delta_1b(client=0, N=10 ** 9, scale=1e-3, device="cuda"):
    """One client's full fp32 update of the 10^9-parameter model before
    sparsification: i.i.d. Laplace(0, 1e-3) deltas (the distribution whose
    top-10% the sparse workload stands in for)."""
    return laplace(N, scale, generator(CFG_SPARSE_1B, ROLE_VALUES, 1000 + client, device), device)
