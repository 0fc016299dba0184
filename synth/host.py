"""Host-side (numpy) seeded generators for inputs the CPU oracle can handle.

Random draws only: sample counts, Gaussian values, Bernoulli presence masks,
Laplace deltas with their top-p% support.  The bf16 encoding of generated
values uses torch's CPU dtype conversion (a library primitive), so no rounding
code of the method is involved.
"""

import math

import numpy as np

from .configs import ROLE_COUNTS, ROLE_BASE, ROLE_VALUES, ROLE_SUPPORT


def rng(cfg, role, client=0):
    """Generator keyed by SeedSequence([2026, cfg, role, client])."""
    return np.random.default_rng(np.random.SeedSequence([2026, int(cfg), int(role), int(client)]))


def sample_counts(cfg, K, lo, hi):
    """n_k ~ uniform integers in [lo, hi] (both ends included), int64."""
    return rng(cfg, ROLE_COUNTS).integers(lo, hi + 1, size=K, dtype=np.int64)


def normal_f32(cfg, role, client, N, sigma):
    """N(0, sigma) values (sigma is the standard deviation) as float32."""
    return (rng(cfg, role, client).standard_normal(N) * sigma).astype(np.float32)


def bf16_bits_from_f32(a):
    """uint16 bf16 bit patterns of float32 values, via torch's CPU conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def f32_from_bf16_bits(b):
    """float32 values of uint16 bf16 bit patterns (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def dense_clients_f32(cfg, K, N, sigma):
    """K independent fp32 client vectors ~N(0, sigma)."""
    return [normal_f32(cfg, ROLE_VALUES, k, N, sigma) for k in range(K)]


def dense_clients_bf16(cfg, K, N, base_sigma, pert_sigma):
    """Returns (base fp32, [bf16 bits of base + N(0, pert_sigma)] per client):
    clients are perturbed copies of one global model."""
    base = normal_f32(cfg, ROLE_BASE, 0, N, base_sigma)
    xs = []
    for k in range(K):
        pert = rng(cfg, ROLE_VALUES, k).standard_normal(N) * pert_sigma
        xs.append(bf16_bits_from_f32((base.astype(np.float64) + pert).astype(np.float32)))
    return base, xs


def adapter_presence(cfg, K, n_modules, p):
    """present[k, m] ~ Bernoulli(p), independent per (client, module)."""
    r = rng(cfg, ROLE_SUPPORT)
    return (r.random((K, n_modules)) < p).astype(np.uint8)


def topk_sparse_deltas(cfg, client, N, frac, scale):
    """Literal top-frac |delta| of N i.i.d. Laplace(0, scale) deltas: exactly
    floor(frac*N) entries, ties broken toward the lower index.  Returns sorted
    int64 indices and their float32 values."""
    d = rng(cfg, ROLE_VALUES, client).laplace(0.0, scale, N).astype(np.float32)
    k = int(math.floor(frac * N))
    order = np.lexsort((np.arange(N), -np.abs(d)))[:k]
    idx = np.sort(order).astype(np.int64)
    return idx, d[idx]


def uniform_sparse_support(cfg, client, N, k):
    """A uniformly random k-subset of [0, N) as sorted int64 indices (the
    support of a top-k of i.i.d. draws is such a subset)."""
    r = rng(cfg, ROLE_SUPPORT, client)
    return np.sort(r.choice(N, size=k, replace=False)).astype(np.int64)


def laplace_tail_values(cfg, client, k, frac, scale):
    """Values distributed as the entries of a Laplace(0, scale) sample whose
    |value| lies in the top `frac` tail: sign uniform, magnitude
    t + Exp(scale) with t = scale*ln(1/frac) (memorylessness of the tail)."""
    r = rng(cfg, ROLE_VALUES, client)
    t = scale * math.log(1.0 / frac)
    mag = t + r.exponential(scale, k)
    sign = np.where(r.random(k) < 0.5, -1.0, 1.0)
    return (sign * mag).astype(np.float32)
