"""The seeded input generators on the CPU (torch's CPU generator draws the
same kind of stream the GPU tests and the benchmark draw on the device)."""

import torch

import synth
import synth.device as sd


def test_laplace_has_no_infinities_where_the_uniform_draw_hits_its_lower_end():
    """uniform_ draws from [-0.5, 0.5): this stream holds u = -0.5, which the
    inverse CDF would turn into -inf.  The generator keeps every value finite
    and the draws Laplace(0, b) (mean |x| = b)."""
    N, b = 1 << 25, 1e-3
    g = sd.generator(synth.CFG_SPARSE_1B, synth.ROLE_VALUES, 5000, device="cpu")
    u = torch.empty(N).uniform_(-0.5, 0.5, generator=g)
    assert int((u == -0.5).sum()) >= 1
    g = sd.generator(synth.CFG_SPARSE_1B, synth.ROLE_VALUES, 5000, device="cpu")
    x = sd.laplace(N, b, g, device="cpu")
    assert bool(torch.isfinite(x).all())
    assert abs(float(x.abs().double().mean()) / b - 1) < 1e-3
    assert float(x.abs().max()) <= b * 24 * 0.6931472 * 1.0001      # -b ln(2^-24)
