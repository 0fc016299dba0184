"""Comparison of library outputs with the oracle's, to the stated bar.

* fp32 output: |g - ref32| <= 1e-6 * max(|ref32|, M), M the oracle's error
  scale |base| + sum n_k |x_k| / W (a pure |ref32|-relative bound cannot hold
  for any fp32 accumulator where the clients' terms cancel).
* bf16 output: |g - ref32| <= max(ulp_bf16(ref32), 1e-6 * M), where
  ulp_bf16(v) = 2^(floor(log2|v|) - 7), at least the bf16 subnormal spacing
  2^-133: within one bf16 ulp of the fp32-rounded exact result.
* Parameters no client sent: bit-identical copy of base (rounded to
  nearest-even first when base is fp32 and the output bf16).
* NaN matches NaN; infinities must match exactly.
"""

import numpy as np

import oracle
import synth


def _bf16_ulp(ref):
    a = np.abs(ref.astype(np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.exp2(e - 7)
    return np.maximum(ulp, 2.0 ** -133)


def check(got, ref32, mag, out_dtype, copied=None, copy_expect=None, label=""):
    """got: output values (float32 array, or uint16 bf16 bits when out_dtype is
    'bf16').  copied: boolean mask of parameters that must equal copy_expect
    bit for bit.  Raises AssertionError with a summary on failure; returns
    the largest error divided by its bound."""
    ref32 = np.asarray(ref32, dtype=np.float32)
    mag = np.asarray(mag, dtype=np.float64)
    if out_dtype == "bf16":
        bits = np.asarray(got, dtype=np.uint16)
        g = synth.f32_from_bf16_bits(bits).astype(np.float64)
    else:
        bits = np.asarray(got, dtype=np.float32).view(np.uint32)
        g = np.asarray(got, dtype=np.float32).astype(np.float64)
    r = ref32.astype(np.float64)
    nan_r, nan_g = np.isnan(r), np.isnan(g)
    assert np.array_equal(nan_r, nan_g), f"{label}: NaN pattern differs at {np.nonzero(nan_r != nan_g)[0][:10]}"
    inf_r = np.isinf(r)
    assert np.array_equal(g[inf_r], r[inf_r]), f"{label}: infinities differ"
    fin = ~nan_r & ~inf_r
    if out_dtype == "bf16":
        bound = np.maximum(_bf16_ulp(r), 1e-6 * mag)
    else:
        bound = 1e-6 * np.maximum(np.abs(r), mag)
    err = np.abs(g - r)
    bad = fin & (err > bound)
    if bad.any():
        i = np.nonzero(bad)[0][:8]
        raise AssertionError(f"{label}: {int(bad.sum())} of {len(r)} outside tolerance; first at {i}: "
                             f"got {g[i]}, ref {r[i]}, bound {bound[i]}")
    if copied is not None and copied.any():
        want = np.asarray(copy_expect)
        if out_dtype == "bf16":
            assert np.array_equal(bits[copied], want[copied]), f"{label}: unsent parameters not copied from base"
        else:
            assert np.array_equal(bits[copied], np.asarray(want, np.float32).view(np.uint32)[copied]), \
                f"{label}: unsent parameters not copied from base"
    ratio = np.where(fin, err / np.maximum(bound, 1e-300), 0.0)
    return float(ratio.max()) if len(ratio) else 0.0


def base_copy_expect(base, base_dtype, out_dtype):
    """What an unsent parameter must hold: base itself, rounded to bf16 when
    the output is bf16 and base fp32 (via the oracle's rounding)."""
    if out_dtype == "bf16":
        if base_dtype == "bf16":
            return np.asarray(base, dtype=np.uint16)
        return oracle.round_to_bf16(np.asarray(base, dtype=np.float32))
    if base_dtype == "bf16":
        return synth.f32_from_bf16_bits(base)
    return np.asarray(base, dtype=np.float32)
