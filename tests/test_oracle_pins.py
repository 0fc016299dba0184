"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than its own formula:
hand-worked values, the exact-rational brute force, closed forms and
invariants of a weighted mean, or a library routine for a special case.
Together they are chosen so that a dropped term, a wrong sign, a wrong index,
a swapped operand or a wrong denominator fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import exact
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _f32(vals):
    return np.asarray(vals, dtype=np.float32)


def _mode(name):
    return oracle.DELTAS if name == "deltas" else oracle.WEIGHTS


# --------------------------------------------------------------------------
# hand-worked examples
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", _golden()["dense"], ids=lambda c: c["name"])
def test_hand_worked_dense(case):
    base = _f32(case["base"]) if "base" in case else None
    ref, mag, cnt, ws = oracle.weighted_average([_f32(x) for x in case["x"]], case["n"],
                                                mode=_mode(case["mode"]), base=base)
    np.testing.assert_array_equal(ref, _f32(case["expect"]))
    for r, h in zip(ref, case.get("expect_hex", [])):
        if h is not None:
            assert int(np.float32(r).view(np.uint32)) == int(h, 16)


@pytest.mark.parametrize("case", _golden()["masked"], ids=lambda c: c["name"])
def test_hand_worked_masked(case):
    bounds = case["segments"]
    N = bounds[-1]
    sent = []
    for pres in case["present"]:
        s = np.zeros(N, np.uint8)
        for t, p in enumerate(pres):
            s[bounds[t]:bounds[t + 1]] = p
        sent.append(s)
    ref, mag, cnt, ws = oracle.weighted_average([_f32(x) for x in case["x"]], case["n"],
                                                mode=_mode(case["mode"]), base=_f32(case["base"]),
                                                sent=sent)
    np.testing.assert_array_equal(ref, _f32(case["expect"]))
    np.testing.assert_array_equal(cnt, case["expect_count"])


@pytest.mark.parametrize("case", _golden()["sparse"], ids=lambda c: c["name"])
def test_hand_worked_sparse(case):
    ref, mag, cnt, ws = oracle.sparse_average(case["idx"], case["val"], case["n"], case["N"],
                                              mode=_mode(case["mode"]), base=_f32(case["base"]))
    np.testing.assert_array_equal(ref, _f32(case["expect"]))
    np.testing.assert_array_equal(cnt, case["expect_count"])
    np.testing.assert_array_equal(ws, case["expect_wsum"])


# --------------------------------------------------------------------------
# exact-rational brute force on tiny random inputs
# --------------------------------------------------------------------------

def _special_values():
    f = np.float32
    return np.array([0.0, -0.0, 1.0, -1.0, f(1e-40), f(-3e-39), f(1e-45), f(3.3e38), f(-3.3e38),
                     f(1.5), f(0.1), f(-2.5e-8), f(65504.0), f(1.17549435e-38)], dtype=np.float32)


@pytest.mark.parametrize("K", [1, 2, 3, 5])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["weights", "deltas"])
def test_brute_force_dense(K, dtype, mode):
    r = np.random.default_rng(100 + K)
    N = 48
    xs32 = [(r.standard_normal(N) * 10.0 ** r.integers(-3, 3)).astype(np.float32) for _ in range(K)]
    xs32[0][:8] = _special_values()[:8]
    n = r.integers(0, 2000, size=K)
    n[0] = max(n[0], 1)
    base32 = (r.standard_normal(N) * 0.02).astype(np.float32)
    if dtype == "bf16":
        xs = [synth.bf16_bits_from_f32(x) for x in xs32]
        vals = [synth.f32_from_bf16_bits(x) for x in xs]
        dt = oracle.BF16
    else:
        xs, vals, dt = xs32, xs32, oracle.F32
    base = base32 if mode == "deltas" else None
    ref, mag, cnt, ws = oracle.weighted_average(xs, n, mode=_mode(mode), base=base, x_dtype=dt)
    want = exact.weighted_average_exact([v.astype(np.float64).tolist() for v in vals], n.tolist(),
                                        mode=mode, base=None if base is None else base.tolist())
    want = np.asarray(want, dtype=np.float32)
    # fp64 accumulation can only differ from the exact result within 64*2^-53*M
    # of a rounding boundary; on these inputs that never happens
    np.testing.assert_array_equal(ref, want)


def test_brute_force_masked_and_sparse():
    r = np.random.default_rng(7)
    K, N = 4, 40
    xs = [r.standard_normal(N).astype(np.float32) for _ in range(K)]
    sent = [(r.random(N) < 0.5).astype(np.uint8) for _ in range(K)]
    n = r.integers(1, 100, size=K)
    base = r.standard_normal(N).astype(np.float32)
    ref, _, cnt, ws = oracle.weighted_average(xs, n, mode=oracle.DELTAS, base=base, sent=sent)
    want = exact.weighted_average_exact([x.tolist() for x in xs], n.tolist(), mode="deltas",
                                        base=base.tolist(), sent=[s.tolist() for s in sent])
    np.testing.assert_array_equal(ref, np.asarray(want, np.float32))
    # the same data expressed as sparse lists
    idx = [np.nonzero(s)[0] for s in sent]
    val = [x[i] for x, i in zip(xs, idx)]
    sref, _, scnt, sws = oracle.sparse_average(idx, val, n, N, mode=oracle.DELTAS, base=base)
    np.testing.assert_array_equal(sref, ref)
    np.testing.assert_array_equal(scnt, cnt)
    np.testing.assert_array_equal(sws, ws)


def test_exact_rounding_helper_against_numpy():
    # the brute force's own fp32 rounding agrees with numpy's binary32
    # conversion of doubles whose value it represents exactly
    r = np.random.default_rng(3)
    vals = np.concatenate([r.standard_normal(500) * 10.0 ** r.integers(-40, 38, 500),
                           [1e-45, 7e-46, 3.5e-45, 3.4028235e38, 3.4028236e38, 1e39]])
    from fractions import Fraction
    for v in vals:
        assert exact.round_fp32(Fraction(float(v))) == float(np.float32(v)) or \
            (math.isinf(exact.round_fp32(Fraction(float(v)))) and math.isinf(np.float32(v)))


# --------------------------------------------------------------------------
# closed forms and invariants of a weighted mean
# --------------------------------------------------------------------------

def test_single_client_is_identity():
    x = synth.normal_f32(1, synth.ROLE_VALUES, 0, 10000, 0.02)
    for nk in (1, 3, 977, 2 ** 24):
        ref, mag, cnt, ws = oracle.weighted_average([x], [nk])
        np.testing.assert_array_equal(ref, x)
        assert (cnt == 1).all() and (ws == nk).all()


def test_identical_clients_reproduce_input():
    x = synth.normal_f32(1, synth.ROLE_VALUES, 1, 5000, 0.02)
    n = synth.sample_counts(1, 16, 100, 1000)
    ref, *_ = oracle.weighted_average([x] * 16, n)
    np.testing.assert_array_equal(ref, x)
    bits = synth.bf16_bits_from_f32(x)
    ref, *_ = oracle.weighted_average([bits] * 16, n, x_dtype=oracle.BF16)
    np.testing.assert_array_equal(ref, synth.f32_from_bf16_bits(bits))


def test_normalised_weights_sum_to_one():
    # all-ones clients give exactly 1 only if the weights n_k/W sum to 1
    n = synth.sample_counts(3, 32, 100, 10000)
    ones = [np.ones(64, np.float32)] * 32
    ref, *_ = oracle.weighted_average(ones, n)
    np.testing.assert_array_equal(ref, np.ones(64, np.float32))
    w = n.astype(np.float64) / n.sum()
    assert abs(w.sum() - 1.0) <= 32 * 2.0 ** -53


def test_linearity():
    K, N = 6, 3000
    n = synth.sample_counts(1, K, 100, 1000)
    X = synth.dense_clients_f32(1, K, N, 0.02)
    Y = synth.dense_clients_f32(9, K, N, 0.5)
    a, b = 0.75, -3.0  # exact in binary32 combinations below
    Z = [(a * x.astype(np.float64) + b * y.astype(np.float64)).astype(np.float32) for x, y in zip(X, Y)]
    rx, mx, *_ = oracle.weighted_average(X, n)
    ry, my, *_ = oracle.weighted_average(Y, n)
    rz, mz, *_ = oracle.weighted_average(Z, n)
    lhs = rz.astype(np.float64)
    rhs = a * rx.astype(np.float64) + b * ry.astype(np.float64)
    scale = np.maximum(mz, abs(a) * mx + abs(b) * my)
    assert np.all(np.abs(lhs - rhs) <= 4 * 2.0 ** -24 * scale)


def test_weight_scale_invariance():
    K, N = 5, 2000
    n = synth.sample_counts(1, K, 100, 1000)
    X = synth.dense_clients_f32(2, K, N, 0.02)
    r1, *_ = oracle.weighted_average(X, n)
    r2, *_ = oracle.weighted_average(X, n * 8)      # power of two: bit-identical
    np.testing.assert_array_equal(r1, r2)
    r3, *_ = oracle.weighted_average(X, n * 3)
    assert np.max(np.abs(r3.view(np.int32).astype(np.int64) - r1.view(np.int32).astype(np.int64))) <= 1


def test_client_permutation():
    K, N = 7, 2000
    n = synth.sample_counts(4, K, 100, 1000)
    X = synth.dense_clients_f32(4, K, N, 0.02)
    perm = np.random.default_rng(0).permutation(K)
    r1, *_ = oracle.weighted_average(X, n)
    r2, *_ = oracle.weighted_average([X[p] for p in perm], n[perm])
    d = np.abs(r1.view(np.int32).astype(np.int64) - r2.view(np.int32).astype(np.int64))
    assert d.max() <= 1


def test_uniform_weights_equal_numpy_mean():
    K, N = 9, 4000
    X = synth.dense_clients_f32(5, K, N, 0.02)
    ref, *_ = oracle.weighted_average(X, [42] * K)
    want = np.mean(np.stack(X).astype(np.float64), axis=0).astype(np.float32)
    d = np.abs(ref.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert d.max() <= 1 and (d == 0).mean() > 0.999


def test_masks_all_one_and_none():
    K, N = 4, 1000
    n = synth.sample_counts(2, K, 500, 5000)
    X = synth.dense_clients_f32(2, K, N, 0.01)
    base = synth.normal_f32(2, synth.ROLE_BASE, 0, N, 0.01)
    dense, *_ = oracle.weighted_average(X, n)
    allsent, *_ = oracle.weighted_average(X, n, base=base, sent=[np.ones(N, np.uint8)] * K)
    np.testing.assert_array_equal(dense, allsent)
    none, _, cnt, ws = oracle.weighted_average(X, n, base=base, sent=[np.zeros(N, np.uint8)] * K)
    np.testing.assert_array_equal(none, base)
    assert (cnt == 0).all() and (ws == 0).all()
    # exactly one sender per parameter: that sender's value
    owner = np.random.default_rng(1).integers(0, K, N)
    sent = [(owner == k).astype(np.uint8) for k in range(K)]
    one, *_ = oracle.weighted_average(X, n, base=base, sent=sent)
    np.testing.assert_array_equal(one, np.choose(owner, X))


def test_no_sender_and_no_base_is_an_error():
    with pytest.raises(oracle.OracleError):
        oracle.weighted_average([np.ones(4, np.float32)], [1], sent=[np.zeros(4, np.uint8)])
    with pytest.raises(oracle.OracleError):
        oracle.weighted_average([np.ones(4, np.float32)], [-1])


def test_sparse_full_support_equals_dense_deltas():
    K, N = 5, 3000
    n = synth.sample_counts(5, K, 100, 1000)
    D = synth.dense_clients_f32(5, K, N, 1e-3)
    base = synth.normal_f32(5, synth.ROLE_BASE, 0, N, 0.02)
    full = [np.arange(N)] * K
    sref, _, scnt, sws = oracle.sparse_average(full, D, n, N, base=base)
    dref, *_ = oracle.weighted_average(D, n, mode=oracle.DELTAS, base=base)
    np.testing.assert_array_equal(sref, dref)
    assert (scnt == K).all() and (sws == n.sum()).all()


def test_sparse_disjoint_supports_add_the_delta():
    K, N = 4, 4000
    n = synth.sample_counts(5, K, 100, 1000)
    owner = np.random.default_rng(2).integers(-1, K, N)   # -1: nobody
    base = synth.normal_f32(5, synth.ROLE_BASE, 0, N, 0.02)
    D = synth.dense_clients_f32(6, K, N, 1e-3)
    idx = [np.nonzero(owner == k)[0] for k in range(K)]
    val = [D[k][i] for k, i in enumerate(idx)]
    ref, _, cnt, ws = oracle.sparse_average(idx, val, n, N, base=base)
    want = base.copy()
    for k in range(K):
        want[idx[k]] = base[idx[k]] + val[k]   # binary32 add is correctly rounded
    np.testing.assert_array_equal(ref, want)
    np.testing.assert_array_equal(cnt, (owner >= 0).astype(np.uint32))


def test_sparse_counts_and_weight_sums_are_bincounts():
    K, N = 6, 5000
    n = synth.sample_counts(5, K, 100, 1000)
    base = synth.normal_f32(5, synth.ROLE_BASE, 0, N, 0.02)
    idx, val = zip(*[synth.topk_sparse_deltas(5, k, N, 0.1, 1e-3) for k in range(K)])
    ref, _, cnt, ws = oracle.sparse_average(idx, val, n, N, base=base)
    allidx = np.concatenate(idx)
    np.testing.assert_array_equal(cnt, np.bincount(allidx, minlength=N))
    wts = np.concatenate([np.full(len(i), n[k], np.float64) for k, i in enumerate(idx)])
    np.testing.assert_array_equal(ws, np.bincount(allidx, weights=wts, minlength=N).astype(np.uint64))
    # unsent parameters keep the base bit for bit
    np.testing.assert_array_equal(ref[cnt == 0], base[cnt == 0])


def test_sparse_at_matches_full():
    K, N = 5, 6000
    n = synth.sample_counts(5, K, 100, 1000)
    base = synth.normal_f32(5, synth.ROLE_BASE, 0, N, 0.02)
    idx, val = zip(*[synth.topk_sparse_deltas(5, k, N, 0.1, 1e-3) for k in range(K)])
    ref, mag, cnt, ws = oracle.sparse_average(idx, val, n, N, base=base)
    at = np.random.default_rng(0).choice(N, 500, replace=False)
    r2, m2, c2, w2 = oracle.sparse_average_at(idx, val, n, N, at, base=base)
    np.testing.assert_array_equal(r2, ref[at])
    np.testing.assert_array_equal(c2, cnt[at])
    np.testing.assert_array_equal(w2, ws[at])


def test_sparse_rejects_unsorted_or_out_of_range():
    base = np.zeros(8, np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.sparse_average([[3, 2]], [[1.0, 1.0]], [1], 8, base=base)
    with pytest.raises(oracle.OracleError):
        oracle.sparse_average([[1, 1]], [[1.0, 1.0]], [1], 8, base=base)
    with pytest.raises(oracle.OracleError):
        oracle.sparse_average([[8]], [[1.0]], [1], 8, base=base)


def test_nan_propagates_and_zero_weight_nan_is_skipped():
    x0 = np.array([np.nan, 1.0], np.float32)
    x1 = np.array([2.0, 3.0], np.float32)
    ref, *_ = oracle.weighted_average([x0, x1], [1, 1])
    assert math.isnan(ref[0]) and ref[1] == 2.0
    ref, *_ = oracle.weighted_average([x0, x1], [0, 1])
    np.testing.assert_array_equal(ref, x1)


def test_bf16_rounding_matches_library_conversion():
    # round-to-nearest-even to bf16 is what torch's dtype conversion does
    import torch
    r = np.random.default_rng(11)
    a = np.concatenate([r.standard_normal(20000).astype(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.4028235e38, 1e-40,
                                  -1e-45, 1.0039062, 1.0117188], np.float32)])
    # exact ties: low half exactly 0x8000 with odd and even upper halves
    ties = (np.arange(0x3f80, 0x3f90, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    a = np.concatenate([a, ties])
    ours = oracle.round_to_bf16(a)
    lib = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, lib)
    q = oracle.round_to_bf16(np.array([np.nan, -np.nan], np.float32))
    assert all((v & 0x7f80) == 0x7f80 and (v & 0x7f) != 0 for v in q)


def test_checksum_split_additivity_and_sensitivity():
    r = np.random.default_rng(5)
    a = r.standard_normal(1000).astype(np.float32)
    h = oracle.checksum(a, oracle.F32)
    # the checksum of a buffer equals the sum (mod 2^64) of its pieces', for
    # any split, so it does not depend on the order elements are visited
    for m in (1, 333, 999):
        parts = oracle.checksum(a[:m], oracle.F32) + oracle.checksum(a[m:], oracle.F32, first=m)
        assert h == parts % 2 ** 64
    b = a.copy()
    b[500] = np.nextafter(b[500], np.float32(np.inf))
    assert oracle.checksum(b, oracle.F32) != h
    # swapping two different values changes it (indices are part of the hash)
    c = a.copy()
    c[[3, 4]] = c[[4, 3]]
    assert oracle.checksum(c, oracle.F32) != h
    # bf16 buffers hash their 16-bit patterns
    bits = synth.bf16_bits_from_f32(a)
    assert oracle.checksum(bits, oracle.BF16) != oracle.checksum(bits ^ np.uint16(1), oracle.BF16)


def test_topk_generator_support_and_tail():
    N = 10007
    idx, val = synth.topk_sparse_deltas(5, 0, N, 0.1, 1e-3)
    assert len(idx) == N // 10
    assert np.all(np.diff(idx) > 0) and idx[0] >= 0 and idx[-1] < N
    # top-10% of Laplace(0,b) magnitudes sit above about b*ln(10)
    assert np.quantile(np.abs(val), 0.05) > 0.8 * 1e-3 * math.log(10)


# ---------------------------------------------------------------- top-k selection

def _bits_array(case):
    if case["dtype"] == "f32":
        return np.array([int(h, 16) for h in case["x_hex"]], np.uint32).view(np.float32), oracle.F32
    return np.array([int(h, 16) for h in case["x_hex"]], np.uint16), oracle.BF16


@pytest.mark.parametrize("case", _golden()["topk"], ids=lambda c: c["name"])
def test_hand_worked_topk(case):
    x, dt = _bits_array(case)
    for c in case["cases"]:
        idx, val = oracle.topk(x, dt, c["k"])
        assert idx.tolist() == c["idx"], c
        want = x[idx] if dt == oracle.F32 else synth.f32_from_bf16_bits(x[idx])
        assert np.array_equal(val.view(np.uint32), np.asarray(want, np.float32).view(np.uint32))


def _dominates(keys, S):
    """S (a set of indices) is the top-k: every chosen entry outranks every
    other -- larger key, or equal key and lower index."""
    out = [j for j in range(len(keys)) if j not in S]
    return all(keys[i] > keys[j] or (keys[i] == keys[j] and i < j) for i in S for j in out)


def test_topk_brute_force_over_all_subsets():
    import itertools
    r = np.random.default_rng(5)
    pool = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.inf, -np.inf, np.nan, 1e-40, 3.0], np.float32)
    for trial in range(60):
        N = int(r.integers(1, 9))
        x = r.choice(pool, N)
        # rank by |x| with NaN above infinity, compared as tuples so that no
        # comparison ever involves a NaN
        rank_key = [(2 if np.isnan(v) else 1 if np.isinf(v) else 0, 0.0 if np.isnan(v) or np.isinf(v)
                     else float(abs(v))) for v in x]
        for k in range(N + 1):
            winners = [set(S) for S in itertools.combinations(range(N), k) if _dominates(rank_key, set(S))]
            assert len(winners) == 1
            idx, _ = oracle.topk(x, oracle.F32, k)
            assert set(idx.tolist()) == winners[0] and list(idx) == sorted(idx)


def test_topk_magnitude_order_for_finite_values():
    r = np.random.default_rng(6)
    x = (r.standard_normal(20000) * np.exp(r.uniform(-30, 30, 20000))).astype(np.float32)
    x[::97] = 0.0
    x[::89] *= -1
    k = 777
    idx, val = oracle.topk(x, oracle.F32, k)
    a = np.abs(x.astype(np.float64))
    chosen = np.zeros(len(x), bool)
    chosen[idx] = True
    assert a[chosen].min() >= a[~chosen].max()
    # distinct magnitudes: a plain stable sort by magnitude gives the same set
    u = np.unique(a, return_index=True)[1]
    xd = x[np.sort(u)]
    kd = 500
    got, _ = oracle.topk(xd, oracle.F32, kd)
    want = np.sort(np.argsort(-np.abs(xd.astype(np.float64)), kind="stable")[:kd])
    assert np.array_equal(got, want)


def test_topk_bf16_equals_widened_fp32_and_edge_counts():
    r = np.random.default_rng(7)
    bits = synth.bf16_bits_from_f32((r.standard_normal(5000) * 0.01).astype(np.float32))
    wide = synth.f32_from_bf16_bits(bits)
    for k in (0, 1, 500, 4999, 5000):
        a = oracle.topk(bits, oracle.BF16, k)
        b = oracle.topk(wide, oracle.F32, k)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    with pytest.raises(oracle.OracleError):
        oracle.topk(wide, oracle.F32, 5001)


# ---------------------------------------------------------------- zero-fill denominator

def test_zero_fill_brute_force_masked_sparse_and_sampled():
    """Zero-fill delta mode (unsent entries count as zero deltas, so the mean
    divides by the total weight of all clients) against the exact-rational
    statement, through the dense-with-masks, sparse and sampled entry points."""
    r = np.random.default_rng(17)
    K, N = 5, 60
    xs = [(r.standard_normal(N) * 10.0 ** r.integers(-3, 2)).astype(np.float32) for _ in range(K)]
    sent = [(r.random(N) < 0.4).astype(np.uint8) for _ in range(K)]
    for s_ in sent:
        s_[:3] = 0                               # nobody sent 0..2: base kept
    n = r.integers(0, 900, size=K)
    n[1] = 0                                     # a zero-weight client is no client at all
    n[0] = max(n[0], 1)
    base = r.standard_normal(N).astype(np.float32)
    want = np.asarray(exact.weighted_average_exact([x.tolist() for x in xs], n.tolist(),
                                                   mode="deltas_zero_fill", base=base.tolist(),
                                                   sent=[s_.tolist() for s_ in sent]), np.float32)
    ref, _, cnt, ws = oracle.weighted_average(xs, n, mode=oracle.DELTAS_ZERO_FILL, base=base, sent=sent)
    np.testing.assert_array_equal(ref, want)
    assert np.array_equal(ref[:3].view(np.uint32), base[:3].view(np.uint32))
    idx = [np.nonzero(s_)[0] for s_ in sent]
    val = [x[i] for x, i in zip(xs, idx)]
    sref, _, scnt, sws = oracle.sparse_average(idx, val, n, N, mode=oracle.DELTAS_ZERO_FILL, base=base)
    np.testing.assert_array_equal(sref, want)
    np.testing.assert_array_equal(scnt, cnt)
    at = np.array([0, 5, 17, 59], np.int64)
    aref, _, _, _ = oracle.sparse_average_at(idx, val, n, N, at, mode=oracle.DELTAS_ZERO_FILL, base=base)
    np.testing.assert_array_equal(aref, want[at])


def test_zero_fill_special_cases():
    r = np.random.default_rng(18)
    K, N = 4, 500
    xs = [(r.standard_normal(N) * 1e-3).astype(np.float32) for _ in range(K)]
    n = np.array([3, 5, 7, 11])
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    # everyone sends everything: W_i = S, the two readings coincide
    a = oracle.weighted_average(xs, n, mode=oracle.DELTAS_ZERO_FILL, base=base)[0]
    b = oracle.weighted_average(xs, n, mode=oracle.DELTAS, base=base)[0]
    assert np.array_equal(a, b)
    # disjoint supports: each parameter gets base + n_k * d / S exactly rounded
    owner = r.integers(0, K, N)
    sent = [(owner == k).astype(np.uint8) for k in range(K)]
    z = oracle.weighted_average(xs, n, mode=oracle.DELTAS_ZERO_FILL, base=base, sent=sent)[0]
    S = int(n.sum())
    want = np.array([float(base[i]) + n[owner[i]] * float(xs[owner[i]][i]) / S for i in range(N)])
    assert np.max(np.abs(z - want.astype(np.float32))) <= 2 * np.spacing(np.abs(want).astype(np.float32)).max()


@pytest.mark.parametrize("case", _golden()["sparse_zero_fill"], ids=lambda c: c["name"])
def test_hand_worked_sparse_zero_fill(case):
    idx = [np.array(i, np.int64) for i in case["idx"]]
    val = [np.array(v, np.float32) for v in case["val"]]
    base = np.array(case["base"], np.float32)
    ref, _, _, _ = oracle.sparse_average(idx, val, case["n"], case["N"], mode=oracle.DELTAS_ZERO_FILL,
                                         base=base)
    assert ref.tolist() == case["expect"]


# ---------------------------------------------------------------- sample allocation

import oracle.controller as controller


@pytest.mark.parametrize("case", _golden()["controller"]["cases"], ids=lambda c: c["name"])
def test_hand_worked_controller(case):
    state = None
    for rnd in case["rounds"]:
        got, state = controller.controller_step(rnd["t"], rnd["e"], rnd["n"], case["total"], case["w_time"],
                                                case["w_energy"], case["ema"], case["deadband"], state)
        assert got == rnd["expect"], (case["name"], got)


def test_controller_invariants():
    r = np.random.default_rng(9)
    for trial in range(200):
        P = int(r.integers(1, 12))
        n = r.integers(1, 5000, P).tolist()
        t = (r.random(P) * 100 + 0.01).tolist()
        e = (r.random(P) * 50 + 0.01).tolist()
        total = int(r.integers(P, 100_000))
        wt, we = float(r.random()), float(r.random())
        got, (tau, eps) = controller.controller_step(t, e, n, total, wt, we, 1.0, 0.0)
        assert sum(got) == total and min(got) >= 1
        # lower cost never gets fewer samples than a higher cost (up to one
        # sample of rounding); medians by numpy
        mt, me = float(np.median(tau)), float(np.median(eps))
        c = [wt * tau[i] / mt + we * eps[i] / me for i in range(P)]
        for i in range(P):
            for j in range(P):
                if c[i] < c[j]:
                    assert got[i] + 1 >= got[j]
    # rescaling every time by the same factor changes nothing (median normalisation)
    a, _ = controller.controller_step([3, 5, 7], [1, 1, 1], [10, 10, 10], 999, 1.0, 0.0, 1.0, 0.0)
    b, _ = controller.controller_step([30, 50, 70], [1, 1, 1], [10, 10, 10], 999, 1.0, 0.0, 1.0, 0.0)
    assert a == b


def _fsum(a):
    # Python's math.fsum returns the correctly rounded sum of its floats
    return math.fsum(np.asarray(a, np.float64).tolist())


@pytest.mark.parametrize("period", [0, 1, 7])
def test_value_sum_is_the_correctly_rounded_exact_sum(period):
    """Pinned to math.fsum (an independent correctly rounded summation) on
    values spread over fp32's whole range, subnormals included, with heavy
    cancellation; also with the carry pass run after every few additions."""
    oracle.set_sum_carry_period(period)
    try:
        r = np.random.default_rng(31 + period)
        cases = [
            r.standard_normal(10_000).astype(np.float32),
            # log-uniform magnitudes over 2^-149 .. 2^127, random signs
            (np.exp2(r.uniform(-149, 127, 5000)) * r.choice([-1.0, 1.0], 5000)).astype(np.float32),
            # many values cancelling around a few large ones
            np.concatenate([np.float32([3e38, -3e38, 1e30, -1e30]),
                            r.standard_normal(3000).astype(np.float32) * np.float32(1e-30)]),
            np.full(100_000, np.float32(3.4e38)),
            r.integers(-(1 << 24), 1 << 24, 20_000).astype(np.float32) * np.float32(2.0 ** -149),
        ]
        for a in cases:
            a = r.permutation(a)
            assert oracle.value_sum(a, oracle.F32) == _fsum(a)
            bits = synth.bf16_bits_from_f32(a)
            widened = (bits.astype(np.uint32) << 16).view(np.float32)
            assert oracle.value_sum(bits, oracle.BF16) == _fsum(widened)
    finally:
        oracle.set_sum_carry_period(0)


def test_value_sum_rounds_once_with_ties_to_even():
    """Exact sums halfway between fp64 neighbours round to the even one;
    anything beyond halfway rounds away; a naive fp64 loop loses the small
    terms these cases hinge on."""
    t = np.float32(2.0 ** 53)
    assert oracle.value_sum(np.float32([t, 1.0]), oracle.F32) == 2.0 ** 53
    assert oracle.value_sum(np.float32([t, 3.0]), oracle.F32) == 2.0 ** 53 + 4
    assert oracle.value_sum(np.float32([t, 1.0, 2.0 ** -20]), oracle.F32) == 2.0 ** 53 + 2
    assert oracle.value_sum(np.float32([t, 1.0, -(2.0 ** -20)]), oracle.F32) == 2.0 ** 53
    assert oracle.value_sum(np.float32([-t, -1.0, -(2.0 ** -20)]), oracle.F32) == -(2.0 ** 53 + 2)
    assert oracle.value_sum(np.float32([1e30, 1.0, -1e30]), oracle.F32) == 1.0
    assert oracle.value_sum(np.float32([2.0 ** -149] * 3), oracle.F32) == 3 * 2.0 ** -149


def test_value_sum_special_values():
    inf, nan = np.float32(np.inf), np.float32(np.nan)
    assert math.isnan(oracle.value_sum(np.float32([1.0, nan, 2.0]), oracle.F32))
    assert math.isnan(oracle.value_sum(np.float32([inf, 1.0, -inf]), oracle.F32))
    assert oracle.value_sum(np.float32([inf, -3e38, -3e38]), oracle.F32) == math.inf
    assert oracle.value_sum(np.float32([-inf, 3e38]), oracle.F32) == -math.inf
    z = oracle.value_sum(np.float32([-0.0, -0.0]), oracle.F32)
    assert z == 0.0 and math.copysign(1.0, z) == 1.0
    assert oracle.value_sum(np.float32([5.0, -5.0]), oracle.F32) == 0.0
    assert oracle.value_sum(np.zeros(0, np.float32), oracle.F32) == 0.0
    assert oracle.value_sum(np.uint16([0x7F80, 0x3F80]), oracle.BF16) == math.inf
    assert math.isnan(oracle.value_sum(np.uint16([0xFFC1, 0x3F80]), oracle.BF16))


# ---------------------------------------------------------------- fp32 mirror

def _np_f32_sequence(xs, n, sent, mode, base, S_all):
    """With weights that are powers of two, fp32(n_k) * x is exact, so each
    fused multiply-add is one IEEE fp32 addition: numpy's float32 arithmetic
    computes the same sequence independently."""
    N = len(xs[0])
    acc = np.zeros(N, np.float32)
    W = np.zeros(N, np.int64)
    for k in range(len(xs)):
        if n[k] == 0:
            continue
        on = np.ones(N, bool) if sent is None else sent[k].astype(bool)
        prod = np.float32(n[k]) * xs[k]                      # exact for n_k = 2^j
        acc = np.where(on, (acc + prod).astype(np.float32), acc)
        W = W + np.where(on, n[k], 0)
    D = np.float32(S_all) if mode == oracle.DELTAS_ZERO_FILL else W.astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = (acc / D).astype(np.float32)
    r = q if mode == oracle.WEIGHTS else (base + q).astype(np.float32)
    return np.where(W > 0, r, base if base is not None else r).astype(np.float32)


@pytest.mark.parametrize("mode", [oracle.WEIGHTS, oracle.DELTAS, oracle.DELTAS_ZERO_FILL])
def test_mirror_equals_float32_arithmetic_for_power_of_two_weights(mode):
    r = np.random.default_rng(70 + mode)
    N, K = 5000, 7
    xs = [(r.standard_normal(N) * 10.0 ** r.integers(-4, 2)).astype(np.float32) for _ in range(K)]
    n = [int(2 ** r.integers(0, 12)) for _ in range(K)]
    n[2] = 0
    sent = [(r.random(N) < 0.6).astype(np.uint8) for _ in range(K)]
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    S_all = sum(v for v in n if v > 0)
    got = oracle.mirror_f32(xs, n, mode=mode, base=base, sent=sent)
    want = _np_f32_sequence(xs, n, sent, mode, base, S_all)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_mirror_follows_client_order_with_one_rounding_per_step():
    """1 + 2^-24 is a tie and rounds back to 1, while 2^-24 + 2^-24 + 1 is
    exact: the same three clients in two orders give different bits, as the
    fp32 steps in client order say they must."""
    one, tiny = np.float32(1.0), np.float32(2.0 ** -24)
    a = oracle.mirror_f32([np.float32([one]), np.float32([tiny]), np.float32([tiny])], [1, 1, 1])
    b = oracle.mirror_f32([np.float32([tiny]), np.float32([tiny]), np.float32([one])], [1, 1, 1])
    assert a[0] == np.float32(1.0) / np.float32(3.0)
    assert b[0] == np.float32(1.0 + 2.0 ** -23) / np.float32(3.0)
    assert a[0] != b[0]


@pytest.mark.parametrize("x_dtype,out_dtype", [(oracle.F32, oracle.F32), (oracle.BF16, oracle.BF16),
                                               (oracle.BF16, oracle.F32), (oracle.F32, oracle.BF16)])
def test_mirror_within_the_rounding_bound_of_the_definition(x_dtype, out_dtype):
    """General weights (fused products not exact): the mirror stays within
    the fp32 tolerance of the fp64 definition, and parameters nobody sent
    are the base rounded to the output type."""
    from parity import check
    r = np.random.default_rng(90 + x_dtype + 2 * out_dtype)
    N, K = 4000, 9
    x32 = [(r.standard_normal(N) * 1e-2).astype(np.float32) for _ in range(K)]
    xs = [synth.bf16_bits_from_f32(x) for x in x32] if x_dtype == oracle.BF16 else x32
    n = synth.sample_counts(3, K, 100, 10000)
    sent = [(r.random(N) < 0.4).astype(np.uint8) for _ in range(K)]
    sent[0][:50] = 1
    for s_ in sent:
        s_[50:60] = 0                        # nobody sent these
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    for mode in (oracle.WEIGHTS, oracle.DELTAS):
        got = oracle.mirror_f32(xs, n, mode=mode, base=base, x_dtype=x_dtype, out_dtype=out_dtype, sent=sent)
        ref, mag, cnt, _ = oracle.weighted_average(xs, n, mode=mode, base=base, x_dtype=x_dtype, sent=sent)
        odt = "bf16" if out_dtype == oracle.BF16 else "f32"
        expect_copy = oracle.round_to_bf16(base) if out_dtype == oracle.BF16 else base
        check(got, ref, mag, odt, copied=cnt == 0, copy_expect=expect_copy)


def test_mirror_products_are_fused():
    """The rounding error of an fp32 product is itself an fp32 number: when
    the accumulator holds -RN(3x), a fused multiply-add of 3 * x leaves
    exactly that error, where a rounded product and a separate addition
    leave 0.  The result divides by W = 1 + 3 = 4, exactly."""
    r = np.random.default_rng(5)
    x = (1.0 + r.random(64)).astype(np.float32)
    rn3x = (np.float32(3.0) * x).astype(np.float32)          # numpy: one IEEE rounding
    err = 3.0 * x.astype(np.float64) - rn3x.astype(np.float64)  # exact in float64
    assert (err != 0).sum() > 32
    got = oracle.mirror_f32([-rn3x, x], [1, 3])
    assert np.array_equal(got, (err / 4.0).astype(np.float32))


# ---------------------------------------------------------------- sparse fp32 mirror

def _sparse_lists(r, N, K, p):
    idx = [np.flatnonzero(r.random(N) < p).astype(np.int64) for _ in range(K)]
    val = [(r.standard_normal(i.size) * 10.0 ** r.integers(-4, 1)).astype(np.float32) for i in idx]
    return idx, val


def _dense_of(idx, val, N):
    xs, sent = [], []
    for i, v in zip(idx, val):
        x = np.zeros(N, np.float32)
        s_ = np.zeros(N, np.uint8)
        x[i] = v
        s_[i] = 1
        xs.append(x)
        sent.append(s_)
    return xs, sent


@pytest.mark.parametrize("mode", [oracle.WEIGHTS, oracle.DELTAS, oracle.DELTAS_ZERO_FILL])
def test_sparse_mirror_equals_float32_arithmetic_for_power_of_two_weights(mode):
    """Power-of-two weights make every product exact, so numpy's float32
    additions in client order give the same bits; counts and weight sums are
    bincounts of the lists."""
    r = np.random.default_rng(120 + mode)
    N, K = 6000, 9
    idx, val = _sparse_lists(r, N, K, 0.3)
    n = [int(2 ** r.integers(0, 12)) for _ in range(K)]
    n[4] = 0
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    out, cnt, ws = oracle.sparse_mirror_f32(idx, val, n, 0, N, mode=mode, base=base)
    xs, sent = _dense_of(idx, val, N)
    want = _np_f32_sequence(xs, n, sent, mode, base, sum(v for v in n if v > 0))
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32))
    live = [k for k in range(K) if n[k] > 0]
    assert np.array_equal(cnt, np.bincount(np.concatenate([idx[k] for k in live]), minlength=N))
    wb = np.bincount(np.concatenate([idx[k] for k in live]),
                     weights=np.concatenate([np.full(idx[k].size, float(n[k])) for k in live]), minlength=N)
    assert np.array_equal(ws, wb.astype(np.uint64))


def test_sparse_mirror_follows_client_order_and_fuses_products():
    one, tiny = np.float32(1.0), np.float32(2.0 ** -24)
    i0 = np.array([3], np.int64)
    base = np.zeros(5, np.float32)
    a, _, _ = oracle.sparse_mirror_f32([i0] * 3, [np.float32([one]), np.float32([tiny]), np.float32([tiny])],
                                       [1, 1, 1], 0, 5, mode=oracle.WEIGHTS, base=base)
    b, _, _ = oracle.sparse_mirror_f32([i0] * 3, [np.float32([tiny]), np.float32([tiny]), np.float32([one])],
                                       [1, 1, 1], 0, 5, mode=oracle.WEIGHTS, base=base)
    assert a[3] == np.float32(1.0) / np.float32(3.0)
    assert b[3] == np.float32(1.0 + 2.0 ** -23) / np.float32(3.0)
    # fused: -RN(3x) then 3 * x leaves the product's exact rounding error
    r = np.random.default_rng(6)
    x = (1.0 + r.random(40)).astype(np.float32)
    rn3x = (np.float32(3.0) * x).astype(np.float32)
    err = 3.0 * x.astype(np.float64) - rn3x.astype(np.float64)
    ii = np.arange(40, dtype=np.int64)
    got, _, _ = oracle.sparse_mirror_f32([ii, ii], [-rn3x, x], [1, 3], 0, 40, mode=oracle.WEIGHTS,
                                         base=np.zeros(40, np.float32))
    assert np.array_equal(got, (err / 4.0).astype(np.float32))


def test_sparse_mirror_within_tolerance_of_the_definition_and_windows_agree():
    """General weights: within the fp32 tolerance of the fp64 sparse
    definition, unsent parameters a bit copy of base; a window computed
    alone equals the same slice of the whole range, bit for bit."""
    from parity import check
    r = np.random.default_rng(130)
    N, K = 20_000, 12
    idx, val = _sparse_lists(r, N, K, 0.15)
    n = synth.sample_counts(130, K, 100, 1000)
    base = (r.standard_normal(N) * 0.02).astype(np.float32)
    for mode in (oracle.WEIGHTS, oracle.DELTAS, oracle.DELTAS_ZERO_FILL):
        out, cnt, ws = oracle.sparse_mirror_f32(idx, val, n, 0, N, mode=mode, base=base)
        ref, mag, c64, w64 = oracle.sparse_average(idx, val, n, N, mode=mode, base=base)
        check(out, ref, mag, "f32", copied=c64 == 0, copy_expect=base)
        assert np.array_equal(cnt, c64) and np.array_equal(ws, w64)
        lo, hi = 3_333, 15_001
        wi = [i[(i >= lo) & (i < hi)] for i in idx]
        wv = [v[(i >= lo) & (i < hi)] for i, v in zip(idx, val)]
        # zero fill divides by every client's weight, also one with no entry in the window
        o2, c2, w2 = oracle.sparse_mirror_f32(wi, wv, n, lo, hi - lo, mode=mode, base=base[lo:hi])
        assert np.array_equal(o2.view(np.uint32), out[lo:hi].view(np.uint32))
        assert np.array_equal(c2, cnt[lo:hi]) and np.array_equal(w2, ws[lo:hi])


def test_sparse_mirror_rejects_entries_outside_the_window_or_unsorted():
    base = np.zeros(10, np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.sparse_mirror_f32([np.array([2, 12], np.int64)], [np.ones(2, np.float32)], [1], 5, 10,
                                 base=base)
    with pytest.raises(oracle.OracleError):
        oracle.sparse_mirror_f32([np.array([7, 6], np.int64)], [np.ones(2, np.float32)], [1], 5, 10,
                                 base=base)
