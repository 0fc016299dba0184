"""Per-round sample allocation by the measurement-based adaptive controller --
TEST INFRASTRUCTURE ONLY (see the package docstring).

The gist.science summary of the adaptive data partitioning paper, section
"The adaptive controller", gives the steps; they are followed here in its
order, in plain Python floats (IEEE binary64):

  1. measurement: at the end of round r each participant i reports its
     processing time t_i, its energy e_i and its sample count n_i;
  2. per-sample costs tau_i = t_i / n_i and eps_i = e_i / n_i, each smoothed by
     an exponential moving average;
  3. a dimensionless combined cost with user weights w_t and w_e, each term
     normalised by the median over the participants:
        c_i = w_t * tau_i / median(tau) + w_e * eps_i / median(eps);
  4. allocation: participants receive samples in inverse proportion to c_i,
     and a deadband keeps the current allocation when the change would be
     insignificant.

Readings where the page is silent (stated again in the design notes):
  * EMA: s <- alpha * x + (1 - alpha) * s, started at the first measurement;
  * median of an even number of values: the mean of the two middle ones;
  * a term whose weight is 0 is left out (its median may then be 0);
  * integer counts from the proportional targets total * (1/c_i) / sum_j 1/c_j
    by largest remainder (floors first, then one more sample to the largest
    fractional parts, ties to the lower index), so they sum to `total`; every
    participant keeps at least one sample (taken from the largest count,
    lowest index first) so its per-sample cost stays measurable;
  * deadband: the current counts are kept when no participant's new count
    differs from its current one by more than `deadband` times the current
    count.
"""

import math


def _median(v):
    s = sorted(v)
    m = len(s)
    return s[m // 2] if m % 2 else (s[m // 2 - 1] + s[m // 2]) / 2.0


def controller_step(t, e, n, total, w_time, w_energy, alpha, deadband, state=None):
    """One round.  t, e: per-participant time and energy (>= 0); n: the
    current counts (> 0); total: samples to hand out next round (>= P).
    state: None on the first round, else the (tau, eps) EMAs from the last
    call.  Returns (next counts, new state)."""
    P = len(n)
    if P < 1 or len(t) != P or len(e) != P or total < P:
        raise ValueError("bad sizes")
    if any(x <= 0 for x in n) or any(x < 0 for x in t) or any(x < 0 for x in e):
        raise ValueError("bad measurement")
    tau = [t[i] / n[i] for i in range(P)]
    eps = [e[i] / n[i] for i in range(P)]
    if state is not None:
        tau = [alpha * tau[i] + (1.0 - alpha) * state[0][i] for i in range(P)]
        eps = [alpha * eps[i] + (1.0 - alpha) * state[1][i] for i in range(P)]
    c = [0.0] * P
    if w_time != 0.0:
        mt = _median(tau)
        if mt <= 0.0:
            raise ValueError("median time cost is zero")
        for i in range(P):
            c[i] += w_time * tau[i] / mt
    if w_energy != 0.0:
        me = _median(eps)
        if me <= 0.0:
            raise ValueError("median energy cost is zero")
        for i in range(P):
            c[i] += w_energy * eps[i] / me
    if any(ci <= 0.0 for ci in c):
        raise ValueError("a combined cost is not positive")
    inv = [1.0 / ci for ci in c]
    z = 0.0
    for v in inv:
        z += v
    target = [total * (inv[i] / z) for i in range(P)]
    base = [int(math.floor(x)) for x in target]
    left = total - sum(base)
    order = sorted(range(P), key=lambda i: (-(target[i] - base[i]), i))
    for i in order[:left]:
        base[i] += 1
    for i in range(P):
        while base[i] < 1:
            j = max(range(P), key=lambda q: (base[q], -q))
            base[j] -= 1
            base[i] += 1
    keep = all(abs(base[i] - n[i]) <= deadband * n[i] for i in range(P)) and sum(n) == total
    return (list(n) if keep else base), (tau, eps)
