"""The library's sample-allocation step (fedavg_controller_step, host code)
against the oracle's statement of the same steps: equal integer counts and
equal smoothed costs, bit for bit, over random rounds.  No device needed."""

import numpy as np
import pytest

import oracle.controller as controller
import weighted_model_update_amd as fa


def test_library_matches_oracle_over_random_rounds():
    r = np.random.default_rng(12)
    for trial in range(100):
        P = int(r.integers(1, 40))
        wt, we = float(r.choice([0.0, r.random()])), float(r.random())
        if wt == 0.0 and we == 0.0:
            we = 0.5
        ema = float(r.choice([1.0, r.random() * 0.9 + 0.05]))
        dead = float(r.choice([0.0, 0.02, 0.2]))
        lib = fa.SampleController(P, w_time=wt, w_energy=we, ema=ema, deadband=dead)
        state = None
        n = r.integers(1, 3000, P).tolist()
        total = int(sum(n))
        for rnd in range(4):
            t = (r.random(P) * 10 + 0.001).tolist()
            e = (r.random(P) * 5 + 0.001).tolist()
            want, state = controller.controller_step(t, e, n, total, wt, we, ema, dead, state)
            got = lib.step(t, e, n, total)
            assert got == want, (trial, rnd)
            tau, eps = lib.state()
            assert np.array_equal(np.array(tau), np.array(state[0]))
            assert np.array_equal(np.array(eps), np.array(state[1]))
            n = got
            if rnd == 2:
                total += int(r.integers(0, 500))


def test_library_rejects_bad_rounds():
    c = fa.SampleController(3)
    with pytest.raises(fa.FedAvgError) as e:
        c.step([1, 1, 1], [0, 0, 0], [1, 0, 1], 10)          # a participant without samples
    assert e.value.code == -1
    with pytest.raises(fa.FedAvgError) as e:
        c.step([1, 1, 1], [0, 0, 0], [1, 1, 1], 2)           # fewer samples than participants
    assert e.value.code == -3
    with pytest.raises(fa.FedAvgError) as e:
        c.step([0, 0, 0], [0, 0, 0], [1, 1, 1], 10)          # zero median time cost
    assert e.value.code == -1
    with pytest.raises(fa.FedAvgError) as e:
        fa.SampleController(2, w_time=0.0, w_energy=0.0).step([1, 1], [1, 1], [1, 1], 4)
    assert e.value.code == -1
