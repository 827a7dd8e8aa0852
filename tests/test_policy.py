"""Block-size policy (no GPU): the oracle's definition pinned to the distribution it models,
then the library's host function dflash_choose_gamma checked against it."""
import math

import numpy as np
import pytest

from oracle import policy as P


# ----------------------------------------------------------------------------- oracle pins

@pytest.mark.parametrize("p", [0.0, 0.3, 0.845, 0.99, 1.0])
@pytest.mark.parametrize("g", [2, 5, 16])
def test_expected_tokens_is_the_mean_of_the_accept_length(p, g):
    dist = P.tau_distribution(p, g)
    assert math.isclose(sum(dist.values()), 1.0, rel_tol=0, abs_tol=1e-12)
    mean = sum(t * q for t, q in dist.items())
    assert math.isclose(P.expected_tokens(p, g), mean, rel_tol=1e-12, abs_tol=1e-12)


def test_expected_tokens_matches_simulated_verification():
    """Simulate the run of agreeing drafts position by position (a draft is accepted only if
    every earlier one was) and compare the mean accept length with E(g)."""
    rng = np.random.default_rng(7)
    p, g, n = 0.8, 16, 200_000
    agree = rng.random((n, g - 1)) < p
    k = np.where(agree.all(axis=1), g - 1, np.argmin(agree, axis=1))      # leading agreeing drafts
    tau = k + 1
    sem = tau.std() / math.sqrt(n)
    assert abs(tau.mean() - P.expected_tokens(p, g)) < 4 * sem


def test_estimate_hand_worked():
    # cycles (3 of 16), (16 of 16: nothing rejected), (1 of 16): 17 accepted, 2 rejected positions
    assert P.estimate_accept([3, 16, 1], [16, 16, 16], 0.5, 0.0) == pytest.approx(17 / 19, abs=1e-15)
    # pseudo-counts: 4 of weight at 0.8 add 3.2 accepted and 0.8 rejected
    assert P.estimate_accept([3, 16, 1], [16, 16, 16], 0.8, 4.0) == pytest.approx((17 + 3.2) / (19 + 4), abs=1e-15)
    assert P.estimate_accept([], [], 0.7, 0.0) == 0.7


def test_estimate_maximises_the_likelihood():
    rng = np.random.default_rng(3)
    g = rng.integers(2, 17, size=40)
    t = np.minimum(rng.geometric(0.3, size=40), g)
    p0, w = 0.6, 2.0

    def loglik(p):
        ll = sum(math.log(P.tau_distribution(p, int(gi))[int(ti)]) for ti, gi in zip(t, g))
        return ll + w * p0 * math.log(p) + w * (1 - p0) * math.log(1 - p)     # Beta pseudo-counts

    ph = P.estimate_accept(t, g, p0, w)
    for q in np.linspace(0.01, 0.99, 99):
        assert loglik(ph) >= loglik(q) - 1e-9
    for d in (1e-4, -1e-4):
        assert loglik(ph) >= loglik(ph + d)


def test_estimate_recovers_the_simulated_rate():
    rng = np.random.default_rng(11)
    p, g, n = 0.85, 16, 20_000
    agree = rng.random((n, g - 1)) < p
    tau = np.where(agree.all(axis=1), g - 1, np.argmin(agree, axis=1)) + 1
    assert abs(P.estimate_accept(tau, [g] * n, 0.5, 0.0) - p) < 0.01


def test_choice_cases():
    flat = [0.0, 0.0] + [900.0] * 15
    assert P.choose_gamma([2, 3], [16, 16], flat, 2, 16, 0.8, 0.0)[0] == 16     # flat cost: the largest block
    lin = [0.0, 0.0] + [100.0 * g for g in range(2, 17)]
    # p = 0.5, cost proportional to g: E(g)/g = (2 - 2^(1-g)) / g falls with g
    assert P.choose_gamma([1, 2], [16, 16], lin, 2, 16, 0.5, 0.0)[0] == 2
    # p = 2/3, cost a + b g (a compute-bound batch): interior optimum, checked by brute force
    aff = [0.0, 0.0] + [200.0 + 100.0 * g for g in range(2, 17)]
    gbest, p = P.choose_gamma([3, 4, 2], [16, 16, 16], aff, 2, 16, 0.85, 0.0)
    rates = {g: P.expected_tokens(p, g) / aff[g] for g in range(2, 17)}
    assert gbest == max(rates, key=rates.get) and 2 < gbest < 16


# ----------------------------------------------------------------------------- the library's function

def _lib_choose(*args, **kw):
    import block_diffusion_drafter_states_amd as dfl
    return dfl.choose_gamma(*args, **kw)


def test_library_matches_oracle_on_random_histories():
    rng = np.random.default_rng(2026)
    for it in range(400):
        gmin = int(rng.integers(2, 9))
        gmax = int(rng.integers(gmin, 17))
        n = int(rng.integers(0, 30))
        g = rng.integers(2, 17, size=n)
        t = np.minimum(rng.geometric(float(rng.uniform(0.05, 0.95)), size=n), g)
        kind = it % 3
        gs = np.arange(gmax + 1)
        cost = {0: 800.0 + 3.0 * gs, 1: 300.0 + 150.0 * gs * rng.uniform(0.5, 1.5), 2: rng.uniform(100, 2000, gmax + 1)}[kind]
        cost = np.asarray(cost, dtype=np.float32)
        cost[rng.random(gmax + 1) < 0.15] = 0.0                 # some sizes not measured
        if not (cost[gmin:gmax + 1] > 0).any():
            cost[gmax] = 500.0
        p0, w = float(rng.uniform(0, 1)), float(rng.choice([0.0, 1.0, 4.0]))
        cl = [float(c) for c in cost]
        got_g, got_p = _lib_choose(list(map(int, t)), list(map(int, g)), cl, gmin, gmax, p0, w)
        ref_g, ref_p = P.choose_gamma(list(map(int, t)), list(map(int, g)), cl, gmin, gmax, p0, w)
        assert got_p == pytest.approx(ref_p, rel=0, abs=1e-12)
        if got_g != ref_g:      # only a tie within rounding may be resolved differently
            r = lambda x: P.expected_tokens(ref_p, x) / cl[x]
            assert abs(r(got_g) - r(ref_g)) <= 1e-12 * r(ref_g)


def test_library_rejects_bad_arguments():
    import block_diffusion_drafter_states_amd as dfl
    cost = [0.0, 0.0] + [500.0] * 15
    for args in [([5], [4], cost, 2, 16),          # tau > gamma
                 ([0], [4], cost, 2, 16),          # tau < 1
                 ([1], [17], cost, 2, 16),         # gamma beyond 16
                 ([1], [4], cost, 1, 16),          # gamma_min < 2
                 ([1], [4], cost, 9, 8),           # empty range
                 ([1], [4], [0.0] * 17, 2, 16)]:   # no candidate with a cost
        with pytest.raises(dfl.DFlashError):
            dfl.choose_gamma(*args)
    with pytest.raises(dfl.DFlashError):
        dfl.choose_gamma([1], [4], cost, 2, 16, prior_p=1.5)
