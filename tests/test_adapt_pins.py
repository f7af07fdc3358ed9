"""Pins of the adaptive block-size oracle (oracle/adapt.py): closed-form and
enumerated expected acceptance, recovery of known (a, gamma), forgetting,
and the choice rule (kongchang.com "D-Flash", "Ablations" and
"Limitations"; Google Developers Blog, "Scaling theory", "Predictability")."""
import itertools

import numpy as np
import pytest

from oracle import adapt as OA


def _enumerated_tau(K, a, g):
    """E[tau] by enumerating all 2^K agreement patterns."""
    p = [a * g ** i for i in range(K)]
    e = 0.0
    for pat in itertools.product((0, 1), repeat=K):
        pr = 1.0
        for i, bit in enumerate(pat):
            pr *= p[i] if bit else 1.0 - p[i]
        n = 0
        while n < K and pat[n]:
            n += 1
        e += pr * (1 + n)
    return e


@pytest.mark.parametrize("K,a,g", [(1, 0.7, 0.9), (5, 0.9, 0.97), (8, 0.6, 0.8), (10, 1.0, 0.5)])
def test_expected_tau_matches_enumeration(K, a, g):
    assert abs(OA.expected_tau(K, a, g) - _enumerated_tau(K, a, g)) < 1e-12


def test_expected_tau_published_values():
    """Values of the agreement model at a = 0.9, gamma = 0.97 (also pinned
    for the drafter's synthetic verifier)."""
    assert OA.expected_tau(16, 0.9, 0.97) == pytest.approx(5.4710, abs=5e-5)
    assert OA.expected_tau(8, 0.9, 0.97) == pytest.approx(5.1053, abs=5e-5)
    assert OA.expected_tau(10, 0.9, 0.97) == pytest.approx(5.3232, abs=5e-5)
    assert OA.expected_tau(64, 0.9, 0.97) == pytest.approx(5.4765, abs=5e-5)


def test_observe_counts():
    s = OA.AdaptStats(8, decay=1.0)
    s.observe(4, 5)          # all 4 positions agreed
    s.observe(4, 1)          # position 0 reached, disagreed
    s.observe(6, 3)          # positions 0, 1 agreed; 2 reached, disagreed
    assert s.reached.tolist() == [3, 2, 2, 1, 0, 0, 0, 0]
    assert s.agreed.tolist() == [2, 2, 1, 1, 0, 0, 0, 0]


def test_estimate_is_exact_on_expected_counts():
    """Counts equal to their expectations over 1e9 steps give back (a, gamma)."""
    a, g, K = 0.83, 0.91, 16
    s = OA.AdaptStats(K, decay=1.0)
    reach = 1e9
    for i in range(K):
        p = a * g ** i
        s.reached[i] = reach
        s.agreed[i] = reach * p
        reach *= p
    ea, eg = s.estimate()
    assert abs(ea - a) < 1e-6 and abs(eg - g) < 1e-6


def test_estimate_recovers_a_and_gamma_from_sampled_steps():
    rng = np.random.default_rng(0)
    a, g, K = 0.85, 0.93, 16
    s = OA.AdaptStats(K, decay=1.0)
    p = a * g ** np.arange(K)
    for _ in range(20000):
        agree = rng.random(K) < p
        n = int(np.argmin(agree)) if not agree.all() else K
        s.observe(K, n + 1)
    ea, eg = s.estimate()
    assert abs(ea - a) < 0.01 and abs(eg - g) < 0.01


def test_forgetting_tracks_a_change_of_regime():
    rng = np.random.default_rng(1)
    K, g = 16, 0.95
    fast, slow = OA.AdaptStats(K, decay=0.99), OA.AdaptStats(K, decay=1.0)
    for a in (0.95, 0.5):
        p = a * g ** np.arange(K)
        for _ in range(3000):
            agree = rng.random(K) < p
            tau = (int(np.argmin(agree)) if not agree.all() else K) + 1
            fast.observe(K, tau)
            slow.observe(K, tau)
    assert abs(fast.estimate()[0] - 0.5) < 0.05
    assert fast.estimate()[0] < slow.estimate()[0]


def test_prior_until_enough_data():
    s = OA.AdaptStats(8, decay=1.0, prior=(0.7, 0.9))
    assert s.estimate() == (0.7, 0.9)
    s.observe(8, 1)
    assert s.estimate() == (0.7, 0.9)


def test_choice_rule():
    Ks = [4, 8, 16, 32]
    # flat cost: the largest block (E[tau] grows with K)
    assert OA.choose(Ks, [1, 1, 1, 1], 0.9, 0.97)[0] == 32
    # hand-computed: a = gamma = 1 gives E = K + 1
    assert OA.choose([4, 16], [1.0, 2.0], 1.0, 1.0) == (16, 8.5)
    # a = 0.5, gamma = 1: E(4) = 1.9375, E(16) < 2: the cheaper block wins
    assert OA.choose([4, 16], [1.0, 2.0], 0.5, 1.0)[0] == 4
    # scaling every cost leaves the choice unchanged
    c = [1.0, 1.1, 1.3, 1.9]
    for a, g in ((0.9, 0.97), (0.6, 0.9), (0.99, 0.99)):
        assert OA.choose(Ks, c, a, g)[0] == OA.choose(Ks, [7.0 * x for x in c], a, g)[0]
    # ties go to the smaller K
    assert OA.choose([4, 8], [5.0, 9.0], 1.0, 1.0)[0] == 4
