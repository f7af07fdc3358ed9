"""The library's adaptive block-size policy (dflash_adapt_*, host code
called through the C ABI) against oracle/adapt.py on the same observation
streams: (a, gamma) to 1e-12, the chosen K exactly wherever the best and
second-best candidates differ by more than 1e-9 in expected tokens per
cost."""
import numpy as np
import pytest

import block_diffusion_drafting_amd as dfl
from oracle import adapt as OA

KS = [4, 8, 16, 32, 64]
COST = [0.50 + 2.90, 0.52 + 3.10, 0.55 + 3.35, 0.60 + 3.80, 0.70 + 4.60]   # draft + verify ms, illustrative


def _stream(rng, phases, K_of):
    """(K, tau) pairs: agreement a * gamma^i per position, (a, gamma, steps)
    per phase, K chosen by K_of(step)."""
    t = 0
    for a, g, n in phases:
        for _ in range(n):
            K = K_of(t)
            p = a * g ** np.arange(K)
            agree = rng.random(K) < p
            yield K, (int(np.argmin(agree)) if not agree.all() else K) + 1
            t += 1


@pytest.mark.parametrize("decay", [1.0, 0.98, 0.9])
def test_policy_matches_oracle(decay):
    rng = np.random.default_rng(7)
    pol = dfl.AdaptPolicy(64, decay=decay, min_count=4.0, a0=0.8, gamma0=0.95)
    ora = OA.AdaptStats(64, decay=decay, min_count=4.0, prior=(0.8, 0.95))
    phases = [(0.95, 0.98, 150), (0.6, 0.85, 150), (0.9, 0.95, 150)]   # code-like, chat-like, mixed
    compared = 0
    for K, tau in _stream(rng, phases, lambda t: KS[(t * 7) % len(KS)]):
        pol.observe(K, tau)
        ora.observe(K, tau)
        Kc, a, g, v = pol.choose(KS, COST)
        ea, eg = ora.estimate()
        assert abs(a - ea) <= 1e-12 * max(1.0, ea) and abs(g - eg) <= 1e-12 * max(1.0, eg)
        vals = sorted((OA.expected_tau(k, ea, eg) / c for k, c in zip(KS, COST)), reverse=True)
        if vals[0] - vals[1] > 1e-9 * vals[0]:
            assert Kc == OA.choose(KS, COST, ea, eg)[0]
            assert abs(v - vals[0]) <= 1e-12 * vals[0]
            compared += 1
    assert compared > 400


def test_policy_follows_the_load():
    """A steeper cost of large blocks (heavier verification load) moves the
    choice to smaller K; with acceptance near 1 and flat cost the largest."""
    pol = dfl.AdaptPolicy(64, decay=1.0)
    for _ in range(50):
        pol.observe(16, 17)
    assert pol.choose(KS, [1.0] * 5)[0] == 64
    steep = [1.0, 1.6, 2.8, 5.5, 11.0]
    assert pol.choose(KS, steep)[0] < 64


def test_policy_argument_errors():
    with pytest.raises(dfl.DFlashError):
        dfl.AdaptPolicy(0)
    with pytest.raises(dfl.DFlashError):
        dfl.AdaptPolicy(8, decay=0.0)
    pol = dfl.AdaptPolicy(8)
    for K, tau in ((9, 1), (4, 0), (4, 6)):
        with pytest.raises(dfl.DFlashError):
            pol.observe(K, tau)
    with pytest.raises(dfl.DFlashError):
        pol.choose([8, 4], [1.0, 1.0])          # not increasing
    with pytest.raises(dfl.DFlashError):
        pol.choose([4, 8], [1.0, 0.0])          # cost must be > 0
    assert pol.choose([], [])[0] == 0
