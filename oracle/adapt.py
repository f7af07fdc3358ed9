"""Oracle of the adaptive block-size policy (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module.  It shares no code with the library.

Sources (page title, section):
  [K-ABL]   kongchang.com, "D-Flash: diffusion drafting speeds LLM inference
            3.5x", "Ablations": a drafter trained on a large block works at
            smaller blocks at inference, so the block size can be lowered
            with the load to control verification cost; "Limitations":
            adaptive block-size scheduling is not yet built.
  [G-SCALE] Google Developers Blog (zh translation, aihot.virxact.com),
            "Scaling theory": a per-position acceptance probability a with
            positional decay; K = 16 captures most of the attainable
            speed-up and raising a is worth more than raising K.
  [G-PRED]  same post, "Predictability": acceptance decays along the block,
            slowly for math and code, quickly for chat.

Readings where the pages are silent:
  * acceptance model: position i of a block agrees with probability
    p_i = a * gamma^i, independently; tau = 1 + the leading run of
    agreements (the extra one is the target's own token);
  * statistics: per position i, with exponential forgetting by `decay` at
    each observed step, the weighted count of steps that reached i (all
    earlier positions agreed, i < K) and of those that agreed at i;
  * estimate: weighted least squares of log p_hat_i = log a + i log gamma
    with p_hat_i = (agreed_i + 1/2) / (reached_i + 1) and weights reached_i,
    over positions with reached_i >= min_count; a and gamma are clamped to
    [1e-6, 1]; with fewer than two such positions the prior (a0, gamma0)
    is returned;
  * choice: among candidate block sizes the K that maximises the expected
    accepted tokens per unit cost, E[tau | K] / cost(K), where cost(K) is
    the caller's per-step cost (draft + verify latency at K); ties go to
    the smaller K.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np


def expected_tau(K: int, a: float, gamma: float) -> float:
    """E[tau] = 1 + sum_{m=1..K} prod_{i<m} a gamma^i  [G-SCALE]."""
    e, run = 1.0, 1.0
    for i in range(K):
        run *= a * gamma ** i
        e += run
    return e


class AdaptStats:
    """Per-position agreement counts with exponential forgetting."""

    def __init__(self, kmax: int, decay: float, min_count: float = 4.0,
                 prior: Tuple[float, float] = (0.8, 0.95)):
        self.kmax, self.decay, self.min_count, self.prior = kmax, decay, min_count, prior
        self.reached = np.zeros(kmax)
        self.agreed = np.zeros(kmax)

    def observe(self, K: int, tau: int) -> None:
        """One step at block size K with acceptance length tau in [1, K+1]:
        positions 0..tau-2 agreed; position tau-1 (if < K) was reached and
        disagreed; later positions were not reached."""
        assert 1 <= K <= self.kmax and 1 <= tau <= K + 1
        self.reached *= self.decay
        self.agreed *= self.decay
        n_agree = tau - 1
        last = min(tau - 1, K - 1)          # last position reached
        self.reached[:last + 1] += 1.0
        self.agreed[:n_agree] += 1.0

    def estimate(self) -> Tuple[float, float]:
        """(a, gamma) by weighted least squares on smoothed log rates."""
        idx = [i for i in range(self.kmax) if self.reached[i] >= self.min_count]
        if len(idx) < 2:
            return self.prior
        w = np.array([self.reached[i] for i in idx])
        x = np.array(idx, dtype=np.float64)
        y = np.array([math.log((self.agreed[i] + 0.5) / (self.reached[i] + 1.0)) for i in idx])
        sw, sx, sy = w.sum(), (w * x).sum(), (w * y).sum()
        sxx, sxy = (w * x * x).sum(), (w * x * y).sum()
        den = sw * sxx - sx * sx
        slope = (sw * sxy - sx * sy) / den
        icpt = (sy - slope * sx) / sw
        a = min(1.0, max(1e-6, math.exp(icpt)))
        g = min(1.0, max(1e-6, math.exp(slope)))
        return a, g


def choose(Ks: Sequence[int], cost: Sequence[float], a: float, gamma: float) -> Tuple[int, float]:
    """The candidate K maximising E[tau | K] / cost(K) (smallest on ties),
    and that ratio [K-ABL]."""
    best, best_v = None, -1.0
    for K, c in zip(Ks, cost):
        v = expected_tau(K, a, gamma) / c
        if v > best_v:
            best, best_v = K, v
    return best, best_v
