"""Pins of the loss-decay weighted cross-entropy oracle (oracle/loss.py)
against closed forms, an independent scalar writing, finite differences and
invariants (kongchang.com "D-Flash", sections "Innovation 3: random anchor
sampling" and "Innovation 4: loss-decay weighted training")."""
import math

import numpy as np
import pytest

from oracle import loss as OL


def _brute(logits, targets, block, gamma):
    """Scalar pure-Python loss and gradient (no NumPy arithmetic)."""
    R, V = len(logits), len(logits[0])
    ws, ces = [], []
    for r in range(R):
        row = [float(x) for x in logits[r]]
        t = int(targets[r])
        if t < 0:
            ws.append(0.0)
            ces.append(0.0)
            continue
        m = max(row)
        s = 0.0
        for x in row:
            s += math.exp(x - m)
        lse = m + math.log(s)
        ws.append(gamma ** (r % block))
        ces.append(lse - row[t])
    W = sum(ws)
    loss = sum(w * c for w, c in zip(ws, ces)) / W if W > 0 else 0.0
    grad = [[0.0] * V for _ in range(R)]
    if W > 0:
        for r in range(R):
            if ws[r] == 0.0:
                continue
            row = [float(x) for x in logits[r]]
            m = max(row)
            s = sum(math.exp(x - m) for x in row)
            for v in range(V):
                p = math.exp(row[v] - m) / s
                grad[r][v] = (p - (1.0 if v == int(targets[r]) else 0.0)) * ws[r] / W
    return loss, np.array(grad)


def test_uniform_logits_give_log_vocab():
    V = 37
    L = np.zeros((12, V))
    t = np.arange(12) % V
    loss, _, ce = OL.decay_ce(L, t, block=4, gamma=0.7)
    assert np.allclose(ce, math.log(V), rtol=0, atol=1e-12)
    assert abs(loss - math.log(V)) < 1e-12


@pytest.mark.parametrize("gamma", [1.0, 0.8, 0.5])
def test_matches_scalar_brute_force(gamma):
    rng = np.random.default_rng(3)
    R, V, block = 9, 6, 3
    L = rng.normal(0, 2, size=(R, V))
    t = rng.integers(0, V, size=R)
    t[4] = OL.IGNORE
    loss, grad, _ = OL.decay_ce(L, t, block, gamma)
    bl, bg = _brute(L.tolist(), t.tolist(), block, gamma)
    assert abs(loss - bl) < 1e-12
    assert np.max(np.abs(grad - bg)) < 1e-13


def test_gradient_matches_finite_differences():
    rng = np.random.default_rng(5)
    R, V, block, gamma = 6, 5, 3, 0.6
    L = rng.normal(0, 1.5, size=(R, V))
    t = rng.integers(0, V, size=R)
    t[2] = OL.IGNORE
    _, grad, _ = OL.decay_ce(L, t, block, gamma)
    eps = 1e-6
    num = np.zeros_like(L)
    for r in range(R):
        for v in range(V):
            a = L.copy()
            b = L.copy()
            a[r, v] += eps
            b[r, v] -= eps
            num[r, v] = (OL.decay_ce(a, t, block, gamma, False)[0] - OL.decay_ce(b, t, block, gamma, False)[0]) / (2 * eps)
    assert np.max(np.abs(num - grad)) < 1e-8


def test_gradient_rows_sum_to_zero_and_ignored_rows_are_inert():
    rng = np.random.default_rng(7)
    R, V, block = 8, 11, 4
    L = rng.normal(0, 3, size=(R, V))
    t = rng.integers(0, V, size=R)
    t[[1, 6]] = OL.IGNORE
    loss, grad, _ = OL.decay_ce(L, t, block, 0.9)
    assert np.max(np.abs(grad.sum(axis=1))) < 1e-15
    assert np.all(grad[[1, 6]] == 0.0)
    L2 = L.copy()
    L2[[1, 6]] = rng.normal(0, 3, size=(2, V))
    assert OL.decay_ce(L2, t, block, 0.9)[0] == pytest.approx(loss, abs=1e-15)


def test_position_weights_decay_geometrically():
    """The same row at in-block positions 0 and k: equal CE, gradient ratio
    gamma^k (earlier positions weigh more)."""
    rng = np.random.default_rng(9)
    V, block, gamma = 13, 8, 0.75
    row = rng.normal(0, 1, size=V)
    L = np.tile(row, (block, 1))
    t = np.full(block, 4)
    _, grad, ce = OL.decay_ce(L, t, block, gamma)
    assert np.allclose(ce, ce[0], atol=1e-15)
    for k in range(1, block):
        assert np.allclose(grad[k], grad[0] * gamma ** k, rtol=1e-12, atol=1e-18)
    assert np.allclose(OL.decay_weights(block, gamma), [gamma ** k for k in range(block)])


def test_confident_prediction_has_near_zero_loss():
    V = 50
    L = np.zeros((2, V))
    L[0, 3] = 50.0
    L[1, 7] = 50.0
    loss, _, _ = OL.decay_ce(L, np.array([3, 7]), block=2, gamma=0.5)
    assert 0.0 <= loss < V * math.exp(-50) * 1.01


def test_all_rows_ignored():
    L = np.ones((4, 3))
    loss, grad, _ = OL.decay_ce(L, np.full(4, OL.IGNORE), block=2, gamma=0.9)
    assert loss == 0.0 and np.all(grad == 0.0)


def test_block_targets_follow_the_anchor():
    """Row k of the block anchored at position a predicts token a + 1 + k;
    rows past the end of the response are ignored."""
    tokens = np.arange(10, 20)
    got = OL.block_targets(tokens, np.array([0, 7, 9]), K=4)
    assert got.tolist() == [[11, 12, 13, 14], [18, 19, -1, -1], [-1, -1, -1, -1]]
