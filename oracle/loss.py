"""fp64 oracle of the loss-decay weighted cross-entropy used to train the
block drafter (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module.  It shares no code with the HIP library.

Sources (page title, section):
  [K-ANCH]  kongchang.com, "D-Flash: diffusion drafting speeds LLM inference
            3.5x", section "Innovation 3: random anchor sampling": clean tokens
            sampled at random from the response serve as the anchors of the
            mask blocks, and the tokens after each anchor are predicted in
            parallel.
  [K-DECAY] same page, "Innovation 4: loss-decay weighted training": the
            cross-entropy of the token at in-block position k is weighted by
            gamma^k, so earlier positions weigh more (an early error voids the
            rest of the block).

Readings where the pages are silent:
  * block row k (k = 0 .. K-1) predicts the response token at anchor + 1 + k
    (the same shift as the draft block: row i proposes position ctx_len+1+i)
    and carries weight gamma^k; rows past the response end are ignored;
  * the loss is the weighted mean over rows with a target,
    sum_r w_r CE_r / sum_r w_r, and 0 when no row has one;
  * CE_r = logsumexp(l_r) - l_r[t_r], computed from the exact input values.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

IGNORE = -1


def block_targets(tokens: np.ndarray, anchors: np.ndarray, K: int) -> np.ndarray:
    """[K-ANCH]: targets [len(anchors), K]; row k of the block anchored at a
    is tokens[a + 1 + k], or IGNORE past the end of the response."""
    tokens = np.asarray(tokens)
    out = np.full((len(anchors), K), IGNORE, dtype=np.int64)
    for n, a in enumerate(anchors):
        for k in range(K):
            p = int(a) + 1 + k
            if 0 <= p < len(tokens):
                out[n, k] = int(tokens[p])
    return out


def decay_weights(block: int, gamma: float) -> np.ndarray:
    """[K-DECAY]: weight gamma^k of in-block position k."""
    return np.power(float(gamma), np.arange(block, dtype=np.float64))


def decay_ce(logits: np.ndarray, targets: np.ndarray, block: int, gamma: float,
             want_grad: bool = True) -> Tuple[float, Optional[np.ndarray], np.ndarray]:
    """Weighted cross-entropy of rows [R, V] laid out as blocks of `block`
    rows (row r at in-block position r % block).

    Returns (loss, grad [R, V] or None, ce [R]) with
      w_r   = gamma^(r % block) for rows with a target (>= 0), else 0,
      CE_r  = logsumexp(l_r) - l_r[t_r],
      loss  = sum_r w_r CE_r / sum_r w_r   (0 if sum_r w_r = 0),
      grad  = d loss / d l = w_r / sum w * (softmax(l_r) - onehot(t_r)).
    """
    L = np.asarray(logits, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64).reshape(-1)
    R, V = L.shape
    pos = np.arange(R) % block
    valid = t >= 0
    w = np.where(valid, decay_weights(block, gamma)[pos], 0.0)
    mx = L.max(axis=1, keepdims=True) if V else np.zeros((R, 1))
    lse = (mx + np.log(np.exp(L - mx).sum(axis=1, keepdims=True))).reshape(-1)
    tl = np.where(valid, L[np.arange(R), np.where(valid, t, 0)], 0.0)
    ce = np.where(valid, lse - tl, 0.0)
    W = w.sum()
    loss = float((w * ce).sum() / W) if W > 0 else 0.0
    grad = None
    if want_grad:
        grad = np.zeros_like(L)
        if W > 0:
            p = np.exp(L - lse[:, None])
            p[np.arange(R)[valid], t[valid]] -= 1.0
            grad = p * (w / W)[:, None]
    return loss, grad, ce
