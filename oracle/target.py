"""fp64 oracle of target-side block verification (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module.  It shares no code with the HIP library; it reuses
the elementary steps of ``oracle/dflash.py`` (RMSNorm, RoPE, SwiGLU,
exact upcast), which are pinned there.

Sources (page title, section):
  [G-AR]    Google Developers Blog (zh translation, aihot.virxact.com),
            "Overcoming the autoregressive bottleneck": the target checks the
            whole draft block in one parallel forward and keeps the longest
            agreeing prefix plus its own next token.
  [G-KFLAT] same post, "K-Flat": verifying a block costs about the same at
            any block size while weight loading dominates.
  [G-DUAL]  same post, "Dual cache for attention": the target keeps its own
            (paged) cache of the committed positions, separate from the
            drafter's static cache.
  [G-META]  same post, "Bridging the metadata gap in TPU inference": state
            tracks the accepted count, never the drafts under verification.
  [K-ARCH]  kongchang.com, "D-Flash: diffusion drafting speeds LLM inference
            3.5x", "System architecture": hidden states of several target
            layers, concatenated, are the drafter's context features.

Readings where the pages are silent:
  * the target is a decoder of the same layer form as the drafter (RMSNorm,
    GQA attention with rotate-half RoPE, SwiGLU MLP, final RMSNorm, LM head)
    but causal: block row i sees the committed positions and block rows
    0..i;
  * the verified block is [anchor, d_0, ..., d_{K-1}] at positions
    ctx_len .. ctx_len + K; row i's argmax is the target's token for
    position ctx_len + 1 + i, compared with d_i (so the drafter's row i and
    the target's row i predict the same position);
  * after acceptance of tau, the first tau block rows (the anchor and the
    tau - 1 accepted drafts) are committed: their K/V stay in the cache and
    ctx_len grows by tau; the next anchor is the target's token at row
    tau - 1;
  * a tapped hidden state is the residual stream after the tapped layer
    (before any norm), taps given as layer indices; their concatenation in
    tap order is the drafter's feature row of that position.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

from oracle.dflash import Model, rms_norm, rope, silu


@dataclasses.dataclass
class TargetState:
    """Committed positions of one sequence in the target's cache [G-DUAL]."""
    ctx_len: int = 0
    k: Optional[List[np.ndarray]] = None     # per layer [ctx_len, nkv, d], RoPE applied
    v: Optional[List[np.ndarray]] = None     # per layer [ctx_len, nkv, d]


def new_target_state(model: Model) -> TargetState:
    s = model.shape
    return TargetState(0, [np.zeros((0, s.n_kv_heads, s.head_dim)) for _ in range(s.n_layers)],
                       [np.zeros((0, s.n_kv_heads, s.head_dim)) for _ in range(s.n_layers)])


@dataclasses.dataclass
class VerifyOut:
    target: np.ndarray        # [K1] int64: the target's token for position ctx_len + 1 + i
    logits: np.ndarray        # [K1, V]
    taps: np.ndarray          # [K1, n_taps * H] residual after each tapped layer
    k_new: List[np.ndarray]   # per layer [K1, nkv, d] (RoPE applied), not yet committed
    v_new: List[np.ndarray]


def _causal_attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, n_ctx: int, nq: int,
                      nkv: int) -> np.ndarray:
    """Causal GQA attention: q [K1, nq, d]; keys, vals [n_ctx + K1, nkv, d].
    Block row i sees keys 0 .. n_ctx + i; q head h reads KV head h // (nq/nkv)."""
    K1, _, d = q.shape
    rep = nq // nkv
    n = keys.shape[0]
    visible = np.arange(n)[None, :] <= (n_ctx + np.arange(K1))[:, None]     # [K1, n]
    out = np.empty((K1, nq, d))
    for h in range(nq):
        g = h // rep
        sc = (q[:, h, :] @ keys[:, g, :].T) / np.sqrt(d)
        sc = np.where(visible, sc, -np.inf)
        sc = sc - sc.max(axis=1, keepdims=True)
        p = np.exp(sc)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vals[:, g, :]
    return out


def verify(model: Model, state: TargetState, ids: np.ndarray, taps: Sequence[int] = ()) -> VerifyOut:
    """One target forward over the block ``ids`` [K1] at positions
    ctx_len .. ctx_len + K1 - 1, attending to the committed cache and
    causally within the block [G-AR]; the cache is not changed."""
    s = model.shape
    ids = np.asarray(ids, dtype=np.int64)
    K1 = ids.shape[0]
    pos = np.arange(state.ctx_len, state.ctx_len + K1, dtype=np.int64)
    x = model.embed_rows(ids)
    tapped = {}
    k_new, v_new = [], []
    for l in range(s.n_layers):
        p = f"layers.{l}."
        u = rms_norm(x, model.f64(p + "attn_norm"), s.rms_eps)
        q = rope((u @ model.f64(p + "wq").T).reshape(K1, s.n_q_heads, s.head_dim), pos, s.rope_theta)
        k = rope((u @ model.f64(p + "wk").T).reshape(K1, s.n_kv_heads, s.head_dim), pos, s.rope_theta)
        v = (u @ model.f64(p + "wv").T).reshape(K1, s.n_kv_heads, s.head_dim)
        k_new.append(k)
        v_new.append(v)
        keys = np.concatenate([state.k[l], k], axis=0)
        vals = np.concatenate([state.v[l], v], axis=0)
        o = _causal_attention(q, keys, vals, state.ctx_len, s.n_q_heads, s.n_kv_heads)
        x = x + o.reshape(K1, s.q_dim) @ model.f64(p + "wo").T
        w = rms_norm(x, model.f64(p + "mlp_norm"), s.rms_eps)
        x = x + (silu(w @ model.f64(p + "w_gate").T) * (w @ model.f64(p + "w_up").T)) @ model.f64(p + "w_down").T
        if l in taps:
            tapped[l] = x.copy()
    z = rms_norm(x, model.f64("final_norm"), s.rms_eps)
    logits = z @ model.f64("lm_head").T
    tap_rows = (np.concatenate([tapped[l] for l in taps], axis=1) if len(taps)
                else np.zeros((K1, 0)))
    return VerifyOut(np.argmax(logits, axis=1), logits, tap_rows, k_new, v_new)


def commit(state: TargetState, out: VerifyOut, n: int) -> None:
    """Keep the first n verified rows (the anchor and the n - 1 accepted
    drafts) in the cache; ctx_len grows by n [G-META]."""
    assert 0 <= n <= out.target.shape[0]
    for l in range(len(state.k)):
        state.k[l] = np.concatenate([state.k[l], out.k_new[l][:n]], axis=0)
        state.v[l] = np.concatenate([state.v[l], out.v_new[l][:n]], axis=0)
    state.ctx_len += n


def forward_full(model: Model, ids: np.ndarray, taps: Sequence[int] = ()) -> VerifyOut:
    """The causal forward of a whole sequence from an empty cache."""
    return verify(model, new_target_state(model), ids, taps)
