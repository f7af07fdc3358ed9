"""fp64 NumPy oracle of the DFlash draft-block hot path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module.

Everything is computed in float64 from the exact values of the (bf16 or
float32) inputs; no intermediate is rounded to a narrower type.

Sources (page title, section):
  [K-ARCH]  kongchang.com, "D-Flash: diffusion drafting speeds LLM inference
            3.5x", section "System architecture".
  [K-INJ]   same page, "Innovation 2: target-feature KV injection".
  [K-PAR]   same page, "Innovation 1: block-diffusion parallel drafting".
  [K-ANCH]  same page, "Innovation 3: random anchor sampling".
  [G-DUAL]  Google Developers Blog (zh translation, aihot.virxact.com),
            "Dual cache for attention".
  [G-CTX]   same post, "Smart context management".
  [G-META]  same post, "Bridging the metadata gap in TPU inference".
  [G-AR]    same post, "Overcoming the autoregressive bottleneck".
  [G-BENCH] same post, table 2 caption (greedy decoding).

Readings where the pages are silent:
  * block row i sits at position ctx_len + i; its argmax is the draft for
    position ctx_len + 1 + i, so all K rows are drafts and the acceptance
    length is in [1, K + 1];
  * no bias anywhere, no norm after the context projection, no norm on the
    context feature before the K/V projections, which are the draft layer's
    own W_k and W_v;
  * RoPE in rotate-half form (pairs m and m + d/2), angle p * theta^(-2m/d);
  * attention scale 1/sqrt(d), query head h reads KV head h // (nq / nkv);
  * no mask inside the block and none between block and context;
  * RMSNorm(x) = x / sqrt(mean(x^2) + eps) times a per-channel gain, before
    attention, before the MLP and before the LM head;
  * SwiGLU MLP: W_down (silu(W_gate w) * (W_up w)), silu(t) = t / (1 + e^-t);
  * argmax ties go to the lowest index;
  * the context capacity is a power of two, grown to the next power of two of
    the new length only when an append would overflow it.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# exact upcast of stored values
# --------------------------------------------------------------------------
def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored tensor (bf16 bits or float32)."""
    if dtype == "bf16":
        a = np.asarray(a, dtype=np.uint16)
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


class Model:
    """Drafter weights, upcast to float64 on demand.

    ``keep`` keeps every upcast copy (small shapes); otherwise the vocabulary
    tables (embedding, LM head) are upcast again at each use so that at most
    one of them is held in float64 at a time.
    """

    def __init__(self, shape, weights: Dict[str, np.ndarray], keep: Optional[bool] = None):
        self.shape = shape
        self.w = weights
        if keep is None:
            keep = shape.vocab * shape.hidden <= (1 << 24)
        self.keep = keep
        self._cache: Dict[str, np.ndarray] = {}

    def f64(self, name: str) -> np.ndarray:
        if name in self._cache:
            return self._cache[name]
        v = to_f64(self.w[name], self.shape.dtype)
        if self.keep or name not in ("embed", "lm_head"):
            self._cache[name] = v
        return v

    def embed_rows(self, ids: np.ndarray) -> np.ndarray:
        return to_f64(self.w["embed"][np.asarray(ids, dtype=np.int64)], self.shape.dtype)


# --------------------------------------------------------------------------
# elementary steps
# --------------------------------------------------------------------------
def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis with a per-channel gain [K-ARCH]."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gain


def rope(v: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE.  ``v``: [n, heads, d]; ``pos``: [n] integer positions.

    Channel pair (m, m + d/2) is rotated by the angle pos * theta^(-2m/d).
    The pages name a RoPE offset kept in sync with the accepted length
    [G-META]; the rotate-half form is the reading taken here.
    """
    d = v.shape[-1]
    half = d // 2
    m = np.arange(half, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * m / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = v[..., :half]
    x2 = v[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(t: np.ndarray) -> np.ndarray:
    return t / (1.0 + np.exp(-t))


def next_pow2(n: int) -> int:
    c = 1
    while c < n:
        c <<= 1
    return c


# --------------------------------------------------------------------------
# per-sequence proposer state
# --------------------------------------------------------------------------
@dataclasses.dataclass
class SeqState:
    """State that persists across steps for one sequence [G-META]: the
    context buffer, the positions held in the KV caches, and their count.

    ``cap`` is the power-of-two capacity of the static buffers [G-CTX];
    ``cap == 0`` means nothing has been appended yet.
    """
    ctx_len: int = 0
    cap: int = 0
    pos: Optional[np.ndarray] = None         # [ctx_len] int64
    ctx: Optional[np.ndarray] = None         # [ctx_len, H] projected features
    k: Optional[List[np.ndarray]] = None     # per layer [ctx_len, nkv, d], RoPE applied
    v: Optional[List[np.ndarray]] = None     # per layer [ctx_len, nkv, d]
    grow_events: int = 0
    store: dict = dataclasses.field(default_factory=dict, repr=False)   # backing arrays


def new_state(model: Model) -> SeqState:
    s = model.shape
    return SeqState(ctx_len=0, cap=0, pos=np.zeros(0, np.int64),
                    ctx=np.zeros((0, s.hidden)),
                    k=[np.zeros((0, s.n_kv_heads, s.head_dim)) for _ in range(s.n_layers)],
                    v=[np.zeros((0, s.n_kv_heads, s.head_dim)) for _ in range(s.n_layers)])


def _append_rows(state: SeqState, key, cur: np.ndarray, new: np.ndarray) -> np.ndarray:
    """``cur`` with the rows ``new`` appended, as a view of the first rows of
    a backing array kept in ``state`` that grows by a quarter when full, so
    that a long session of small appends copies each row a bounded number
    of times (storage only: the values are those of a concatenation).  An
    array that is not the view handed out last (a test replaced it) starts a
    new backing array."""
    n0, n1 = cur.shape[0], cur.shape[0] + new.shape[0]
    back = state.store.get(key)
    if (back is None or cur.base is not back or cur.shape[1:] != back.shape[1:]
            or cur.__array_interface__["data"][0] != back.__array_interface__["data"][0]
            or n1 > back.shape[0]):
        cap = n1 + max(64, n1 // 4)
        nb = np.empty((cap,) + tuple(cur.shape[1:]), dtype=np.result_type(cur, new))
        nb[:n0] = cur
        back = nb
        state.store[key] = back
    back[n0:n1] = new
    return back[:n1]


def grow_rule(ctx_len: int, cap: int, n_new: int) -> int:
    """New capacity after appending n_new rows: unchanged while it fits,
    otherwise the next power of two of the new length [G-CTX]."""
    need = ctx_len + n_new
    if need <= cap:
        return cap
    return next_pow2(need)


# --------------------------------------------------------------------------
# (a1)-(a3): context projection, append, KV injection
# --------------------------------------------------------------------------
def project_ctx(model: Model, state: SeqState, feats: np.ndarray,
                positions: Optional[Sequence[int]] = None) -> None:
    """Append newly accepted positions to one sequence's context.

    c_j = W_fc [h^1_j || ... || h^n_j] projects the concatenated target
    hidden states to hidden size [K-ARCH]; only the new positions are
    projected and appended, each exactly once [G-CTX].  For every draft
    layer, K_j = RoPE(W_k c_j, pos_j) and V_j = W_v c_j are stored in that
    layer's static KV cache for reuse at every step [K-INJ], [G-DUAL].
    ``positions`` defaults to ctx_len + j.
    """
    s = model.shape
    f = to_f64(feats, s.dtype) if feats.dtype != np.float64 else feats
    n_new = f.shape[0]
    if n_new == 0:
        return
    assert f.shape[1] == s.n_feat * s.hidden
    if positions is None:
        pos = np.arange(state.ctx_len, state.ctx_len + n_new, dtype=np.int64)
    else:
        pos = np.asarray(positions, dtype=np.int64)
        assert pos.shape == (n_new,)
    c = f @ model.f64("fc").T                                  # [n_new, H]
    for l in range(s.n_layers):
        p = f"layers.{l}."
        kk = (c @ model.f64(p + "wk").T).reshape(n_new, s.n_kv_heads, s.head_dim)
        vv = (c @ model.f64(p + "wv").T).reshape(n_new, s.n_kv_heads, s.head_dim)
        state.k[l] = _append_rows(state, ("k", l), state.k[l], rope(kk, pos, s.rope_theta))
        state.v[l] = _append_rows(state, ("v", l), state.v[l], vv)
    state.ctx = _append_rows(state, "ctx", state.ctx, c)
    state.pos = _append_rows(state, "pos", state.pos, pos)
    new_cap = grow_rule(state.ctx_len, state.cap, n_new)
    if new_cap != state.cap:
        state.grow_events += 1
    state.cap = new_cap
    state.ctx_len += n_new


# --------------------------------------------------------------------------
# (a4)-(a9): one draft block
# --------------------------------------------------------------------------
@dataclasses.dataclass
class DraftOut:
    draft: np.ndarray      # [B, K] int64
    logits: np.ndarray     # [B, K, V]
    hidden: np.ndarray     # [B, K, H] final-normed hidden states


def _attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, nq: int, nkv: int,
               capture: Optional[dict] = None) -> np.ndarray:
    """Bidirectional GQA attention of the block queries over every key given.

    q: [K, nq, d]; keys, vals: [n, nkv, d].  No mask: the block is denoised
    in one non-causal forward [K-ARCH], [G-DUAL].
    """
    Kq, _, d = q.shape
    rep = nq // nkv
    out = np.empty((Kq, nq, d))
    probs = [] if capture is not None else None
    for h in range(nq):
        g = h // rep
        sc = (q[:, h, :] @ keys[:, g, :].T) / np.sqrt(d)        # [K, n]
        sc = sc - sc.max(axis=1, keepdims=True)
        p = np.exp(sc)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vals[:, g, :]
        if probs is not None:
            probs.append(p)
    if capture is not None:
        capture.setdefault("attn_probs", []).append(np.stack(probs, axis=1))  # [K, nq, n]
    return out


def draft_one(model: Model, state: SeqState, ids: np.ndarray,
              block_pos: Optional[np.ndarray] = None,
              capture: Optional[dict] = None):
    """Draft block of one sequence.  Returns (draft [K], logits [K,V], z [K,H]).

    The block is the clean anchor followed by mask tokens [K-ARCH], [K-ANCH];
    all rows go through the draft layers together in one forward [K-PAR].
    Each layer: RMSNorm, Q/K/V projections with RoPE at the block positions,
    attention over [context KV || block KV] with no mask, output projection
    and residual, RMSNorm, SwiGLU MLP and residual [K-ARCH], [K-INJ].  The
    final RMSNorm is followed by the LM head and a per-row argmax [K-ARCH],
    [G-BENCH].  ``block_pos`` overrides the positions ctx_len + i (tests).
    """
    s = model.shape
    ids = np.asarray(ids, dtype=np.int64)
    K = ids.shape[0]
    if block_pos is None:
        block_pos = np.arange(state.ctx_len, state.ctx_len + K, dtype=np.int64)
    x = model.embed_rows(ids)                                     # [K, H]
    if capture is not None:
        capture.setdefault("x", []).append(x.copy())
    for l in range(s.n_layers):
        p = f"layers.{l}."
        u = rms_norm(x, model.f64(p + "attn_norm"), s.rms_eps)
        q = (u @ model.f64(p + "wq").T).reshape(K, s.n_q_heads, s.head_dim)
        k = (u @ model.f64(p + "wk").T).reshape(K, s.n_kv_heads, s.head_dim)
        v = (u @ model.f64(p + "wv").T).reshape(K, s.n_kv_heads, s.head_dim)
        q = rope(q, block_pos, s.rope_theta)
        k = rope(k, block_pos, s.rope_theta)
        keys = np.concatenate([state.k[l], k], axis=0)
        vals = np.concatenate([state.v[l], v], axis=0)
        o = _attention(q, keys, vals, s.n_q_heads, s.n_kv_heads, capture)
        if capture is not None:
            capture.setdefault("v_block", []).append(v.copy())
            capture.setdefault("attn_out", []).append(o.copy())
        x = x + o.reshape(K, s.q_dim) @ model.f64(p + "wo").T
        w = rms_norm(x, model.f64(p + "mlp_norm"), s.rms_eps)
        a = silu(w @ model.f64(p + "w_gate").T) * (w @ model.f64(p + "w_up").T)
        x = x + a @ model.f64(p + "w_down").T
        if capture is not None:
            capture["x"].append(x.copy())
    z = rms_norm(x, model.f64("final_norm"), s.rms_eps)
    logits = z @ model.f64("lm_head").T
    draft = np.argmax(logits, axis=1)          # first (lowest) index on ties
    return draft, logits, z


def draft_block(model: Model, states: Sequence[SeqState], ids: np.ndarray) -> DraftOut:
    """Batched draft block: sequence b uses its own context (variable length)."""
    ids = np.asarray(ids)
    B, K = ids.shape
    assert len(states) == B
    s = model.shape
    draft = np.empty((B, K), np.int64)
    logits = np.empty((B, K, s.vocab))
    hidden = np.empty((B, K, s.hidden))
    for b in range(B):
        draft[b], logits[b], hidden[b] = draft_one(model, states[b], ids[b])
    return DraftOut(draft, logits, hidden)


# --------------------------------------------------------------------------
# (a10)-(a11): acceptance and state advance
# --------------------------------------------------------------------------
def accept(draft: np.ndarray, target: np.ndarray) -> np.ndarray:
    """Greedy longest-prefix acceptance [G-AR], [G-BENCH]:
    tau_b = 1 + the number of leading block positions where the draft equals
    the target's token; the extra one is the target's own token at the first
    mismatch (or after a fully accepted block)."""
    draft = np.asarray(draft)
    target = np.asarray(target)
    B, K = draft.shape
    tau = np.empty(B, np.int32)
    for b in range(B):
        n = 0
        while n < K and draft[b, n] == target[b, n]:
            n += 1
        tau[b] = 1 + n
    return tau


def check_state(state: SeqState, committed: int) -> List[str]:
    """Invariants of one sequence's proposer state; returns the violations.

    ``committed`` is the number of tokens truly accepted so far (prefill plus
    every step's acceptance length).  The state must count exactly those
    positions, never the drafts still under verification [G-META]; the
    buffer must be a power of two no smaller than what it holds, and the
    positions must be contiguous with none lost or repeated [G-CTX].
    """
    errs = []
    if state.ctx_len != committed:
        errs.append(f"ctx_len {state.ctx_len} != committed tokens {committed}")
    if state.ctx_len > 0 and (state.cap & (state.cap - 1)) != 0:
        errs.append(f"cap {state.cap} is not a power of two")
    if state.cap < state.ctx_len:
        errs.append(f"cap {state.cap} < ctx_len {state.ctx_len}")
    if state.pos is not None and len(state.pos) != state.ctx_len:
        errs.append(f"{len(state.pos)} positions stored for ctx_len {state.ctx_len}")
    if state.pos is not None and len(state.pos):
        srt = np.sort(state.pos)
        if not np.array_equal(srt, np.arange(len(srt))):
            errs.append("context positions are not exactly 0..ctx_len-1")
    return errs


# --------------------------------------------------------------------------
# session: draft -> verify (stand-in) -> accept -> project accepted -> advance
# --------------------------------------------------------------------------
@dataclasses.dataclass
class StepRecord:
    draft: np.ndarray
    target: np.ndarray
    tau: np.ndarray
    ctx_len: np.ndarray     # after the step
    cap: np.ndarray         # after the step
    write_start: np.ndarray  # first context row written by the step
    logits: Optional[np.ndarray] = None
    hidden: Optional[np.ndarray] = None
    block_ids: Optional[np.ndarray] = None


class Session:
    """Speculative steps over a synthetic workload (``synth.Workload``).

    Each step [G-META], [K-ANCH]: the block is [anchor, masks]; the draft
    block gives K drafts; the stand-in verifier gives the target's tokens;
    tau = accept(...); the tau newly committed positions (the anchor and the
    tau - 1 accepted drafts) are projected into the context; the next anchor
    (the target's own token after the accepted prefix, at position ctx_len)
    is the verifier's independent draw ``bonus``, so that it never depends
    on the drafted tokens.

    ``draft=False`` skips the forward and accepts a dummy draft: tau depends
    only on the verifier's agreement draws, so the state advances exactly as
    with the real draft (used to advance long sessions cheaply).

    ``n_new_override`` replaces tau as the appended count (used by a test
    that reproduces the "sequence-length inflation" mistake).
    """

    def __init__(self, model: Model, wl, keep_outputs: bool = False,
                 seqs: Optional[Sequence[int]] = None):
        import synth
        self.synth = synth
        self.model = model
        self.wl = wl
        self.seqs = list(range(wl.batch)) if seqs is None else list(seqs)
        self.states = [new_state(model) for _ in self.seqs]
        self.committed = [0] * len(self.seqs)
        self.keep_outputs = keep_outputs
        self.step_idx = 0
        s = model.shape
        self.anchor = []
        for i, b in enumerate(self.seqs):
            n0 = wl.ctx0[b]
            project_ctx(model, self.states[i], synth.prefill_features(s, wl.seed, b, n0))
            self.committed[i] = n0
            self.anchor.append(synth.first_anchor(wl.seed, b, s.vocab))

    def block(self, i: int, K: Optional[int] = None) -> np.ndarray:
        K = self.wl.K if K is None else K
        b = self.seqs[i]
        ids = self.synth.block_ids(self.wl.seed, b, self.step_idx, K, self.model.shape.vocab)
        ids = ids.copy()
        ids[0] = self.anchor[i]
        return ids

    def step(self, n_new_override: Optional[int] = None, draft: bool = True) -> StepRecord:
        s, wl, syn = self.model.shape, self.wl, self.synth
        K = wl.K
        ids = np.stack([self.block(i) for i in range(len(self.seqs))])
        if draft:
            out = draft_block(self.model, self.states, ids)
        else:
            out = DraftOut(np.zeros(ids.shape, np.int64), None, None)
        targets = np.empty_like(ids)
        bonus = []
        for i, b in enumerate(self.seqs):
            d = syn.verifier_draws(wl.seed, b, self.step_idx, K, s.vocab, wl.a[b], wl.gamma)
            targets[i] = syn.target_tokens(out.draft[i], d, s.vocab)
            bonus.append(d.bonus)
        tau = accept(out.draft, targets)
        write_start = np.array([st.ctx_len for st in self.states], np.int64)
        for i, b in enumerate(self.seqs):
            n_new = int(tau[i]) if n_new_override is None else int(n_new_override)
            f = syn.step_features(s, wl.seed, b, self.step_idx, n_new)
            project_ctx(self.model, self.states[i], f)
            self.committed[i] += int(tau[i])
            self.anchor[i] = bonus[i]
        self.step_idx += 1
        return StepRecord(draft=out.draft, target=targets, tau=tau,
                          ctx_len=np.array([st.ctx_len for st in self.states], np.int64),
                          cap=np.array([st.cap for st in self.states], np.int64),
                          write_start=write_start,
                          logits=out.logits if self.keep_outputs else None,
                          hidden=out.hidden if self.keep_outputs else None,
                          block_ids=ids)

    def violations(self) -> List[str]:
        errs = []
        for i, st in enumerate(self.states):
            errs += [f"seq {self.seqs[i]}: {e}" for e in check_state(st, self.committed[i])]
        return errs
