"""Seeded synthetic workloads for the DFlash draft block.

This module only draws random numbers and lays them out. It holds none of the
draft-block arithmetic (no projection, attention, norm, RoPE or acceptance):
both the fp64 oracle under ``oracle/`` and the HIP path's Python driver read
their inputs from here, and nothing else is shared between them.

Sources for the shapes and the input recipe:
  * kongchang.com, "D-Flash: diffusion drafting speeds LLM inference 3.5x",
    section "System architecture": hidden states of several target layers are
    concatenated and projected; a clean anchor token plus mask tokens form the
    block.
  * Google Developers Blog (zh translation on aihot.virxact.com), "Scaling
    theory" and "Predictability": a per-position acceptance probability that
    decays along the block.
The concrete sizes (Qwen3-4B- and Llama-3.1-8B-shaped drafters, the tiny fp32
drafter, block sizes, context lengths, a and gamma) are the benchmark
workloads this project measures; the pages give no numbers for them.

Random streams: tensor/step ``name`` with integer indices ``idx`` is drawn from
``PCG64(SeedSequence(entropy=seed, spawn_key=(crc32(name), *idx)))``.  Large
tensors are drawn in chunks of ``CHUNK`` elements, chunk ``c`` from the stream
with ``idx + (c,)``, so that generation can run on several threads and still
give the same values on any machine.

Value conventions:
  * bf16 tensors are returned as ``uint16`` arrays of raw bf16 bits, obtained
    from float32 draws by round-to-nearest-even on the bit pattern;
  * fp32 tensors are returned as ``float32`` arrays;
  * linear weights are row-major ``[out_features, in_features]``.
"""
from __future__ import annotations

import dataclasses
import math
import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

CHUNK = 1 << 22
WEIGHT_STD = 0.02


# --------------------------------------------------------------------------
# shapes and workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Shape:
    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_feat: int
    rope_theta: float
    rms_eps: float = 1e-6
    dtype: str = "bf16"          # "bf16" or "f32"
    tied: bool = False           # LM head shares the embedding table

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark/parity workload: a drafter shape plus a session recipe."""
    name: str
    shape: Shape
    batch: int
    K: int
    ctx0: Tuple[int, ...]            # initial context length per sequence
    steps: int                       # session steps used for parity
    a: Tuple[float, ...]             # per-sequence acceptance probability
    gamma: float                     # positional decay of acceptance
    seed: int
    k_sweep: Tuple[int, ...] = ()    # block sizes timed by the K sweep

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY = Shape(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64,
             intermediate=704, vocab=1024, n_feat=3, rope_theta=1e4,
             dtype="f32", tied=False)
QWEN3_4B = Shape(hidden=2560, n_layers=5, n_q_heads=32, n_kv_heads=8,
                 head_dim=128, intermediate=9728, vocab=151936, n_feat=5,
                 rope_theta=1e6, dtype="bf16", tied=True)
LLAMA31_8B = Shape(hidden=4096, n_layers=5, n_q_heads=32, n_kv_heads=8,
                   head_dim=128, intermediate=14336, vocab=128256, n_feat=5,
                   rope_theta=5e5, dtype="bf16", tied=False)


# Verification target of the Qwen3-4B shape (36 layers; the drafter's
# shape has 5), with five tapped layers spread from shallow to deep as the
# drafter's n_feat = 5 feature sources.
QWEN3_4B_TARGET = QWEN3_4B.replace(n_layers=36)
QWEN3_4B_TAPS = (1, 9, 17, 25, 33)


def _config4_ctx(seed: int, batch: int) -> Tuple[int, ...]:
    g = stream(seed, "ctx0")
    u = g.uniform(math.log(1024.0), math.log(32768.0), size=batch)
    return tuple(int(math.floor(math.exp(v))) for v in u)


def _config4_a(seed: int, batch: int) -> Tuple[float, ...]:
    g = stream(seed, "accept_a")
    return tuple(float(v) for v in g.uniform(0.6, 0.95, size=batch))


def workloads() -> List[Workload]:
    """The five workloads, indexed 0..4."""
    w0 = Workload("tiny-fp32", TINY, batch=1, K=8, ctx0=(64,), steps=8,
                  a=(0.9,), gamma=0.97, seed=1000)
    w1 = Workload("qwen3-4b-shape", QWEN3_4B, batch=1, K=16, ctx0=(2048,),
                  steps=16, a=(0.9,), gamma=0.97, seed=1001)
    w2 = Workload("llama3.1-8b-shape", LLAMA31_8B, batch=1, K=10,
                  ctx0=(4096,), steps=64, a=(0.9,), gamma=0.97, seed=1002)
    w3 = Workload("qwen3-4b-shape-ksweep", QWEN3_4B, batch=1, K=16,
                  ctx0=(4096,), steps=0, a=(0.9,), gamma=0.97, seed=1003,
                  k_sweep=(16, 32, 64, 128, 1024))
    w4 = Workload("qwen3-4b-shape-b16-longctx", QWEN3_4B, batch=16, K=16,
                  ctx0=_config4_ctx(1004, 16), steps=32,
                  a=_config4_a(1004, 16), gamma=0.95, seed=1004)
    return [w0, w1, w2, w3, w4]


def workload(i: int) -> Workload:
    return workloads()[i]


# --------------------------------------------------------------------------
# random streams
# --------------------------------------------------------------------------
def stable_hash(name: str) -> int:
    return zlib.crc32(name.encode("utf-8")) & 0xFFFFFFFF


def stream(seed: int, name: str, *idx: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed,
                                spawn_key=(stable_hash(name),) + tuple(int(i) for i in idx))
    return np.random.Generator(np.random.PCG64(ss))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return raw bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def normal(seed: int, name: str, shape: Sequence[int], std: float, dtype: str,
           mean: float = 0.0, idx: Tuple[int, ...] = ()) -> np.ndarray:
    """N(mean, std^2) tensor drawn in float32 chunks; bf16 bits or float32."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        v = stream(seed, name, *idx, c).standard_normal(hi - lo, dtype=np.float32)
        v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        out[lo:hi] = f32_to_bf16_bits(v) if dtype == "bf16" else v

    if nchunks <= 2:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(tuple(shape))


def ones(shape: Sequence[int], dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return np.full(tuple(shape), 0x3F80, dtype=np.uint16)
    return np.ones(tuple(shape), dtype=np.float32)


# --------------------------------------------------------------------------
# weights, features, block ids, verifier draws
# --------------------------------------------------------------------------
LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate",
              "w_up", "w_down")


def weights(shape: Shape, seed: int, gain_std: float = 0.0) -> Dict[str, np.ndarray]:
    """Random-init drafter weights.

    Linear maps, the embedding, the LM head and the context projection are
    N(0, 0.02^2).  Norm gains are 1.0, or 1 + N(0, gain_std^2) when
    ``gain_std`` > 0 (used by unit tests so that the gain multiply matters).
    Keys: ``embed``, ``lm_head`` (the same array object when tied), ``fc``,
    ``final_norm`` and ``layers.{l}.{attn_norm,wq,wk,wv,wo,mlp_norm,w_gate,
    w_up,w_down}``.
    """
    s, dt, H = shape, shape.dtype, shape.hidden
    w: Dict[str, np.ndarray] = {}
    w["embed"] = normal(seed, "embed", (s.vocab, H), WEIGHT_STD, dt)
    w["lm_head"] = w["embed"] if s.tied else normal(seed, "lm_head", (s.vocab, H), WEIGHT_STD, dt)
    w["fc"] = normal(seed, "fc", (H, s.n_feat * H), WEIGHT_STD, dt)

    def gain(name: str) -> np.ndarray:
        if gain_std > 0.0:
            return normal(seed, name, (H,), gain_std, dt, mean=1.0)
        return ones((H,), dt)

    w["final_norm"] = gain("final_norm")
    for l in range(s.n_layers):
        p = f"layers.{l}."
        w[p + "attn_norm"] = gain(p + "attn_norm")
        w[p + "wq"] = normal(seed, p + "wq", (s.q_dim, H), WEIGHT_STD, dt)
        w[p + "wk"] = normal(seed, p + "wk", (s.kv_dim, H), WEIGHT_STD, dt)
        w[p + "wv"] = normal(seed, p + "wv", (s.kv_dim, H), WEIGHT_STD, dt)
        w[p + "wo"] = normal(seed, p + "wo", (H, s.q_dim), WEIGHT_STD, dt)
        w[p + "mlp_norm"] = gain(p + "mlp_norm")
        w[p + "w_gate"] = normal(seed, p + "w_gate", (s.intermediate, H), WEIGHT_STD, dt)
        w[p + "w_up"] = normal(seed, p + "w_up", (s.intermediate, H), WEIGHT_STD, dt)
        w[p + "w_down"] = normal(seed, p + "w_down", (H, s.intermediate), WEIGHT_STD, dt)
    return w


def features(shape: Shape, seed: int, name: str, rows: int, *idx: int) -> np.ndarray:
    """Stand-in target hidden states: ``rows`` x (n_feat*hidden), N(0, 1)."""
    return normal(seed, "feat:" + name, (rows, shape.n_feat * shape.hidden), 1.0,
                  shape.dtype, idx=tuple(idx))


def prefill_features(shape: Shape, seed: int, b: int, rows: int) -> np.ndarray:
    return features(shape, seed, "prefill", rows, b)


def step_features(shape: Shape, seed: int, b: int, step: int, rows: int) -> np.ndarray:
    """Features of the positions accepted at ``step``: the first ``rows`` of
    K+1 possible rows, so the values do not depend on how many are taken."""
    return features(shape, seed, "step", rows, b, step)


def block_ids(seed: int, b: int, step: int, K: int, vocab: int) -> np.ndarray:
    """Row 0 stands for the anchor, rows 1..K-1 for mask tokens; all ids are
    uniform in [0, vocab) so rows are distinguishable in tests."""
    return stream(seed, "block_ids", b, step).integers(0, vocab, size=K, dtype=np.int64).astype(np.int32)


def first_anchor(seed: int, b: int, vocab: int) -> int:
    """The last verified token before the first step (uniform in [0, vocab))."""
    return int(stream(seed, "first_anchor", b).integers(0, vocab))


@dataclasses.dataclass
class VerifierDraws:
    agree: np.ndarray      # bool [K]: block position i agrees with the draft
    shift: np.ndarray      # int  [K]: offset in [0, V-2] for disagreeing tokens
    bonus: int             # the target's own token after the accepted prefix
                           # (the next anchor), independent of the draft


def verifier_draws(seed: int, b: int, step: int, K: int, vocab: int, a: float,
                   gamma: float) -> VerifierDraws:
    """Draws of the stand-in target verifier: agreement at block position i
    with probability a * gamma**i, independently per position."""
    g = stream(seed, "verify", b, step)
    u = g.random(K)
    shift = g.integers(0, max(vocab - 1, 1), size=K, dtype=np.int64)
    bonus = int(g.integers(0, vocab))
    p = a * np.power(gamma, np.arange(K, dtype=np.float64))
    return VerifierDraws(agree=u < p, shift=shift, bonus=bonus)


def target_tokens(draft: np.ndarray, d: VerifierDraws, vocab: int) -> np.ndarray:
    """The stand-in target's tokens for one sequence: equal to the draft where
    ``agree`` holds, a different token otherwise."""
    draft = np.asarray(draft, dtype=np.int64)
    other = (draft + 1 + d.shift) % vocab
    return np.where(d.agree, draft, other).astype(np.int32)



# --------------------------------------------------------------------------
# drafter-training logits (loss-decay weighted cross-entropy)
# --------------------------------------------------------------------------
def ce_inputs(seed: int, rows: int, vocab: int, block: int, dtype: str, std: float = 2.0,
              boost: Tuple[float, float] = (0.0, 12.0), cut_frac: float = 0.25,
              masked_tail: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Logits [rows, vocab] and targets [rows] int32 of drafter blocks of
    ``block`` rows (kongchang.com, "D-Flash", "Innovation 3: random anchor
    sampling"; "Innovation 4: loss-decay weighted training").

    Logits are N(0, std^2); the target's logit is then raised by a per-row
    amount uniform in ``boost`` (rows range from confident to wrong).  A
    fraction ``cut_frac`` of the blocks run past the end of their response:
    their last u rows (u uniform in [1, block]) get the target -1.  The last
    ``masked_tail`` vocabulary entries are -inf (padding of the vocabulary)
    and never targets.  bf16 logits come back as raw bits (uint16)."""
    L = normal(seed, "ce_logits", (rows, vocab), std, dtype)
    g = stream(seed, "ce_targets")
    live = vocab - masked_tail
    t = g.integers(0, live, size=rows, dtype=np.int64)
    up = g.uniform(boost[0], boost[1], size=rows).astype(np.float32)
    nblk = (rows + block - 1) // block
    cut = g.random(nblk) < cut_frac
    ulen = g.integers(1, block + 1, size=nblk)
    r = np.arange(rows)
    if dtype == "bf16":
        cur = (L[r, t].astype(np.uint32) << np.uint32(16)).view(np.float32)
        L[r, t] = f32_to_bf16_bits(cur + up)
        if masked_tail:
            L[:, live:] = 0xFF80
    else:
        L[r, t] += up
        if masked_tail:
            L[:, live:] = -np.inf
    pos = r % block
    blk = r // block
    blen = np.minimum(block, rows - blk * block)  # the last block may be short
    dead = cut[blk] & (pos >= blen - ulen[blk])
    t = np.where(dead, -1, t).astype(np.int32)
    return L, t
