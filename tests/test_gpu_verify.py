"""GPU parity of target-side block verification (dflash_verify_block,
dflash_commit) against the fp64 oracle (oracle/target.py) on the same seeded
inputs.

Google Developers Blog (zh translation, aihot.virxact.com), "Overcoming the
autoregressive bottleneck", "Dual cache for attention", "Bridging the
metadata gap in TPU inference"; kongchang.com "D-Flash", "System
architecture".

Tolerances are those of the draft block: per-row relative error of the
logits and of the tapped hidden rows 2e-2 for bf16 models (fp16 attention
operands in the cache) and 1e-4 for fp32; the argmax is exact where the
oracle's top-1/top-2 margin exceeds 0.05.
"""
import numpy as np
import pytest
import torch

import block_diffusion_drafting_amd as dfl
import synth
from oracle import dflash as O
from oracle import target as OT
from tests.gpu_util import check_argmax, check_rows, d2h, say

pytestmark = pytest.mark.gpu

TINY_T = synth.Shape(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=704,
                     vocab=1024, n_feat=2, rope_theta=1e4, dtype="f32")
SMALL_T = synth.Shape(hidden=512, n_layers=3, n_q_heads=8, n_kv_heads=2, head_dim=64, intermediate=1024,
                      vocab=4096, n_feat=2, rope_theta=1e4, dtype="bf16")


def _tol(shape):
    return 2e-2 if shape.dtype == "bf16" else 1e-4


class VerifyPair:
    """A GPU target context and the oracle's per-sequence target states,
    driven in lockstep."""

    def __init__(self, shape, taps, batch, seed, gain_std=0.1, init_cap=None):
        self.shape, self.taps, self.B = shape, tuple(taps), batch
        w = synth.weights(shape, seed, gain_std=gain_std)
        self.wd = dfl.weights_to_device(w)
        self.model = dfl.Model(shape, self.wd, taps=taps)
        self.ctx = dfl.Context(self.model, batch, init_cap=init_cap)
        self.om = O.Model(shape, w)
        self.states = [OT.new_target_state(self.om) for _ in range(batch)]
        self.last = None

    def verify(self, ids):
        B, K1 = ids.shape
        d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
        tgt = torch.empty(B, K1, dtype=torch.int32, device="cuda")
        logits = torch.empty(B, K1, self.shape.vocab, dtype=torch.float32, device="cuda")
        tdt = torch.bfloat16 if self.shape.dtype == "bf16" else torch.float32
        taps = torch.empty(B, K1, len(self.taps) * self.shape.hidden, dtype=tdt, device="cuda")
        dfl.dflash_verify_block(self.ctx, d_ids, K1, tgt, logits, taps)
        torch.cuda.synchronize()
        self.last = [OT.verify(self.om, self.states[b], ids[b], self.taps) for b in range(B)]
        return tgt.cpu().numpy(), logits.cpu().numpy(), taps.float().cpu().numpy()

    def check(self, ids, name):
        tgt, logits, taps = self.verify(ids)
        t = _tol(self.shape)
        for b, o in enumerate(self.last):
            check_rows(f"{name} logits b{b}", logits[b], o.logits, t)
            if len(self.taps):
                for k in range(len(self.taps)):
                    H = self.shape.hidden
                    check_rows(f"{name} tap{k} b{b}", taps[b][:, k * H:(k + 1) * H], o.taps[:, k * H:(k + 1) * H], t)
            check_argmax(tgt[b], o.logits)
        return tgt

    def commit(self, n):
        dfl.dflash_commit(self.ctx, n)
        for b in range(self.B):
            OT.commit(self.states[b], self.last[b], int(n[b]))
        lens, caps = self.ctx.query()
        assert lens == [st.ctx_len for st in self.states]
        for c, l in zip(caps, lens):
            assert c >= l and (c & (c - 1)) == 0


def _ids(rng, B, K1, V):
    return rng.integers(0, V, size=(B, K1))


def test_verify_tiny_fp32_prefill_then_partial_commits():
    say("verify tiny fp32")
    p = VerifyPair(TINY_T, (0, 1), 1, seed=21)
    rng = np.random.default_rng(1)
    p.check(_ids(rng, 1, 37, TINY_T.vocab), "prefill")
    p.commit([37])
    for step, n in enumerate([0, 9, 1, 4, 7, 2]):
        p.check(_ids(rng, 1, 9, TINY_T.vocab), f"step{step}")
        p.commit([n])


@pytest.mark.parametrize("K1", [1, 16, 17, 40])
def test_verify_bf16_batch2_ragged_contexts(K1):
    """Two sequences with different committed lengths; capacity grows when
    the block does not fit (60 -> 64 -> 128)."""
    say(f"verify bf16 batch 2 K1={K1}")
    p = VerifyPair(SMALL_T, (0, 2), 2, seed=22)
    rng = np.random.default_rng(2)
    pre = _ids(rng, 2, 60, SMALL_T.vocab)
    p.check(pre, "prefill")
    p.commit([60, 23])
    for step in range(3):
        p.check(_ids(rng, 2, K1, SMALL_T.vocab), f"step{step}")
        p.commit([K1 if step == 0 else rng.integers(0, K1 + 1), rng.integers(0, K1 + 1)])


@pytest.mark.parametrize("stream", [False, True])
@pytest.mark.parametrize("K1", [16, 40])
def test_verify_bf16_d128_long_splits(monkeypatch, K1, stream):
    """head_dim 128 with bf16 weights (fp16 attention operands staged by
    direct loads to LDS), causal, with 1024-key splits: a 700-row prefill
    (11 chunks) and blocks over ragged contexts of several chunks each."""
    say(f"verify bf16 d128 long splits K1={K1} stream={stream}")
    monkeypatch.setenv("DFLASH_ATTN_MIN_SPLIT", "1024")
    monkeypatch.setenv("DFLASH_ATTN_STREAM_MB", "0" if stream else "1048576")
    shape = SMALL_T.replace(head_dim=128)
    p = VerifyPair(shape, (0, 2), 2, seed=26)
    rng = np.random.default_rng(6)
    p.check(_ids(rng, 2, 700, shape.vocab), "prefill")
    p.commit([700, 431])
    for step in range(2):
        p.check(_ids(rng, 2, K1, shape.vocab), f"step{step}")
        p.commit([rng.integers(0, K1 + 1), K1])


def test_verify_cache_holds_the_committed_keys():
    """After verify + commit the cache rows [0, ctx_len) are the committed
    rows' RoPE'd keys and values (fp32 model: compared to 1e-4)."""
    say("verify cache rows")
    p = VerifyPair(TINY_T.replace(n_feat=0), (), 1, seed=23)
    rng = np.random.default_rng(3)
    p.check(_ids(rng, 1, 20, TINY_T.vocab), "prefill")
    p.commit([20])
    p.check(_ids(rng, 1, 8, TINY_T.vocab), "block")
    p.commit([5])
    _, kp, vp, phys = p.ctx.buffers(0)
    s = TINY_T
    n = 25
    nb = s.n_layers * s.n_kv_heads * phys * s.head_dim * 4
    k = d2h(kp, nb).view(np.float32).reshape(s.n_layers, s.n_kv_heads, phys, s.head_dim)
    v = d2h(vp, nb).view(np.float32).reshape(s.n_layers, s.n_kv_heads, s.head_dim, phys)
    st = p.states[0]
    for l in range(s.n_layers):
        ref_k = st.k[l].transpose(1, 0, 2)                 # [nkv, n, d]
        ref_v = st.v[l].transpose(1, 2, 0)                 # [nkv, d, n]
        assert np.max(np.abs(k[l, :, :n] - ref_k)) <= 1e-4 * np.max(np.abs(ref_k))
        assert np.max(np.abs(v[l, :, :, :n] - ref_v)) <= 1e-4 * np.max(np.abs(ref_v))


def test_verify_qwen3_4b_layer_shape():
    """The Qwen3-4B target's layer and vocabulary shapes (2 of its 36
    layers): d = 128, 32 query / 8 KV heads, V = 151936, tied embedding."""
    say("verify qwen3-4b layer shape")
    shape = synth.QWEN3_4B.replace(n_layers=2, n_feat=2)
    p = VerifyPair(shape, (0, 1), 1, seed=24, gain_std=0.0)
    rng = np.random.default_rng(4)
    p.check(_ids(rng, 1, 300, shape.vocab), "prefill")
    p.commit([300])
    p.check(_ids(rng, 1, 17, shape.vocab), "block")
    p.commit([6])
    p.check(_ids(rng, 1, 17, shape.vocab), "block2")


def test_verify_and_commit_errors():
    p = VerifyPair(TINY_T, (0, 1), 1, seed=25)
    ids = torch.zeros(1, 4, dtype=torch.int32, device="cuda")
    out = torch.zeros(1, 4, dtype=torch.int32, device="cuda")
    with pytest.raises(dfl.DFlashError):
        dfl.dflash_commit(p.ctx, [1])                       # nothing verified yet
    dfl.dflash_verify_block(p.ctx, ids, 4, out)
    with pytest.raises(dfl.DFlashError):
        dfl.dflash_commit(p.ctx, [5])                       # more rows than verified
    dfl.dflash_commit(p.ctx, [4])
    with pytest.raises(dfl.DFlashError):
        dfl.dflash_commit(p.ctx, [1])                       # the verification was consumed
    with pytest.raises(dfl.DFlashError):
        dfl.dflash_draft_block(p.ctx, ids, 4, out)          # a target context does not draft
    assert p.ctx.query()[0] == [4]
