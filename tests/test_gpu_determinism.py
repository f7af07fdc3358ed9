"""Run-to-run determinism of the draft path: the same inputs give the same
bits.  Every reduction in the kernels has a fixed order (the waves' sums
through LDS in wave order, split-K partials added split 0 first whichever
split finishes last, attention splits merged in split order, argmax keys
combined with an order-free max), so two draft blocks over the same
context, and two contexts built by the same calls, agree bit for bit:
draft ids, logits, final hidden rows, and the context buffers and caches.

Cases: one m-tile (output projection over the whole reduction, down split
with the last split adding the partials), two m-tiles (both projections
split that way), five m-tiles (split products and the residual pass), and
the single-launch block.
"""
import numpy as np
import pytest
import torch

import block_diffusion_drafting_amd as dfl
import synth
from tests.gpu_util import d2h, say, to_dev

pytestmark = pytest.mark.gpu

SMALL = synth.Shape(hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                    intermediate=1408, vocab=4003, n_feat=3, rope_theta=1e6, dtype="bf16")
SEED = 91
REPEATS = 3


def _ctx(model, lens):
    c = dfl.Context(model, len(lens))
    feats = [synth.prefill_features(SMALL, SEED, b, n) for b, n in enumerate(lens)]
    dfl.dflash_project_ctx(c, to_dev(np.concatenate(feats, axis=0)), lens)
    return c


def _step(c, K, step):
    """dflash_step: append 3 positions per sequence, draft K; returns raw bytes."""
    B, s = c.batch, SMALL
    feats = np.concatenate([synth.prefill_features(s, SEED + 1 + step, b, 3) for b in range(B)], axis=0)
    ids = np.stack([synth.block_ids(SEED, b, step, K, s.vocab) for b in range(B)]).astype(np.int32)
    dr = torch.empty(B, K, dtype=torch.int32, device="cuda")
    lg = torch.empty(B, K, s.vocab, dtype=torch.float32, device="cuda")
    hd = torch.empty(B, K, s.hidden, dtype=torch.uint16, device="cuda")
    dfl.dflash_step(c, to_dev(feats), [3] * B, to_dev(ids), K, dr, lg, hd)
    torch.cuda.synchronize()
    return ids, _raw(dr, lg, hd)


def _draft(c, ids, K):
    B, s = c.batch, SMALL
    dr = torch.empty(B, K, dtype=torch.int32, device="cuda")
    lg = torch.empty(B, K, s.vocab, dtype=torch.float32, device="cuda")
    hd = torch.empty(B, K, s.hidden, dtype=torch.uint16, device="cuda")
    dfl.dflash_draft_block(c, to_dev(ids), K, dr, lg, hd)
    torch.cuda.synchronize()
    return _raw(dr, lg, hd)


def _raw(dr, lg, hd):
    return {"draft": dr.cpu().numpy().copy(), "logits": lg.cpu().numpy().view(np.uint32).copy(),
            "hidden": hd.cpu().numpy().copy()}


def _state(c):
    """Raw bytes of every sequence's valid context rows and cache rows."""
    s = SMALL
    lens, _ = c.query()
    out = []
    for b, n in enumerate(lens):
        cptr, kptr, vptr, phys = c.buffers(b)
        es = s.elem_bytes
        L, nkv, d = s.n_layers, s.n_kv_heads, s.head_dim
        ctxb = d2h(cptr, n * s.hidden * 4)
        k = d2h(kptr, L * nkv * phys * d * es).reshape(L, nkv, phys, d * es)[:, :, :n]
        v = d2h(vptr, L * nkv * d * phys * es).reshape(L, nkv, d, phys * es)[:, :, :, :n * es]
        out.append((np.ascontiguousarray(ctxb), np.ascontiguousarray(k), np.ascontiguousarray(v)))
    return out


def _same(name, a, b):
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{name}: {k} differs in {int(np.sum(a[k] != b[k]))} entries"


@pytest.mark.parametrize("lens,K,persistent", [([700], 16, False), ([700, 333], 16, False),
                                               ([700, 333], 40, False), ([700], 16, True)],
                         ids=["1mtile", "2mtiles", "5mtiles", "single-launch"])
def test_draft_path_is_bitwise_deterministic(lens, K, persistent):
    say(f"case: determinism lens={lens} K={K} persistent={persistent}")
    w = synth.weights(SMALL, SEED, gain_std=0.1)
    model = dfl.Model(SMALL, dfl.weights_to_device(w))
    a, b = _ctx(model, lens), _ctx(model, lens)
    for c in (a, b):
        c.set_persistent(persistent)
    if persistent:
        if not a.persistent_path(K):
            pytest.skip("the single-launch block is not available for this shape on this device")
    # the same step on two contexts built by the same calls
    ids, ra = _step(a, K, 0)
    _, rb = _step(b, K, 0)
    _same("two contexts, fused step", ra, rb)
    for (ca, ka, va), (cb, kb, vb) in zip(_state(a), _state(b)):
        assert np.array_equal(ca, cb) and np.array_equal(ka, kb) and np.array_equal(va, vb), "state differs"
    # the same block drafted again and again on one context (no state change)
    first = _draft(a, ids, K)
    for r in range(REPEATS):
        _same(f"repeat {r}", first, _draft(a, ids, K))
        _same(f"other context, repeat {r}", first, _draft(b, ids, K))
    if persistent:
        a.check()
        b.check()
    for o in (a, b, model):
        o.close()
