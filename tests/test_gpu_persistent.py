"""GPU parity of the single-launch draft block (bf16, batch * K <= 16)
against the fp64 oracle, through the C ABI.

Same bar as the other parity tests: per-row max |gpu - oracle| / max |oracle|
<= 2e-2 for logits and final hidden states, argmax exact where the oracle's
top-1/top-2 margin exceeds 0.05.  Every test also asks the library whether
a launch was abandoned (dflash_ctx_check) and asserts that the block really
took the single-launch path.
"""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import Pair, check_argmax, check_rows, say

pytestmark = pytest.mark.gpu

SMALL = synth.Shape(hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                    intermediate=1408, vocab=4003, n_feat=3, rope_theta=1e6, dtype="bf16")
# head_dim 64, one query head per KV head, intermediate not a multiple of 32
SMALL64 = synth.Shape(hidden=256, n_layers=3, n_q_heads=4, n_kv_heads=4, head_dim=64,
                      intermediate=696, vocab=2053, n_feat=2, rope_theta=1e4, dtype="bf16")


def _prefill(p, lens, seed=5):
    feats = [synth.prefill_features(p.shape, seed, b, n) for b, n in enumerate(lens)]
    p.project(feats)


def _ids(seed, B, K, V, step=0):
    return np.stack([synth.block_ids(seed, b, step, K, V) for b in range(B)])


def _persistent(p, K):
    p.ctx.set_persistent(True)
    assert p.ctx.persistent_path(K), "block should take the single-launch path"


@pytest.mark.parametrize("shape_name,B,lens,K", [
    ("small", 1, [200], 16),
    ("small", 2, [300, 317], 5),      # ragged contexts: different split counts
    ("small", 4, [0, 1, 64, 129], 4),  # empty context, one key, chunk edges
    ("small", 1, [1000], 1),          # one row
    ("small64", 1, [77], 16),
    ("small64", 3, [5, 130, 64], 3),
])
def test_persistent_block_matches_oracle(shape_name, B, lens, K):
    shape = SMALL if shape_name == "small" else SMALL64
    say(f"case: persistent {shape_name} B={B} ctx={lens} K={K}")
    p = Pair(shape, 41, B, gain_std=0.1)
    _prefill(p, lens)
    _persistent(p, K)
    p.compare(_ids(43, B, K, shape.vocab))
    p.ctx.check()


def test_persistent_matches_multikernel_path():
    """The two paths run the same arithmetic up to summation order."""
    say("case: persistent vs per-product kernels")
    p = Pair(SMALL, 51, 1, gain_std=0.1)
    _prefill(p, [333])
    ids = _ids(52, 1, 16, SMALL.vocab)
    _persistent(p, 16)
    a = p.gpu_draft(ids)
    p.ctx.set_persistent(False)
    assert not p.ctx.persistent_path(16)
    b = p.gpu_draft(ids)
    p.ctx.set_persistent(True)
    check_rows("logits persistent vs kernels", a["logits"][0], b["logits"][0], 1e-2)
    check_rows("hidden persistent vs kernels", a["hidden"][0], b["hidden"][0], 1e-2)
    _, l_o, _ = p.oracle_draft(0, ids[0])
    check_argmax(a["draft"][0], l_o)
    check_argmax(b["draft"][0], l_o)
    p.ctx.check()


def test_persistent_padding_rows_never_leak():
    """NaN in every cache row past ctx_len must not reach any output."""
    say("case: persistent, NaN-poisoned padding")
    p = Pair(SMALL, 61, 2, gain_std=0.1)
    _prefill(p, [65, 3])
    p.poison_padding()
    _persistent(p, 8)
    g, _ = p.compare(_ids(62, 2, 8, SMALL.vocab))
    assert np.all(np.isfinite(g["logits"]))
    p.ctx.check()


def test_persistent_repeated_launches_and_appends():
    """Back-to-back launches (the barrier flags advance, the split counters
    reset themselves) interleaved with appends of 1-11 rows, each block
    checked against the oracle; the state stays exact."""
    say("case: persistent, 6 steps with appends")
    p = Pair(SMALL, 71, 1, gain_std=0.1)
    _prefill(p, [120])
    rng = np.random.default_rng(72)
    for t in range(6):
        ids = _ids(73, 1, 10, SMALL.vocab, step=t)
        _persistent(p, 10)
        p.compare(ids)
        n = int(rng.integers(1, 12))
        p.project([synth.step_features(SMALL, 74, 0, t, n)])
        p.check_state()
    p.ctx.check()


def test_persistent_launches_without_sync_in_between():
    """Several blocks enqueued back to back with no host synchronisation,
    outputs kept apart: every one equals the block run alone."""
    say("case: persistent, 5 blocks without sync")
    p = Pair(SMALL, 81, 1, gain_std=0.1)
    _prefill(p, [257])
    K = 16
    _persistent(p, K)
    idss = [_ids(82, 1, K, SMALL.vocab, step=t) for t in range(5)]
    outs = []
    for ids in idss:
        dr = torch.empty(1, K, dtype=torch.int32, device="cuda")
        lg = torch.empty(1, K, SMALL.vocab, dtype=torch.float32, device="cuda")
        p.dfl.dflash_draft_block(p.ctx, torch.from_numpy(ids.astype(np.int32)).cuda(), K, dr, lg, None)
        outs.append((dr, lg))
    torch.cuda.synchronize()
    p.ctx.check()
    for ids, (dr, lg) in zip(idss, outs):
        ref = p.gpu_draft(ids)
        assert np.array_equal(dr.cpu().numpy(), ref["draft"])
        assert np.array_equal(lg.cpu().numpy(), ref["logits"])


@pytest.mark.slow
def test_persistent_workload1_qwen3_4b_shape_full_size():
    """The Qwen3-4B-shaped drafter at full size (context 2048, K = 16): one
    block through the single-launch path against the oracle."""
    wl = synth.workload(1)
    say(f"case: persistent {wl.name} full size")
    p = Pair(wl.shape, wl.seed, 1)
    _prefill(p, list(wl.ctx0), seed=wl.seed)
    _persistent(p, wl.K)
    ids = _ids(wl.seed, 1, wl.K, wl.shape.vocab)
    p.compare(ids, hidden=True)
    p.ctx.check()
