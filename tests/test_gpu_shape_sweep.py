"""Seeded sweep over random small drafter shapes and block sizes, each
against the fp64 oracle: the product planning's corner cases (tile counts
that do not divide into workgroups, k-block counts that do not divide into
splits, padded m-groups, one to eighteen m-tiles, so every residual form),
GQA ratios, head sizes, tiny and odd vocabularies, tied and untied LM
heads, bf16 and fp32, ragged contexts and appends, a sequence with an empty
context and a step that appends nothing.

Per case: a prefill of ragged contexts (state compared: context buffer and
caches), a draft block (logits, final hidden rows, argmax), then one fused
step (dflash_step) appending a random number of positions per sequence,
including none, compared with the oracle's projection + draft.
"""
import numpy as np
import pytest

import synth
from oracle import dflash as O
from tests.gpu_util import Pair, check_argmax, check_rows, say, tol

pytestmark = pytest.mark.gpu

N_CASES = 48


def _case(i):
    rng = np.random.default_rng(7000 + i)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    head_dim = int(rng.choice([64, 128]))
    nkv = int(rng.choice([1, 2, 4]))
    rep = int(rng.choice([1, 2, 4, 8]))
    shape = synth.Shape(hidden=64 * int(rng.integers(1, 10)), n_layers=int(rng.integers(1, 4)),
                        n_q_heads=nkv * rep, n_kv_heads=nkv, head_dim=head_dim,
                        intermediate=8 * int(rng.integers(4, 91)), vocab=int(rng.integers(2, 3001)),
                        n_feat=int(rng.integers(1, 4)), rope_theta=float(rng.choice([1e4, 5e5, 1e6])),
                        dtype=dtype, tied=bool(rng.random() < 0.5))
    B = int(rng.integers(1, 5))
    K = int(rng.choice([1, 2, 3, 5, 8, 16, 17, 33, 48, 64, 70]))
    lens = [int(x) for x in rng.integers(0, 401, size=B)]
    n_new = [int(x) for x in rng.integers(0, 21, size=B)]
    # degenerate cases the draws rarely reach: a sequence with no context
    # at all, a step that appends nothing, a vocabulary of a few tokens
    if i % 6 == 5:
        lens[0] = 0
    if i % 12 == 11:
        n_new = [0] * B
    if i % 8 == 3:
        shape = shape.replace(vocab=int(rng.integers(2, 20)))
    return shape, B, K, lens, n_new


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_against_oracle(i):
    shape, B, K, lens, n_new = _case(i)
    say(f"case {i}: {shape} B={B} K={K} ctx={lens} append={n_new}")
    seed = 7100 + i
    p = Pair(shape, seed, B, gain_std=0.1)
    feats = [synth.prefill_features(shape, seed, b, n) for b, n in enumerate(lens)]
    p.project(feats)
    p.check_state()
    ids = np.stack([synth.block_ids(seed, b, 0, K, shape.vocab) for b in range(B)])
    p.compare(ids)
    # one fused step: append n_new[b] positions to sequence b, draft again
    t = tol(shape)
    new = [synth.step_features(shape, seed, b, 1, n) for b, n in enumerate(n_new)]
    ids2 = np.stack([synth.block_ids(seed, b, 1, K, shape.vocab) for b in range(B)])
    g = p.gpu_step(new, ids2)
    for b in range(B):
        if n_new[b]:
            O.project_ctx(p.om, p.ost[b], new[b])
        d_o, l_o, z_o = p.oracle_draft(b, ids2[b])
        check_rows(f"step logits[{b}]", g["logits"][b], l_o, t)
        check_rows(f"step hidden[{b}]", g["hidden"][b], z_o, t)
        check_argmax(g["draft"][b], l_o)
    p.check_state()
