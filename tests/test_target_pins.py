"""Pins of the target-verification oracle (oracle/target.py) against an
independent scalar writing, the incremental-decoding invariant, causality,
closed forms and the commit rule (Google Developers Blog, "Overcoming the
autoregressive bottleneck", "Dual cache for attention", "Bridging the
metadata gap in TPU inference"; kongchang.com "D-Flash", "System
architecture")."""
import numpy as np
import pytest

import synth
from oracle import brute
from oracle import dflash as O
from oracle import target as OT

MICRO = synth.Shape(hidden=16, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=4, intermediate=24,
                    vocab=37, n_feat=0, rope_theta=1e4, dtype="f32")
SMALL = synth.Shape(hidden=64, n_layers=3, n_q_heads=4, n_kv_heads=2, head_dim=16, intermediate=96,
                    vocab=97, n_feat=0, rope_theta=1e4, dtype="bf16")


def _model(shape, seed=3):
    w = synth.weights(shape, seed, gain_std=0.1)
    return O.Model(shape, w, keep=True), w


def _seq(n, vocab, seed=4):
    return np.random.default_rng(seed).integers(0, vocab, size=n)


def test_full_forward_matches_scalar_brute_force():
    m, w = _model(MICRO)
    ids = _seq(9, MICRO.vocab)
    out = OT.forward_full(m, ids, taps=(0, 1))
    D, L, T = brute.target_forward(MICRO, w, ids, taps=(0, 1))
    assert np.max(np.abs(out.logits - np.array(L))) < 1e-12
    assert np.max(np.abs(out.taps - np.array(T))) < 1e-12
    assert out.target.tolist() == D


@pytest.mark.parametrize("shape", [MICRO, SMALL])
def test_incremental_verify_equals_full_forward(shape):
    """Blocks verified against the committed cache, with partial commits,
    give the same logits as a fresh causal forward over everything committed
    plus the block: the cache holds exactly the committed positions, at the
    right RoPE angles, and the mask is causal."""
    m, _ = _model(shape)
    seq = _seq(60, shape.vocab, seed=5)
    rng = np.random.default_rng(6)
    st = OT.new_target_state(m)
    out = OT.verify(m, st, seq[:11], taps=(1,))
    OT.commit(st, out, 11)
    checked = 0
    while st.ctx_len + 6 <= len(seq):
        block = seq[st.ctx_len:st.ctx_len + 6]
        out = OT.verify(m, st, block, taps=(1,))
        ref = OT.forward_full(m, seq[:st.ctx_len + 6], taps=(1,))
        assert np.max(np.abs(out.logits - ref.logits[-6:])) < 1e-10
        assert np.max(np.abs(out.taps - ref.taps[-6:])) < 1e-10
        assert out.target.tolist() == ref.target[-6:].tolist()
        OT.commit(st, out, int(rng.integers(1, 7)))
        checked += 1
    assert checked >= 5


def test_block_rows_are_causal():
    """Changing block token j leaves rows < j bit-identical and changes row j."""
    m, _ = _model(SMALL)
    st = OT.new_target_state(m)
    OT.commit(st, OT.verify(m, st, _seq(20, SMALL.vocab)), 20)
    block = _seq(8, SMALL.vocab, seed=9)
    a = OT.verify(m, st, block)
    for j in (1, 4, 7):
        b2 = block.copy()
        b2[j] = (b2[j] + 1) % SMALL.vocab
        b = OT.verify(m, st, b2)
        assert np.array_equal(a.logits[:j], b.logits[:j])
        assert np.max(np.abs(a.logits[j] - b.logits[j])) > 1e-6


def test_commit_keeps_exactly_the_first_rows():
    m, _ = _model(MICRO)
    st = OT.new_target_state(m)
    out = OT.verify(m, st, _seq(7, MICRO.vocab))
    OT.commit(st, out, 3)
    assert st.ctx_len == 3
    for l in range(MICRO.n_layers):
        assert np.array_equal(st.k[l], out.k_new[l][:3]) and np.array_equal(st.v[l], out.v_new[l][:3])
    OT.commit(st, OT.verify(m, st, _seq(2, MICRO.vocab)), 0)
    assert st.ctx_len == 3


def test_zero_layers_is_the_lm_head_of_the_normed_embedding():
    shape = MICRO.replace(n_layers=0)
    m, w = _model(shape)
    ids = _seq(5, shape.vocab)
    out = OT.forward_full(m, ids)
    E = O.to_f64(w["embed"], "f32")[ids]
    z = E / np.sqrt(np.mean(E * E, axis=1, keepdims=True) + shape.rms_eps) * O.to_f64(w["final_norm"], "f32")
    assert np.max(np.abs(out.logits - z @ O.to_f64(w["lm_head"], "f32").T)) < 1e-12


def test_last_tap_gives_the_logits_and_taps_match_truncated_models():
    m, w = _model(SMALL)
    ids = _seq(12, SMALL.vocab)
    out = OT.forward_full(m, ids, taps=(0, 2))
    H = SMALL.hidden
    last = out.taps[:, H:]
    z = O.rms_norm(last, m.f64("final_norm"), SMALL.rms_eps)
    assert np.max(np.abs(z @ m.f64("lm_head").T - out.logits)) < 1e-10
    trunc = O.Model(SMALL.replace(n_layers=1), w, keep=True)
    assert np.max(np.abs(OT.forward_full(trunc, ids, taps=(0,)).taps - out.taps[:, :H])) < 1e-12


def test_first_position_attends_only_to_itself():
    """ctx 0, one token: softmax over one key is 1, so attention returns v."""
    m, w = _model(MICRO)
    out = OT.forward_full(m, np.array([5]))
    D, L, _ = brute.target_forward(MICRO, w, [5])
    assert np.max(np.abs(out.logits[0] - np.array(L[0]))) < 1e-12
