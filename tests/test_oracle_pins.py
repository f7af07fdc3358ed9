"""Pins of the fp64 oracle against things other than itself.

Each test checks ``oracle.dflash`` against brute force, a textbook identity, a
special case with a known answer, or an invariance the method must have, so
that a plausible mistake in the oracle (dropped term, wrong sign, wrong index,
transposed operand, wrong head mapping, a causal mask) fails at least one.
"""
import cmath
import math

import numpy as np
import pytest

import synth
from oracle import brute
from oracle import dflash as O

MINI = synth.Shape(hidden=32, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=8,
                   intermediate=48, vocab=64, n_feat=2, rope_theta=1e4, rms_eps=1e-6,
                   dtype="f32", tied=False)


def mini_model(shape=MINI, seed=7, gain_std=0.1, **kw):
    w = synth.weights(shape, seed, gain_std=gain_std)
    for k, v in kw.items():
        w[k] = v
    return O.Model(shape, w, keep=True)


def projected(model, n_ctx, seed=3, positions=None, order=None):
    st = O.new_state(model)
    f = synth.prefill_features(model.shape, seed, 0, n_ctx)
    pos = np.arange(n_ctx) if positions is None else np.asarray(positions)
    if order is not None:
        f, pos = f[order], pos[order]
    O.project_ctx(model, st, f, positions=pos)
    return st, f


def rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(1e-300, np.max(np.abs(b))))


# ---------------------------------------------------------------- P1 brute force
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_brute_force_matches_oracle(dtype):
    shape = MINI.replace(dtype=dtype)
    model = mini_model(shape)
    n_ctx, K = 5, 4
    f = synth.prefill_features(shape, 3, 0, n_ctx)
    ids = synth.block_ids(11, 0, 0, K, shape.vocab)
    d_b, l_b, z_b = brute.forward(shape, model.w, f, ids)
    st = O.new_state(model)
    O.project_ctx(model, st, f)
    d_o, l_o, z_o = O.draft_one(model, st, ids)
    assert rel(l_o, np.array(l_b)) < 1e-12
    assert rel(z_o, np.array(z_b)) < 1e-12
    assert list(d_o) == d_b


def test_brute_force_tiny_fp32_config():
    """The tiny fp32 workload shape itself (small context and block)."""
    shape = synth.TINY.replace(n_layers=1, vocab=128)
    w = synth.weights(shape, 1000, gain_std=0.1)
    model = O.Model(shape, w, keep=True)
    f = synth.prefill_features(shape, 1000, 0, 3)
    ids = synth.block_ids(1000, 0, 0, 2, shape.vocab)
    d_b, l_b, z_b = brute.forward(shape, w, f, ids)
    st = O.new_state(model)
    O.project_ctx(model, st, f)
    d_o, l_o, z_o = O.draft_one(model, st, ids)
    assert rel(l_o, np.array(l_b)) < 1e-12
    assert list(d_o) == d_b


# ---------------------------------------------------------------- RoPE pins
def test_rope_is_complex_rotation():
    """Rotate-half RoPE == multiplying z_m = v_m + i v_{m+d/2} by e^{i p theta_m}."""
    rng = np.random.default_rng(0)
    d, theta = 16, 1e4
    v = rng.standard_normal((5, 3, d))
    pos = np.array([0, 1, 7, 1000, 33000])
    out = O.rope(v, pos, theta)
    for n in range(5):
        for h in range(3):
            for m in range(d // 2):
                z = complex(v[n, h, m], v[n, h, m + d // 2])
                w = z * cmath.exp(1j * pos[n] * theta ** (-2.0 * m / d))
                assert abs(out[n, h, m] - w.real) < 1e-9
                assert abs(out[n, h, m + d // 2] - w.imag) < 1e-9


def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((4, 2, 8))
    assert np.array_equal(O.rope(v, np.zeros(4, np.int64), 1e6), v)
    r = O.rope(v, np.array([3, 50, 999, 12345]), 1e6)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(v, axis=-1), rtol=1e-13)


def test_rope_relative_position_of_dot_products():
    """<RoPE(q, p1), RoPE(k, p2)> depends only on p1 - p2."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 8))
    k = rng.standard_normal((1, 1, 8))
    a = np.sum(O.rope(q, np.array([10]), 1e4) * O.rope(k, np.array([3]), 1e4))
    b = np.sum(O.rope(q, np.array([1007]), 1e4) * O.rope(k, np.array([1000]), 1e4))
    assert abs(a - b) < 1e-10


# ---------------------------------------------------------------- attention special cases
def test_single_key_attention_returns_v():
    """Empty context, K = 1: softmax over one key is 1, so attention == v."""
    model = mini_model()
    st = O.new_state(model)
    cap = {}
    O.draft_one(model, st, np.array([5]), capture=cap)
    s = model.shape
    rep = s.n_q_heads // s.n_kv_heads
    for l in range(s.n_layers):
        o = cap["attn_out"][l][0]            # [nq, d]
        v = cap["v_block"][l][0]             # [nkv, d]
        for h in range(s.n_q_heads):
            assert np.allclose(o[h], v[h // rep], rtol=0, atol=1e-14)


def test_zero_query_weights_average_all_values():
    """W_q = 0 gives uniform attention: the output is the mean of every V row,
    context rows and block rows alike (no mask, no dropped rows)."""
    s = MINI
    w = synth.weights(s, 7, gain_std=0.1)
    for l in range(s.n_layers):
        w[f"layers.{l}.wq"] = np.zeros_like(w[f"layers.{l}.wq"])
    model = O.Model(s, w, keep=True)
    st, _ = projected(model, 6)
    cap = {}
    O.draft_one(model, st, synth.block_ids(1, 0, 0, 3, s.vocab), capture=cap)
    rep = s.n_q_heads // s.n_kv_heads
    for l in range(s.n_layers):
        allv = np.concatenate([st.v[l], cap["v_block"][l]], axis=0)     # [6+3, nkv, d]
        mean = allv.mean(axis=0)
        o = cap["attn_out"][l]
        for i in range(3):
            for h in range(s.n_q_heads):
                assert np.allclose(o[i, h], mean[h // rep], atol=1e-13)


def test_attention_is_non_causal():
    """Changing the last block id changes row 0's output, and row 0 puts
    positive weight on every block key."""
    model = mini_model()
    st, _ = projected(model, 5)
    ids = synth.block_ids(4, 0, 0, 6, MINI.vocab)
    cap = {}
    _, l1, _ = O.draft_one(model, st, ids, capture=cap)
    ids2 = ids.copy()
    ids2[-1] = (ids2[-1] + 1) % MINI.vocab
    _, l2, _ = O.draft_one(model, st, ids2)
    assert np.max(np.abs(l1[0] - l2[0])) > 1e-6
    p = cap["attn_probs"][0]      # [K, nq, n_ctx + K]
    assert np.all(p[0, :, 5:] > 0)
    assert np.allclose(p.sum(-1), 1.0)


# ---------------------------------------------------------------- invariances
def test_context_permutation_invariance():
    """Permuting context rows together with their positions (and so their
    RoPE angles) leaves every output unchanged."""
    model = mini_model()
    n = 9
    perm = np.random.default_rng(5).permutation(n)
    st_a, _ = projected(model, n)
    st_b, _ = projected(model, n, order=perm)
    ids = synth.block_ids(6, 0, 0, 5, MINI.vocab)
    da, la, za = O.draft_one(model, st_a, ids)
    db, lb, zb = O.draft_one(model, st_b, ids)
    assert rel(lb, la) < 1e-12 and np.array_equal(da, db)
    # and the order matters when the positions do not travel with the rows
    st_c = O.new_state(model)
    f = synth.prefill_features(MINI, 3, 0, n)
    O.project_ctx(model, st_c, f[perm])
    _, lc, _ = O.draft_one(model, st_c, ids)
    assert rel(lc, la) > 1e-6


def test_global_position_shift_invariance():
    """Shifting every position (context and block) by the same amount leaves
    the outputs unchanged: RoPE only encodes relative offsets."""
    model = mini_model()
    n, K, D = 7, 4, 12345
    st_a, _ = projected(model, n)
    st_b, _ = projected(model, n, positions=np.arange(n) + D)
    ids = synth.block_ids(8, 0, 0, K, MINI.vocab)
    _, la, _ = O.draft_one(model, st_a, ids)
    _, lb, _ = O.draft_one(model, st_b, ids, block_pos=np.arange(n, n + K) + D)
    assert rel(lb, la) < 1e-9


def test_block_permutation_equivariance():
    """Permuting block rows together with their positions permutes outputs."""
    model = mini_model()
    st, _ = projected(model, 6)
    K = 5
    ids = synth.block_ids(9, 0, 0, K, MINI.vocab)
    perm = np.array([3, 0, 4, 1, 2])
    pos = np.arange(6, 6 + K)
    _, la, za = O.draft_one(model, st, ids)
    _, lb, zb = O.draft_one(model, st, ids[perm], block_pos=pos[perm])
    assert rel(lb, la[perm]) < 1e-12
    assert rel(zb, za[perm]) < 1e-12


def test_gqa_equals_mha_with_duplicated_kv():
    """GQA with nkv < nq equals MHA whose K/V weights repeat each KV head for
    the query heads that share it."""
    s = MINI
    w = synth.weights(s, 7, gain_std=0.1)
    rep = s.n_q_heads // s.n_kv_heads
    s2 = s.replace(n_kv_heads=s.n_q_heads)
    w2 = dict(w)
    for l in range(s.n_layers):
        for nm in ("wk", "wv"):
            W = w[f"layers.{l}.{nm}"].reshape(s.n_kv_heads, s.head_dim, s.hidden)
            w2[f"layers.{l}.{nm}"] = np.repeat(W, rep, axis=0).reshape(s2.kv_dim, s.hidden)
    m1, m2 = O.Model(s, w, keep=True), O.Model(s2, w2, keep=True)
    st1, _ = projected(m1, 5)
    st2, _ = projected(m2, 5)
    ids = synth.block_ids(10, 0, 0, 4, s.vocab)
    _, l1, _ = O.draft_one(m1, st1, ids)
    _, l2, _ = O.draft_one(m2, st2, ids)
    assert rel(l2, l1) < 1e-12


def test_batch_independence():
    """Sequence b's outputs do not depend on the other sequences in the batch."""
    model = mini_model()
    states = [projected(model, n, seed=20 + n)[0] for n in (3, 8, 1)]
    ids = np.stack([synth.block_ids(12, b, 0, 4, MINI.vocab) for b in range(3)])
    out = O.draft_block(model, states, ids)
    for b in range(3):
        d, l, z = O.draft_one(model, states[b], ids[b])
        assert np.array_equal(out.logits[b], l) and np.array_equal(out.draft[b], d)


def test_incremental_projection_equals_one_shot():
    """Appending the context in chunks gives the same buffer and caches as
    appending it at once."""
    model = mini_model()
    n = 17
    f = synth.prefill_features(MINI, 3, 0, n)
    st_a = O.new_state(model)
    O.project_ctx(model, st_a, f)
    st_b = O.new_state(model)
    i = 0
    for c in (1, 3, 11, 2):
        O.project_ctx(model, st_b, f[i:i + c])
        i += c
    assert st_a.ctx_len == st_b.ctx_len == n
    assert np.allclose(st_a.ctx, st_b.ctx, rtol=0, atol=1e-12)
    for l in range(MINI.n_layers):
        assert np.allclose(st_a.k[l], st_b.k[l], atol=1e-12)
        assert np.allclose(st_a.v[l], st_b.v[l], atol=1e-12)


def test_rmsnorm_scale_invariance():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 32))
    g = 1 + 0.1 * rng.standard_normal(32)
    a = O.rms_norm(x, g, 0.0)
    assert np.allclose(O.rms_norm(7.5 * x, g, 0.0), a, rtol=1e-14)
    # unit RMS after the norm when the gain is 1
    u = O.rms_norm(x, np.ones(32), 0.0)
    assert np.allclose(np.sqrt(np.mean(u * u, axis=-1)), 1.0, rtol=1e-14)


def test_zero_layers_reduce_to_lm_head_of_embedding():
    """With no draft layers the block is embedding -> final norm -> LM head;
    checked against a direct product of the stored tables."""
    s = MINI.replace(n_layers=0)
    w = synth.weights(s, 7, gain_std=0.1)
    model = O.Model(s, w, keep=True)
    st = O.new_state(model)
    ids = np.array([0, 63, 17])
    d, l, z = O.draft_one(model, st, ids)
    E = w["embed"].astype(np.float64)[ids]
    g = w["final_norm"].astype(np.float64)
    for i in range(3):
        zi = [E[i, c] * g[c] / math.sqrt(sum(e * e for e in E[i]) / 32 + 1e-6) for c in range(32)]
        li = [sum(w["lm_head"][v, c] * zi[c] for c in range(32)) for v in range(64)]
        assert np.allclose(l[i], li, rtol=1e-12, atol=1e-14)
        assert d[i] == int(np.argmax(li))


def test_argmax_ties_pick_lowest_index():
    """Duplicate LM-head rows give exactly tied logits; the lower index wins."""
    s = MINI.replace(n_layers=0)
    w = synth.weights(s, 7)
    lm = w["lm_head"].copy()
    model0 = O.Model(s, w, keep=True)
    _, l0, _ = O.draft_one(model0, O.new_state(model0), np.array([4]))
    best = int(np.argmax(l0[0]))
    lm[2] = lm[best]             # row 2 now ties with the best row
    lm[60] = lm[best]
    w["lm_head"] = lm
    model = O.Model(s, w, keep=True)
    d, l, _ = O.draft_one(model, O.new_state(model), np.array([4]))
    assert l[0, 2] == l[0, best] == l[0, 60]
    assert d[0] == min(2, best)
