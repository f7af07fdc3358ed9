"""Pins of the acceptance rule, the stand-in verifier and the session state.

  * exhaustive enumeration of every match pattern for small K;
  * the closed form of E[tau] under independent agreement with probability
    a * gamma^i at block position i, against Monte Carlo through the oracle;
  * the claims of the Google Developers Blog post ("Scaling theory") about K,
    stored in tests/golden/pages_claims.json, reproduced on that model;
  * growth and state-advance invariants over a session, and detection of the
    "sequence-length inflation" mistake the post describes ("Bridging the
    metadata gap in TPU inference").
"""
import itertools
import json
import os

import numpy as np
import pytest

import synth
from oracle import dflash as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def expected_tau(a, gamma, K):
    """E[tau] = 1 + sum_{m=1..K} prod_{i<m} a*gamma^i (independent agreement)."""
    tot, run = 1.0, 1.0
    for m in range(1, K + 1):
        run *= a * gamma ** (m - 1)
        tot += run
    return tot


@pytest.mark.parametrize("K", [1, 2, 5, 10])
def test_accept_exhaustive(K):
    draft = np.arange(K)[None, :].repeat(1, 0)
    for pattern in itertools.product([0, 1], repeat=K):
        target = draft.copy()
        for i, ok in enumerate(pattern):
            if not ok:
                target[0, i] += 1000
        lead = 0
        for ok in pattern:
            if not ok:
                break
            lead += 1
        assert int(O.accept(draft, target)[0]) == 1 + lead


def test_accept_batch_rows_independent():
    d = np.array([[1, 2, 3], [1, 2, 3], [1, 2, 3]])
    t = np.array([[1, 2, 3], [9, 2, 3], [1, 2, 9]])
    assert O.accept(d, t).tolist() == [4, 1, 3]


def test_closed_form_values():
    """The closed form itself against an independent evaluation: sum over
    tau of tau * P(tau), with P(tau = n+1) = P(first n agree, n+1-th not)."""
    for a, g, K in [(0.9, 0.97, 16), (0.9, 0.97, 8), (0.7, 0.95, 10)]:
        p = [a * g ** i for i in range(K)]
        e = 0.0
        for n in range(K + 1):
            pr = np.prod(p[:n]) * ((1 - p[n]) if n < K else 1.0)
            e += (n + 1) * pr
        assert abs(e - expected_tau(a, g, K)) < 1e-12


def test_monte_carlo_matches_closed_form():
    """Stand-in verifier + oracle acceptance reproduce E[tau] within 4 sigma."""
    a, g, K, V, N = 0.9, 0.97, 16, 151936, 20000
    taus = np.empty(N)
    draft = np.zeros((1, K), np.int64)
    for t in range(N):
        d = synth.verifier_draws(77, 0, t, K, V, a, g)
        taus[t] = O.accept(draft, synth.target_tokens(draft[0], d, V)[None])[0]
    mu = expected_tau(a, g, K)
    assert abs(taus.mean() - mu) < 4 * taus.std() / np.sqrt(N)
    assert taus.min() >= 1 and taus.max() <= K + 1


def test_disagreeing_targets_always_differ():
    V = 7
    for t in range(200):
        d = synth.verifier_draws(5, 0, t, 8, V, 0.5, 0.9)
        draft = np.random.default_rng(t).integers(0, V, 8)
        tg = synth.target_tokens(draft, d, V)
        assert np.all((tg == draft) == d.agree)
        assert np.all((tg >= 0) & (tg < V))


def test_pages_claims_on_the_agreement_model():
    """The post's scaling claims hold on the a*gamma^i model the workloads
    use (values and citation in tests/golden/pages_claims.json)."""
    with open(os.path.join(GOLDEN, "pages_claims.json")) as f:
        claims = json.load(f)
    c = claims["k16_captures_most_of_max"]
    a, g = c["a"], c["gamma"]
    e16, einf = expected_tau(a, g, 16), expected_tau(a, g, 4096)
    assert e16 / einf >= c["min_fraction"]
    c2 = claims["k16_to_k128_adds_under_one_token"]
    assert expected_tau(a, g, 128) - e16 < c2["max_added_tokens"]
    c3 = claims["config2_accept_range"]
    assert 1 + c3["K"] == c3["max_accepted_positions"]


# ---------------------------------------------------------------- sessions
def _tiny_session(**kw):
    wl = synth.workload(0).replace(ctx0=(61,), steps=8, **kw)
    shape = wl.shape.replace(hidden=64, intermediate=96, vocab=256, n_q_heads=4,
                             n_kv_heads=2, head_dim=16)
    model = O.Model(shape, synth.weights(shape, wl.seed), keep=True)
    return O.Session(model, wl.replace(shape=shape))


def test_session_growth_and_state_invariants():
    sess = _tiny_session()
    st = sess.states[0]
    assert st.ctx_len == 61 and st.cap == 64
    prev_cap, prev_len = st.cap, st.ctx_len
    for _ in range(8):
        rec = sess.step()
        tau = int(rec.tau[0])
        assert 1 <= tau <= sess.wl.K + 1
        assert rec.write_start[0] == prev_len
        assert rec.ctx_len[0] == prev_len + tau
        cap = int(rec.cap[0])
        assert cap & (cap - 1) == 0 and cap >= rec.ctx_len[0]
        if prev_len + tau <= prev_cap:
            assert cap == prev_cap               # grows only on overflow
        else:
            assert cap == 1 << int(np.ceil(np.log2(prev_len + tau)))
        prev_cap, prev_len = cap, int(rec.ctx_len[0])
        assert sess.violations() == []
    assert st.grow_events >= 2                    # 64 -> 128 at least once


def test_sequence_length_inflation_is_detected():
    """Appending the drafted length K instead of the accepted length (the
    metadata mistake the post describes) is caught by the state check."""
    sess = _tiny_session()
    sess.step(n_new_override=sess.wl.K)
    errs = sess.violations()
    assert any("committed" in e for e in errs)


def test_duplicate_or_lost_positions_are_detected():
    sess = _tiny_session()
    st = sess.states[0]
    st.pos = st.pos.copy()
    st.pos[5] = st.pos[4]                          # one position twice, one lost
    assert any("positions" in e for e in O.check_state(st, sess.committed[0]))


def test_session_tau_depends_only_on_verifier_draws():
    """tau is a function of the verifier's agreement draws alone, so two
    implementations that draft different tokens still advance identically."""
    s1 = _tiny_session()
    s2 = _tiny_session()
    # perturb the second session's drafts by changing its LM head
    s2.model = O.Model(s2.model.shape, dict(s2.model.w, lm_head=s2.model.w["lm_head"][::-1].copy()), keep=True)
    for _ in range(6):
        r1, r2 = s1.step(), s2.step()
        assert np.array_equal(r1.tau, r2.tau)
        assert np.array_equal(r1.ctx_len, r2.ctx_len) and np.array_equal(r1.cap, r2.cap)


def test_golden_config0_session():
    """Regression guard: the oracle's tiny fp32 session matches the values
    stored by tests/golden/make_golden.py (which calls only the oracle)."""
    with open(os.path.join(GOLDEN, "config0_session.json")) as f:
        g = json.load(f)
    wl = synth.workload(0)
    model = O.Model(wl.shape, synth.weights(wl.shape, wl.seed), keep=True)
    sess = O.Session(model, wl, keep_outputs=True)
    for t, rec_g in enumerate(g["steps"]):
        rec = sess.step()
        assert rec.tau.tolist() == rec_g["tau"]
        assert rec.ctx_len.tolist() == rec_g["ctx_len"]
        assert rec.cap.tolist() == rec_g["cap"]
        assert rec.draft.tolist() == rec_g["draft"]
        np.testing.assert_allclose(rec.logits[0, :, :8], np.array(rec_g["logits_head"]), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("ctx_len,cap,n_new,want", [
    (0, 0, 1, 1), (0, 0, 2048, 2048), (0, 0, 2049, 4096), (60, 64, 4, 64),
    (60, 64, 5, 128), (64, 64, 0, 64), (4096, 4096, 1, 8192), (100, 128, 1000, 2048)])
def test_growth_boundaries(ctx_len, cap, n_new, want):
    """A buffer filled exactly to capacity does not grow; one row more takes
    it to the next power of two of the new length."""
    assert O.grow_rule(ctx_len, cap, n_new) == want


def test_exact_fill_through_project():
    sess = _tiny_session()
    st = sess.states[0]
    f = synth.step_features(sess.model.shape, 1, 0, 0, 3)
    O.project_ctx(sess.model, st, f)                 # 61 + 3 = 64 == cap
    assert st.ctx_len == 64 and st.cap == 64 and st.grow_events == 1
    O.project_ctx(sess.model, st, f[:1])
    assert st.ctx_len == 65 and st.cap == 128 and st.grow_events == 2
