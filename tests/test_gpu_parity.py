"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances (written here, applied per row): bf16 max |gpu - oracle| /
max |oracle| <= 2e-2, fp32 <= 1e-4, for logits, final hidden states, the
context buffer and both KV caches; argmax bit-exact wherever the oracle's
top-1/top-2 logit margin exceeds 0.05; acceptance lengths, context lengths,
capacities and buffer row indices bit-exact.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import dflash as O
from tests.gpu_util import Pair, check_argmax, check_rows, say, to_dev, tol

pytestmark = pytest.mark.gpu

# Small bf16 drafter: several tiles per matrix, ragged vocab tail (4003 rows),
# GQA with 4 query heads per KV head.
SMALL = synth.Shape(hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                    intermediate=1408, vocab=4003, n_feat=3, rope_theta=1e6, dtype="bf16")
SMALL32 = SMALL.replace(dtype="f32", head_dim=64, n_q_heads=8, n_kv_heads=4)


_WCACHE = {}


def _weights(shape, seed):
    key = (shape, seed)
    if key not in _WCACHE:
        _WCACHE.clear()
        _WCACHE[key] = synth.weights(shape, seed)
    return _WCACHE[key]


def _prefill(p, lens, seed=5):
    feats = [synth.prefill_features(p.shape, seed, b, n) for b, n in enumerate(lens)]
    p.project(feats)
    return feats


def _ids(seed, B, K, V, step=0):
    return np.stack([synth.block_ids(seed, b, step, K, V) for b in range(B)])


def test_mfma_fragment_layout_fp32_tiny():
    """Tiny fp32 drafter (workload 0 shape) with an empty context and K=1:
    exercises every kernel with one row, one key, one tile."""
    say("case: tiny fp32, ctx 0, K 1")
    p = Pair(synth.TINY, 1000, 1, gain_std=0.1)
    ids = _ids(3, 1, 1, synth.TINY.vocab)
    p.compare(ids)


@pytest.mark.parametrize("ctx,K", [(64, 8), (0, 8), (1, 3), (130, 37), (200, 16)])
def test_tiny_fp32_single_block(ctx, K):
    say(f"case: tiny fp32 ctx={ctx} K={K}")
    p = Pair(synth.TINY, 1000, 1, gain_std=0.1)
    if ctx:
        _prefill(p, [ctx])
    p.check_state()
    p.compare(_ids(7, 1, K, synth.TINY.vocab))


@pytest.mark.parametrize("B,ctx,K", [(1, 200, 16), (1, 63, 37), (3, 0, 16), (2, 300, 5),
                                     (1, 100, 128), (2, 70, 130), (1, 5, 300)])
def test_small_bf16_block(B, ctx, K):
    say(f"case: small bf16 B={B} ctx={ctx} K={K}")
    p = Pair(SMALL, 11, B, gain_std=0.1)
    lens = [ctx + 17 * b for b in range(B)]
    _prefill(p, lens)
    p.check_state()
    p.compare(_ids(13, B, K, SMALL.vocab))


def test_small_fp32_block_ragged():
    say("case: small fp32 B=2 ctx ragged K=21")
    p = Pair(SMALL32, 12, 2, gain_std=0.1)
    _prefill(p, [77, 150])
    p.check_state()
    p.compare(_ids(14, 2, 21, SMALL32.vocab))


def test_padding_rows_never_leak():
    """NaN in every cache row past ctx_len must not reach any output."""
    say("case: NaN-poisoned padding")
    p = Pair(SMALL, 21, 2, gain_std=0.1)
    _prefill(p, [65, 3])
    p.poison_padding()
    g, _ = p.compare(_ids(22, 2, 16, SMALL.vocab))
    assert np.all(np.isfinite(g["logits"]))


@pytest.mark.parametrize("stream", [False, True])
@pytest.mark.parametrize("K", [16, 37, 130])
def test_small_bf16_long_splits_poisoned(monkeypatch, K, stream):
    """Key splits of 1024 (16 chunks of 64: the staged attention pipelines'
    steady state and drain), ragged contexts whose last chunk is partial,
    NaN in every cache row past ctx_len; K = 16 (one query group), 37 (two
    query groups, one of them padding) and 130 (nine query groups: workgroups
    of four, two query tiles per wave, the last workgroup mostly padding);
    with `stream` the context K/V is loaded nontemporally."""
    say(f"case: long splits K={K} stream={stream}")
    monkeypatch.setenv("DFLASH_ATTN_MIN_SPLIT", "1024")
    monkeypatch.setenv("DFLASH_ATTN_STREAM_MB", "0" if stream else "1048576")
    p = Pair(SMALL, 41, 2, gain_std=0.1)
    _prefill(p, [1500, 2111])
    p.poison_padding()
    g, _ = p.compare(_ids(42, 2, K, SMALL.vocab))
    assert np.all(np.isfinite(g["logits"]))


@pytest.mark.parametrize("warm", ["16", "0"])
def test_small_bf16_l2_warm_up_settings(monkeypatch, warm):
    """The L2 warm-up workgroups appended to the attention kernel for the
    output projection load weights and discard them: outputs match the
    oracle with them on and off."""
    say(f"case: warm-up O={warm}")
    monkeypatch.setenv("DFLASH_WARM_O", warm)
    p = Pair(SMALL, 43, 2, gain_std=0.1)
    _prefill(p, [200, 77])
    p.compare(_ids(44, 2, 16, SMALL.vocab))


def test_side_stream_growth_and_draft():
    """Every call on a non-default stream, with capacity growth (the library
    frees the old buffers while the copy that reads them is still queued on
    that stream) and torch allocating on its own stream meanwhile: the state
    and the draft match the oracle."""
    say("case: calls on a side stream with growth")
    import block_diffusion_drafting_amd as dfl
    p = Pair(SMALL, 47, 2, gain_std=0.1)
    side = torch.cuda.Stream()
    s = SMALL
    feats0 = [synth.prefill_features(s, 47, b, n) for b, n in enumerate([60, 9])]
    with torch.cuda.stream(side):
        fd = to_dev(np.concatenate(feats0, axis=0))
    dfl.dflash_project_ctx(p.ctx, fd, [60, 9], stream=side)
    for b in range(2):
        O.project_ctx(p.om, p.ost[b], feats0[b])
    for t, n_new in enumerate([(5, 60), (70, 1)]):            # both sequences grow once
        fe = [synth.step_features(s, 47, b, t, n) for b, n in enumerate(n_new)]
        with torch.cuda.stream(side):
            fd = to_dev(np.concatenate(fe, axis=0))
        dfl.dflash_project_ctx(p.ctx, fd, list(n_new), stream=side)
        junk = torch.randn(1 << 20, device="cuda")            # torch reuses memory on its own stream
        del junk
        for b in range(2):
            O.project_ctx(p.om, p.ost[b], fe[b])
    ids = _ids(48, 2, 16, s.vocab)
    with torch.cuda.stream(side):
        idd = to_dev(ids.astype(np.int32))
        dr = torch.empty(2, 16, dtype=torch.int32, device="cuda")
        lg = torch.empty(2, 16, s.vocab, dtype=torch.float32, device="cuda")
    dfl.dflash_draft_block(p.ctx, idd, 16, dr, lg, stream=side)
    side.synchronize()
    p.check_state()
    for b in range(2):
        d_o, l_o, _ = p.oracle_draft(b, ids[b])
        check_rows(f"logits[{b}]", lg.cpu().numpy()[b], l_o, tol(s))
        check_argmax(dr.cpu().numpy()[b], l_o)


def test_non_causal_through_abi():
    """Changing the last block token changes row 0's logits."""
    say("case: non-causal")
    p = Pair(SMALL, 31, 1)
    _prefill(p, [50])
    ids = _ids(32, 1, 8, SMALL.vocab)
    a = p.gpu_draft(ids)["logits"][0, 0]
    ids2 = ids.copy()
    ids2[0, -1] = (ids2[0, -1] + 1) % SMALL.vocab
    b = p.gpu_draft(ids2)["logits"][0, 0]
    assert np.max(np.abs(a - b)) > 1e-3


def test_context_permutation_through_abi():
    """Projecting the context rows in a permuted order together with their
    positions gives the same draft outputs (same set of keys and values)."""
    say("case: context permutation")
    n = 97
    p1 = Pair(SMALL, 41, 1)
    f = synth.prefill_features(SMALL, 42, 0, n)
    p1.project([f])
    perm = np.random.default_rng(0).permutation(n)
    p2 = Pair(SMALL, 41, 1, weights=p1.w)
    p2.project([f[perm]], positions_per_seq=[perm.astype(np.int32)])
    ids = _ids(43, 1, 16, SMALL.vocab)
    a = p1.gpu_draft(ids)
    b = p2.gpu_draft(ids)
    # same key/value set in another order: equal within the path's tolerance
    check_rows("permuted logits", b["logits"][0], a["logits"][0].astype(np.float64), tol(SMALL))
    # and against the oracle with the permuted projection
    p2.compare(ids)


def test_batch_independence_through_abi():
    say("case: batch independence")
    pb = Pair(SMALL, 51, 3)
    lens = [40, 190, 7]
    feats = [synth.prefill_features(SMALL, 52, b, n) for b, n in enumerate(lens)]
    pb.project(feats)
    ids = _ids(53, 3, 16, SMALL.vocab)
    gb = pb.gpu_draft(ids)
    for b in range(3):
        p1 = Pair(SMALL, 51, 1, weights=pb.w)
        p1.project([feats[b]])
        g1 = p1.gpu_draft(ids[b:b + 1])
        check_rows(f"batch row {b}", gb["logits"][b], g1["logits"][0].astype(np.float64), tol(SMALL))


def test_incremental_projection_matches_one_shot():
    say("case: incremental projection")
    f = synth.prefill_features(SMALL, 61, 0, 40)
    p1 = Pair(SMALL, 62, 1)
    p1.project([f])
    p2 = Pair(SMALL, 62, 1, weights=p1.w)
    i = 0
    for c in (1, 3, 11, 2, 23):
        p2.project([f[i:i + c]])
        i += c
    p1.check_state()
    p2.check_state()
    ids = _ids(63, 1, 16, SMALL.vocab)
    a, b = p1.gpu_draft(ids), p2.gpu_draft(ids)
    check_rows("incremental logits", b["logits"][0], a["logits"][0].astype(np.float64), tol(SMALL))


def test_zero_new_rows_and_multi_sequence_append():
    say("case: n_new zero rows")
    p = Pair(SMALL, 71, 3)
    _prefill(p, [10, 0, 33])
    p.project([synth.step_features(SMALL, 72, 0, 0, 0), synth.step_features(SMALL, 72, 1, 0, 5),
               synth.step_features(SMALL, 72, 2, 0, 0)])
    p.check_state()
    p.compare(_ids(73, 3, 4, SMALL.vocab))


def test_accept_kernel_exhaustive_patterns():
    """Every match pattern at K = 10, plus K spanning several waves."""
    import block_diffusion_drafting_amd as dfl
    say("case: accept patterns")
    K = 10
    pats = np.array([[(m >> i) & 1 for i in range(K)] for m in range(1 << K)], np.int32)
    B = len(pats)
    draft = np.tile(np.arange(K, dtype=np.int32), (B, 1))
    target = np.where(pats == 1, draft, draft + 7).astype(np.int32)
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    dfl.dflash_accept(to_dev(draft), to_dev(target), B, K, out)
    assert np.array_equal(out.cpu().numpy(), O.accept(draft, target))
    for K in (1, 63, 64, 65, 130, 1024):
        rng = np.random.default_rng(K)
        B = 50
        d = rng.integers(0, 5, size=(B, K)).astype(np.int32)
        t = d.copy()
        cut = rng.integers(0, K + 1, size=B)
        for b in range(B):
            if cut[b] < K:
                t[b, cut[b]] += 1
        out = torch.empty(B, dtype=torch.int32, device="cuda")
        dfl.dflash_accept(to_dev(d), to_dev(t), B, K, out)
        assert np.array_equal(out.cpu().numpy(), O.accept(d, t))


def _session(shape, wl, steps, check_every=1, batch_seqs=None, tail_check=(), fused=False, keep_vocab=False):
    """GPU session and oracle session in lockstep; tau, ctx_len and cap must
    be identical every step; outputs compared on the checked steps.  With
    `fused`, the accepted positions of step t are appended by the
    dflash_step call that drafts step t + 1 (and by a final
    dflash_project_ctx), so the GPU state lags the oracle's by one append
    between calls.  `keep_vocab` keeps the oracle's float64 LM head between
    drafts (many sequences drafted per checked step)."""
    import block_diffusion_drafting_amd as dfl
    seqs = list(range(wl.batch)) if batch_seqs is None else batch_seqs
    w = _weights(shape, wl.seed)
    p = Pair(shape, wl.seed, wl.batch, weights=w, oracle_seqs=[])
    if keep_vocab:
        p.om.keep = True
    feats = [synth.prefill_features(shape, wl.seed, b, wl.ctx0[b]) for b in range(wl.batch)]
    p.project(feats)                      # GPU only: the oracle session prefills itself
    osess = O.Session(p.om, wl, keep_outputs=True, seqs=seqs)
    p.oseqs = list(seqs)
    p.ost = {b: osess.states[i] for i, b in enumerate(seqs)}
    anchors = [synth.first_anchor(wl.seed, b, shape.vocab) for b in range(wl.batch)]
    p.check_state()
    K = wl.K
    pending = None          # (features per sequence, taus) not yet appended on the GPU
    prev = None             # previous oracle step record
    for t in range(steps):
        ids = np.stack([synth.block_ids(wl.seed, b, t, K, shape.vocab) for b in range(wl.batch)])
        ids[:, 0] = anchors
        check = (t % check_every == 0) or (t in tail_check) or t == steps - 1
        if pending is not None:
            g = p.gpu_step(pending, ids, logits=check, hidden=False)
            lens, caps = p.ctx.query()
            assert [lens[b] for b in seqs] == prev.ctx_len.tolist()
            assert [caps[b] for b in seqs] == prev.cap.tolist()
            pending = None
        else:
            g = p.gpu_draft(ids, logits=check, hidden=False)
        draws = [synth.verifier_draws(wl.seed, b, t, K, shape.vocab, wl.a[b], wl.gamma) for b in range(wl.batch)]
        target = np.stack([synth.target_tokens(g["draft"][b], draws[b], shape.vocab) for b in range(wl.batch)])
        tau_d = torch.empty(wl.batch, dtype=torch.int32, device="cuda")
        dfl.dflash_accept(to_dev(g["draft"].astype(np.int32)), to_dev(target), wl.batch, K, tau_d)
        tau = tau_d.cpu().numpy()
        rec = osess.step(draft=check)
        assert np.array_equal(rec.block_ids, ids[seqs])
        assert np.array_equal(tau[seqs], rec.tau), (t, tau[seqs], rec.tau)
        if check:
            for i, b in enumerate(seqs):
                check_rows(f"step {t} logits[{b}]", g["logits"][b], rec.logits[i], tol(shape))
                check_argmax(g["draft"][b], rec.logits[i])
        # commit tau positions on the GPU side (oracle did it inside step)
        fe = [synth.step_features(shape, wl.seed, b, t, int(tau[b])) for b in range(wl.batch)]
        anchors = [draws[b].bonus for b in range(wl.batch)]
        assert osess.violations() == []
        if fused:
            pending, prev = fe, rec
            say(f"  step {t}: tau={tau.tolist()[:4]} (appended by the next step)")
            continue
        p.dfl.dflash_project_ctx(p.ctx, to_dev(np.concatenate(fe, axis=0)), [int(x) for x in tau])
        lens, caps = p.ctx.query()
        assert [lens[b] for b in seqs] == rec.ctx_len.tolist()
        assert [caps[b] for b in seqs] == rec.cap.tolist()
        say(f"  step {t}: tau={tau.tolist()[:4]} ctx={lens[:4]} cap={caps[:4]}")
    if pending is not None:
        p.dfl.dflash_project_ctx(p.ctx, to_dev(np.concatenate(pending, axis=0)), [len(f) for f in pending])
    p.check_state()
    return p


def test_session_workload0_tiny_fp32():
    """The tiny fp32 workload: 8 steps, every step compared."""
    say("case: session workload 0")
    wl = synth.workload(0)
    _session(wl.shape, wl, wl.steps)


def test_session_small_bf16_growth():
    say("case: session small bf16 with growth")
    wl = synth.workload(2).replace(shape=SMALL, ctx0=(60, 5), batch=2, a=(0.9, 0.7), K=10)
    _session(SMALL, wl, 12)


def test_fused_step_matches_oracle():
    """dflash_step (append + draft in one call, context K/V written by the
    QKV products) against the oracle's project + draft: logits, final hidden
    states, context buffer and caches; two sequences with 5 and 11 new rows,
    then one with none."""
    say("case: fused step small bf16")
    p = Pair(SMALL, 41, 2, gain_std=0.1)
    _prefill(p, [70, 33], seed=41)
    for t, n_new in enumerate([(5, 11), (0, 3), (17, 0)]):
        feats = [synth.step_features(SMALL, 41, b, t, n) for b, n in enumerate(n_new)]
        ids = _ids(41 + t, 2, 16, SMALL.vocab)
        g = p.gpu_step(feats, ids)
        for b in range(2):
            if n_new[b]:
                O.project_ctx(p.om, p.ost[b], feats[b])
            d_o, l_o, z_o = p.oracle_draft(b, ids[b])
            check_rows(f"t{t} logits[{b}]", g["logits"][b], l_o, tol(SMALL))
            check_rows(f"t{t} hidden[{b}]", g["hidden"][b], z_o, tol(SMALL))
            check_argmax(g["draft"][b], l_o)
        p.check_state()


def test_fused_step_fp32_and_large_append():
    """Tiny fp32 model: a fused step (8 rows) and one whose append is too
    large to fuse (two-call path inside dflash_step), both against the
    oracle."""
    say("case: fused step tiny fp32")
    wl = synth.workload(0)
    s = wl.shape
    p = Pair(s, 43, 1, gain_std=0.1)
    _prefill(p, [40], seed=43)
    for t, n in enumerate([8, 70]):
        feats = [synth.step_features(s, 43, 0, t, n)]
        ids = _ids(43 + t, 1, 8, s.vocab)
        g = p.gpu_step(feats, ids)
        O.project_ctx(p.om, p.ost[0], feats[0])
        d_o, l_o, z_o = p.oracle_draft(0, ids[0])
        check_rows(f"t{t} logits", g["logits"][0], l_o, tol(s))
        check_rows(f"t{t} hidden", g["hidden"][0], z_o, tol(s))
        check_argmax(g["draft"][0], l_o)
        p.check_state()


def test_fused_session_small_bf16_growth():
    say("case: fused session small bf16 with growth")
    wl = synth.workload(2).replace(shape=SMALL, ctx0=(60, 5), batch=2, a=(0.9, 0.7), K=10)
    _session(SMALL, wl, 12, fused=True)


@pytest.mark.slow
def test_fused_session_workload1_qwen3_4b_shape():
    """Workload 1 session through dflash_step (16 steps, logits at 0, 7, 15)."""
    say("case: fused session workload 1")
    wl = synth.workload(1)
    _session(wl.shape, wl, wl.steps, check_every=8, fused=True)


@pytest.mark.slow
def test_fused_session_workload2_llama_growth():
    """Workload 2 session through dflash_step: 64 steps with the first
    append growing the buffers from 4096 to 8192 rows."""
    say("case: fused session workload 2")
    wl = synth.workload(2)
    _session(wl.shape, wl, wl.steps, check_every=32, tail_check=(1,), fused=True)


@pytest.mark.slow
def test_workload1_qwen3_4b_shape_full_size():
    """Qwen3-4B-shaped drafter at full size: prefill 2048, one block compared
    in full, then a 16-step session (tau/ctx/cap every step, logits at
    steps 0, 7, 15)."""
    say("case: workload 1 full size")
    wl = synth.workload(1)
    _session(wl.shape, wl, wl.steps, check_every=8)


@pytest.mark.slow
def test_workload2_llama_shape_growth_session():
    """Llama-3.1-8B-shaped drafter, 64 steps of K=10 appends from a full
    4096-row buffer (grows to 8192 on the first step); outputs compared at
    steps 0, 1, 32, 63; tau/ctx/cap every step."""
    say("case: workload 2 full size")
    wl = synth.workload(2)
    _session(wl.shape, wl, wl.steps, check_every=32, tail_check=(1,))


@pytest.mark.slow
@pytest.mark.parametrize("K", [48, 128, 640])
def test_llama_shape_large_block(K):
    """Llama-3.1-8B-shaped drafter, one block over a 1500-row context, above
    the 32 rows where the products' activation precision used to drop:
    K=48 (three 16-row tiles: QKV and the k-split products in 32-row
    groups, gate/up in one 64-row group, the LM head on 64 rows), K=128
    (gate/up in two 64-row groups, the k-split products over 128 rows) and
    K=640 (five 128-row groups: gate/up and the LM head on the
    shared-activation kernel)."""
    say(f"case: llama shape, ctx 1500, K {K}")
    wl = synth.workload(2)
    p = Pair(wl.shape, wl.seed, 1, weights=_weights(wl.shape, wl.seed))
    _prefill(p, [1500], seed=wl.seed)
    ids = _ids(wl.seed + 1, 1, K, wl.shape.vocab)
    p.compare(ids, hidden=(K <= 128))


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_workload4_batched_long_context_all_sequences():
    """Batch 16, contexts 1k-20k (171k positions in all): the GPU runs all
    16 sequences in one ragged launch per kernel and the oracle follows
    every one of them for the whole 32-step session.  After the prefill and
    at the end, every sequence's context buffer and both caches of every
    layer are compared; tau, ctx_len and cap of every sequence are exact at
    every step; logits and argmax of all 16 sequences are compared at steps
    0, 1 and 31 (the oracle advances without drafting in between: tau
    depends only on the verifier's agreement draws)."""
    say("case: workload 4, all 16 sequences")
    wl = synth.workload(4).replace(steps=32)
    _session(wl.shape, wl, wl.steps, check_every=31, tail_check=(1,), keep_vocab=True)


_K_SWEEP = {}


@pytest.mark.slow
@pytest.mark.parametrize("K", [16, 32, 64, 128, 1024])
def test_workload3_k_sweep_blocks(K):
    """Qwen3-4B shape, context 4096, each block size of the sweep (one
    prefilled context shared by the five block sizes)."""
    say(f"case: workload 3 K={K}")
    wl = synth.workload(3)
    if "p" not in _K_SWEEP:
        p = Pair(wl.shape, wl.seed, 1, weights=_weights(wl.shape, wl.seed))
        _prefill(p, [4096], seed=wl.seed)
        p.check_state()
        _K_SWEEP["p"] = p
    p = _K_SWEEP["p"]
    ids = _ids(wl.seed, 1, K, wl.shape.vocab)
    _, stats = p.compare(ids, hidden=(K <= 128))
    say(f"  errors {stats}")
