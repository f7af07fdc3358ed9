"""GPU parity of dflash_decay_ce (loss-decay weighted cross-entropy) against
the fp64 oracle (oracle/loss.py) on the same seeded inputs.

kongchang.com, "D-Flash", "Innovation 4: loss-decay weighted training" and
"Innovation 3: random anchor sampling".

Tolerances follow from the kernel's fp32 arithmetic (sums of exponentials
in fp32 per thread then over the workgroup, about 170 roundings deep, and a
hardware 2^x of about 1 ulp):
  * ce and loss: |gpu - oracle| <= 5e-5 + 1e-5 |oracle|;
  * gradient in fp32: an exponent error of at most ~3e-5 (base 2) gives a
    relative error of at most 4e-5 per element; at the target, where
    p_t - 1 cancels, the bound is 4e-5 of the row scale c_r = w_r / sum w;
  * gradient in bf16: the same plus one rounding to bf16 (7 stored mantissa
    bits: at most 2^-8 relative).
Outputs below 1e-37 may be flushed to zero.
"""
import numpy as np
import pytest
import torch

import block_diffusion_drafting_amd as dfl
import synth
from oracle import dflash as O
from oracle import loss as OL
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _upload(L, dtype, offset=0):
    """Logits to the device; offset > 0 places them `offset` elements into a
    larger buffer (a base that is not 16-byte aligned)."""
    rows, V = L.shape
    flat = np.ascontiguousarray(L).reshape(-1)
    if dtype == "bf16":
        src = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16)
    else:
        src = torch.from_numpy(flat)
    buf = torch.empty(rows * V + offset, dtype=TORCH_DT[dtype], device="cuda")
    buf[offset:].copy_(src.cuda())
    return buf[offset:].view(rows, V)


def _to_np64(t, dtype):
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return O.to_f64(t.view(torch.int16).numpy().view(np.uint16), "bf16")
    return t.numpy().astype(np.float64)


def _gpu(L, t, dtype, block, gamma, want_grad=True, offset=0):
    rows, V = L.shape
    d_L = _upload(L, dtype, offset)
    d_t = torch.from_numpy(np.ascontiguousarray(t, dtype=np.int32)).cuda()
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    ce = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    grad = torch.full((rows, V), float("nan"), dtype=TORCH_DT[dtype], device="cuda") if want_grad else None
    dfl.dflash_decay_ce(d_L, d_t, block, gamma, loss, ce, grad)
    torch.cuda.synchronize()
    return (float(loss.item()), ce.cpu().numpy().astype(np.float64),
            _to_np64(grad, dtype) if want_grad else None)


def _check(L, t, dtype, block, gamma, got, rows_to_check=None):
    loss, ce, grad = got
    Lf = O.to_f64(L, dtype)
    rl, rg, rce = OL.decay_ce(Lf, t, block, gamma, want_grad=grad is not None)
    assert np.isfinite(loss) and abs(loss - rl) <= 5e-5 + 1e-5 * abs(rl), f"loss {loss} vs {rl}"
    err = np.abs(ce - rce)
    assert np.all(err <= 5e-5 + 1e-5 * np.abs(rce)), f"ce: max err {err.max():.3e} at row {err.argmax()}"
    if grad is None:
        return
    rows = np.arange(L.shape[0]) if rows_to_check is None else np.asarray(rows_to_check)
    valid = (t >= 0) & (t < L.shape[1])
    w = np.where(valid, np.power(float(gamma), np.arange(L.shape[0]) % block), 0.0)
    W = w.sum()
    c = w / W if W > 0 else np.zeros_like(w)
    rel = 4e-5 + (2.0 ** -8 if dtype == "bf16" else 0.0)
    for r in rows:
        g, ref = grad[r], rg[r]
        bound = rel * np.abs(ref) + 1e-37
        if valid[r]:
            bound[t[r]] += 4e-5 * c[r]
        bad = np.abs(g - ref) > bound
        assert not bad.any(), (f"grad row {r}: {int(bad.sum())} elements out of bound, e.g. col "
                               f"{int(np.argmax(bad))}: {g[np.argmax(bad)]} vs {ref[np.argmax(bad)]}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1000, 1001, 20000, 8])
def test_decay_ce_matches_oracle(dtype, V):
    """37 rows = two blocks of 16 and a ragged block of 5; V = 1000 (one
    16-byte vector per thread), 1001 (rows not 16-byte aligned: the two-pass
    kernel), 20000 (several register slots), 8 (one vector per row)."""
    say(f"decay_ce dtype={dtype} V={V}")
    L, t = synth.ce_inputs(11, 37, V, 16, dtype)
    _check(L, t, dtype, 16, 0.8, _gpu(L, t, dtype, 16, 0.8))


@pytest.mark.parametrize("dtype,V", [("bf16", 1000), ("f32", 5000), ("bf16", 40000), ("f32", 4000)])
def test_decay_ce_many_rows_per_workgroup(dtype, V):
    """1100 rows: more than the resident workgroups, so each workgroup runs
    several rows, loading its next row while it writes the current one's
    gradient (1, 2, 5 and 1 register slots)."""
    say(f"decay_ce many rows dtype={dtype} V={V}")
    L, t = synth.ce_inputs(18, 1100, V, 16, dtype)
    _check(L, t, dtype, 16, 0.8, _gpu(L, t, dtype, 16, 0.8))
    _check(L, t, dtype, 16, 0.8, _gpu(L, t, dtype, 16, 0.8, want_grad=False))


@pytest.mark.parametrize("block,gamma", [(1, 0.8), (16, 1.0), (16, 0.5), (7, 0.9)])
def test_decay_ce_block_and_gamma(block, gamma):
    say(f"decay_ce block={block} gamma={gamma}")
    L, t = synth.ce_inputs(12, 50, 4096, block, "bf16")
    _check(L, t, "bf16", block, gamma, _gpu(L, t, "bf16", block, gamma))


@pytest.mark.parametrize("dtype,rows", [("bf16", 24), ("f32", 6)])
def test_decay_ce_qwen_vocab_with_masked_tail(dtype, rows):
    """Vocabulary 151936 with its last 267 entries at -inf (never targets):
    bf16 keeps the row in registers (19 slots), fp32 rows exceed the register
    budget and take the two-pass kernel."""
    say(f"decay_ce qwen vocab dtype={dtype} rows={rows}")
    L, t = synth.ce_inputs(13, rows, 151936, 16, dtype, masked_tail=267)
    got = _gpu(L, t, dtype, 16, 0.8)
    _check(L, t, dtype, 16, 0.8, got)
    assert np.all(got[2][:, -267:] == 0.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decay_ce_unaligned_base_takes_two_pass_kernel(dtype):
    say(f"decay_ce unaligned dtype={dtype}")
    L, t = synth.ce_inputs(14, 20, 2048, 16, dtype)
    got = _gpu(L, t, dtype, 16, 0.8, offset=1)
    _check(L, t, dtype, 16, 0.8, got)
    ref = _gpu(L, t, dtype, 16, 0.8)
    assert got[0] == pytest.approx(ref[0], abs=5e-5)


def test_decay_ce_edge_cases():
    say("decay_ce edge cases")
    # no rows: loss 0
    loss = torch.full((1,), 7.0, device="cuda")
    empty = torch.empty((0, 100), dtype=torch.bfloat16, device="cuda")
    dfl.dflash_decay_ce(empty, torch.empty(0, dtype=torch.int32, device="cuda"), 16, 0.8, loss,
                        torch.empty(0, device="cuda"))
    assert loss.item() == 0.0
    # every row without a token: loss 0, ce 0, gradient 0
    L, _ = synth.ce_inputs(15, 20, 512, 16, "bf16")
    t = np.full(20, -1, np.int32)
    t[3] = 512  # out of range counts as no token
    loss_v, ce, grad = _gpu(L, t, "bf16", 16, 0.8)
    assert loss_v == 0.0 and np.all(ce == 0.0) and np.all(grad == 0.0)
    # a single row
    L, t = synth.ce_inputs(16, 1, 300, 16, "f32")
    t[0] = 5
    _check(L, t, "f32", 16, 0.8, _gpu(L, t, "f32", 16, 0.8))


def test_decay_ce_argument_errors():
    L = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    t = torch.zeros(4, dtype=torch.int32, device="cuda")
    loss, ce = torch.zeros(1, device="cuda"), torch.zeros(4, device="cuda")
    for block, gamma in ((0, 0.8), (16, 0.0), (16, -1.0), (16, float("inf")), (16, float("nan"))):
        with pytest.raises(dfl.DFlashError):
            dfl.dflash_decay_ce(L, t, block, gamma, loss, ce)


def test_decay_ce_deterministic_and_grad_optional():
    say("decay_ce determinism")
    L, t = synth.ce_inputs(17, 300, 30000, 16, "bf16")
    a = _gpu(L, t, "bf16", 16, 0.8)
    b = _gpu(L, t, "bf16", 16, 0.8)
    c = _gpu(L, t, "bf16", 16, 0.8, want_grad=False)
    assert a[0] == b[0] == c[0]
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[1], c[1])
    assert np.array_equal(a[2], b[2])


@pytest.mark.timeout(400)
def test_decay_ce_full_size_qwen_vocab():
    """The benchmarked launch: 256 blocks of 16 rows, vocabulary 151936 with a
    267-entry -inf tail, bf16; loss and every row's CE against the oracle,
    the gradient on sampled rows (first, last, ragged spread)."""
    say("decay_ce full size: generating")
    L, t = synth.ce_inputs(2026, 4096, 151936, 16, "bf16", masked_tail=267)
    say("decay_ce full size: gpu")
    got = _gpu(L, t, "bf16", 16, 0.8)
    say("decay_ce full size: oracle")
    rng = np.random.default_rng(0)
    sample = np.unique(np.concatenate([[0, 1, 15, 16, 4095], rng.integers(0, 4096, 27)]))
    _check(L, t, "bf16", 16, 0.8, got, rows_to_check=sample)
