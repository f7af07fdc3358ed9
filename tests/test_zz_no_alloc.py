"""dflash_decay_ce_noalloc (the decay-CE call whose workspace is the
library's static per-GPU array, for callers that cannot allocate) against
dflash_decay_ce with a caller workspace, through the C ABI, on the same
seeded inputs: two calls in a row, the second with fewer rows and a smaller
vocabulary, so the second finds the array holding the first call's weight
sum.  The two entry points run the same kernels in the same order, so the
bar is bitwise equality of the loss, the per-row CE and the gradient (the
decay-CE parity bar against the oracle is met by dflash_decay_ce)."""
import ctypes

import numpy as np
import pytest
import torch

import block_diffusion_drafting_amd as dfl
import synth

pytestmark = pytest.mark.gpu


def _case(rows, vocab, block, gamma, dtype, seed):
    L, t = synth.ce_inputs(seed, rows, vocab, block, dtype)
    if dtype == "bf16":
        d_L = torch.from_numpy(L.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        d_L = torch.from_numpy(L).cuda()
    return d_L, torch.from_numpy(t).cuda()


def _run(fn_name, d_L, d_t, block, gamma):
    rows, vocab = d_L.shape
    loss = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    ce = torch.full((rows,), -1.0, dtype=torch.float32, device="cuda")
    grad = torch.empty_like(d_L)
    dt = dfl.DFLASH_BF16 if d_L.dtype == torch.bfloat16 else dfl.DFLASH_F32
    s = torch.cuda.current_stream().cuda_stream
    f = getattr(dfl.lib, fn_name)
    if fn_name == "dflash_decay_ce":
        ws = torch.zeros(dfl.DECAY_CE_WORKSPACE, dtype=torch.uint8, device="cuda")
        st = f(d_L.data_ptr(), dt, d_t.data_ptr(), rows, vocab, block, ctypes.c_double(gamma), loss.data_ptr(),
               ce.data_ptr(), grad.data_ptr(), ws.data_ptr(), s)
    else:
        st = f(d_L.data_ptr(), dt, d_t.data_ptr(), rows, vocab, block, ctypes.c_double(gamma), loss.data_ptr(),
               ce.data_ptr(), grad.data_ptr(), s)
    assert st == 0, dfl.lib.dflash_last_error()
    torch.cuda.synchronize()
    return loss.cpu().numpy(), ce.cpu().numpy(), grad.view(torch.int16 if d_L.dtype == torch.bfloat16
                                                           else torch.int32).cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_call_twice(dtype):
    cases = [(600, 20000, 16, 0.8, 11), (37, 1001, 8, 0.5, 12)]   # the second call smaller
    for rows, vocab, block, gamma, seed in cases:
        d_L, d_t = _case(rows, vocab, block, gamma, dtype, seed)
        a = _run("dflash_decay_ce_noalloc", d_L, d_t, block, gamma)
        b = _run("dflash_decay_ce", d_L, d_t, block, gamma)
        for x, y, name in zip(a, b, ("loss", "ce", "grad")):
            assert np.array_equal(x, y), f"{dtype} rows={rows} vocab={vocab}: {name} differs"
        assert np.isfinite(a[0]).all() and a[0][0] > 0


def test_noalloc_zero_rows_and_errors():
    loss = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    f = dfl.lib.dflash_decay_ce_noalloc
    assert f(None, dfl.DFLASH_F32, None, 0, 10, 4, ctypes.c_double(0.9), loss.data_ptr(), None, None, s) == 0
    torch.cuda.synchronize()
    assert float(loss.item()) == 0.0
    assert f(None, dfl.DFLASH_F32, None, 3, 10, 4, ctypes.c_double(0.9), loss.data_ptr(), None, None, s) == -1
    assert f(None, dfl.DFLASH_F32, None, 0, 10, 0, ctypes.c_double(0.9), loss.data_ptr(), None, None, s) == -1
    assert f(None, dfl.DFLASH_F32, None, 0, 10, 4, ctypes.c_double(0.0), loss.data_ptr(), None, None, s) == -1
    assert f(None, 7, None, 0, 10, 4, ctypes.c_double(0.9), loss.data_ptr(), None, None, s) == -1
