"""The C ABI library loads, exports every symbol include/dflash.h declares,
and rejects bad arguments on the host (no GPU needed for any of this)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")
LIB = os.path.join(ROOT, "block_diffusion_drafting_amd", "libdflash.so")


def _ensure_built():
    if not os.path.exists(LIB):
        from block_diffusion_drafting_amd import build
        build.build()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("dflash_project_ctx", "dflash_draft_block", "dflash_accept"):
        assert n in names


def test_library_exports_every_declared_symbol():
    _ensure_built()
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_header():
    _ensure_built()
    import block_diffusion_drafting_amd as dfl
    assert set(dfl.EXPORTS) == set(declared_functions())


def test_version_and_abi():
    _ensure_built()
    import block_diffusion_drafting_amd as dfl
    assert dfl.lib.dflash_abi_version() == 1
    assert "gfx950" in dfl.version()


def test_host_side_argument_errors():
    """Calls rejected before any device work: status codes and messages."""
    _ensure_built()
    import block_diffusion_drafting_amd as dfl
    L = dfl.lib
    assert L.dflash_accept(None, None, 1, 4, None, None) == -1
    assert b"NULL" in L.dflash_last_error()
    one = ctypes.c_void_p(16)
    assert L.dflash_accept(one, one, 1, 0, one, None) == -1          # K = 0
    assert L.dflash_accept(one, one, 1, 1025, one, None) == -1       # K too large
    assert L.dflash_accept(one, one, 0, 4, one, None) == -1          # empty batch
    assert L.dflash_draft_block(None, one, 4, one, None, None, None) == -1
    assert L.dflash_project_ctx(None, None, None, None, None) == -1
    h = ctypes.c_void_p()
    assert L.dflash_model_create(None, None, None, None, ctypes.byref(h)) == -1

    class S:
        hidden, n_layers, n_q_heads, n_kv_heads, head_dim = 100, 1, 4, 2, 64
        intermediate, vocab, n_feat, rope_theta, rms_eps, dtype = 64, 10, 1, 1e4, 1e-6, "f32"
    cfg = dfl.config_struct(S)
    w = dfl._Weights()
    assert L.dflash_model_create(ctypes.byref(cfg), ctypes.byref(w), None, None, ctypes.byref(h)) == -2
    assert b"hidden" in L.dflash_last_error()
    S.hidden, S.head_dim = 128, 48
    cfg = dfl.config_struct(S)
    assert L.dflash_model_create(ctypes.byref(cfg), ctypes.byref(w), None, None, ctypes.byref(h)) == -2
    S.head_dim, S.n_q_heads, S.n_kv_heads = 64, 3, 2
    cfg = dfl.config_struct(S)
    assert L.dflash_model_create(ctypes.byref(cfg), ctypes.byref(w), None, None, ctypes.byref(h)) == -2
    S.n_q_heads = 4
    cfg = dfl.config_struct(S)
    # valid shape, NULL weights
    assert L.dflash_model_create(ctypes.byref(cfg), ctypes.byref(w), None, None, ctypes.byref(h)) == -1
    assert L.dflash_ctx_create(None, 1, None, None, None, ctypes.byref(h)) == -1
    assert L.dflash_ctx_query(None, None, None) == -1
