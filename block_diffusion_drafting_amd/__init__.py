"""Python binding of libdflash.so, the DFlash draft-block path for MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in ``include/dflash.h``.  PyTorch supplies device
memory (through the allocator callbacks) and streams.  The library is loaded
on first use; every call raises ImportError if it has not been built.  There
is no other code path.

Entry points keep the C names:
  dflash_model_create / Model      repack drafter weights
  dflash_ctx_create / Context      per-sequence proposer state
  dflash_project_ctx               (a1)-(a3) project + append + KV injection
  dflash_draft_block               (a4)-(a9) one non-causal draft forward
  dflash_accept                    (a10) greedy acceptance
  dflash_decay_ce                  loss-decay weighted cross-entropy (training)
  dflash_target_create / Model(target=True), dflash_verify_block,
  dflash_commit                    target-side block verification
  dflash_adapt_* / AdaptPolicy     adaptive block size (host)
"""
from __future__ import annotations

import atexit
import contextlib
import ctypes
import os
import sys
import weakref
from typing import Dict, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

DFLASH_F32, DFLASH_BF16 = 0, 1
MAX_BATCH, MAX_K = 256, 1024
DECAY_CE_WORKSPACE = 256


class DFlashError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> status {status}: {msg}")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("n_feat", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_double),
                ("dtype", ctypes.c_int)]


class _LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")]


class _Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("fc", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(_LayerWeights))]


_ALLOC_FN = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p)
_FREE_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p)


class _Allocator(ctypes.Structure):
    _fields_ = [("alloc", _ALLOC_FN), ("free", _FREE_FN), ("user", ctypes.c_void_p)]


EXPORTS = ("dflash_version", "dflash_abi_version", "dflash_last_error", "dflash_model_create",
           "dflash_model_destroy", "dflash_model_bytes", "dflash_ctx_create",
           "dflash_ctx_destroy", "dflash_project_ctx", "dflash_draft_block", "dflash_step",
           "dflash_accept", "dflash_decay_ce", "dflash_decay_ce_noalloc", "dflash_target_create", "dflash_verify_block",
           "dflash_commit", "dflash_adapt_create", "dflash_adapt_destroy", "dflash_adapt_observe",
           "dflash_adapt_choose",
           "dflash_ctx_query", "dflash_ctx_buffers", "dflash_ctx_set_persistent",
           "dflash_ctx_persistent_path", "dflash_ctx_check", "dflash_persist_trace",
           "dflash_profile_enable",
           "dflash_profile_read", "dflash_phase_name")
NUM_PHASES = 16


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_diffusion_drafting_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    sig = {
        "dflash_version": ([], ctypes.c_char_p),
        "dflash_abi_version": ([], i32),
        "dflash_last_error": ([], ctypes.c_char_p),
        "dflash_model_create": ([ctypes.POINTER(_Config), ctypes.POINTER(_Weights),
                                 ctypes.POINTER(_Allocator), vp, ctypes.POINTER(vp)], ctypes.c_int),
        "dflash_model_destroy": ([vp], ctypes.c_int),
        "dflash_model_bytes": ([vp, i64p, i64p, i64p], ctypes.c_int),
        "dflash_ctx_create": ([vp, i32, i32p, ctypes.POINTER(_Allocator), vp, ctypes.POINTER(vp)],
                              ctypes.c_int),
        "dflash_ctx_destroy": ([vp], ctypes.c_int),
        "dflash_project_ctx": ([vp, vp, i32p, vp, vp], ctypes.c_int),
        "dflash_draft_block": ([vp, vp, i32, vp, vp, vp, vp], ctypes.c_int),
        "dflash_step": ([vp, vp, ctypes.POINTER(ctypes.c_int32), vp, i32, vp, vp, vp, vp], ctypes.c_int),
        "dflash_accept": ([vp, vp, i32, i32, vp, vp], ctypes.c_int),
        "dflash_decay_ce": ([vp, ctypes.c_int, vp, i32, i32, i32, ctypes.c_double, vp, vp, vp, vp, vp],
                            ctypes.c_int),
        "dflash_decay_ce_noalloc": ([vp, ctypes.c_int, vp, i32, i32, i32, ctypes.c_double, vp, vp, vp, vp],
                                    ctypes.c_int),
        "dflash_target_create": ([ctypes.POINTER(_Config), ctypes.POINTER(_Weights), i32p,
                                  ctypes.POINTER(_Allocator), vp, ctypes.POINTER(vp)], ctypes.c_int),
        "dflash_verify_block": ([vp, vp, i32, vp, vp, vp, vp], ctypes.c_int),
        "dflash_commit": ([vp, i32p, vp], ctypes.c_int),
        "dflash_adapt_create": ([i32, ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                 ctypes.POINTER(vp)], ctypes.c_int),
        "dflash_adapt_destroy": ([vp], ctypes.c_int),
        "dflash_adapt_observe": ([vp, i32, i32], ctypes.c_int),
        "dflash_adapt_choose": ([vp, i32p, ctypes.POINTER(ctypes.c_double), i32, i32p,
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        "dflash_ctx_query": ([vp, i32p, i32p], ctypes.c_int),
        "dflash_ctx_buffers": ([vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                ctypes.POINTER(vp), i32p], ctypes.c_int),
        "dflash_ctx_set_persistent": ([vp, i32], ctypes.c_int),
        "dflash_ctx_persistent_path": ([vp, i32, i32p], ctypes.c_int),
        "dflash_ctx_check": ([vp, vp], ctypes.c_int),
        "dflash_persist_trace": ([vp, ctypes.POINTER(ctypes.c_uint64), ctypes.c_int64, i32p, i32p], ctypes.c_int),
        "dflash_profile_enable": ([vp, ctypes.c_uint32], ctypes.c_int),
        "dflash_profile_read": ([vp, ctypes.POINTER(ctypes.c_double), i64p], ctypes.c_int),
        "dflash_phase_name": ([i32], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


class _Lib:
    """Loads libdflash.so on first use (so that the build step can import
    this package before the library exists); raises ImportError if it is
    missing."""
    _cdll = None

    def __getattr__(self, name):
        if _Lib._cdll is None:
            _Lib._cdll = _load()
        return getattr(_Lib._cdll, name)


lib = _Lib()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise DFlashError(fn, status, lib.dflash_last_error().decode(errors="replace"))


def _stream(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _on(stream: Optional[torch.cuda.Stream]):
    """Makes the call's stream torch's current stream while the library may
    allocate or free (growth, workspaces): TorchAllocator then serves and
    releases blocks on that stream, so torch reuses them only after the work
    queued there."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


# Live handles, closed before interpreter shutdown: destroying a context or a
# model frees device memory through Python callbacks into torch's allocator,
# which must still be alive then.
_LIVE: "weakref.WeakSet" = weakref.WeakSet()


def _close_all() -> None:
    objs = list(_LIVE)
    if not objs:
        return
    try:
        if torch.cuda.is_initialized():
            torch.cuda.synchronize()
    except Exception:
        pass
    for kind in (Context, Model, AdaptPolicy):
        for o in objs:
            if isinstance(o, kind):
                try:
                    o.close()
                except Exception:
                    pass


atexit.register(_close_all)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


class TorchAllocator:
    """Device allocations served by PyTorch's caching allocator on ``device``."""

    def __init__(self, device: torch.device):
        self.device = torch.device(device)
        self.live: Dict[int, torch.Tensor] = {}
        self._a = _ALLOC_FN(self._alloc)
        self._f = _FREE_FN(self._free)
        self.struct = _Allocator(self._a, self._f, None)

    def _alloc(self, n: int, user) -> int:
        try:
            t = torch.empty(int(n), dtype=torch.uint8, device=self.device)
        except Exception:      # out of memory: the library reports DFLASH_E_ALLOC
            return 0
        p = t.data_ptr()
        self.live[p] = t
        return p

    def _free(self, p: int, user, _finalizing=sys.is_finalizing) -> None:
        t = self.live.pop(int(p) if p else 0, None)
        if t is not None and not _finalizing():
            # work queued on the freeing call's stream (torch's current stream
            # during the call) may still use the block: torch reuses it only
            # after that work, also when it was allocated on another stream
            try:
                t.record_stream(torch.cuda.current_stream(self.device))
            except Exception:
                pass

    @property
    def bytes(self) -> int:
        return sum(t.numel() for t in self.live.values())


def config_struct(shape) -> _Config:
    """``shape``: any object with the fields of ``dflash_config`` (dtype "bf16"/"f32")."""
    return _Config(shape.hidden, shape.n_layers, shape.n_q_heads, shape.n_kv_heads,
                   shape.head_dim, shape.intermediate, shape.vocab, shape.n_feat,
                   float(shape.rope_theta), float(shape.rms_eps),
                   DFLASH_BF16 if shape.dtype == "bf16" else DFLASH_F32)


class Model:
    """dflash_model_create / dflash_model_destroy (a drafter), or with
    ``taps`` given, dflash_target_create (a verification target whose
    ``shape.n_feat`` equals ``len(taps)``).

    ``weights``: device tensors keyed ``embed``, ``lm_head``, ``fc`` (drafter
    only), ``final_norm`` and ``layers.{l}.{attn_norm,wq,wk,wv,wo,mlp_norm,
    w_gate,w_up,w_down}`` in the model dtype (bf16 may be given as uint16
    bits).  ``embed`` stays borrowed: this object keeps a reference to it.
    """

    def __init__(self, shape, weights: Dict[str, torch.Tensor], device="cuda",
                 stream: Optional[torch.cuda.Stream] = None, taps: Optional[Sequence[int]] = None):
        self.shape = shape
        self.target = taps is not None
        self.taps = list(taps) if taps is not None else []
        self.device = torch.device(device)
        self.alloc = TorchAllocator(self.device)
        self._embed = weights["embed"]
        L = shape.n_layers
        keys = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")
        layers = (_LayerWeights * max(L, 1))()
        for l in range(L):
            for k in keys:
                setattr(layers[l], k, _ptr(weights[f"layers.{l}.{k}"]))
        w = _Weights(_ptr(weights["embed"]), _ptr(weights["lm_head"]),
                     None if self.target else _ptr(weights["fc"]), _ptr(weights["final_norm"]), layers)
        cfg = config_struct(shape)
        h = ctypes.c_void_p()
        if self.target:
            if len(self.taps) != shape.n_feat:
                raise ValueError("a target's shape.n_feat must equal len(taps)")
            tp = (ctypes.c_int32 * max(len(self.taps), 1))(*[int(t) for t in self.taps])
            with _on(stream):
                _check("dflash_target_create",
                       lib.dflash_target_create(ctypes.byref(cfg), ctypes.byref(w), tp,
                                                ctypes.byref(self.alloc.struct), _stream(stream),
                                                ctypes.byref(h)))
        else:
            with _on(stream):
                _check("dflash_model_create",
                       lib.dflash_model_create(ctypes.byref(cfg), ctypes.byref(w),
                                               ctypes.byref(self.alloc.struct), _stream(stream),
                                               ctypes.byref(h)))
        self.handle = h
        _LIVE.add(self)

    def bytes(self):
        a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check("dflash_model_bytes", lib.dflash_model_bytes(self.handle, ctypes.byref(a),
                                                            ctypes.byref(b), ctypes.byref(c)))
        return {"layers": a.value, "lm_head": b.value, "proj": c.value}

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib.dflash_model_destroy(self.handle)
            self.handle = None

    def __del__(self, _finalizing=sys.is_finalizing):
        # (bound at definition: module globals may already be None at exit)
        if _finalizing():            # closed by the atexit hook, or torch is gone
            return
        try:
            self.close()
        except Exception:
            pass


class Context:
    """dflash_ctx_create / dflash_ctx_destroy: proposer state for ``batch`` sequences."""

    def __init__(self, model: Model, batch: int, init_cap: Optional[Sequence[int]] = None,
                 stream: Optional[torch.cuda.Stream] = None):
        self.model = model
        self.batch = batch
        self.alloc = TorchAllocator(model.device)
        caps = None
        if init_cap is not None:
            caps = (ctypes.c_int32 * batch)(*[int(c) for c in init_cap])
        h = ctypes.c_void_p()
        with _on(stream):
            _check("dflash_ctx_create",
                   lib.dflash_ctx_create(model.handle, batch, caps, ctypes.byref(self.alloc.struct),
                                         _stream(stream), ctypes.byref(h)))
        self.handle = h
        _LIVE.add(self)

    def query(self):
        a = (ctypes.c_int32 * self.batch)()
        b = (ctypes.c_int32 * self.batch)()
        _check("dflash_ctx_query", lib.dflash_ctx_query(self.handle, a, b))
        return list(a), list(b)

    def buffers(self, b: int):
        c, k, v = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        phys = ctypes.c_int32()
        _check("dflash_ctx_buffers", lib.dflash_ctx_buffers(self.handle, b, ctypes.byref(c),
                                                            ctypes.byref(k), ctypes.byref(v),
                                                            ctypes.byref(phys)))
        return c.value, k.value, v.value, phys.value

    def set_persistent(self, enable: bool) -> None:
        """dflash_ctx_set_persistent: the single-launch draft block on / off."""
        _check("dflash_ctx_set_persistent", lib.dflash_ctx_set_persistent(self.handle, 1 if enable else 0))

    def persistent_path(self, K: int) -> bool:
        """dflash_ctx_persistent_path: whether a block of K rows per sequence
        runs as one launch on this device."""
        y = ctypes.c_int32()
        _check("dflash_ctx_persistent_path", lib.dflash_ctx_persistent_path(self.handle, int(K), ctypes.byref(y)))
        return bool(y.value)

    def check(self, stream: Optional[torch.cuda.Stream] = None) -> None:
        """dflash_ctx_check: raises DFlashError if a single-launch block on
        this context was abandoned (an expired barrier wait)."""
        _check("dflash_ctx_check", lib.dflash_ctx_check(self.handle, _stream(stream)))

    def persist_trace(self):
        """dflash_persist_trace: the last profiled single-launch block's
        timeline as a [workgroups, slots] uint64 array of 100 MHz ticks (or
        None)."""
        import numpy as np
        nwg, stride = ctypes.c_int32(), ctypes.c_int32()
        _check("dflash_persist_trace", lib.dflash_persist_trace(self.handle, None, 0, ctypes.byref(nwg),
                                                                ctypes.byref(stride)))
        if nwg.value == 0:
            return None
        out = np.zeros(nwg.value * stride.value, np.uint64)
        _check("dflash_persist_trace",
               lib.dflash_persist_trace(self.handle, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                        out.size, ctypes.byref(nwg), ctypes.byref(stride)))
        return out.reshape(nwg.value, stride.value)

    def profile(self, enable=True) -> None:
        """Time phases with HIP events: True = every phase, False = off, a
        name or a list of names = those phases only."""
        if enable is True:
            mask = (1 << NUM_PHASES) - 1
        elif not enable:
            mask = 0
        else:
            names = [enable] if isinstance(enable, str) else list(enable)
            known = [lib.dflash_phase_name(i).decode() for i in range(NUM_PHASES)]
            mask = 0
            for n in names:
                if n not in known:
                    raise ValueError(f"unknown phase {n!r}")
                mask |= 1 << known.index(n)
        _check("dflash_profile_enable", lib.dflash_profile_enable(self.handle, mask))

    def profile_read(self):
        """{phase name: (total ms, launches)} since the last read."""
        ms = (ctypes.c_double * NUM_PHASES)()
        cnt = (ctypes.c_int64 * NUM_PHASES)()
        _check("dflash_profile_read", lib.dflash_profile_read(self.handle, ms, cnt))
        return {lib.dflash_phase_name(i).decode(): (ms[i], cnt[i]) for i in range(NUM_PHASES) if cnt[i]}

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib.dflash_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self, _finalizing=sys.is_finalizing):
        # (bound at definition: module globals may already be None at exit)
        if _finalizing():            # closed by the atexit hook, or torch is gone
            return
        try:
            self.close()
        except Exception:
            pass


def dflash_project_ctx(ctx: Context, feats: torch.Tensor, n_new: Sequence[int],
                       positions: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None) -> None:
    nn = (ctypes.c_int32 * ctx.batch)(*[int(n) for n in n_new])
    if positions is not None and positions.dtype != torch.int32:
        raise ValueError("positions must be int32")
    with _on(stream):
        _check("dflash_project_ctx",
               lib.dflash_project_ctx(ctx.handle, _ptr(feats) if feats is not None and feats.numel() else None,
                                      nn, _ptr(positions), _stream(stream)))


def dflash_draft_block(ctx: Context, block_ids: torch.Tensor, K: int, draft_ids: torch.Tensor,
                       logits: Optional[torch.Tensor] = None, hidden: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None) -> None:
    for t, dt in ((block_ids, torch.int32), (draft_ids, torch.int32)):
        if t.dtype != dt or t.numel() != ctx.batch * K:
            raise ValueError("block_ids / draft_ids must be int32 [batch, K]")
    if logits is not None and (logits.dtype != torch.float32 or
                               logits.numel() != ctx.batch * K * ctx.model.shape.vocab):
        raise ValueError("logits must be float32 [batch, K, vocab]")
    with _on(stream):
        _check("dflash_draft_block",
               lib.dflash_draft_block(ctx.handle, _ptr(block_ids), int(K), _ptr(draft_ids),
                                      _ptr(logits), _ptr(hidden), _stream(stream)))


def dflash_step(ctx: Context, feats: Optional[torch.Tensor], n_new: Sequence[int], block_ids: torch.Tensor,
                K: int, draft_ids: torch.Tensor, logits: Optional[torch.Tensor] = None,
                hidden: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None) -> None:
    """dflash_project_ctx(feats, n_new) then dflash_draft_block(...), fused."""
    nn = (ctypes.c_int32 * ctx.batch)(*[int(n) for n in n_new])
    for t, dt in ((block_ids, torch.int32), (draft_ids, torch.int32)):
        if t.dtype != dt or t.numel() != ctx.batch * K:
            raise ValueError("block_ids / draft_ids must be int32 [batch, K]")
    if logits is not None and (logits.dtype != torch.float32 or
                               logits.numel() != ctx.batch * K * ctx.model.shape.vocab):
        raise ValueError("logits must be float32 [batch, K, vocab]")
    with _on(stream):
        _check("dflash_step",
               lib.dflash_step(ctx.handle, _ptr(feats) if feats is not None and feats.numel() else None, nn,
                               _ptr(block_ids), int(K), _ptr(draft_ids), _ptr(logits), _ptr(hidden),
                               _stream(stream)))


def dflash_accept(draft_ids: torch.Tensor, target_ids: torch.Tensor, batch: int, K: int,
                  accept_len: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> None:
    for t in (draft_ids, target_ids, accept_len):
        if t.dtype != torch.int32:
            raise ValueError("int32 tensors expected")
    if draft_ids.numel() != batch * K or target_ids.numel() != batch * K or accept_len.numel() != batch:
        raise ValueError("shape mismatch")
    _check("dflash_accept", lib.dflash_accept(_ptr(draft_ids), _ptr(target_ids), int(batch), int(K),
                                              _ptr(accept_len), _stream(stream)))


def dflash_decay_ce(logits: torch.Tensor, targets: torch.Tensor, block: int, gamma: float,
                    loss: torch.Tensor, ce: torch.Tensor, grad: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None) -> None:
    """Loss-decay weighted cross-entropy of logits [rows, vocab] (float32 or
    bfloat16): loss [1] float32, per-row ce [rows] float32 and, if given,
    grad [rows, vocab] in the logits' dtype.  workspace: a device tensor of
    at least DECAY_CE_WORKSPACE bytes (allocated here if None)."""
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [rows, vocab] tensor")
    if logits.dtype == torch.bfloat16:
        dt = DFLASH_BF16
    elif logits.dtype == torch.float32:
        dt = DFLASH_F32
    else:
        raise ValueError("logits must be float32 or bfloat16")
    rows, vocab = logits.shape
    if targets.dtype != torch.int32 or targets.numel() != rows:
        raise ValueError("targets must be int32 [rows]")
    if loss.dtype != torch.float32 or loss.numel() < 1 or ce.dtype != torch.float32 or ce.numel() != rows:
        raise ValueError("loss [1] and ce [rows] must be float32")
    if grad is not None and (grad.dtype != logits.dtype or grad.shape != logits.shape or
                             not grad.is_contiguous()):
        raise ValueError("grad must match logits")
    if workspace is None:
        workspace = torch.empty(DECAY_CE_WORKSPACE, dtype=torch.uint8, device=logits.device)
    elif workspace.numel() * workspace.element_size() < DECAY_CE_WORKSPACE:
        raise ValueError("workspace too small")
    _check("dflash_decay_ce",
           lib.dflash_decay_ce(_ptr(logits), dt, _ptr(targets), int(rows), int(vocab), int(block),
                               float(gamma), _ptr(loss), _ptr(ce), _ptr(grad), _ptr(workspace),
                               _stream(stream)))


def dflash_decay_ce_noalloc(logits: torch.Tensor, targets: torch.Tensor, block: int, gamma: float,
                            loss: torch.Tensor, ce: torch.Tensor, grad: Optional[torch.Tensor] = None,
                            stream: Optional[torch.cuda.Stream] = None) -> None:
    """dflash_decay_ce with the library's static per-GPU workspace: nothing
    is allocated, here or in the library."""
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [rows, vocab] tensor")
    if logits.dtype == torch.bfloat16:
        dt = DFLASH_BF16
    elif logits.dtype == torch.float32:
        dt = DFLASH_F32
    else:
        raise ValueError("logits must be float32 or bfloat16")
    rows, vocab = logits.shape
    if targets.dtype != torch.int32 or targets.numel() != rows:
        raise ValueError("targets must be int32 [rows]")
    if loss.dtype != torch.float32 or loss.numel() < 1 or ce.dtype != torch.float32 or ce.numel() != rows:
        raise ValueError("loss [1] and ce [rows] must be float32")
    if grad is not None and (grad.dtype != logits.dtype or grad.shape != logits.shape or
                             not grad.is_contiguous()):
        raise ValueError("grad must match logits")
    _check("dflash_decay_ce_noalloc",
           lib.dflash_decay_ce_noalloc(_ptr(logits), dt, _ptr(targets), int(rows), int(vocab), int(block),
                                       float(gamma), _ptr(loss), _ptr(ce), _ptr(grad), _stream(stream)))


def dflash_verify_block(ctx: Context, block_ids: torch.Tensor, K1: int, target_ids: torch.Tensor,
                        logits: Optional[torch.Tensor] = None, taps: Optional[torch.Tensor] = None,
                        stream: Optional[torch.cuda.Stream] = None) -> None:
    """One causal target forward over blocks [B, K1] (the anchor and K1 - 1
    drafts): target_ids [B, K1] int32 out (the target's token for the
    position after each row), optional float32 logits [B, K1, V] and taps
    [B, K1, n_taps * H] in the model dtype."""
    for t in (block_ids, target_ids):
        if t.dtype != torch.int32 or t.numel() != ctx.batch * K1:
            raise ValueError("block_ids / target_ids must be int32 [batch, K1]")
    sh = ctx.model.shape
    if logits is not None and (logits.dtype != torch.float32 or logits.numel() != ctx.batch * K1 * sh.vocab):
        raise ValueError("logits must be float32 [batch, K1, vocab]")
    if taps is not None and taps.numel() != ctx.batch * K1 * len(ctx.model.taps) * sh.hidden:
        raise ValueError("taps must be [batch, K1, n_taps * hidden]")
    with _on(stream):
        _check("dflash_verify_block",
               lib.dflash_verify_block(ctx.handle, _ptr(block_ids), int(K1), _ptr(target_ids), _ptr(logits),
                                       _ptr(taps), _stream(stream)))


def dflash_commit(ctx: Context, n_acc: Sequence[int], stream: Optional[torch.cuda.Stream] = None) -> None:
    """Keep the first n_acc[b] rows of the last verified block in sequence
    b's cache (host counts)."""
    nn = (ctypes.c_int32 * ctx.batch)(*[int(n) for n in n_acc])
    _check("dflash_commit", lib.dflash_commit(ctx.handle, nn, _stream(stream)))


class AdaptPolicy:
    """dflash_adapt_create / observe / choose / destroy: the block size per
    step from running acceptance statistics (host computation)."""

    def __init__(self, kmax: int, decay: float = 0.98, min_count: float = 4.0, a0: float = 0.8,
                 gamma0: float = 0.95):
        h = ctypes.c_void_p()
        _check("dflash_adapt_create", lib.dflash_adapt_create(int(kmax), float(decay), float(min_count),
                                                              float(a0), float(gamma0), ctypes.byref(h)))
        self.handle = h
        _LIVE.add(self)

    def observe(self, K: int, tau: int) -> None:
        _check("dflash_adapt_observe", lib.dflash_adapt_observe(self.handle, int(K), int(tau)))

    def choose(self, Ks: Sequence[int], cost: Sequence[float]):
        """(K, a, gamma, expected tokens per unit cost) for candidates Ks
        (increasing) with per-step costs."""
        n = len(Ks)
        ks = (ctypes.c_int32 * max(n, 1))(*[int(k) for k in Ks])
        cs = (ctypes.c_double * max(n, 1))(*[float(c) for c in cost])
        K, a, g, v = ctypes.c_int32(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        _check("dflash_adapt_choose", lib.dflash_adapt_choose(self.handle, ks, cs, n, ctypes.byref(K),
                                                              ctypes.byref(a), ctypes.byref(g), ctypes.byref(v)))
        return K.value, a.value, g.value, v.value

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib.dflash_adapt_destroy(self.handle)
            self.handle = None

    def __del__(self, _finalizing=sys.is_finalizing):
        # (bound at definition: module globals may already be None at exit)
        if _finalizing():            # closed by the atexit hook, or torch is gone
            return
        try:
            self.close()
        except Exception:
            pass


def version() -> str:
    return lib.dflash_version().decode()


def weights_to_device(weights: Dict, device="cuda") -> Dict[str, torch.Tensor]:
    """Host arrays (bf16 bits as uint16, or float32) -> device tensors; tied
    tables stay one tensor."""
    out: Dict[str, torch.Tensor] = {}
    seen: Dict[int, torch.Tensor] = {}
    for k, v in weights.items():
        if id(v) in seen:
            out[k] = seen[id(v)]
            continue
        t = torch.from_numpy(v).to(device)
        seen[id(v)] = t
        out[k] = t
    return out
