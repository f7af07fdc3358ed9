"""Helpers for the GPU parity tests: drive the C ABI through the binding on
seeded inputs and compare with the fp64 oracle on the same inputs."""
import ctypes
import sys

import numpy as np
import torch

import synth
from oracle import dflash as O

BF16_TOL = 2e-2      # max |gpu - oracle| / max |oracle| per row, bf16 configs
F32_TOL = 1e-4       # same, fp32 configs
ARGMAX_MARGIN = 0.05


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tol(shape):
    return BF16_TOL if shape.dtype == "bf16" else F32_TOL


def row_rel(gpu, ora):
    gpu = np.asarray(gpu, np.float64).reshape(-1, np.shape(ora)[-1])
    ora = np.asarray(ora, np.float64).reshape(-1, np.shape(ora)[-1])
    den = np.maximum(np.max(np.abs(ora), axis=1), 1e-30)
    return np.max(np.abs(gpu - ora), axis=1) / den


def check_rows(name, gpu, ora, t):
    r = row_rel(gpu, ora)
    assert np.all(np.isfinite(np.asarray(gpu, np.float64))), f"{name}: non-finite values"
    assert float(r.max()) <= t, f"{name}: max row-relative error {r.max():.3e} > {t:.1e} (row {int(r.argmax())})"
    return float(r.max())


def check_argmax(gpu_ids, ora_logits):
    """Bit-exact where the oracle's top-1/top-2 margin exceeds 0.05; otherwise
    the pick must be within 0.05 of the oracle's maximum."""
    L = np.asarray(ora_logits, np.float64).reshape(-1, np.shape(ora_logits)[-1])
    g = np.asarray(gpu_ids).reshape(-1)
    top = np.argmax(L, axis=1)
    srt = np.sort(L, axis=1)
    margin = srt[:, -1] - srt[:, -2] if L.shape[1] > 1 else np.full(len(L), np.inf)
    exact = margin > ARGMAX_MARGIN
    bad = exact & (g != top)
    assert not bad.any(), f"argmax differs on {int(bad.sum())} rows with margin > {ARGMAX_MARGIN}"
    near = L[np.arange(len(L)), g] >= srt[:, -1] - ARGMAX_MARGIN
    assert near.all(), "argmax pick far from the oracle maximum"
    return int(exact.sum()), len(L)


_hip = None


def hip():
    global _hip
    if _hip is None:
        for n in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                _hip = ctypes.CDLL(n)
                break
            except OSError:
                pass
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
        _hip.hipMemset2D.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_size_t, ctypes.c_size_t]
    return _hip


def d2h(ptr, nbytes):
    torch.cuda.synchronize()
    out = np.empty(nbytes, np.uint8)
    assert hip().hipMemcpy(out.ctypes.data, ptr, nbytes, 2) == 0
    return out


def as_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    return O.to_f64(raw.view(np.uint16) if dtype == "bf16" else raw.view(np.float32), dtype)


def cache_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """KV-cache bytes -> float64: fp16 for bf16 models, fp32 for fp32 models."""
    return raw.view(np.float16 if dtype == "bf16" else np.float32).astype(np.float64)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Pair:
    """A GPU model/context and an oracle model/states driven in lockstep."""

    def __init__(self, shape, seed, batch, gain_std=0.0, weights=None, oracle_seqs=None):
        import block_diffusion_drafting_amd as dfl
        self.dfl = dfl
        self.shape = shape
        self.seed = seed
        self.batch = batch
        self.w = weights if weights is not None else synth.weights(shape, seed, gain_std=gain_std)
        self.wd = dfl.weights_to_device(self.w)
        self.model = dfl.Model(shape, self.wd)
        self.ctx = dfl.Context(self.model, batch)
        self.om = O.Model(shape, self.w)
        self.oseqs = list(range(batch)) if oracle_seqs is None else list(oracle_seqs)
        self.ost = {b: O.new_state(self.om) for b in self.oseqs}

    def project(self, feats_per_seq, positions_per_seq=None):
        n_new = [len(f) for f in feats_per_seq]
        nonempty = [f for f in feats_per_seq if len(f)]
        if nonempty:
            cat = np.concatenate(nonempty, axis=0)
            fd = to_dev(cat)
        else:
            fd = None
        pd = None
        if positions_per_seq is not None:
            pd = to_dev(np.concatenate([np.asarray(p, np.int32) for p in positions_per_seq]).astype(np.int32))
        self.dfl.dflash_project_ctx(self.ctx, fd, n_new, pd)
        for b in self.oseqs:
            if n_new[b]:
                O.project_ctx(self.om, self.ost[b], feats_per_seq[b],
                              positions=None if positions_per_seq is None else positions_per_seq[b])

    def gpu_draft(self, ids, logits=True, hidden=True):
        B, K = ids.shape
        s = self.shape
        idd = to_dev(ids.astype(np.int32))
        dr = torch.empty(B, K, dtype=torch.int32, device="cuda")
        lg = torch.empty(B, K, s.vocab, dtype=torch.float32, device="cuda") if logits else None
        hd = (torch.empty(B, K, s.hidden, dtype=torch.uint16 if s.dtype == "bf16" else torch.float32,
                          device="cuda") if hidden else None)
        self.dfl.dflash_draft_block(self.ctx, idd, K, dr, lg, hd)
        torch.cuda.synchronize()
        out = {"draft": dr.cpu().numpy()}
        if logits:
            out["logits"] = lg.cpu().numpy()
        if hidden:
            h = hd.cpu().numpy()
            out["hidden"] = O.to_f64(h, s.dtype)
        return out

    def gpu_step(self, feats_per_seq, ids, logits=True, hidden=True):
        """dflash_step: append feats_per_seq[b] to sequence b and draft ids
        (the oracle states are advanced by the caller)."""
        B, K = ids.shape
        s = self.shape
        n_new = [len(f) for f in feats_per_seq]
        nonempty = [f for f in feats_per_seq if len(f)]
        fd = to_dev(np.concatenate(nonempty, axis=0)) if nonempty else None
        idd = to_dev(ids.astype(np.int32))
        dr = torch.empty(B, K, dtype=torch.int32, device="cuda")
        lg = torch.empty(B, K, s.vocab, dtype=torch.float32, device="cuda") if logits else None
        hd = (torch.empty(B, K, s.hidden, dtype=torch.uint16 if s.dtype == "bf16" else torch.float32,
                          device="cuda") if hidden else None)
        self.dfl.dflash_step(self.ctx, fd, n_new, idd, K, dr, lg, hd)
        torch.cuda.synchronize()
        out = {"draft": dr.cpu().numpy()}
        if logits:
            out["logits"] = lg.cpu().numpy()
        if hidden:
            out["hidden"] = O.to_f64(hd.cpu().numpy(), s.dtype)
        return out

    def oracle_draft(self, b, ids_b):
        return O.draft_one(self.om, self.ost[b], ids_b)

    def compare(self, ids, logits=True, hidden=True):
        g = self.gpu_draft(ids, logits, hidden)
        t = tol(self.shape)
        stats = {}
        for b in self.oseqs:
            d_o, l_o, z_o = self.oracle_draft(b, ids[b])
            if logits:
                stats[f"logits{b}"] = check_rows(f"logits[{b}]", g["logits"][b], l_o, t)
            if hidden:
                stats[f"hidden{b}"] = check_rows(f"hidden[{b}]", g["hidden"][b], z_o, t)
            ex, tot = check_argmax(g["draft"][b], l_o)
            stats[f"argmax_exact{b}"] = f"{ex}/{tot}"
        say(f"  max row-relative errors: {stats}")
        return g, stats

    def check_state(self):
        """ctx_len / cap exact; context buffer and caches against the oracle."""
        s = self.shape
        lens, caps = self.ctx.query()
        t = tol(s)
        for b in self.oseqs:
            st = self.ost[b]
            assert lens[b] == st.ctx_len, (b, lens[b], st.ctx_len)
            assert caps[b] == st.cap, (b, caps[b], st.cap)
            if st.ctx_len == 0:
                continue
            cptr, kptr, vptr, phys = self.ctx.buffers(b)
            es = s.elem_bytes                    # cache element: fp16 (bf16 models) or fp32
            n = st.ctx_len
            ctxb = d2h(cptr, n * s.hidden * 4).view(np.float32).astype(np.float64).reshape(n, s.hidden)
            check_rows(f"ctxbuf[{b}]", ctxb, st.ctx, t)
            L, nkv, d = s.n_layers, s.n_kv_heads, s.head_dim
            raw_k = d2h(kptr, L * nkv * phys * d * es).reshape(L, nkv, phys, d * es)
            raw_v = d2h(vptr, L * nkv * d * phys * es).reshape(L, nkv, d, phys * es)
            kall = cache_f64(np.ascontiguousarray(raw_k[:, :, :n, :]), s.dtype).reshape(L, nkv, n, d)
            vall = cache_f64(np.ascontiguousarray(raw_v[:, :, :, :n * es]), s.dtype).reshape(L, nkv, d, n)
            for l in range(L):
                kg = kall[l].transpose(1, 0, 2)                   # [n, nkv, d]
                vg = vall[l].transpose(2, 0, 1)                   # [n, nkv, d]
                check_rows(f"k[{b}][{l}]", kg.reshape(n, -1), st.k[l].reshape(n, -1), t)
                check_rows(f"v[{b}][{l}]", vg.reshape(n, -1), st.v[l].reshape(n, -1), t)

    def poison_padding(self):
        """Fill every cache row past ctx_len with NaN bytes."""
        s = self.shape
        lens, _ = self.ctx.query()
        es = s.elem_bytes
        torch.cuda.synchronize()
        for b in range(self.batch):
            cptr, kptr, vptr, phys = self.ctx.buffers(b)
            if not kptr:
                continue
            n = lens[b]
            if n >= phys:
                continue
            L, nkv, d = s.n_layers, s.n_kv_heads, s.head_dim
            for lg in range(L * nkv):
                assert hip().hipMemset(kptr + (lg * phys + n) * d * es, 0xFF, (phys - n) * d * es) == 0
            assert hip().hipMemset2D(vptr + n * es, phys * es, 0xFF, (phys - n) * es, L * nkv * d) == 0
        torch.cuda.synchronize()
