"""Scalar pure-Python version of the draft forward, for tiny shapes only.

TEST INFRASTRUCTURE ONLY (same import rule as the rest of ``oracle/``).

It follows the same description as ``oracle.dflash`` (kongchang.com "D-Flash"
page, sections "System architecture" and "Innovation 2: target-feature KV
injection"; Google Developers Blog, "Dual cache for attention" and "Smart
context management") but is written independently: every product is an
explicit loop over Python floats, RoPE rotates each channel pair on its own,
softmax and argmax are hand-rolled.  Its only purpose is to pin the NumPy
oracle against a mistake in vectorisation (a transposed operand, a wrong
axis, a wrong head mapping).
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple


def _val(a, dtype: str) -> List:
    """Nested Python lists of exact float values of a stored array."""
    import numpy as np
    if dtype == "bf16":
        f = (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    else:
        f = np.asarray(a, dtype=np.float32)
    return f.astype(float).tolist()


def _matvec(W: List[List[float]], x: List[float]) -> List[float]:
    out = []
    for row in W:
        acc = 0.0
        for j in range(len(x)):
            acc += row[j] * x[j]
        out.append(acc)
    return out


def _rmsnorm(x: List[float], g: List[float], eps: float) -> List[float]:
    ss = 0.0
    for v in x:
        ss += v * v
    r = 1.0 / math.sqrt(ss / len(x) + eps)
    return [x[i] * r * g[i] for i in range(len(x))]


def _rope_head(v: List[float], pos: int, theta: float) -> List[float]:
    d = len(v)
    h = d // 2
    out = list(v)
    for m in range(h):
        ang = pos * theta ** (-2.0 * m / d)
        c, s = math.cos(ang), math.sin(ang)
        a, b = v[m], v[m + h]
        out[m] = a * c - b * s
        out[m + h] = b * c + a * s
    return out


def forward(shape, weights: Dict, feats, ids: Sequence[int],
            positions: Sequence[int] = None) -> Tuple[List[int], List[List[float]], List[List[float]]]:
    """Project ``feats`` (ctx rows) into an empty context, then draft ``ids``.

    Returns (draft ids, logits rows, final-normed hidden rows).
    """
    s = shape
    dt = s.dtype
    H, d = s.hidden, s.head_dim
    nq, nkv = s.n_q_heads, s.n_kv_heads
    F = _val(feats, dt)
    n_ctx = len(F)
    ctx_pos = list(range(n_ctx)) if positions is None else [int(p) for p in positions]
    Wfc = _val(weights["fc"], dt)
    C = [_matvec(Wfc, F[j]) for j in range(n_ctx)]

    # per layer context K (rotated) and V, as [pos][head][d]
    ctxK, ctxV = [], []
    for l in range(s.n_layers):
        Wk = _val(weights[f"layers.{l}.wk"], dt)
        Wv = _val(weights[f"layers.{l}.wv"], dt)
        Kl, Vl = [], []
        for j in range(n_ctx):
            kf = _matvec(Wk, C[j])
            vf = _matvec(Wv, C[j])
            Kl.append([_rope_head(kf[g * d:(g + 1) * d], ctx_pos[j], s.rope_theta) for g in range(nkv)])
            Vl.append([vf[g * d:(g + 1) * d] for g in range(nkv)])
        ctxK.append(Kl)
        ctxV.append(Vl)

    E = _val(weights["embed"], dt)
    K = len(ids)
    X = [list(E[int(t)]) for t in ids]
    blk_pos = [n_ctx + i for i in range(K)]
    for l in range(s.n_layers):
        p = f"layers.{l}."
        g1 = _val(weights[p + "attn_norm"], dt)
        Wq, Wk, Wv = (_val(weights[p + n], dt) for n in ("wq", "wk", "wv"))
        Wo = _val(weights[p + "wo"], dt)
        U = [_rmsnorm(X[i], g1, s.rms_eps) for i in range(K)]
        Q, Kb, Vb = [], [], []
        for i in range(K):
            qf, kf, vf = _matvec(Wq, U[i]), _matvec(Wk, U[i]), _matvec(Wv, U[i])
            Q.append([_rope_head(qf[h * d:(h + 1) * d], blk_pos[i], s.rope_theta) for h in range(nq)])
            Kb.append([_rope_head(kf[g * d:(g + 1) * d], blk_pos[i], s.rope_theta) for g in range(nkv)])
            Vb.append([vf[g * d:(g + 1) * d] for g in range(nkv)])
        keys = ctxK[l] + Kb
        vals = ctxV[l] + Vb
        group = nq // nkv
        for i in range(K):
            o = []
            for h in range(nq):
                g = h // group
                sc = []
                for j in range(len(keys)):
                    dot = 0.0
                    for c in range(d):
                        dot += Q[i][h][c] * keys[j][g][c]
                    sc.append(dot / math.sqrt(d))
                mx = max(sc)
                e = [math.exp(v - mx) for v in sc]
                tot = sum(e)
                for c in range(d):
                    acc = 0.0
                    for j in range(len(keys)):
                        acc += e[j] / tot * vals[j][g][c]
                    o.append(acc)
            att = _matvec(Wo, o)
            X[i] = [X[i][c] + att[c] for c in range(H)]
        g2 = _val(weights[p + "mlp_norm"], dt)
        Wg, Wu, Wd = (_val(weights[p + n], dt) for n in ("w_gate", "w_up", "w_down"))
        for i in range(K):
            w = _rmsnorm(X[i], g2, s.rms_eps)
            gt, up = _matvec(Wg, w), _matvec(Wu, w)
            act = [gt[c] / (1.0 + math.exp(-gt[c])) * up[c] for c in range(len(gt))]
            dn = _matvec(Wd, act)
            X[i] = [X[i][c] + dn[c] for c in range(H)]
    gf = _val(weights["final_norm"], dt)
    Wlm = _val(weights["lm_head"], dt)
    Z, L, D = [], [], []
    for i in range(K):
        z = _rmsnorm(X[i], gf, s.rms_eps)
        lg = _matvec(Wlm, z)
        best = 0
        for v in range(1, len(lg)):
            if lg[v] > lg[best]:
                best = v
        Z.append(z)
        L.append(lg)
        D.append(best)
    return D, L, Z


def target_forward(shape, weights: Dict, ids: Sequence[int],
                   taps: Sequence[int] = ()) -> Tuple[List[int], List[List[float]], List[List[float]]]:
    """Causal forward of a whole sequence from an empty cache (the target of
    block verification; Google Developers Blog, "Overcoming the
    autoregressive bottleneck"): position i attends to positions 0..i.

    Returns (argmax per position, logits rows, tapped residual rows: the
    residual after each layer in ``taps``, concatenated in tap order).
    """
    s = shape
    dt = s.dtype
    H, d = s.hidden, s.head_dim
    nq, nkv = s.n_q_heads, s.n_kv_heads
    E = _val(weights["embed"], dt)
    n = len(ids)
    X = [list(E[int(t)]) for t in ids]
    T = [[] for _ in range(n)]
    for l in range(s.n_layers):
        p = f"layers.{l}."
        g1 = _val(weights[p + "attn_norm"], dt)
        Wq, Wk, Wv = (_val(weights[p + nm], dt) for nm in ("wq", "wk", "wv"))
        Wo = _val(weights[p + "wo"], dt)
        Q, Kr, Vr = [], [], []
        for i in range(n):
            u = _rmsnorm(X[i], g1, s.rms_eps)
            qf, kf, vf = _matvec(Wq, u), _matvec(Wk, u), _matvec(Wv, u)
            Q.append([_rope_head(qf[h * d:(h + 1) * d], i, s.rope_theta) for h in range(nq)])
            Kr.append([_rope_head(kf[g * d:(g + 1) * d], i, s.rope_theta) for g in range(nkv)])
            Vr.append([vf[g * d:(g + 1) * d] for g in range(nkv)])
        group = nq // nkv
        newX = []
        for i in range(n):
            o = []
            for h in range(nq):
                g = h // group
                sc = []
                for j in range(i + 1):            # causal: keys 0..i only
                    dot = 0.0
                    for c in range(d):
                        dot += Q[i][h][c] * Kr[j][g][c]
                    sc.append(dot / math.sqrt(d))
                mx = max(sc)
                e = [math.exp(v - mx) for v in sc]
                tot = sum(e)
                for c in range(d):
                    acc = 0.0
                    for j in range(i + 1):
                        acc += e[j] / tot * Vr[j][g][c]
                    o.append(acc)
            att = _matvec(Wo, o)
            newX.append([X[i][c] + att[c] for c in range(H)])
        X = newX
        g2 = _val(weights[p + "mlp_norm"], dt)
        Wg, Wu, Wd = (_val(weights[p + nm], dt) for nm in ("w_gate", "w_up", "w_down"))
        for i in range(n):
            w = _rmsnorm(X[i], g2, s.rms_eps)
            gt, up = _matvec(Wg, w), _matvec(Wu, w)
            act = [gt[c] / (1.0 + math.exp(-gt[c])) * up[c] for c in range(len(gt))]
            dn = _matvec(Wd, act)
            X[i] = [X[i][c] + dn[c] for c in range(H)]
        if l in taps:
            for i in range(n):
                T[i] = T[i] + list(X[i])
    gf = _val(weights["final_norm"], dt)
    Wlm = _val(weights["lm_head"], dt)
    L, D = [], []
    for i in range(n):
        lg = _matvec(Wlm, _rmsnorm(X[i], gf, s.rms_eps))
        best = 0
        for v in range(1, len(lg)):
            if lg[v] > lg[best]:
                best = v
        L.append(lg)
        D.append(best)
    return D, L, T
