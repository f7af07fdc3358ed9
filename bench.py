#!/usr/bin/env python3
"""Benchmark of the DFlash draft-block hot path on one MI355X.

A step is one speculative step of the whole hot path for every sequence of
the batch, enqueued on one stream with no host synchronisation:
    dflash_step (append the positions accepted at the previous step and
    draft K block rows, one call)  ->  dflash_accept.
The same work as three calls (dflash_draft_block -> dflash_accept ->
dflash_project_ctx) is timed as well and reported beside it.
The accepted counts come from the seeded stand-in verifier (they depend only
on its agreement draws, so they are known ahead); its target tokens are
pre-generated.  Inputs are resident in device memory before timing starts.

Prints ONE JSON line: drafted tokens per second (batch * K / step time),
the step time, the draft-block-only latency, a live roofline of the dominant
kernel (LM head + argmax, measured with HIP events on the launch stream
during the timed steps), and the fp64 oracle timed on this host's cores on a
bounded sample of the same workload.

    python bench.py [--steps 50] [--warmup 10] [--workload 1]
    python bench.py --ksweep          # block-size sweep, one line per K
    python bench.py --decay-ce        # drafter-training loss kernel instead
    python bench.py --verify-sweep    # target-side verification latency vs block size
    python bench.py --adaptive        # draft-verify loop, adaptive vs fixed block size
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 matrix peak
METRIC = "draft-block latency (ms) & drafted tok/s at K=16, Qwen3-4B shape; % HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=1)
    ap.add_argument("--K", type=int, default=0, help="override the block size")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=25)
    ap.add_argument("--ksweep", action="store_true")
    ap.add_argument("--draft-iters", type=int, default=50)
    ap.add_argument("--dist-iters", type=int, default=200,
                    help="timed draft blocks per warm / cold latency distribution")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the cold-cache, K-flat, MFMA and Llama-shaped figures")
    ap.add_argument("--persistent", action="store_true",
                    help="draft with the single-launch block where it applies (batch * K <= 16)")
    ap.add_argument("--trace", action="store_true",
                    help="report the single-launch block's per-phase timeline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--decay-ce", action="store_true",
                    help="benchmark the loss-decay weighted cross-entropy (drafter training) instead")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows of the decay-CE oracle sample timed on the host")
    ap.add_argument("--verify-sweep", action="store_true",
                    help="benchmark target-side verification latency vs block size instead")
    ap.add_argument("--adaptive", action="store_true",
                    help="benchmark the draft-verify loop with the adaptive block size instead")
    ap.add_argument("--loop-steps", type=int, default=300, help="steps per session of --adaptive")
    return ap.parse_args()


# dominant kernel -> (counter summary, the sources its code comes from)
TRAFFIC = {
    "lm_head": ("lm_head_argmax_qwen3_4b_k16_traffic.txt",
                ["gemm_kernel.h", "gemm_argmax.hip", "gemm.hip", "kernels.h", "common.h"]),
    "persistent_draft": ("persistent_draft_qwen3_4b_k16_traffic.txt",
                         ["persist.hip", "kernels.h", "common.h"]),
    "decay_ce": ("decay_ce_row_qwen_vocab_traffic.txt", ["loss.hip", "common.h"]),
}

# Loss-decay weighted CE workload: 256 drafter blocks of K = 16 rows over the
# Qwen3 vocabulary (151936, of which the last 267 are padding at -inf), bf16
# logits and gradient, gamma 0.8.
CE_ROWS, CE_VOCAB, CE_BLOCK, CE_GAMMA, CE_MASKED, CE_SEED = 4096, 151936, 16, 0.8, 267, 2026
CE_WORKLOAD = (f"decay-CE {CE_ROWS // CE_BLOCK} blocks x {CE_BLOCK} rows, vocab {CE_VOCAB} "
               f"({CE_MASKED} masked), bf16, gamma {CE_GAMMA}")


def kernel_source_hash(kernel: str):
    """sha256 over the sources of a kernel (counter readings taken from an
    older build are not reported)."""
    import hashlib
    h = hashlib.sha256()
    for n in TRAFFIC[kernel][1]:
        with open(os.path.join(ROOT, "block_diffusion_drafting_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str, K: int):
    """HBM bytes per launch of `kernel` from its committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), or None when
    the summary is missing, was taken on another workload, or the kernel
    sources changed since."""
    try:
        vals = {}
        with open(os.path.join(ROOT, "profiles", TRAFFIC[kernel][0])) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    vals[k.strip()] = v.strip()
        if vals.get("source_sha256") != kernel_source_hash(kernel):
            return None
        if vals.get("workload") != f"{workload} K={K}":
            return None
        return int(vals["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(torch):
    """A plain device copy of 1 GiB, three times: the HBM counters read for
    it give the bytes-per-count scale of FETCH_SIZE / WRITE_SIZE."""
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 3 copies of {n} bytes")
    del a, b


def persist_timeline(tr, n_layers):
    """Per-phase figures (us) from a single-launch block's timeline
    [workgroups, 8 slots per phase] of 100 MHz ticks: for each phase (mean
    over layers), the median and slowest workgroup's time from the phase
    start to each mark inside it (1-5) and to its barrier arrival (6), and
    the barrier's latency from the last arrival to the first release."""
    names = ["embed"] + [n for _ in range(n_layers) for n in ("qkv", "attention", "attn_merge", "o_proj", "gate_up",
                                                              "down")]
    names.append("lm_head")
    tr = tr.astype(np.int64).reshape(tr.shape[0], -1, 8)
    acc = {}
    for p, name in enumerate(names):
        ph = tr[:, p, :]
        st = ph[:, 0]
        d = acc.setdefault(name, {"n": 0})
        d["n"] += 1
        for k in range(1, 7):
            ok = ph[:, k] > 0
            if not ok.any():
                continue
            dt = (ph[ok, k] - st[ok]) / 100.0
            key = "arrive" if k == 6 else f"m{k}"
            d[key + "_med"] = d.get(key + "_med", 0.0) + float(np.median(dt))
            d[key + "_max"] = d.get(key + "_max", 0.0) + float(dt.max())
        if ph[:, 7].max() > 0:
            d["barrier"] = d.get("barrier", 0.0) + (ph[:, 7].min() - ph[:, 6].max()) / 100.0
    res = {}
    for name, d in acc.items():
        n = d.pop("n")
        res[name] = {k: round(v / n, 2) for k, v in d.items()}
    res["total_us"] = round((tr[:, -1, 6].max() - tr[:, 0, 0].min()) / 100.0, 2)
    return res


def setup(wl, K, dfl, torch):
    import synth
    t0 = time.time()
    w = synth.weights(wl.shape, wl.seed)
    log(f"[bench] weights generated in {time.time() - t0:.1f}s")
    wd = dfl.weights_to_device(w)
    model = dfl.Model(wl.shape, wd)
    ctx = dfl.Context(model, wl.batch)
    if getattr(setup, "persistent", False):
        ctx.set_persistent(True)
    feats = [synth.prefill_features(wl.shape, wl.seed, b, wl.ctx0[b]) for b in range(wl.batch)]
    t0 = time.time()
    dfl.dflash_project_ctx(ctx, torch.from_numpy(np.concatenate(feats)).cuda(), list(wl.ctx0))
    torch.cuda.synchronize()
    log(f"[bench] prefill of {sum(wl.ctx0)} positions in {time.time() - t0:.1f}s")
    return w, wd, model, ctx


def kv_bytes(shape, ctx_lens, K, batch):
    per_pos = shape.n_layers * 2 * shape.kv_dim * shape.elem_bytes
    return sum((c + K) * per_pos for c in ctx_lens)


def block_bytes(shape, model_bytes, ctx_lens, K, batch):
    """Algorithmic bytes of one draft block: every streamed weight once
    (logical sizes, no padding) plus each sequence's context and block KV."""
    s = shape
    e = s.elem_bytes
    layer = s.n_layers * e * s.hidden * ((s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim
                                         + s.q_dim + 3 * s.intermediate)
    lm = s.vocab * s.hidden * e
    return layer + lm + kv_bytes(s, ctx_lens, K, batch)


def plan_steps(wl, K, n_steps):
    """Block ids, pre-generated targets and accepted counts of every step."""
    import synth
    s = wl.shape
    anchors = [synth.first_anchor(wl.seed, b, s.vocab) for b in range(wl.batch)]
    steps = []
    for t in range(n_steps):
        ids = np.stack([synth.block_ids(wl.seed, b, t, K, s.vocab) for b in range(wl.batch)])
        ids[:, 0] = anchors
        draws = [synth.verifier_draws(wl.seed, b, t, K, s.vocab, wl.a[b], wl.gamma)
                 for b in range(wl.batch)]
        tau = [1 + int(np.argmin(np.append(d.agree, False))) for d in draws]
        target = np.stack([synth.target_tokens(np.zeros(K, np.int64), d, s.vocab) for d in draws])
        feats = np.concatenate([synth.step_features(s, wl.seed, b, t, tau[b]) for b in range(wl.batch)])
        steps.append((ids.astype(np.int32), target, tau, feats))
        anchors = [d.bonus for d in draws]
    return steps


def cpu_baseline(wl, K, w, n_steps):
    """The fp64 oracle, as it stands, on this host: prefill untimed, then
    n_steps whole steps (draft block + accept + projection) timed."""
    import synth
    from oracle import dflash as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    model = O.Model(wl.shape, w)
    wl2 = wl.replace(K=K)
    t0 = time.time()
    sess = O.Session(model, wl2)
    log(f"[bench] oracle prefill {time.time() - t0:.1f}s")
    sess.step()                       # upcasts the cached matrices once (untimed)
    t0 = time.time()
    for _ in range(n_steps):
        sess.step()
    dt = (time.time() - t0) / n_steps
    cpu_model, host_cores = host_cpu()
    return {"value": round(wl.batch * K / dt, 3), "unit": "drafted tok/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model, "host_cores_available": host_cores,
            "sample": f"{n_steps} whole steps (fp64 draft block + accept + projection) of workload "
                      f"'{wl.name}' after an untimed prefill and one untimed step; {dt:.2f} s/step; "
                      f"'cores' is the BLAS thread count the oracle ran with"}


def host_cpu():
    """(CPU model name, cores this process may run on)."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


def block_flops(shape, ctx_lens, K, batch):
    """Algorithmic flops of one draft block: every weight product once
    (2 flops per multiply-add; the hi/lo activation pair the kernels issue
    for precision is not counted) plus attention (Q K^T and P V over each
    sequence's context and block keys)."""
    s = shape
    M = batch * K
    params = s.n_layers * s.hidden * ((s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim + s.q_dim
                                      + 3 * s.intermediate) + s.vocab * s.hidden
    attn = sum(4 * K * s.n_q_heads * s.head_dim * (c + K) * s.n_layers for c in ctx_lens)
    return 2 * M * params, attn


def event_times(torch, stream, fn, iters, flush=None):
    """Per-call milliseconds of fn() from HIP events recorded on `stream`
    around each call; with `flush` (a 1 GiB device buffer) every call is
    preceded, outside its events, by a write of the whole buffer, which
    evicts the L2 caches and the 256 MB Infinity Cache."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i, (a, b) in enumerate(evs):
        if flush is not None:
            flush.fill_(float(i & 7))
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def spread(ms):
    return {"median": round(float(np.median(ms)), 4), "p10": round(float(np.percentile(ms, 10)), 4),
            "p90": round(float(np.percentile(ms, 90)), 4), "mean": round(float(ms.mean()), 4), "n": int(ms.size)}


def headline_extras(args, torch, dfl, wl, model, ctx, K, ids0, lens0, mb):
    """The figures the goal names beside the headline step: draft-block
    latency warm and cold (median / p10 / p90), MFMA utilisation, the
    draft latency at K = 16 and K = 128 over a 4096-position context (the
    K sweep's context, same drafter shape), and the Llama-3.1-8B-shaped
    drafter's block at K = 10 over 4096 positions."""
    import synth
    stream = torch.cuda.current_stream()
    s = wl.shape
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    it = args.dist_iters
    out = {}
    draft = torch.empty(wl.batch, K, dtype=torch.int32, device="cuda")

    def block():
        dfl.dflash_draft_block(ctx, ids0, K, draft)

    lens0, _ = ctx.query()           # the context as the timed steps left it
    warm = event_times(torch, stream, block, it)
    cold = event_times(torch, stream, block, it, flush)
    byt = block_bytes(s, mb, lens0, K, wl.batch)
    out["draft_block_warm_ms"] = spread(warm)
    out["draft_block_cold_ms"] = spread(cold)
    out["draft_block_cold_hbm_frac"] = round(byt / (np.median(cold) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    fp, fa = block_flops(s, lens0, K, wl.batch)
    med = float(np.median(warm))
    out["mfma"] = {"flops_per_block": int(fp + fa), "product_flops": int(fp), "attention_flops": int(fa),
                   "achieved_tflops": round((fp + fa) / (med * 1e-3) / 1e12, 2),
                   "peak_tflops": MFMA_PEAK_TFLOPS, "frac": round((fp + fa) / (med * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 5),
                   "timing": "warm median draft block", "dtype": "bf16 products (hi/lo activation pair), "
                                                            "fp16 attention"}
    log(f"[bench] draft block warm median {med:.4f} ms, cold median {np.median(cold):.4f} ms")

    # K-flat: the K sweep's 4096-position context on the same drafter shape
    w3 = synth.workload(3)
    c3 = dfl.Context(model, 1)
    f3 = synth.prefill_features(w3.shape, w3.seed, 0, w3.ctx0[0])
    dfl.dflash_project_ctx(c3, torch.from_numpy(f3).cuda(), [w3.ctx0[0]])
    del f3
    kf = {"ctx": w3.ctx0[0]}
    for Kx in (16, 128):
        ids = torch.from_numpy(synth.block_ids(w3.seed, 0, 0, Kx, s.vocab)).cuda().view(1, Kx)
        dr = torch.empty(1, Kx, dtype=torch.int32, device="cuda")

        def fn(ids=ids, dr=dr, Kx=Kx):
            dfl.dflash_draft_block(c3, ids, Kx, dr)

        for _ in range(3):
            fn()
        wm = event_times(torch, stream, fn, it)
        cm = event_times(torch, stream, fn, it, flush)
        kf[f"K{Kx}_warm_ms"] = spread(wm)
        kf[f"K{Kx}_cold_ms"] = spread(cm)
    kf["ratio_K128_over_K16_warm"] = round(kf["K128_warm_ms"]["median"] / kf["K16_warm_ms"]["median"], 4)
    kf["ratio_K128_over_K16_cold"] = round(kf["K128_cold_ms"]["median"] / kf["K16_cold_ms"]["median"], 4)
    kf["target"] = "<= 1.2"
    out["k_flat"] = kf
    c3.close()
    log(f"[bench] K-flat at ctx 4096: {kf['ratio_K128_over_K16_warm']} warm, {kf['ratio_K128_over_K16_cold']} cold")

    # Llama-3.1-8B-shaped drafter, K = 10, 4096 positions
    w2 = synth.workload(2)
    t0 = time.time()
    wts = synth.weights(w2.shape, w2.seed)
    m2 = dfl.Model(w2.shape, dfl.weights_to_device(wts))
    del wts
    c2 = dfl.Context(m2, 1)
    f2 = synth.prefill_features(w2.shape, w2.seed, 0, w2.ctx0[0])
    dfl.dflash_project_ctx(c2, torch.from_numpy(f2).cuda(), [w2.ctx0[0]])
    del f2
    log(f"[bench] llama-shaped drafter set up in {time.time() - t0:.1f}s")
    ids = torch.from_numpy(synth.block_ids(w2.seed, 0, 0, w2.K, w2.shape.vocab)).cuda().view(1, w2.K)
    dr = torch.empty(1, w2.K, dtype=torch.int32, device="cuda")

    def fl():
        dfl.dflash_draft_block(c2, ids, w2.K, dr)

    for _ in range(3):
        fl()
    wm = event_times(torch, stream, fl, it)
    cm = event_times(torch, stream, fl, it, flush)
    b2 = block_bytes(w2.shape, m2.bytes(), [w2.ctx0[0]], w2.K, 1)
    out[w2.name] = {"K": w2.K, "ctx": w2.ctx0[0], "bytes_per_block": int(b2),
                    "draft_block_warm_ms": spread(wm), "draft_block_cold_ms": spread(cm),
                    "drafted_tok_s_warm": round(w2.K / (np.median(wm) * 1e-3), 1),
                    "hbm_frac_warm": round(b2 / (np.median(wm) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "hbm_frac_cold": round(b2 / (np.median(cm) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    c2.close()
    m2.close()
    del flush
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def decay_ce_cpu_baseline(L, t, n_rows):
    """The fp64 oracle on the first n_rows rows (whole blocks) of the decay-CE
    workload, loss and gradient."""
    from oracle import dflash as O
    from oracle import loss as OL
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    n_rows = max(CE_BLOCK, n_rows // CE_BLOCK * CE_BLOCK)
    Lf = O.to_f64(L[:n_rows], "bf16")
    t0 = time.time()
    OL.decay_ce(Lf, t[:n_rows], CE_BLOCK, CE_GAMMA, want_grad=True)
    dt = time.time() - t0
    return {"value": round(n_rows / dt, 2), "unit": "rows/s", "cores": int(threads), "kind": "oracle",
            "sample": f"loss and gradient of the first {n_rows} rows ({n_rows // CE_BLOCK} blocks) of the "
                      f"same logits in fp64 (bf16 to fp64 conversion untimed); {dt:.2f} s"}


def bench_decay_ce(args, torch, dfl):
    """Loss-decay weighted CE + gradient of one batch of drafter logits per
    step (three launches: weight sum and row scales, rows, loss)."""
    import synth
    log(f"[bench] decay-CE inputs: {CE_WORKLOAD}")
    L, t = synth.ce_inputs(CE_SEED, CE_ROWS, CE_VOCAB, CE_BLOCK, "bf16", masked_tail=CE_MASKED)
    d_L = torch.from_numpy(L.view(np.int16)).view(torch.bfloat16).cuda()
    d_t = torch.from_numpy(t).cuda()
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    ce = torch.empty(CE_ROWS, dtype=torch.float32, device="cuda")
    grad = torch.empty_like(d_L)
    ws = torch.empty(dfl.DECAY_CE_WORKSPACE, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        dfl.dflash_decay_ce(d_L, d_t, CE_BLOCK, CE_GAMMA, loss, ce, grad, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = e0.elapsed_time(e1) / args.steps
    ms_step = wall * 1e3 / args.steps
    bytes_per_call = 2 * CE_ROWS * CE_VOCAB * 2   # one read of the logits, one write of the gradient
    achieved = bytes_per_call / (call_ms * 1e-3) / 1e9
    out = {
        "metric": "loss-decay weighted CE + gradient over drafter logits (rows/s); % HBM peak",
        "value": round(CE_ROWS / (wall / args.steps), 1),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": CE_WORKLOAD, "rows": CE_ROWS, "vocab": CE_VOCAB, "block": CE_BLOCK,
                   "gamma": CE_GAMMA, "parallelism": "1 GPU"},
        "loss": round(float(loss.item()), 6),
        "roofline": {"kernel": "dflash_decay_ce call (ce_scale, ce_row_kernel<bf16, 19>, ce_loss launches)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decay_ce", CE_WORKLOAD, CE_BLOCK),
                     "avg_launch_ms": round(call_ms, 5), "launches": args.steps,
                     "bytes_per_launch": int(bytes_per_call)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = decay_ce_cpu_baseline(L, t, args.cpu_rows)
    print(json.dumps(out))


VERIFY_K1 = (16, 32, 64, 128, 256, 512, 1024)
VERIFY_CTX, VERIFY_SEED = 4096, 1005


def verify_cpu_baseline(shape, taps, n_layers=4, ctx=256, K1=16):
    """The fp64 target oracle on a bounded sample: a K1-row block verified
    against a ctx-position cache of the first n_layers layers (prefill
    untimed), scaled to the whole target by its layer count."""
    import synth
    from oracle import dflash as O
    from oracle import target as OT
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    sub = shape.replace(n_layers=n_layers)
    w = synth.weights(sub, VERIFY_SEED)
    m = O.Model(sub, w)
    rng = np.random.default_rng(0)
    st = OT.new_target_state(m)
    OT.commit(st, OT.verify(m, st, rng.integers(0, sub.vocab, ctx)), ctx)
    OT.verify(m, st, rng.integers(0, sub.vocab, K1))        # upcasts the weights once (untimed)
    t0 = time.time()
    OT.verify(m, st, rng.integers(0, sub.vocab, K1), tuple(t for t in taps if t < n_layers))
    dt = time.time() - t0
    scaled = dt * shape.n_layers / n_layers
    return {"value": round(scaled * 1e3, 1), "unit": "ms per verify (scaled)", "cores": int(threads),
            "kind": "oracle",
            "sample": f"one {K1}-row block verified in fp64 by the first {n_layers} of {shape.n_layers} layers "
                      f"(plus LM head) over a {ctx}-position cache: {dt:.2f} s, scaled by "
                      f"{shape.n_layers}/{n_layers}"}


def bench_verify(args, torch, dfl):
    """Latency of one target verification vs block size at a fixed context:
    the pages' K-Flat claim, on a 36-layer Qwen3-4B-shaped target."""
    import synth
    shape = synth.QWEN3_4B_TARGET
    taps = synth.QWEN3_4B_TAPS
    shape = shape.replace(n_feat=len(taps))
    t0 = time.time()
    w = synth.weights(shape, VERIFY_SEED)
    log(f"[bench] target weights generated in {time.time() - t0:.1f}s")
    wd = dfl.weights_to_device(w)
    del w
    model = dfl.Model(shape, wd, taps=taps)
    for k in list(wd):
        if k != "embed":
            del wd[k]
    torch.cuda.empty_cache()
    ctx = dfl.Context(model, 1)
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda")
    g.manual_seed(VERIFY_SEED)
    maxk = max(VERIFY_K1)
    tgt = torch.empty(1, maxk, dtype=torch.int32, device="cuda")
    done = 0
    while done < VERIFY_CTX:          # prefill: verify + commit in blocks of up to 1024
        n = min(1024, VERIFY_CTX - done)
        ids = torch.randint(0, shape.vocab, (1, n), dtype=torch.int32, device="cuda", generator=g)
        dfl.dflash_verify_block(ctx, ids, n, tgt[:, :n].contiguous() if n != maxk else tgt)
        dfl.dflash_commit(ctx, [n])
        done += n
    torch.cuda.synchronize()
    mb = model.bytes()
    weight_bytes = mb["layers"] + mb["lm_head"]
    kv_per_pos = shape.n_layers * 2 * shape.n_kv_heads * shape.head_dim * 2
    sweep = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for K1 in VERIFY_K1:
        ids = torch.randint(0, shape.vocab, (1, K1), dtype=torch.int32, device="cuda", generator=g)
        out = torch.empty(1, K1, dtype=torch.int32, device="cuda")
        for _ in range(args.warmup):
            dfl.dflash_verify_block(ctx, ids, K1, out)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            dfl.dflash_verify_block(ctx, ids, K1, out)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        byt = weight_bytes + (VERIFY_CTX + K1) * kv_per_pos
        flops = 2.0 * K1 * (weight_bytes / 2) + 4.0 * shape.n_layers * shape.n_q_heads * shape.head_dim * \
            K1 * (VERIFY_CTX + K1 / 2)
        sweep.append({"K1": K1, "verify_ms": round(ms, 4), "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "mfma_frac": round(flops / (ms * 1e-3) / 2.5e15, 4)})
        log(f"[bench] verify K1={K1}: {ms:.3f} ms")
    ctx.profile(True)
    ids = torch.randint(0, shape.vocab, (1, 16), dtype=torch.int32, device="cuda", generator=g)
    out = torch.empty(1, 16, dtype=torch.int32, device="cuda")
    for _ in range(3):
        dfl.dflash_verify_block(ctx, ids, 16, out)
    ph = {k: round(v[0] / 3, 4) for k, v in ctx.profile_read().items()}
    ctx.profile(False)
    lat = {r["K1"]: r["verify_ms"] for r in sweep}
    r16 = sweep[0]
    out = {
        "metric": "target verification latency vs block size (36-layer Qwen3-4B-shaped target, ctx 4096)",
        "value": r16["verify_ms"], "unit": "ms per verify at K1 = 16", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"target verify, 36 layers, H 2560, 32q/8kv x 128, I 9728, V 151936, "
                               f"taps {list(taps)}, ctx {VERIFY_CTX}", "batch": 1, "parallelism": "1 GPU"},
        "sweep": sweep,
        "latency_ratio_K1_128_over_16": round(lat[128] / lat[16], 4),
        "latency_ratio_K1_1024_over_16": round(lat[1024] / lat[16], 4),
        "phase_ms_at_K1_16": ph,
        "roofline": {"kernel": "whole verification at K1 = 16 (36 layers + LM head, events on the stream)",
                     "bound": "hbm", "achieved": round((weight_bytes + (VERIFY_CTX + 16) * kv_per_pos) /
                                                       (r16["verify_ms"] * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": r16["hbm_frac"], "traffic": None,
                     "bytes_per_launch": int(weight_bytes + (VERIFY_CTX + 16) * kv_per_pos)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = verify_cpu_baseline(shape, taps)
    print(json.dumps(out))


ADAPT_KS = (4, 8, 16, 32, 64)
# acceptance regimes of one session (a, gamma, steps as a share of the
# session): code-like, chat-like, mixed
ADAPT_PHASES = ((0.95, 0.98, 1 / 3), (0.6, 0.85, 1 / 3), (0.9, 0.95, 1 / 3))


def bench_adaptive(args, torch, dfl):
    """The whole speculative loop on one GPU, per step: draft K rows
    (drafter), verify the K + 1 rows [anchor, drafts] (36-layer target),
    acceptance length from the seeded agreement model (a, gamma per phase),
    commit tau rows in the target, project tau feature rows into the
    drafter.  Block size per step from dflash_adapt_choose (costs = the
    draft + verify latencies measured here), or fixed."""
    import synth
    wl = synth.workload(1)
    dshape = wl.shape
    tshape = synth.QWEN3_4B_TARGET.replace(n_feat=len(synth.QWEN3_4B_TAPS))
    w = synth.weights(dshape, wl.seed)
    dwd = dfl.weights_to_device(w)
    dmodel = dfl.Model(dshape, dwd)
    tw = synth.weights(tshape, VERIFY_SEED)
    twd = dfl.weights_to_device(tw)
    del tw
    tmodel = dfl.Model(tshape, twd, taps=synth.QWEN3_4B_TAPS)
    for k in list(twd):
        if k != "embed":
            del twd[k]
    torch.cuda.empty_cache()
    ctx0 = wl.ctx0[0]
    pre_feats = torch.from_numpy(synth.prefill_features(dshape, wl.seed, 0, ctx0)).cuda()
    kmax = max(ADAPT_KS)
    step_feats = torch.from_numpy(synth.step_features(dshape, wl.seed, 0, 0, kmax + 1)).cuda()
    g = torch.Generator(device="cuda")
    g.manual_seed(VERIFY_SEED)
    pre_ids = torch.randint(0, tshape.vocab, (1, ctx0), dtype=torch.int32, device="cuda", generator=g)

    def fresh():
        dctx = dfl.Context(dmodel, 1)
        dfl.dflash_project_ctx(dctx, pre_feats, [ctx0])
        tctx = dfl.Context(tmodel, 1)
        done = 0
        while done < ctx0:
            n = min(1024, ctx0 - done)
            out = torch.empty(1, n, dtype=torch.int32, device="cuda")
            dfl.dflash_verify_block(tctx, pre_ids[:, done:done + n].contiguous(), n, out)
            dfl.dflash_commit(tctx, [n])
            done += n
        return dctx, tctx

    draft = torch.empty(1, kmax, dtype=torch.int32, device="cuda")
    vids = torch.empty(1, kmax + 1, dtype=torch.int32, device="cuda")
    vout = torch.empty(1, kmax + 1, dtype=torch.int32, device="cuda")

    def one_step(dctx, tctx, d_ids, K, anchor, tau):
        """Enqueue one step (no host synchronisation)."""
        dk = draft[:, :K]
        dfl.dflash_draft_block(dctx, d_ids, K, dk)
        vids[:, 0] = anchor
        vids[:, 1:K + 1] = dk
        dfl.dflash_verify_block(tctx, vids[:, :K + 1], K + 1, vout[:, :K + 1])
        dfl.dflash_commit(tctx, [tau])
        dfl.dflash_project_ctx(dctx, step_feats[:tau], [tau])

    # per-step cost of each candidate at the starting context (ms)
    dctx, tctx = fresh()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    costs = []
    for K in ADAPT_KS:
        d_ids = torch.from_numpy(synth.block_ids(wl.seed, 0, 0, K, dshape.vocab).reshape(1, K)).cuda()
        vid = torch.randint(0, tshape.vocab, (1, K + 1), dtype=torch.int32, device="cuda", generator=g)
        for _ in range(3):
            dfl.dflash_draft_block(dctx, d_ids, K, draft[:, :K])
            dfl.dflash_verify_block(tctx, vid, K + 1, vout[:, :K + 1])
        e0.record()
        for _ in range(10):
            dfl.dflash_draft_block(dctx, d_ids, K, draft[:, :K])
            dfl.dflash_verify_block(tctx, vid, K + 1, vout[:, :K + 1])
        e1.record()
        torch.cuda.synchronize()
        costs.append(e0.elapsed_time(e1) / 10)
    del dctx, tctx
    log(f"[bench] per-step cost (draft + verify ms) at K {list(ADAPT_KS)}: {[round(c, 3) for c in costs]}")

    S = args.loop_steps
    bounds = []
    acc = 0
    for a, gm, share in ADAPT_PHASES:
        n = int(round(S * share))
        bounds.append((acc, acc + n, (a, gm)))
        acc += n

    def phase_of(t):
        for lo, hi, ph in bounds:
            if lo <= t < hi:
                return ph
        return bounds[-1][2]

    def plan(policy_K):
        """Block size, block ids and acceptance length of every step.  The
        acceptance lengths come from the seeded agreement model, not from
        the GPU's tokens, so the policy's choices can be made here, exactly
        as they would be online."""
        pol = dfl.AdaptPolicy(kmax, decay=0.95) if policy_K is None else None
        anchor = synth.first_anchor(wl.seed, 0, dshape.vocab)
        steps = []
        for t in range(acc):
            K = pol.choose(ADAPT_KS, costs)[0] if pol is not None else policy_K
            ids = synth.block_ids(wl.seed, 0, t, K, dshape.vocab)
            ids[0] = anchor
            a, gm = phase_of(t)
            dr = synth.verifier_draws(wl.seed, 0, t, K, dshape.vocab, a, gm)
            tau = 1 + int(np.argmin(np.append(dr.agree, False)))
            if pol is not None:
                pol.observe(K, tau)
            steps.append((K, ids, tau, anchor))
            anchor = dr.bonus
        return steps

    def session(policy_K):
        steps = plan(policy_K)
        flat = torch.from_numpy(np.concatenate([st[1] for st in steps]).astype(np.int32)).cuda()
        offs = np.cumsum([0] + [st[0] for st in steps])
        dctx, tctx = fresh()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for (K, _, tau, anchor), off in zip(steps, offs):
            one_step(dctx, tctx, flat[off:off + K].view(1, K), K, anchor, tau)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        tokens = sum(st[2] for st in steps)
        return tokens / wall, wall * 1e3 / acc, tokens / acc, [st[0] for st in steps]

    results = {}
    for K in ADAPT_KS:
        results[K] = session(K)
        log(f"[bench] fixed K={K}: {results[K][0]:.1f} accepted tok/s, {results[K][1]:.3f} ms/step, "
            f"mean tau {results[K][2]:.2f}")
    ad = session(None)
    log(f"[bench] adaptive: {ad[0]:.1f} accepted tok/s, {ad[1]:.3f} ms/step, mean tau {ad[2]:.2f}")
    per_phase = []
    for lo, hi, ph in bounds:
        ks = ad[3][lo:hi]
        per_phase.append({"a": ph[0], "gamma": ph[1], "steps": hi - lo,
                          "K_counts": {str(k): ks.count(k) for k in ADAPT_KS if ks.count(k)}})
    best_fixed = max(ADAPT_KS, key=lambda k: results[k][0])
    out = {
        "metric": "accepted tokens/s of the draft-verify loop with the adaptive block size "
                  "(Qwen3-4B-shaped drafter + 36-layer target, one GPU)",
        "value": round(ad[0], 1), "unit": "accepted tok/s", "n_gpus": 1, "steps": acc, "warmup": 0,
        "ms_per_step": round(ad[1], 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"draft-verify loop, ctx {ctx0}, candidates K {list(ADAPT_KS)}, acceptance "
                               f"a*gamma^i in phases {[(p[0], p[1]) for p in ADAPT_PHASES]}, policy decay 0.95",
                   "batch": 1, "parallelism": "1 GPU"},
        "cost_ms_per_step": {str(k): round(c, 4) for k, c in zip(ADAPT_KS, costs)},
        "fixed_K": {str(k): {"tok_s": round(results[k][0], 1), "ms_per_step": round(results[k][1], 4),
                             "mean_tau": round(results[k][2], 3)} for k in ADAPT_KS},
        "adaptive_mean_tau": round(ad[2], 3),
        "adaptive_over_K16": round(ad[0] / results[16][0], 4),
        "adaptive_over_best_fixed": round(ad[0] / results[best_fixed][0], 4),
        "best_fixed_K": best_fixed,
        "adaptive_K_per_phase": per_phase,
    }
    print(json.dumps(out))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; sharding across GPUs is not "
                                   "implemented", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import block_diffusion_drafting_amd as dfl
    import synth

    torch.cuda.set_device(0)
    if args.decay_ce:
        if args.copy_calibration:
            copy_calibration(torch)
        bench_decay_ce(args, torch, dfl)
        return
    if args.verify_sweep:
        bench_verify(args, torch, dfl)
        return
    if args.adaptive:
        bench_adaptive(args, torch, dfl)
        return
    if args.copy_calibration:
        copy_calibration(torch)
    wl = synth.workload(3 if args.ksweep else args.workload)
    Ks = list(wl.k_sweep) if args.ksweep else [args.K or wl.K]
    setup.persistent = args.persistent
    w, wd, model, ctx = setup(wl, Ks[0], dfl, torch)
    mb = model.bytes()
    stream = torch.cuda.current_stream()
    results = []
    for K in Ks:
        steps = plan_steps(wl, K, (args.warmup + 2 * args.steps + 10) if not args.ksweep
                           else args.warmup + args.steps)
        dev = [(torch.from_numpy(i).cuda(), torch.from_numpy(t).cuda(), tau, torch.from_numpy(f).cuda())
               for (i, t, tau, f) in steps]
        draft = torch.empty(wl.batch, K, dtype=torch.int32, device="cuda")
        acc = torch.empty(wl.batch, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

        # draft-block-only latency at the current context (events on the stream)
        ids0 = dev[0][0]
        for _ in range(5):
            dfl.dflash_draft_block(ctx, ids0, K, draft)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.draft_iters):
            dfl.dflash_draft_block(ctx, ids0, K, draft)
        e1.record(stream)
        torch.cuda.synchronize()
        draft_ms = e0.elapsed_time(e1) / args.draft_iters
        lens0, _ = ctx.query()

        if args.ksweep:
            # draft forward + acceptance at a fixed context, per block size
            e0.record(stream)
            for t in range(args.steps):
                i, tg, tau, f = dev[t % len(dev)]
                dfl.dflash_draft_block(ctx, i, K, draft)
                dfl.dflash_accept(draft, tg, wl.batch, K, acc)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            byt = block_bytes(wl.shape, mb, lens0, K, wl.batch)
            # per-phase times of a separate profiled pass
            ctx.profile(True)
            for _ in range(3):
                dfl.dflash_draft_block(ctx, ids0, K, draft)
            ph = {k: round(v[0] / 3, 4) for k, v in ctx.profile_read().items()}
            ctx.profile(False)
            results.append({"K": K, "draft_accept_ms": round(ms, 4), "draft_block_ms": round(draft_ms, 4),
                            "hbm_frac": round(byt / (draft_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "phase_ms": ph})
            log(f"[bench] K={K}: draft+accept {ms:.3f} ms, draft {draft_ms:.3f} ms")
            continue

        # The production step: dflash_step appends the positions accepted
        # at the previous step and drafts this block in one call (the
        # context K/V written by the QKV products), then dflash_accept.
        pending = [None]

        def fused(t):
            i, tg, tau, f = dev[t]
            if pending[0] is None:
                dfl.dflash_draft_block(ctx, i, K, draft)
            else:
                pf, ptau = pending[0]
                dfl.dflash_step(ctx, pf, ptau, i, K, draft)
            dfl.dflash_accept(draft, tg, wl.batch, K, acc)
            pending[0] = (f, tau)

        def flush():
            if pending[0] is not None:
                dfl.dflash_project_ctx(ctx, pending[0][0], pending[0][1])
                pending[0] = None

        # The same step as three calls: draft, accept, project.
        def unfused(t):
            i, tg, tau, f = dev[t]
            dfl.dflash_draft_block(ctx, i, K, draft)
            dfl.dflash_accept(draft, tg, wl.batch, K, acc)
            dfl.dflash_project_ctx(ctx, f, tau)

        # the dominant kernel: the whole block as one launch where the
        # single-launch path applies, else the LM head product
        persistent = ctx.persistent_path(K)
        dom = "persistent_draft" if persistent else "lm_head"
        for t in range(args.warmup):
            fused(t)
        torch.cuda.synchronize()
        lens_start, _ = ctx.query()
        ctx.profile(dom)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(args.warmup, args.warmup + args.steps):
            fused(t)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        prof = ctx.profile_read()
        ctx.profile(False)
        lens_end, caps = ctx.query()
        ms_step = wall * 1e3 / args.steps
        toks = wl.batch * K / (wall / args.steps)

        flush()
        t1 = args.warmup + args.steps
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(t1, t1 + args.steps):
            unfused(t)
        torch.cuda.synchronize()
        ms_unfused = (time.perf_counter() - t0) * 1e3 / args.steps

        dom_ms, dom_n = prof.get(dom, (0.0, 0))
        s = wl.shape
        M = wl.batch * K
        mean_ctx = [(a + b) / 2 for a, b in zip(lens_start, lens_end)]
        byt = block_bytes(s, mb, mean_ctx, K, wl.batch)
        if persistent:
            dom_bytes = byt
            dom_name = "persistent draft block (persist_draft_kernel: embed, 5 layers, LM head + argmax)"
        else:
            dom_bytes = s.vocab * s.hidden * s.elem_bytes + M * s.hidden * s.elem_bytes + M * 4
            dom_name = "LM head product + argmax (gemm_kernel, EPI_ARGMAX)"
        dom_avg = dom_ms / max(dom_n, 1)
        achieved = dom_bytes / (dom_avg * 1e-3) / 1e9 if dom_avg > 0 else 0.0
        # per-phase times of a separate pass of fused steps (every launch
        # timed), outside the timed regions so that the event records do not
        # slow the step loop
        n_ph = max(1, min(args.warmup, 10))
        t2 = t1 + args.steps
        ctx.profile(True)
        for t in range(t2, t2 + n_ph):
            fused(t)
        allp = ctx.profile_read()
        ctx.profile(False)
        flush()
        phases = {k: round(v[0] / n_ph, 4) for k, v in allp.items()}
        timeline = None
        if args.trace and persistent:
            ctx.profile("persistent_draft")
            for _ in range(3):
                dfl.dflash_draft_block(ctx, dev[0][0], K, draft)
            ctx.profile_read()
            ctx.profile(False)
            timeline = persist_timeline(ctx.persist_trace(), s.n_layers)
            for k, v in timeline.items():
                log(f"[bench] timeline {k}: {v}")
        out = {
            "metric": METRIC,
            "value": round(toks, 1),
            "unit": "drafted tok/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms_step, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16" if s.dtype == "bf16" else "f32",
            "data": "synthetic",
            "config": {"workload": wl.name, "batch": wl.batch, "K": K, "ctx0": list(wl.ctx0)[:4],
                       "hidden": s.hidden, "layers": s.n_layers, "vocab": s.vocab,
                       "parallelism": "1 GPU"},
            "unfused_ms_per_step": round(ms_unfused, 4),
            "draft_block_ms": round(draft_ms, 4),
            "draft_block_hbm_frac": round(block_bytes(s, mb, lens0, K, wl.batch) / (draft_ms * 1e-3) / 1e9
                                          / HBM_PEAK_GBS, 4),
            "step_hbm_frac": round(byt / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "phase_ms_per_step": phases,
            "draft_path": "single launch" if persistent else "per-product kernels",
            "persist_timeline_us": timeline,
            "roofline": {"kernel": dom_name,
                         "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(dom, wl.name, K), "avg_launch_ms": round(dom_avg, 5),
                         "launches": dom_n, "bytes_per_launch": int(dom_bytes)},
        }
        if not args.no_extras and args.workload == 1 and not args.K:
            out.update(headline_extras(args, torch, dfl, wl, model, ctx, K, dev[0][0], lens0, mb))
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(wl, K, w, args.cpu_steps)
        results.append(out)
        log(f"[bench] ctx {lens_start[:4]} -> {lens_end[:4]} cap {caps[:4]}")
    if args.ksweep:
        r16 = [r for r in results if r["K"] == 16]
        r128 = [r for r in results if r["K"] == 128]
        flat = (r128[0]["draft_block_ms"] / r16[0]["draft_block_ms"]) if (r16 and r128) else None
        print(json.dumps({"metric": "draft-block latency vs block size (Qwen3-4B shape, ctx 4096)",
                          "unit": "ms", "n_gpus": 1, "data": "synthetic", "dtype": "bf16",
                          "higher_is_better": False, "sweep": results,
                          "latency_ratio_K128_over_K16": round(flat, 4) if flat else None}))
    else:
        print(json.dumps(results[0]))
    # release the library's device memory while torch is fully alive
    torch.cuda.synchronize()
    ctx.close()
    model.close()


if __name__ == "__main__":
    main()
