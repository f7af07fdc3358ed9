"""Drives the host-side code of a libdflash build with no GPU work: run as a
script with the library's path, in a process that has the sanitizer
runtime preloaded (tests/test_host_sanitizers.py).  Every call returns
before any device work: version and error strings, the adaptive block-size
policy (host code), phase names, and the argument checks of the entry
points (NULL pointers, out-of-range values, malformed configurations, a
seeded fuzz of configurations and of the policy's calls).  Exits 0 when
every status is the expected one; a sanitizer report ends the process with
a nonzero status.  Pure Python and ctypes (no numpy or torch in the
sanitized process)."""
import ctypes as C
import random
import sys

OK, E_ARG, E_SHAPE = 0, -1, -2
MAX_K, MAX_BATCH = 1024, 256
F32, BF16 = 0, 1


class Config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_layers", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("intermediate", C.c_int32),
                ("vocab", C.c_int32), ("n_feat", C.c_int32), ("rope_theta", C.c_double),
                ("rms_eps", C.c_double), ("dtype", C.c_int32)]


class Layer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")]


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("lm_head", C.c_void_p), ("fc", C.c_void_p),
                ("final_norm", C.c_void_p), ("layers", C.POINTER(Layer))]


def good_config(**kw):
    c = Config(hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, intermediate=1408,
               vocab=4003, n_feat=3, rope_theta=1e6, rms_eps=1e-6, dtype=BF16)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


class Checker:
    def __init__(self, lib):
        self.lib = lib
        self.n = 0

    def expect(self, what, got, want):
        self.n += 1
        ok = got == want if not isinstance(want, tuple) else got in want
        if not ok:
            err = self.lib.dflash_last_error()
            sys.stderr.write(f"{what}: status {got}, expected {want} ({err!r})\n")
            sys.exit(3)
        if got != OK:
            msg = self.lib.dflash_last_error()
            if not msg:
                sys.stderr.write(f"{what}: error {got} without a message\n")
                sys.exit(3)


def main(path):
    lib = C.CDLL(path)
    lib.dflash_version.restype = C.c_char_p
    lib.dflash_last_error.restype = C.c_char_p
    lib.dflash_phase_name.restype = C.c_char_p
    ck = Checker(lib)
    assert lib.dflash_version().startswith(b"dflash")
    assert lib.dflash_abi_version() == 1
    for ph in range(-5, 40):
        lib.dflash_phase_name(ph)

    # configurations: each field out of range in turn, then a seeded fuzz
    out = C.c_void_p()
    bad = [dict(hidden=0), dict(hidden=100), dict(hidden=-64), dict(n_layers=-1), dict(n_layers=257),
           dict(head_dim=96), dict(head_dim=0), dict(n_q_heads=0), dict(n_kv_heads=0), dict(n_q_heads=6, n_kv_heads=4),
           dict(intermediate=0), dict(intermediate=1410), dict(vocab=0), dict(n_feat=0),
           dict(n_feat=1 << 20), dict(rope_theta=1.0), dict(rope_theta=float("nan")), dict(rms_eps=-1.0),
           dict(rms_eps=float("nan")), dict(dtype=7)]
    for kw in bad:
        cfg = good_config(**kw)
        st = lib.dflash_model_create(C.byref(cfg), None, None, None, C.byref(out))
        ck.expect(f"model_create {kw}", st, (E_ARG, E_SHAPE))
        assert out.value is None
    cfg = good_config()
    ck.expect("model_create out=NULL", lib.dflash_model_create(C.byref(cfg), None, None, None, None), E_ARG)
    ck.expect("model_create cfg=NULL", lib.dflash_model_create(None, None, None, None, C.byref(out)), E_ARG)
    # a valid configuration with missing weight pointers (never dereferenced)
    fake = 0x10000
    layers = (Layer * 2)(*[Layer(*([fake] * 9)) for _ in range(2)])
    for missing in ["embed", "lm_head", "fc", "final_norm", "layers", "wq", "w_down"]:
        w = Weights(fake, fake, fake, fake, layers)
        ls = (Layer * 2)(*[Layer(*([fake] * 9)) for _ in range(2)])
        w.layers = ls
        if missing in ("wq", "w_down"):
            setattr(ls[1], missing, None)
        elif missing == "layers":
            w.layers = C.POINTER(Layer)()
        else:
            setattr(w, missing, None)
        ck.expect(f"model_create without {missing}", lib.dflash_model_create(C.byref(cfg), C.byref(w), None, None,
                                                                             C.byref(out)), E_ARG)
    # target: malformed tap lists (checked before any device work)
    w = Weights(fake, fake, None, fake, layers)
    tcfg = good_config(n_feat=2)
    for taps in ([1, 0], [0, 0], [-1, 1], [0, 2], [5, 6]):
        t = (C.c_int32 * 2)(*taps)
        ck.expect(f"target_create taps {taps}", lib.dflash_target_create(C.byref(tcfg), C.byref(w), t, None, None,
                                                                         C.byref(out)), E_ARG)
    ck.expect("target_create taps NULL", lib.dflash_target_create(C.byref(tcfg), C.byref(w), None, None, None,
                                                                  C.byref(out)), E_ARG)
    rng = random.Random(2024)
    fields = [f for f, _ in Config._fields_]
    for i in range(2000):
        cfg = good_config()
        for _ in range(rng.randint(1, 3)):
            f = rng.choice(fields)
            if f in ("rope_theta", "rms_eps"):
                setattr(cfg, f, rng.choice([-1.0, 0.0, 0.5, 1.0, float("inf"), float("nan")]))
            else:
                setattr(cfg, f, rng.choice([-(1 << 31), -1, 0, 1, 3, 17, 63, 96, 1 << 20, (1 << 31) - 1]))
        st = lib.dflash_model_create(C.byref(cfg), None, None, None, C.byref(out))
        ck.expect(f"fuzz config {i}", st, (E_ARG, E_SHAPE))

    # contexts and the block calls on a NULL context
    n = C.c_int32()
    ck.expect("ctx_create out=NULL", lib.dflash_ctx_create(None, 1, None, None, None, None), E_ARG)
    ck.expect("ctx_create model=NULL", lib.dflash_ctx_create(None, 1, None, None, None, C.byref(out)), E_ARG)
    ck.expect("ctx_destroy NULL", lib.dflash_ctx_destroy(None), OK)
    ck.expect("model_destroy NULL", lib.dflash_model_destroy(None), OK)
    ck.expect("ctx_query NULL", lib.dflash_ctx_query(None, C.byref(n), C.byref(n)), E_ARG)

    # acceptance and the loss: argument errors
    buf = (C.c_int32 * 64)()
    ck.expect("accept NULL", lib.dflash_accept(None, buf, 1, 4, buf, None), E_ARG)
    for batch, K in ((0, 4), (-3, 4), (1, 0), (1, MAX_K + 1), ((1 << 20) + 1, 4)):
        ck.expect(f"accept batch={batch} K={K}", lib.dflash_accept(buf, buf, batch, K, buf, None), E_ARG)
    ws = (C.c_double * 4)()
    loss = (C.c_float * 4)()
    mis = C.c_void_p(C.addressof(ws) + 4)
    cases = [dict(loss=None), dict(workspace=None), dict(workspace=mis), dict(dtype=5), dict(rows=-1),
             dict(vocab=0), dict(block=0), dict(gamma=0.0), dict(gamma=float("nan")), dict(gamma=float("inf")),
             dict(logits=None), dict(targets=None), dict(ce=None)]
    for kw in cases:
        a = dict(logits=C.addressof(buf), dtype=F32, targets=C.addressof(buf), rows=4, vocab=8, block=4,
                 gamma=0.8, loss=C.addressof(loss), ce=C.addressof(loss), grad=None, workspace=C.addressof(ws))
        a.update(kw)
        ck.expect(f"decay_ce {kw}", lib.dflash_decay_ce(
            C.c_void_p(a["logits"]), a["dtype"], C.c_void_p(a["targets"]), a["rows"], a["vocab"], a["block"],
            C.c_double(a["gamma"]), C.c_void_p(a["loss"]), C.c_void_p(a["ce"]), None,
            a["workspace"] if isinstance(a["workspace"], C.c_void_p) else C.c_void_p(a["workspace"]), None), E_ARG)
        if "workspace" in kw:
            continue
        ck.expect(f"decay_ce_noalloc {kw}", lib.dflash_decay_ce_noalloc(
            C.c_void_p(a["logits"]), a["dtype"], C.c_void_p(a["targets"]), a["rows"], a["vocab"], a["block"],
            C.c_double(a["gamma"]), C.c_void_p(a["loss"]), C.c_void_p(a["ce"]), None, None), E_ARG)

    # the adaptive block-size policy (host code): argument errors, then a
    # seeded session of observations and choices
    p = C.c_void_p()
    D = C.c_double
    for args in ((0, 0.9, 4.0, 0.8, 0.95), (MAX_K + 1, 0.9, 4.0, 0.8, 0.95), (16, 0.0, 4.0, 0.8, 0.95),
                 (16, 1.5, 4.0, 0.8, 0.95), (16, 0.9, -1.0, 0.8, 0.95), (16, 0.9, 4.0, 0.0, 0.95),
                 (16, 0.9, 4.0, 0.8, 1.5), (16, float("nan"), 4.0, 0.8, 0.95)):
        k, *r = args
        ck.expect(f"adapt_create {args}", lib.dflash_adapt_create(k, *[D(x) for x in r], C.byref(p)), E_ARG)
    ck.expect("adapt_create out=NULL", lib.dflash_adapt_create(16, D(0.9), D(4.0), D(0.8), D(0.95), None), E_ARG)
    ck.expect("adapt_observe NULL", lib.dflash_adapt_observe(None, 4, 2), E_ARG)
    Kout, a_out, g_out, v_out = C.c_int32(), D(), D(), D()
    ck.expect("adapt_choose NULL", lib.dflash_adapt_choose(None, None, None, 0, None, None, None, None), E_ARG)
    for kmax in (1, 2, 16, 128, MAX_K):
        ck.expect(f"adapt_create kmax={kmax}", lib.dflash_adapt_create(kmax, D(0.97), D(2.0), D(0.8), D(0.95),
                                                                        C.byref(p)), OK)
        for K, tau in ((0, 1), (kmax + 1, 1), (1, 0), (1, 3), (kmax, kmax + 2)):
            ck.expect(f"adapt_observe K={K} tau={tau}", lib.dflash_adapt_observe(p, K, tau), E_ARG)
        for i in range(3000 if kmax <= 128 else 300):
            K = rng.randint(1, kmax)
            ck.expect("adapt_observe", lib.dflash_adapt_observe(p, K, rng.randint(1, K + 1)), OK)
            if i % 7 == 0:
                m = rng.randint(0, 6)
                ks = sorted(rng.sample(range(1, MAX_K + 1), m))
                cs = [rng.uniform(0.5, 3.0) for _ in ks]
                bad = rng.random() < 0.2 and m > 0
                if bad:
                    j = rng.randrange(m)
                    if rng.random() < 0.5:
                        cs[j] = rng.choice([0.0, -1.0, float("nan"), float("inf")])
                    else:
                        ks[j] = rng.choice([0, -5, MAX_K + 1, ks[j - 1] if j > 0 else 0])
                KA = (C.c_int32 * max(m, 1))(*ks)
                CA = (C.c_double * max(m, 1))(*cs)
                st = lib.dflash_adapt_choose(p, KA, CA, m, C.byref(Kout), C.byref(a_out), C.byref(g_out),
                                             C.byref(v_out))
                ck.expect("adapt_choose", st, E_ARG if bad else OK)
                if not bad and m > 0:
                    assert Kout.value in ks, (Kout.value, ks)
                    assert 0.0 < a_out.value <= 1.0 and 0.0 < g_out.value <= 1.0, (a_out.value, g_out.value)
        ck.expect("adapt_choose outputs NULL", lib.dflash_adapt_choose(p, KA, CA, 0, None, None, None, None), OK)
        ck.expect("adapt_destroy", lib.dflash_adapt_destroy(p), OK)
    ck.expect("adapt_destroy NULL", lib.dflash_adapt_destroy(None), OK)
    print(f"host ABI driver: {ck.n} calls with the expected status")


if __name__ == "__main__":
    main(sys.argv[1])
