// C-ABI of the DFlash draft-block path (declared in include/dflash.h):
// model repacking, proposer state, buffer growth and launch sequencing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <string>
#include <vector>

#include "../../include/dflash.h"
#include "kernels.h"

using namespace dflash;

namespace {

thread_local std::string g_err;

dflash_status fail(dflash_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_TRY(expr)                                                                 \
  do {                                                                                \
    hipError_t e_ = (expr);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(DFLASH_E_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), \
                  __FILE__, __LINE__);                                                \
  } while (0)

struct Alloc {
  dflash_allocator a{};
  bool custom = false;
  void* get(size_t n) {
    if (n == 0) n = 256;
    if (custom) return a.alloc(n, a.user);
    void* p = nullptr;
    if (hipMalloc(&p, n) != hipSuccess) return nullptr;
    return p;
  }
  void put(void* p) {
    if (!p) return;
    if (custom)
      a.free(p, a.user);
    else
      (void)hipFree(p);
  }
};

int env_int(const char* name, int dflt, int lo, int hi) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  const int x = atoi(v);
  return x < lo ? lo : (x > hi ? hi : x);
}

int64_t next_pow2(int64_t n) {
  int64_t c = 1;
  while (c < n) c <<= 1;
  return c;
}
int round_up(int v, int m) { return (v + m - 1) / m * m; }

}  // namespace

struct dflash_model {
  dflash_config cfg{};
  int es = 2;   // element size of weights and features
  int ces = 2;  // element size of the attention operands (fp16 / fp32)
  Alloc alloc;
  std::vector<void*> owned;
  const void* embed = nullptr;
  float* gains = nullptr;      // [(2L+1)][H]: attn_norm l, mlp_norm l, final
  double* inv_freq = nullptr;  // [d/2]
  std::vector<Packed> qkv, o, gu, down;
  Packed lm, fc, kv;
  PLayer* players = nullptr;   // device [L]: the layer table of the persistent draft kernel
  int64_t layer_bytes = 0, lm_bytes = 0, proj_bytes = 0;
  // a verification target (dflash_target_create): causal, no context
  // projection; tapped layers in increasing order (cfg.n_feat of them)
  bool target = false;
  std::vector<int> taps;

  const float* attn_gain(int l) const { return gains + (size_t)(2 * l) * cfg.hidden; }
  const float* mlp_gain(int l) const { return gains + (size_t)(2 * l + 1) * cfg.hidden; }
  const float* final_gain() const { return gains + (size_t)(2 * cfg.n_layers) * cfg.hidden; }
};

struct Buf {
  void* p = nullptr;
  size_t bytes = 0;
};

enum Phase {
  PH_EMBED, PH_QKV, PH_ATTN, PH_O, PH_GU, PH_DOWN, PH_LM, PH_FINAL, PH_FC, PH_KV, PH_GROW, PH_ROWMAP,
  PH_COMBINE, PH_RESID, PH_FCFIN, PH_PERSIST
};
static const char* kPhaseNames[DFLASH_NUM_PHASES] = {
    "embed", "qkv", "attention", "o_proj", "gate_up", "down", "lm_head", "finalize", "fc", "kv_inject",
    "grow", "rowmap", "attn_combine", "resid_norm", "fc_finalize", "persistent_draft"};

struct Profiler {
  uint32_t mask = 0;   // bit p: time phase p
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<std::pair<int, size_t>> recs;  // (phase, index of start event)
  hipEvent_t get() {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
  ~Profiler() {
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
  }
};

struct dflash_ctx {
  const dflash_model* m = nullptr;
  Profiler prof;
  int B = 0;
  int verified = 0;   // target contexts: rows of the last verified block (0 after a commit)
  Alloc alloc;
  std::vector<DevSeq> seq;  // host mirror (ctx_len, cap, phys, pointers)
  DevSeq* seq_dev = nullptr;
  // workspaces
  Buf x, ssq, q, bk, bvt, keys, part, attn_part, rowmap;
  Buf fixcnt;   // arrival counters of split-K products (zero between launches)
  Buf xg_hi, xg_lo, o_hi, o_lo, act_hi, act_lo, c_hi, c_lo;   // frag-layout activations
  // L2 warm-up of the output projection's weights by spare blocks of the
  // attention kernel (fragments per product wave; measured on the
  // Qwen3-4B-shaped K = 16 block: its whole weight set pays, 0.4865 ->
  // 0.4813 ms)
  int warm_o = 16;
  // attention grid: 8-wave workgroup equivalents per compute unit, and the
  // shortest key split (a multiple of 64)
  int attn_wgs_per_cu = 2;
  int attn_min_split = 128;
  // context K/V per block (MiB, all layers) above which attention loads it
  // nontemporally
  int attn_stream_mb = 128;
  // persistent single-launch draft block (see persist.hip)
  struct Persist {
    bool enabled = false;   // opt in: measured slower than the per-product kernels
    int nwg = 0;            // workgroups (compute units); 0 = not probed yet, -1 = unavailable
    int down_splits = 8;
    unsigned epoch = 0;     // launches since the barrier flags were last cleared
    int K = 0, max_splits = 0;   // shape the per-launch buffers were sized for
    Buf scratch;            // activations of every layer and phase (one launch)
    Buf apart;              // attention partials
    Buf sync;               // counters, flags, error word (zeroed once)
    size_t off_err = 0;     // byte offset of the error word in `sync`
    Buf trace;              // timeline of the last profiled launch
    int trace_nwg = 0, trace_stride = 0;
  } pst;
};

namespace {

dflash_status ensure(Alloc& al, Buf& b, size_t bytes) {
  if (b.bytes >= bytes && b.p) return DFLASH_OK;
  al.put(b.p);
  b.p = nullptr;
  b.bytes = 0;
  void* p = al.get(bytes);
  if (!p) return fail(DFLASH_E_ALLOC, "allocation of %zu bytes failed", bytes);
  b.p = p;
  b.bytes = bytes;
  return DFLASH_OK;
}

// A zero-filled frag-layout activation matrix of at least `mtiles` x `nkb`
// fragments (a hi/lo pair for bf16 models).
dflash_status ensure_frag(dflash_ctx* c, Buf& hi, Buf& lo, bool pair, int mtiles, int nkb, hipStream_t s,
                          Frag& out) {
  const size_t bytes = (size_t)mtiles * nkb * BLOCK_BYTES;
  for (int i = 0; i < (pair ? 2 : 1); ++i) {
    Buf& b = i ? lo : hi;
    if (b.bytes < bytes || !b.p) {
      dflash_status st = ensure(c->alloc, b, bytes);
      if (st) return st;
      HIP_TRY(launch_fill_u32((unsigned*)b.p, bytes / 4, 0u, s));
    }
  }
  out.hi = (u32x4*)hi.p;
  out.lo = pair ? (u32x4*)lo.p : nullptr;
  out.mtiles = mtiles;
  out.nkb = nkb;
  return DFLASH_OK;
}

// Records a start event now and the end event when destroyed (profiling on).
struct PhaseTimer {
  dflash_ctx* c;
  hipStream_t s;
  hipEvent_t end = nullptr;
  PhaseTimer(dflash_ctx* c_, int ph, hipStream_t s_) : c(c_), s(s_) {
    if (!(c->prof.mask >> ph & 1u)) return;
    hipEvent_t a = c->prof.get();
    hipEvent_t b = c->prof.get();
    if (!a || !b) return;
    if (hipEventRecord(a, s) != hipSuccess) return;
    c->prof.recs.push_back({ph, c->prof.used - 2});
    end = b;
  }
  ~PhaseTimer() {
    if (end) (void)hipEventRecord(end, s);
  }
};

dflash_status check_config(const dflash_config* c, bool target = false) {
  if (!c) return fail(DFLASH_E_ARG, "config is NULL");
  const int32_t dt = abi_int(c->dtype);
  if (dt != DFLASH_F32 && dt != DFLASH_BF16) return fail(DFLASH_E_ARG, "bad dtype %d", dt);
  if (c->hidden <= 0 || c->hidden % 64) return fail(DFLASH_E_SHAPE, "hidden %d must be a positive multiple of 64", c->hidden);
  if (c->n_layers < 0 || c->n_layers > 256) return fail(DFLASH_E_SHAPE, "n_layers %d out of range", c->n_layers);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(DFLASH_E_SHAPE, "head_dim %d: 64 or 128 supported", c->head_dim);
  if (c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->n_q_heads % c->n_kv_heads)
    return fail(DFLASH_E_SHAPE, "n_q_heads %d must be a positive multiple of n_kv_heads %d", c->n_q_heads, c->n_kv_heads);
  if (c->intermediate <= 0 || c->intermediate % 8) return fail(DFLASH_E_SHAPE, "intermediate %d must be a positive multiple of 8", c->intermediate);
  if (c->vocab <= 0) return fail(DFLASH_E_SHAPE, "vocab %d", c->vocab);
  if (c->n_feat < (target ? 0 : 1) || (int64_t)c->n_feat * c->hidden > (1 << 24))
    return fail(DFLASH_E_SHAPE, "n_feat %d", c->n_feat);
  if (!(c->rope_theta > 1.0) || !(c->rms_eps >= 0.0)) return fail(DFLASH_E_ARG, "rope_theta must be > 1 and rms_eps >= 0");
  return DFLASH_OK;
}

// Build a packed matrix from a host table of source-row addresses.
dflash_status pack(dflash_model* m, const std::vector<uint64_t>& rows, int kd, hipStream_t s, Packed& out) {
  const int es = m->es;
  const int kpl = 16 / es;
  if (kd % kpl) return fail(DFLASH_E_SHAPE, "reduction length %d not a multiple of %d", kd, kpl);
  const int n_rows = (int)rows.size();
  const int n_pad = round_up(n_rows, 16);
  const int nkb = (kd * es + 63) / 64;
  std::vector<uint64_t> tbl(rows);
  tbl.resize(n_pad, 0);
  const size_t bytes = (size_t)(n_pad / 16) * nkb * BLOCK_BYTES;
  void* dst = m->alloc.get(bytes);
  if (!dst) return fail(DFLASH_E_ALLOC, "allocation of %zu bytes for packed weights failed", bytes);
  m->owned.push_back(dst);
  uint64_t* dtbl = nullptr;
  HIP_TRY(hipMalloc((void**)&dtbl, tbl.size() * sizeof(uint64_t)));
  hipError_t e = hipMemcpyAsync(dtbl, tbl.data(), tbl.size() * sizeof(uint64_t), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = m->cfg.dtype == DFLASH_BF16 ? launch_pack<bf16_t>(dtbl, n_pad, kd, nkb, (uint8_t*)dst, s)
                                                       : launch_pack<float>(dtbl, n_pad, kd, nkb, (uint8_t*)dst, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(dtbl);
  if (e != hipSuccess) return fail(DFLASH_E_HIP, "weight packing failed: %s", hipGetErrorString(e));
  out.w = (const uint8_t*)dst;
  out.n_rows = n_rows;
  out.n_tiles = n_pad / 16;
  out.kd = kd;
  out.nkb = nkb;
  return DFLASH_OK;
}

int64_t packed_bytes(const Packed& p) { return (int64_t)p.n_tiles * p.nkb * BLOCK_BYTES; }

// Rows of one head's W_q or W_k in RoPE pair order: tile t of the head holds
// pairs 8t..8t+7, row 2q+c of the tile = channel (8t+q) + c*d/2.
void rope_rows(std::vector<uint64_t>& rows, const uint8_t* w, int head, int d, int row_bytes) {
  for (int t = 0; t < d / 16; ++t)
    for (int rr = 0; rr < 16; ++rr) {
      const int p = 8 * t + rr / 2;
      const int f = p + (rr % 2) * (d / 2);
      rows.push_back((uint64_t)(w + (size_t)(head * d + f) * row_bytes));
    }
}
void plain_rows(std::vector<uint64_t>& rows, const uint8_t* w, int n, int row_bytes) {
  for (int r = 0; r < n; ++r) rows.push_back((uint64_t)(w + (size_t)r * row_bytes));
}

bool valid_stream_ptrs(const dflash_weights* w, int L, bool target = false) {
  if (!w || !w->embed || !w->lm_head || (!target && !w->fc) || !w->final_norm) return false;
  if (L > 0 && !w->layers) return false;
  for (int l = 0; l < L; ++l) {
    const dflash_layer_weights& lw = w->layers[l];
    if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.mlp_norm || !lw.w_gate ||
        !lw.w_up || !lw.w_down)
      return false;
  }
  return true;
}

}  // namespace

// For the host-only sources of the library (C++ linkage, not exported).
dflash_status dflash_set_error(dflash_status st, const char* msg) { return fail(st, "%s", msg); }

extern "C" {

const char* dflash_version(void) { return "dflash-mi355x 0.1 (gfx950)"; }
int32_t dflash_abi_version(void) { return DFLASH_ABI_VERSION; }
const char* dflash_last_error(void) { return g_err.c_str(); }

}  // extern "C"

static dflash_status model_create(const dflash_config* cfg, const dflash_weights* w, const int32_t* taps,
                                  bool target, const dflash_allocator* alloc, void* stream, dflash_model** out) {
  if (!out) return fail(DFLASH_E_ARG, "out is NULL");
  *out = nullptr;
  dflash_status st = check_config(cfg, target);
  if (st) return st;
  if (!valid_stream_ptrs(w, cfg->n_layers, target)) return fail(DFLASH_E_ARG, "a weight pointer is NULL");
  if (alloc && (!alloc->alloc || !alloc->free)) return fail(DFLASH_E_ARG, "allocator callbacks are NULL");
  if (target) {
    if (cfg->n_feat > 0 && !taps) return fail(DFLASH_E_ARG, "taps is NULL");
    for (int i = 0; i < cfg->n_feat; ++i)
      if (taps[i] < 0 || taps[i] >= cfg->n_layers || (i > 0 && taps[i] <= taps[i - 1]))
        return fail(DFLASH_E_ARG, "taps must be increasing layer indices in [0, %d)", cfg->n_layers);
  }
  hipStream_t s = (hipStream_t)stream;
  dflash_model* m = new dflash_model();
  m->cfg = *cfg;
  m->target = target;
  if (target) m->taps.assign(taps, taps + cfg->n_feat);
  m->es = cfg->dtype == DFLASH_BF16 ? 2 : 4;
  m->ces = m->es;
  if (alloc) {
    m->alloc.a = *alloc;
    m->alloc.custom = true;
  }
  m->embed = w->embed;
  const int H = cfg->hidden, L = cfg->n_layers, d = cfg->head_dim, nq = cfg->n_q_heads,
            nkv = cfg->n_kv_heads, I = cfg->intermediate, es = m->es;
  auto cleanup = [&](dflash_status r) {
    dflash_model_destroy(m);
    return r;
  };

  // gains -> fp32, inverse RoPE frequencies
  m->gains = (float*)m->alloc.get((size_t)(2 * L + 1) * H * sizeof(float));
  m->inv_freq = (double*)m->alloc.get((size_t)(d / 2) * sizeof(double));
  if (!m->gains || !m->inv_freq) return cleanup(fail(DFLASH_E_ALLOC, "allocation failed"));
  m->owned.push_back(m->gains);
  m->owned.push_back(m->inv_freq);
  auto conv = [&](const void* src, float* dst) {
    return cfg->dtype == DFLASH_BF16 ? launch_to_f32<bf16_t>(src, dst, H, s) : launch_to_f32<float>(src, dst, H, s);
  };
  for (int l = 0; l < L; ++l) {
    if (conv(w->layers[l].attn_norm, (float*)m->attn_gain(l)) != hipSuccess ||
        conv(w->layers[l].mlp_norm, (float*)m->mlp_gain(l)) != hipSuccess)
      return cleanup(fail(DFLASH_E_HIP, "gain conversion failed"));
  }
  if (conv(w->final_norm, (float*)m->final_gain()) != hipSuccess) return cleanup(fail(DFLASH_E_HIP, "gain conversion failed"));
  {
    std::vector<double> inv(d / 2);
    for (int i = 0; i < d / 2; ++i) inv[i] = pow(cfg->rope_theta, -2.0 * i / d);
    if (hipMemcpyAsync(m->inv_freq, inv.data(), inv.size() * sizeof(double), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return cleanup(fail(DFLASH_E_HIP, "upload of RoPE frequencies failed"));
  }

  const int rowH = H * es;
  m->qkv.resize(L);
  m->o.resize(L);
  m->gu.resize(L);
  m->down.resize(L);
  for (int l = 0; l < L; ++l) {
    const dflash_layer_weights& lw = w->layers[l];
    std::vector<uint64_t> rows;
    for (int h = 0; h < nq; ++h) rope_rows(rows, (const uint8_t*)lw.wq, h, d, rowH);
    for (int g = 0; g < nkv; ++g) rope_rows(rows, (const uint8_t*)lw.wk, g, d, rowH);
    plain_rows(rows, (const uint8_t*)lw.wv, nkv * d, rowH);
    if ((st = pack(m, rows, H, s, m->qkv[l]))) return cleanup(st);
    rows.clear();
    plain_rows(rows, (const uint8_t*)lw.wo, H, nq * d * es);
    if ((st = pack(m, rows, nq * d, s, m->o[l]))) return cleanup(st);
    rows.clear();
    for (int t = 0; t < I / 8; ++t)
      for (int rr = 0; rr < 16; ++rr) {
        const int g4 = rr / 4, j = rr % 4;
        const int f = 8 * t + 2 * g4 + j / 2;
        const uint8_t* base = (const uint8_t*)((j % 2 == 0) ? lw.w_gate : lw.w_up);
        rows.push_back((uint64_t)(base + (size_t)f * rowH));
      }
    if ((st = pack(m, rows, H, s, m->gu[l]))) return cleanup(st);
    rows.clear();
    plain_rows(rows, (const uint8_t*)lw.w_down, H, I * es);
    if ((st = pack(m, rows, I, s, m->down[l]))) return cleanup(st);
    m->layer_bytes += packed_bytes(m->qkv[l]) + packed_bytes(m->o[l]) + packed_bytes(m->gu[l]) +
                      packed_bytes(m->down[l]);
  }
  {
    std::vector<uint64_t> rows;
    plain_rows(rows, (const uint8_t*)w->lm_head, cfg->vocab, rowH);
    if ((st = pack(m, rows, H, s, m->lm))) return cleanup(st);
    m->lm_bytes = packed_bytes(m->lm);
    rows.clear();
  }
  if (!target) {
    std::vector<uint64_t> rows;
    plain_rows(rows, (const uint8_t*)w->fc, H, cfg->n_feat * H * es);
    if ((st = pack(m, rows, cfg->n_feat * H, s, m->fc))) return cleanup(st);
    rows.clear();
    for (int l = 0; l < L; ++l) {
      for (int g = 0; g < nkv; ++g) rope_rows(rows, (const uint8_t*)w->layers[l].wk, g, d, rowH);
      plain_rows(rows, (const uint8_t*)w->layers[l].wv, nkv * d, rowH);
    }
    if (L > 0) {
      if ((st = pack(m, rows, H, s, m->kv))) return cleanup(st);
    }
    m->proj_bytes = packed_bytes(m->fc) + (L > 0 ? packed_bytes(m->kv) : 0);
  }
  if (L > 0 && !target) {
    std::vector<PLayer> tbl(L);
    for (int l = 0; l < L; ++l) {
      tbl[l].qkv = m->qkv[l];
      tbl[l].o = m->o[l];
      tbl[l].gu = m->gu[l];
      tbl[l].down = m->down[l];
      tbl[l].attn_gain = m->attn_gain(l);
      tbl[l].mlp_gain = m->mlp_gain(l);
    }
    m->players = (PLayer*)m->alloc.get(sizeof(PLayer) * L);
    if (!m->players) return cleanup(fail(DFLASH_E_ALLOC, "allocation failed"));
    m->owned.push_back(m->players);
    if (hipMemcpyAsync(m->players, tbl.data(), sizeof(PLayer) * L, hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return cleanup(fail(DFLASH_E_HIP, "upload of the layer table failed"));
  }
  *out = m;
  return DFLASH_OK;
}

extern "C" {

dflash_status dflash_model_create(const dflash_config* cfg, const dflash_weights* w,
                                  const dflash_allocator* alloc, void* stream, dflash_model** out) {
  return model_create(cfg, w, nullptr, false, alloc, stream, out);
}

dflash_status dflash_target_create(const dflash_config* cfg, const dflash_weights* w, const int32_t* taps,
                                   const dflash_allocator* alloc, void* stream, dflash_model** out) {
  return model_create(cfg, w, taps, true, alloc, stream, out);
}

dflash_status dflash_model_destroy(dflash_model* m) {
  if (!m) return DFLASH_OK;
  for (void* p : m->owned) m->alloc.put(p);
  delete m;
  return DFLASH_OK;
}

dflash_status dflash_model_bytes(const dflash_model* m, int64_t* layer_bytes, int64_t* lm_head_bytes,
                                 int64_t* proj_bytes) {
  if (!m) return fail(DFLASH_E_ARG, "model is NULL");
  if (layer_bytes) *layer_bytes = m->layer_bytes;
  if (lm_head_bytes) *lm_head_bytes = m->lm_bytes;
  if (proj_bytes) *proj_bytes = m->proj_bytes;
  return DFLASH_OK;
}

}  // extern "C"

static dflash_status alloc_seq(dflash_ctx* c, int b, int cap, DevSeq& out) {
  const dflash_model* m = c->m;
  const int phys = cap < 64 ? 64 : cap;
  const size_t ces = m->ces;
  // attention addresses one layer and KV head's slab with 32-bit offsets
  if ((size_t)phys * m->cfg.head_dim * ces >= ((size_t)1 << 31))
    return fail(DFLASH_E_ARG, "context capacity %d exceeds the per-head cache slab limit (2^31 bytes)", cap);
  const size_t kvn = (size_t)m->cfg.n_layers * m->cfg.n_kv_heads * phys * m->cfg.head_dim;
  DevSeq v{};
  v.ctx_len = c->seq[b].ctx_len;
  v.cap = cap;
  v.phys = phys;
  v.ctxbuf = m->target ? nullptr : c->alloc.get((size_t)phys * m->cfg.hidden * sizeof(float));
  v.k = c->alloc.get(kvn * ces);
  v.vt = c->alloc.get(kvn * ces);
  if ((!m->target && !v.ctxbuf) || !v.k || !v.vt) {
    c->alloc.put(v.ctxbuf);
    c->alloc.put(v.k);
    c->alloc.put(v.vt);
    return fail(DFLASH_E_ALLOC, "allocation of context buffers (cap %d) failed", cap);
  }
  out = v;
  return DFLASH_OK;
}

extern "C" {

dflash_status dflash_ctx_create(const dflash_model* m, int32_t batch, const int32_t* init_cap,
                                const dflash_allocator* alloc, void* stream, dflash_ctx** out) {
  if (!out) return fail(DFLASH_E_ARG, "out is NULL");
  *out = nullptr;
  if (!m) return fail(DFLASH_E_ARG, "model is NULL");
  if (batch < 1 || batch > DFLASH_MAX_BATCH) return fail(DFLASH_E_ARG, "batch %d out of [1, %d]", batch, DFLASH_MAX_BATCH);
  if (alloc && (!alloc->alloc || !alloc->free)) return fail(DFLASH_E_ARG, "allocator callbacks are NULL");
  if (init_cap)
    for (int b = 0; b < batch; ++b)
      if (init_cap[b] < 0 || init_cap[b] > (1 << 30) || (init_cap[b] & (init_cap[b] - 1)))
        return fail(DFLASH_E_ARG, "init_cap[%d] = %d is not a power of two (or 0)", b, init_cap[b]);
  hipStream_t s = (hipStream_t)stream;
  dflash_ctx* c = new dflash_ctx();
  c->m = m;
  c->B = batch;
  if (alloc) {
    c->alloc.a = *alloc;
    c->alloc.custom = true;
  }
  c->seq.assign(batch, DevSeq{});
  c->pst.enabled = env_int("DFLASH_PERSISTENT", 0, 0, 1) != 0;
  c->warm_o = env_int("DFLASH_WARM_O", c->warm_o, 0, 64);
  c->attn_wgs_per_cu = env_int("DFLASH_ATTN_WGS_PER_CU", c->attn_wgs_per_cu, 1, 16);
  c->attn_min_split = round_up(env_int("DFLASH_ATTN_MIN_SPLIT", c->attn_min_split, 64, 1 << 20), 64);
  c->attn_stream_mb = env_int("DFLASH_ATTN_STREAM_MB", c->attn_stream_mb, 0, 1 << 20);
  c->seq_dev = (DevSeq*)c->alloc.get(sizeof(DevSeq) * batch);
  if (!c->seq_dev) {
    delete c;
    return fail(DFLASH_E_ALLOC, "allocation failed");
  }
  for (int b = 0; b < batch; ++b) {
    const int cap = init_cap ? init_cap[b] : 0;
    if (cap > 0) {
      DevSeq v;
      dflash_status st = alloc_seq(c, b, cap, v);
      if (st) {
        dflash_ctx_destroy(c);
        return st;
      }
      c->seq[b] = v;
    }
    if (launch_set_seq(c->seq_dev, b, c->seq[b], s) != hipSuccess) {
      dflash_ctx_destroy(c);
      return fail(DFLASH_E_HIP, "descriptor upload failed");
    }
  }
  *out = c;
  return DFLASH_OK;
}

dflash_status dflash_ctx_destroy(dflash_ctx* c) {
  if (!c) return DFLASH_OK;
  for (DevSeq& v : c->seq) {
    c->alloc.put(v.ctxbuf);
    c->alloc.put(v.k);
    c->alloc.put(v.vt);
  }
  c->alloc.put(c->seq_dev);
  for (Buf* b : {&c->x, &c->ssq, &c->q, &c->bk, &c->bvt, &c->keys, &c->part, &c->attn_part, &c->rowmap, &c->fixcnt,
                 &c->xg_hi, &c->xg_lo, &c->o_hi, &c->o_lo, &c->act_hi, &c->act_lo, &c->c_hi, &c->c_lo,
                 &c->pst.scratch, &c->pst.apart, &c->pst.sync, &c->pst.trace})
    c->alloc.put(b->p);
  delete c;
  return DFLASH_OK;
}

dflash_status dflash_ctx_query(const dflash_ctx* c, int32_t* ctx_len, int32_t* cap) {
  if (!c) return fail(DFLASH_E_ARG, "ctx is NULL");
  for (int b = 0; b < c->B; ++b) {
    if (ctx_len) ctx_len[b] = c->seq[b].ctx_len;
    if (cap) cap[b] = c->seq[b].cap;
  }
  return DFLASH_OK;
}

dflash_status dflash_ctx_buffers(const dflash_ctx* c, int32_t b, const void** ctxbuf, const void** k_cache,
                                 const void** v_cache, int32_t* phys_rows) {
  if (!c) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (b < 0 || b >= c->B) return fail(DFLASH_E_ARG, "sequence %d out of range", b);
  if (ctxbuf) *ctxbuf = c->seq[b].ctxbuf;
  if (k_cache) *k_cache = c->seq[b].k;
  if (v_cache) *v_cache = c->seq[b].vt;
  if (phys_rows) *phys_rows = c->seq[b].phys;
  return DFLASH_OK;
}

}  // extern "C"

static EpiArgs base_epi(const dflash_ctx* c, int M) {
  const dflash_model* m = c->m;
  EpiArgs e{};
  e.M = M;
  e.eps = (float)m->cfg.rms_eps;
  e.nq = m->cfg.n_q_heads;
  e.nkv = m->cfg.n_kv_heads;
  e.d = m->cfg.head_dim;
  e.H = m->cfg.hidden;
  e.I = m->cfg.intermediate;
  e.V = m->cfg.vocab;
  e.L = m->cfg.n_layers;
  e.seqs = c->seq_dev;
  e.inv_freq = m->inv_freq;
  return e;
}

// One weight product.  X: frag-layout activations, or (Xrow != null) the
// caller's row-major features.  Returns the plan (for split-K consumers).
template <typename T>
static dflash_status run_gemm(dflash_ctx* c, int phase, int epi, const Packed& W, const Frag& X,
                              const void* Xrow, int ldx, int M, EpiArgs e, hipStream_t s,
                              GemmPlan* plan_out = nullptr, bool force_split = false) {
  GemmPlan p = plan_gemm(epi, W, M, sizeof(T) == 2, Xrow != nullptr);
  if (force_split && sizeof(T) == 2) p.split = true;
  dflash_status st;
  if (p.part_floats && (st = ensure(c->alloc, c->part, p.part_floats * sizeof(float)))) return st;
  GemmArgs g{};
  g.W = W;
  g.X = X;
  g.Xrow = Xrow;
  g.ldx = ldx;
  g.M = M;
  e.part = (float*)c->part.p;
  e.part_ntiles = W.n_tiles;
  e.part_mtiles = (M + 15) / 16;
  if (epi == EPI_PARTRES) {
    if (p.nsplit > MAX_SPLITS) return fail(DFLASH_E_ARG, "split product: %d splits", p.nsplit);
    // one counter per (tile group, m-group), zero-filled when allocated;
    // every launch leaves its counters at zero
    const size_t bytes = (size_t)p.n_groups * p.m_groups * sizeof(unsigned);
    if (c->fixcnt.bytes < bytes || !c->fixcnt.p) {
      if ((st = ensure(c->alloc, c->fixcnt, bytes))) return st;
      HIP_TRY(launch_fill_u32((unsigned*)c->fixcnt.p, c->fixcnt.bytes / 4, 0u, s));
    }
    e.fix_cnt = (unsigned*)c->fixcnt.p;
  }
  {
    PhaseTimer tm(c, phase, s);
    HIP_TRY(launch_gemm<T>(epi, p, g, e, s));
  }
  if (plan_out) *plan_out = p;
  return DFLASH_OK;
}

// Warm-up descriptor for the product `epi` over W with M activation rows,
// planned exactly as run_gemm will launch it (see Warm in kernels.h);
// `frags` weight fragments per product wave (0 = none).
template <typename T>
static Warm make_warm(int epi, const Packed& W, int M, int frags, bool force_split = false) {
  Warm w{};
  if (frags <= 0) return w;
  GemmPlan p = plan_gemm(epi, W, M, sizeof(T) == 2, false);
  (void)force_split;   // the hi/lo choice does not change which weights a workgroup reads
  // another tile-to-workgroup map: not warmed
  if (p.wide || uses_head_kernel(epi, p, W.n_tiles, (int)sizeof(T))) return w;
  w.w = W.w;
  w.nkb = W.nkb;
  w.n_tiles = W.n_tiles;
  w.n_groups = p.n_groups;
  w.nsplit = p.nsplit;
  w.kbu = p.kbu;
  w.waves = p.fixed ? 4 : (p.mtt == 4 ? 4 : 8);
  w.frags = frags;
  w.consumers = p.n_groups * p.nsplit;
  return w;
}

// (a2) growth: a sequence whose append would overflow its capacity gets
// buffers of the next power of two of the new length, the held rows copied
// (host-authoritative; enqueued before anything reads the buffers).
template <typename T>
static dflash_status grow_for(dflash_ctx* c, const int32_t* n_new, hipStream_t s) {
  const dflash_model* m = c->m;
  const int B = c->B, H = m->cfg.hidden;
  for (int b = 0; b < B; ++b) {
    DevSeq& v = c->seq[b];
    const int64_t need = (int64_t)v.ctx_len + n_new[b];
    if (n_new[b] == 0 || need <= v.cap) continue;
    const int cap = (int)next_pow2(need);
    DevSeq nv;
    dflash_status st = alloc_seq(c, b, cap, nv);
    if (st) return st;
    if (v.k) {
      PhaseTimer tm(c, PH_GROW, s);
      hipError_t e = launch_grow_copy<typename CacheOf<T>::type>(v, nv, m->cfg.n_layers, m->cfg.n_kv_heads,
                                                                m->cfg.head_dim, H, s);
      if (e != hipSuccess) return fail(DFLASH_E_HIP, "growth copy failed: %s", hipGetErrorString(e));
    }
    HIP_TRY(launch_set_seq(c->seq_dev, b, nv, s));
    c->alloc.put(v.ctxbuf);
    c->alloc.put(v.k);
    c->alloc.put(v.vt);
    v = nv;
  }
  return DFLASH_OK;
}

// Row starts of an append and the host context lengths before it.
static RowInfo row_info(const dflash_ctx* c, const int32_t* n_new) {
  RowInfo ri;
  ri.start[0] = 0;
  for (int b = 0; b < c->B; ++b) {
    ri.start[b + 1] = ri.start[b] + n_new[b];
    ri.ctx0[b] = c->seq[b].ctx_len;
  }
  return ri;
}

template <typename T>
static dflash_status project_impl(dflash_ctx* c, const void* feats, const int32_t* n_new,
                                  const int32_t* positions, hipStream_t s) {
  const dflash_model* m = c->m;
  const int B = c->B, H = m->cfg.hidden;
  dflash_status st;
  if ((st = grow_for<T>(c, n_new, s))) return st;
  const RowInfo ri = row_info(c, n_new);
  const int total = ri.start[B];
  if (total == 0) return DFLASH_OK;
  const int mtiles = (total + 15) / 16;
  Frag cb;
  if ((st = ensure(c->alloc, c->rowmap, sizeof(RowMap) * total)) ||
      (st = ensure_frag(c, c->c_hi, c->c_lo, sizeof(T) == 2, mtiles, m->fc.n_tiles * 16 * m->es / 64, s, cb)))
    return st;
  EpiArgs e = base_epi(c, total);
  e.cbuf = cb;
  e.rowmap = (const RowMap*)c->rowmap.p;
  const Frag none{};
  if (mtiles <= 4) {
    // few rows: split the reduction over workgroups, then add the splits
    // (and map the rows) in one pass
    GemmPlan p;
    if ((st = run_gemm<T>(c, PH_FC, EPI_PART, m->fc, none, feats, m->cfg.n_feat * H, total, e, s, &p))) return st;
    PhaseTimer tm(c, PH_FCFIN, s);
    HIP_TRY(launch_fc_finalize<T>((const float*)c->part.p, p.nsplit, mtiles, total, H, ri, B, positions,
                                  (RowMap*)c->rowmap.p, c->seq_dev, cb, 0, s));
  } else {
    {
      PhaseTimer tm(c, PH_ROWMAP, s);
      HIP_TRY(launch_rowmap(ri, B, total, positions, c->seq_dev, (RowMap*)c->rowmap.p, s));
    }
    if ((st = run_gemm<T>(c, PH_FC, EPI_FC, m->fc, none, feats, m->cfg.n_feat * H, total, e, s))) return st;
  }
  if (m->cfg.n_layers > 0)
    if ((st = run_gemm<T>(c, PH_KV, EPI_KV, m->kv, cb, nullptr, 0, total, e, s))) return st;
  for (int b = 0; b < B; ++b) c->seq[b].ctx_len += n_new[b];
  return DFLASH_OK;
}

extern "C" {

dflash_status dflash_project_ctx(dflash_ctx* c, const void* feats, const int32_t* n_new,
                                 const int32_t* positions, void* stream) {
  if (!c) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (c->m->target) return fail(DFLASH_E_STATE, "a target context verifies blocks (dflash_verify_block)");
  if (!n_new) return fail(DFLASH_E_ARG, "n_new is NULL");
  int64_t total = 0;
  for (int b = 0; b < c->B; ++b) {
    if (n_new[b] < 0) return fail(DFLASH_E_ARG, "n_new[%d] = %d is negative", b, n_new[b]);
    if ((int64_t)c->seq[b].ctx_len + n_new[b] > (1 << 30))
      return fail(DFLASH_E_SHAPE, "sequence %d would exceed 2^30 positions", b);
    total += n_new[b];
  }
  if (total > (1 << 30)) return fail(DFLASH_E_SHAPE, "too many rows in one call");
  if (total > 0 && !feats) return fail(DFLASH_E_ARG, "feats is NULL");
  hipStream_t s = (hipStream_t)stream;
  return c->m->cfg.dtype == DFLASH_BF16 ? project_impl<bf16_t>(c, feats, n_new, positions, s)
                                        : project_impl<float>(c, feats, n_new, positions, s);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// persistent single-launch draft block (persist.hip): bf16 drafters whose
// block has at most 16 rows in all
// ---------------------------------------------------------------------------

// Workgroups of the persistent kernel (one per compute unit), or -1 when
// the device cannot run it (no cooperative launch, occupancy, grid shape).
static int persist_nwg(dflash_ctx* c) {
  auto& P = c->pst;
  if (P.nwg != 0) return P.nwg;
  P.nwg = -1;
  P.down_splits = env_int("DFLASH_DOWN_SPLITS", 8, 1, 32);

  int dev = 0, coop = 0, n = 0, occ = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return -1;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (persist_occupancy(c->m->cfg.head_dim, &occ) != hipSuccess || occ < 1) return -1;
  // the flag barrier reads at most 256 flags; the down projection's splits
  // must divide the grid
  if (n < 8 || n > 256 || n % P.down_splits) return -1;
  P.nwg = n;
  return n;
}

static bool persist_ok(dflash_ctx* c, int K) {
  const dflash_config& cf = c->m->cfg;
  if (!c->pst.enabled || cf.dtype != DFLASH_BF16 || cf.n_layers < 1 || cf.n_layers > PERSIST_MAX_LAYERS) return false;
  if ((int64_t)c->B * K > 16) return false;                       // one 16-row activation tile
  if ((int64_t)(cf.n_q_heads / cf.n_kv_heads) * K > 64) return false;  // one query group per KV head
  if (cf.head_dim != 64 && cf.head_dim != 128) return false;
  if (cf.hidden > 4096) return false;                              // norm loads per thread
  if (persist_nwg(c) <= 0) return false;
  const dflash_model* m = c->m;
  return persist_passes_fit(c->pst.nwg, c->pst.down_splits, cf.n_layers, m->qkv[0].n_tiles, m->o[0].n_tiles,
                            m->gu[0].n_tiles, m->down[0].n_tiles, m->lm.n_tiles);
}

static dflash_status persist_draft(dflash_ctx* c, const int32_t* ids, int K, int32_t* draft, float* logits,
                                   void* hidden, hipStream_t s) {
  const dflash_model* m = c->m;
  const dflash_config& cf = m->cfg;
  auto& P = c->pst;
  const int B = c->B, H = cf.hidden, L = cf.n_layers, d = cf.head_dim, nq = cf.n_q_heads, nkv = cf.n_kv_heads;
  const int nwg = P.nwg, S = P.down_splits;
  const int Kpad = round_up(K, 64);
  // attention: the smallest split length (a multiple of 64, at least 128)
  // whose (sequence, KV head, split) units fit one round of the grid
  int max_len = 0;
  for (int b = 0; b < B; ++b) max_len = c->seq[b].ctx_len > max_len ? c->seq[b].ctx_len : max_len;
  int chunk = c->attn_min_split;
  for (;; chunk += 64) {
    int64_t units = 0;
    for (int b = 0; b < B; ++b) units += (int64_t)nkv * ((c->seq[b].ctx_len + chunk - 1) / chunk + (K + chunk - 1) / chunk);
    if (units <= nwg || chunk >= max_len + K) break;
  }
  int max_splits = 0;
  for (int b = 0; b < B; ++b) {
    const int ns = (c->seq[b].ctx_len + chunk - 1) / chunk + (K + chunk - 1) / chunk;
    max_splits = ns > max_splits ? ns : max_splits;
  }
  const int nkb_h = H / 32, nkb_o = nq * d / 32, nkb_i = m->down[0].nkb, T_h = H / 16;
  // per-launch buffers
  auto al = [](size_t& off, size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  size_t off = 0;
  al(off, (size_t)(2 * L + 1) * 16 * H * 4);                          // xs
  const size_t o_xg = al(off, (size_t)(2 * L + 1) * 2 * nkb_h * BLOCK_BYTES);
  const size_t o_ssq = al(off, (size_t)(2 * L + 1) * H * 4);
  const size_t o_q = al(off, (size_t)L * 16 * nq * d * 2);
  const size_t o_bk = al(off, (size_t)L * B * nkv * Kpad * d * 2);
  const size_t o_bvt = al(off, (size_t)L * B * nkv * Kpad * d * 2);
  const size_t o_of = al(off, (size_t)L * 2 * nkb_o * BLOCK_BYTES);
  const size_t o_act = al(off, (size_t)L * 2 * nkb_i * BLOCK_BYTES);
  const size_t o_dp = al(off, (size_t)L * S * T_h * 256 * 4);
  dflash_status st;
  if (P.scratch.bytes < off || !P.scratch.p) {
    if ((st = ensure(c->alloc, P.scratch, off))) return st;
    // zero: the k-block padding of the SwiGLU output is never written
    HIP_TRY(launch_fill_u32((unsigned*)P.scratch.p, P.scratch.bytes / 4, 0u, s));
  }
  const size_t apart_bytes = (size_t)L * B * nkv * max_splits * 4 * (d * 16 + 32) * 4;
  if ((st = ensure(c->alloc, P.apart, apart_bytes))) return st;
  size_t soff = 0;
  const size_t o_keys = al(soff, 16 * 8);
  const size_t o_acnt = al(soff, (size_t)L * B * nkv * 4);
  const size_t o_dcnt = al(soff, (size_t)L * T_h * 4);
  const size_t o_lm = al(soff, 4);
  const size_t o_err = al(soff, 4);
  const size_t o_flags = al(soff, (size_t)nwg * 4);
  const size_t o_zero = al(soff, BLOCK_BYTES);
  if (P.sync.bytes < soff || !P.sync.p) {
    if ((st = ensure(c->alloc, P.sync, soff))) return st;
    HIP_TRY(launch_fill_u32((unsigned*)P.sync.p, P.sync.bytes / 4, 0u, s));
    P.epoch = 0;
  }
  P.off_err = o_err;
  uint8_t* sb = (uint8_t*)P.scratch.p;
  uint8_t* yb = (uint8_t*)P.sync.p;
  PArgs a{};
  a.layers = m->players;
  a.lm = m->lm;
  a.embed = (const bf16_t*)m->embed;
  a.final_gain = m->final_gain();
  a.inv_freq = m->inv_freq;
  a.seqs = c->seq_dev;
  a.ids = ids;
  a.draft = draft;
  a.logits = logits;
  a.hidden = hidden;
  a.B = B;
  a.K = K;
  a.M = B * K;
  a.H = H;
  a.nq = nq;
  a.nkv = nkv;
  a.d = d;
  a.I = cf.intermediate;
  a.V = cf.vocab;
  a.L = L;
  a.Kpad = Kpad;
  a.nkb_i = nkb_i;
  a.eps = (float)cf.rms_eps;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
  a.chunk = chunk;
  a.max_splits = max_splits;
  a.down_splits = S;
  a.xs = (float*)sb;
  a.xg = (u32x4*)(sb + o_xg);
  a.ssq = (float*)(sb + o_ssq);
  a.q = (f16_t*)(sb + o_q);
  a.bk = (f16_t*)(sb + o_bk);
  a.bvt = (f16_t*)(sb + o_bvt);
  a.apart = (float*)P.apart.p;
  a.of = (u32x4*)(sb + o_of);
  a.act = (u32x4*)(sb + o_act);
  a.dpart = (float*)(sb + o_dp);
  a.keys = (unsigned long long*)(yb + o_keys);
  a.acnt = (unsigned*)(yb + o_acnt);
  a.dcnt = (unsigned*)(yb + o_dcnt);
  a.lmcnt = (unsigned*)(yb + o_lm);
  a.err = (unsigned*)(yb + o_err);
  a.flags = (unsigned*)(yb + o_flags);
  a.zero_frag = yb + o_zero;
  a.base = P.epoch * persist_steps(L);
  if (c->prof.mask >> PH_PERSIST & 1u) {
    // timeline of this launch (profiling only)
    const int stride = 8 * ((int)persist_steps(L) + 1);
    if ((st = ensure(c->alloc, P.trace, (size_t)nwg * stride * 8))) return st;
    HIP_TRY(launch_fill_u32((unsigned*)P.trace.p, (size_t)nwg * stride * 2, 0u, s));
    a.trace = (unsigned long long*)P.trace.p;
    a.trace_stride = stride;
    P.trace_nwg = nwg;
    P.trace_stride = stride;
  }
  {
    PhaseTimer tm(c, PH_PERSIST, s);
    const hipError_t e = launch_persist_draft(a, nwg, s);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(DFLASH_E_HIP, "persistent draft launch failed: %s", hipGetErrorString(e));
    }
  }
  P.epoch += 1;
  P.K = K;
  P.max_splits = max_splits;
  return DFLASH_OK;
}

// Context rows of a fused step: projected features in the QKV activation
// matrix from m-tile mt0 on, row map in the context's row-map buffer.
struct FusedCtx {
  int n_ctx = 0;
  int mt0 = 0;
  Frag x{};
  bool embedded = false;   // the block rows were embedded with the context rows' finalize
};

// Block verification by a target model: the same layer sequence, causal,
// the block rows' K/V written to the cache, tapped hidden states copied out.
struct VerifyOpts {
  bool on = false;
  void* taps = nullptr;   // [M][n_taps*H] model type, or null
};

template <typename T>
static dflash_status draft_impl(dflash_ctx* c, const int32_t* ids, int K, int32_t* draft, float* logits,
                                void* hidden, hipStream_t s, const FusedCtx& fused = FusedCtx{},
                                const VerifyOpts& vo = VerifyOpts{}) {
  using CT = typename CacheOf<T>::type;
  if (!vo.on && fused.n_ctx == 0 && persist_ok(c, K)) return persist_draft(c, ids, K, draft, logits, hidden, s);
  const dflash_model* m = c->m;
  const dflash_config& cf = m->cfg;
  const int B = c->B, M = B * K, H = cf.hidden, L = cf.n_layers, d = cf.head_dim;
  const int nq = cf.n_q_heads, nkv = cf.n_kv_heads, I = cf.intermediate;
  const int Kpad = round_up(K, 64), G = H / 64, mtiles = (M + 15) / 16;
  const int ces = m->ces;
  const bool pair = sizeof(T) == 2;
  dflash_status st;
  Frag xg, of, af;
  if ((st = ensure(c->alloc, c->x, (size_t)M * H * 4)) || (st = ensure(c->alloc, c->ssq, (size_t)(H / 16) * M * 4)) ||
      (st = ensure(c->alloc, c->q, (size_t)M * nq * d * ces)) ||
      (st = ensure(c->alloc, c->bk, (size_t)B * nkv * Kpad * d * ces)) ||
      (st = ensure(c->alloc, c->bvt, (size_t)B * nkv * Kpad * d * ces)) ||
      (st = ensure(c->alloc, c->keys, (size_t)M * 8)) ||
      (st = ensure_frag(c, c->xg_hi, c->xg_lo, pair, mtiles, H * m->es / 64, s, xg)) ||
      (st = ensure_frag(c, c->o_hi, c->o_lo, pair, mtiles, nq * d * m->es / 64, s, of)) ||
      (st = ensure_frag(c, c->act_hi, c->act_lo, pair, mtiles, (I * m->es + 63) / 64, s, af)))
    return st;
  // attention plan from the host mirror of the context lengths
  const int rep = nq / nkv;
  const int qtiles = (K * rep + 15) / 16;
  const int qgroups = (qtiles + 3) / 4;
  int max_len = 0;
  for (int b = 0; b < B; ++b) max_len = c->seq[b].ctx_len > max_len ? c->seq[b].ctx_len : max_len;
  // Keys per split: the smallest multiple of 64, at least the minimum (128),
  // whose workgroups fit one round of the chip (two 4-wave workgroups or one
  // 8-wave workgroup per CU); at short contexts the split count, not the
  // split length, sets the cost of the combine.
  // Rounds (measured): one-group workgroups (4 waves, two per CU) take
  // attn_wgs_per_cu rounds; workgroups of two or four query groups carry
  // enough work per chunk that one round of longer splits beats two of short
  // ones, except a non-causal block of more than 256 rows, whose own keys
  // form splits too long to sit beside one-round context splits.
  const int qg_per_wg = attn_groups_per_wg(ces, qgroups);
  const int64_t wg_per_split = (int64_t)nkv * ((qgroups + qg_per_wg - 1) / qg_per_wg);
  const int rounds = qg_per_wg == 1 || (!vo.on && K > 256) ? c->attn_wgs_per_cu : (c->attn_wgs_per_cu + 1) / 2;
  const int64_t round_wgs = (qg_per_wg == 1 ? 2 : 1) * (int64_t)rounds * 256;
  auto splits = [&](int len, int ch) {
    return vo.on ? (len + K + ch - 1) / ch : (len + ch - 1) / ch + (K + ch - 1) / ch;
  };
  int chunk = c->attn_min_split;
  for (;; chunk += 64) {
    int64_t wgs = 0;
    for (int b = 0; b < B; ++b) wgs += wg_per_split * splits(c->seq[b].ctx_len, chunk);
    if (wgs <= round_wgs || chunk >= max_len + K) break;
  }
  const int max_splits = splits(max_len, chunk);
  if ((st = ensure(c->alloc, c->attn_part, attn_part_floats(B, nkv, qgroups, max_splits, d, attn_part_o_bytes(ces, qgroups, d)) * sizeof(float))))
    return st;

  if (!fused.embedded) {
    PhaseTimer tm(c, PH_EMBED, s);
    HIP_TRY(launch_embed<T>(ids, m->embed, L > 0 ? m->attn_gain(0) : m->final_gain(), M, H, cf.vocab,
                            (float*)c->x.p, xg, (float*)c->ssq.p, (unsigned long long*)c->keys.p, s));
  }
  EpiArgs e = base_epi(c, M);
  e.Kblk = K;
  e.Kpad = Kpad;
  e.ssq = (const float*)c->ssq.p;
  e.ssq_groups = G;
  e.norm_dim = H;
  e.q = c->q.p;
  e.bk = c->bk.p;
  e.bvt = c->bvt.p;
  e.act = af;
  e.logits = logits;
  e.keys = (unsigned long long*)c->keys.p;

  AttnArgs a{};
  a.q = c->q.p;
  a.bk = c->bk.p;
  a.bvt = c->bvt.p;
  a.seqs = c->seq_dev;
  a.part = (float*)c->attn_part.p;
  a.B = B;
  a.K = K;
  a.Kpad = Kpad;
  a.nq = nq;
  a.nkv = nkv;
  a.d = d;
  a.qgroups = qgroups;
  a.chunk = chunk;
  a.max_splits = max_splits;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
  a.causal = vo.on ? 1 : 0;
  // Context K/V read per block (all layers): the default load policy lets a
  // small one stay in the caches from one block to the next (the weights
  // stream nontemporally, so they do not evict it; measured at batch 1,
  // ctx 2048: 42 MB); beyond attn_stream_mb (128 MiB) nothing stays, and
  // nontemporal loads stream it faster (batch 16, 3.5 GB per block: -12 %).
  {
    double kv = 0.0;
    for (int b = 0; b < B; ++b) kv += (double)(c->seq[b].ctx_len + (vo.on ? K : 0));
    kv *= (double)nkv * d * 2.0 * ces * L;
    a.stream = kv > (double)c->attn_stream_mb * (1 << 20) ? 1 : 0;
  }

  const Frag none{};
  for (int l = 0; l < L; ++l) {
    if (fused.n_ctx > 0) {
      // block rows and the appended context rows in one product: the
      // context rows' K/V land in layer l's caches before its attention
      EpiArgs ef = e;
      ef.ctx_mt0 = fused.mt0;
      ef.n_ctx = fused.n_ctx;
      ef.layer = l;
      ef.rowmap = (const RowMap*)c->rowmap.p;
      if ((st = run_gemm<T>(c, PH_QKV, EPI_QKV, m->qkv[l], fused.x, nullptr, 0, fused.mt0 * 16 + fused.n_ctx, ef,
                            s, nullptr, true)))
        return st;
    } else if (vo.on) {
      EpiArgs ev = e;   // the block rows' K/V go to layer l of the cache
      ev.kv_cache = 1;
      ev.layer = l;
      if ((st = run_gemm<T>(c, PH_QKV, EPI_QKV, m->qkv[l], xg, nullptr, 0, M, ev, s))) return st;
    } else if ((st = run_gemm<T>(c, PH_QKV, EPI_QKV, m->qkv[l], xg, nullptr, 0, M, e, s))) {
      return st;
    }
    a.layer = l;
    // the attention kernel's spare blocks warm the output projection's weights
    a.warm = make_warm<T>(mtiles == 1 ? EPI_RESNORM : mtiles <= 4 ? EPI_PARTRES : EPI_PART, m->o[l], M, c->warm_o);
    {
      PhaseTimer tm(c, PH_ATTN, s);
      HIP_TRY(launch_attention<CT>(a, s));
    }
    {
      PhaseTimer tm(c, PH_COMBINE, s);
      HIP_TRY((launch_attn_combine<CT, T>(a, of, s)));
    }
    // The output projection and the down projection add into the residual
    // and write the next norm's inputs (x * gain in frag layout, sums of
    // squares): for one m-tile the output projection runs over the whole
    // reduction with that epilogue (EPI_RESNORM); the split products of up
    // to four m-tiles end with their last split adding the partials
    // (EPI_PARTRES, sums of squares per 16 columns); with more rows a tile
    // group's partials are too many for one workgroup, and a residual pass
    // over the whole grid adds them (sums of squares per 64 columns).
    // Measured on the Qwen3-4B shape: down at K = 16 11.6 + 4.8 -> 15.1 us
    // per layer with EPI_PARTRES; at K = 128 (eight m-tiles) EPI_PARTRES
    // was 0.10 ms per block slower than the residual pass.
    const bool fix = mtiles <= 4;
    EpiArgs eo = e;
    eo.xres = (float*)c->x.p;
    eo.gain = m->mlp_gain(l);
    eo.xout = xg;
    eo.ssq_out = (float*)c->ssq.p;
    EpiArgs eg = e;
    GemmPlan p;
    if (mtiles == 1 || fix) {
      if ((st = run_gemm<T>(c, PH_O, mtiles == 1 ? EPI_RESNORM : EPI_PARTRES, m->o[l], of, nullptr, 0, M, eo, s)))
        return st;
      eg.ssq_groups = H / 16;
    } else {
      if ((st = run_gemm<T>(c, PH_O, EPI_PART, m->o[l], of, nullptr, 0, M, e, s, &p))) return st;
      PhaseTimer tm(c, PH_RESID, s);
      HIP_TRY(launch_resid_norm<T>((const float*)c->part.p, p.nsplit, mtiles, M, H, (float*)c->x.p,
                                   m->mlp_gain(l), xg, (float*)c->ssq.p, s));
      eg.ssq_groups = G;
    }
    if ((st = run_gemm<T>(c, PH_GU, EPI_SWIGLU, m->gu[l], xg, nullptr, 0, M, eg, s))) return st;
    EpiArgs ed = eo;
    ed.gain = l + 1 < L ? m->attn_gain(l + 1) : m->final_gain();
    if (fix) {
      if ((st = run_gemm<T>(c, PH_DOWN, EPI_PARTRES, m->down[l], af, nullptr, 0, M, ed, s))) return st;
      e.ssq_groups = H / 16;   // the next layer's QKV, the LM head and the final norm
    } else {
      if ((st = run_gemm<T>(c, PH_DOWN, EPI_PART, m->down[l], af, nullptr, 0, M, e, s, &p))) return st;
      PhaseTimer tm(c, PH_RESID, s);
      HIP_TRY(launch_resid_norm<T>((const float*)c->part.p, p.nsplit, mtiles, M, H, (float*)c->x.p, ed.gain, xg,
                                   (float*)c->ssq.p, s));
      e.ssq_groups = G;
    }
    if (vo.on && vo.taps) {
      const int nt = (int)m->taps.size();
      for (int ti = 0; ti < nt; ++ti)
        if (m->taps[ti] == l) HIP_TRY(launch_tap<T>((const float*)c->x.p, M, H, ti, nt, vo.taps, s));
    }
  }
  (void)none;
  if ((st = run_gemm<T>(c, PH_LM, EPI_ARGMAX, m->lm, xg, nullptr, 0, M, e, s))) return st;
  {
    PhaseTimer tm(c, PH_FINAL, s);
    HIP_TRY(launch_finalize<T>((const unsigned long long*)c->keys.p, M, draft, (const float*)c->x.p,
                               (const float*)c->ssq.p, e.ssq_groups, m->final_gain(), H, (float)cf.rms_eps, hidden, s));
  }
  return DFLASH_OK;
}

// NEXT step in one call: project and append the accepted positions, then
// draft the next block with their K/V injected by each layer's QKV product
// (whose W_k / W_v stream anyway), so no separate injection product runs.
// Appends too large for one activation matrix take the two-call path.
template <typename T>
static dflash_status step_impl(dflash_ctx* c, const void* feats, const int32_t* n_new, const int32_t* ids, int K,
                               int32_t* draft, float* logits, void* hidden, hipStream_t s) {
  const dflash_model* m = c->m;
  const int B = c->B, H = m->cfg.hidden;
  const RowInfo ri0 = row_info(c, n_new);
  const int total = ri0.start[B];
  const int mtb = (B * K + 15) / 16, mtc = (total + 15) / 16;
  dflash_status st;
  if (total == 0) return draft_impl<T>(c, ids, K, draft, logits, hidden, s);
  if (m->cfg.n_layers == 0 || mtb + mtc > 4 || persist_ok(c, K)) {
    if ((st = project_impl<T>(c, feats, n_new, nullptr, s))) return st;
    return draft_impl<T>(c, ids, K, draft, logits, hidden, s);
  }
  if ((st = grow_for<T>(c, n_new, s))) return st;
  const RowInfo ri = row_info(c, n_new);
  FusedCtx fused;
  fused.n_ctx = total;
  fused.mt0 = mtb;
  // the activation matrix spans whole m-tile groups of the QKV product, so
  // that every load batch is a full one (rows past the data are never stored)
  const int mt_all = mtb + mtc <= 2 ? mtb + mtc : 4;
  if ((st = ensure(c->alloc, c->rowmap, sizeof(RowMap) * total)) ||
      (st = ensure_frag(c, c->xg_hi, c->xg_lo, sizeof(T) == 2, mt_all, H * m->es / 64, s, fused.x)))
    return st;
  // the block rows' residual, norm sums and argmax keys, sized as
  // draft_impl sizes them (which then finds them in place)
  const int Mb = B * K;
  if ((st = ensure(c->alloc, c->x, (size_t)Mb * H * 4)) || (st = ensure(c->alloc, c->ssq, (size_t)(H / 16) * Mb * 4)) ||
      (st = ensure(c->alloc, c->keys, (size_t)Mb * 8)))
    return st;
  EpiArgs e = base_epi(c, total);
  const Frag none{};
  GemmPlan p;
  if ((st = run_gemm<T>(c, PH_FC, EPI_PART, m->fc, none, feats, m->cfg.n_feat * H, total, e, s, &p))) return st;
  {
    // the context rows' finalize and the block rows' embedding, one launch
    PhaseTimer tm(c, PH_FCFIN, s);
    HIP_TRY(launch_fc_finalize_embed<T>((const float*)c->part.p, p.nsplit, mtc, total, H, ri, B,
                                        (RowMap*)c->rowmap.p, c->seq_dev, fused.x, mtb * 16, ids, m->embed,
                                        m->attn_gain(0), Mb, m->cfg.vocab, (float*)c->x.p, fused.x,
                                        (float*)c->ssq.p, (unsigned long long*)c->keys.p, s));
  }
  fused.embedded = true;
  for (int b = 0; b < B; ++b) c->seq[b].ctx_len += n_new[b];
  return draft_impl<T>(c, ids, K, draft, logits, hidden, s, fused);
}

extern "C" {

dflash_status dflash_step(dflash_ctx* c, const void* feats, const int32_t* n_new, const int32_t* block_ids,
                          int32_t K, int32_t* draft_ids, float* logits, void* hidden, void* stream) {
  if (!c) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (c->m->target) return fail(DFLASH_E_STATE, "a target context verifies blocks (dflash_verify_block)");
  if (!n_new) return fail(DFLASH_E_ARG, "n_new is NULL");
  if (!block_ids || !draft_ids) return fail(DFLASH_E_ARG, "block_ids / draft_ids is NULL");
  if (K < 1 || K > DFLASH_MAX_K) return fail(DFLASH_E_ARG, "K = %d out of [1, %d]", K, DFLASH_MAX_K);
  int64_t total = 0;
  for (int b = 0; b < c->B; ++b) {
    if (n_new[b] < 0) return fail(DFLASH_E_ARG, "n_new[%d] = %d is negative", b, n_new[b]);
    if ((int64_t)c->seq[b].ctx_len + n_new[b] > (1 << 30))
      return fail(DFLASH_E_SHAPE, "sequence %d would exceed 2^30 positions", b);
    total += n_new[b];
  }
  if (total > (1 << 30)) return fail(DFLASH_E_SHAPE, "too many rows in one call");
  if (total > 0 && !feats) return fail(DFLASH_E_ARG, "feats is NULL");
  hipStream_t s = (hipStream_t)stream;
  return c->m->cfg.dtype == DFLASH_BF16
             ? step_impl<bf16_t>(c, feats, n_new, block_ids, K, draft_ids, logits, hidden, s)
             : step_impl<float>(c, feats, n_new, block_ids, K, draft_ids, logits, hidden, s);
}

dflash_status dflash_draft_block(dflash_ctx* c, const int32_t* block_ids, int32_t K, int32_t* draft_ids,
                                 float* logits, void* hidden, void* stream) {
  if (!c) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (c->m->target) return fail(DFLASH_E_STATE, "a target context verifies blocks (dflash_verify_block)");
  if (!block_ids || !draft_ids) return fail(DFLASH_E_ARG, "block_ids / draft_ids is NULL");
  if (K < 1 || K > DFLASH_MAX_K) return fail(DFLASH_E_ARG, "K = %d out of [1, %d]", K, DFLASH_MAX_K);
  hipStream_t s = (hipStream_t)stream;
  return c->m->cfg.dtype == DFLASH_BF16 ? draft_impl<bf16_t>(c, block_ids, K, draft_ids, logits, hidden, s)
                                        : draft_impl<float>(c, block_ids, K, draft_ids, logits, hidden, s);
}

dflash_status dflash_verify_block(dflash_ctx* c, const int32_t* block_ids, int32_t K1, int32_t* target_ids,
                                  float* logits, void* taps, void* stream) {
  if (!c) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!c->m->target) return fail(DFLASH_E_STATE, "not a target context (dflash_target_create)");
  if (!block_ids || !target_ids) return fail(DFLASH_E_ARG, "block_ids / target_ids is NULL");
  if (K1 < 1 || K1 > DFLASH_MAX_K) return fail(DFLASH_E_ARG, "K1 = %d out of [1, %d]", K1, DFLASH_MAX_K);
  if (taps && c->m->taps.empty()) return fail(DFLASH_E_ARG, "taps requested from a model without tapped layers");
  std::vector<int32_t> n(c->B, K1);
  for (int b = 0; b < c->B; ++b)
    if ((int64_t)c->seq[b].ctx_len + K1 > (1 << 30))
      return fail(DFLASH_E_SHAPE, "sequence %d would exceed 2^30 positions", b);
  hipStream_t s = (hipStream_t)stream;
  VerifyOpts vo;
  vo.on = true;
  vo.taps = taps;
  dflash_status st;
  // room for the block's K/V at slots ctx_len .. ctx_len + K1 - 1
  if (c->m->cfg.dtype == DFLASH_BF16) {
    if ((st = grow_for<bf16_t>(c, n.data(), s))) return st;
    st = draft_impl<bf16_t>(c, block_ids, K1, target_ids, logits, nullptr, s, FusedCtx{}, vo);
  } else {
    if ((st = grow_for<float>(c, n.data(), s))) return st;
    st = draft_impl<float>(c, block_ids, K1, target_ids, logits, nullptr, s, FusedCtx{}, vo);
  }
  c->verified = st == DFLASH_OK ? K1 : 0;
  return st;
}

dflash_status dflash_commit(dflash_ctx* c, const int32_t* n_acc, void* stream) {
  if (!c) return fail(DFLASH_E_ARG, "ctx is NULL");
  if (!c->m->target) return fail(DFLASH_E_STATE, "not a target context (dflash_target_create)");
  if (!n_acc) return fail(DFLASH_E_ARG, "n_acc is NULL");
  for (int b = 0; b < c->B; ++b)
    if (n_acc[b] < 0 || n_acc[b] > c->verified)
      return fail(DFLASH_E_STATE, "n_acc[%d] = %d: the last verified block has %d rows", b, n_acc[b], c->verified);
  hipStream_t s = (hipStream_t)stream;
  for (int b = 0; b < c->B; ++b) {
    if (n_acc[b] == 0) continue;
    c->seq[b].ctx_len += n_acc[b];
    HIP_TRY(launch_set_seq(c->seq_dev, b, c->seq[b], s));
  }
  c->verified = 0;
  return DFLASH_OK;
}

dflash_status dflash_ctx_set_persistent(dflash_ctx* c, int32_t enable) {
  if (!c) return fail(DFLASH_E_ARG, "ctx is NULL");
  c->pst.enabled = enable != 0;
  return DFLASH_OK;
}

dflash_status dflash_ctx_persistent_path(dflash_ctx* c, int32_t K, int32_t* yes) {
  if (!c || !yes) return fail(DFLASH_E_ARG, "NULL pointer");
  if (K < 1 || K > DFLASH_MAX_K) return fail(DFLASH_E_ARG, "K = %d out of [1, %d]", K, DFLASH_MAX_K);
  *yes = persist_ok(c, K) ? 1 : 0;
  return DFLASH_OK;
}

dflash_status dflash_ctx_check(dflash_ctx* c, void* stream) {
  if (!c) return fail(DFLASH_E_ARG, "ctx is NULL");
  auto& P = c->pst;
  if (!P.sync.p) return DFLASH_OK;
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
  unsigned err = 0;
  HIP_TRY(hipMemcpy(&err, (uint8_t*)P.sync.p + P.off_err, 4, hipMemcpyDeviceToHost));
  if (err) {
    HIP_TRY(hipMemset(P.sync.p, 0, P.sync.bytes));
    HIP_TRY(hipDeviceSynchronize());
    P.epoch = 0;
    return fail(DFLASH_E_HIP, "persistent draft kernel: a barrier wait expired; outputs since the last check are invalid");
  }
  return DFLASH_OK;
}

dflash_status dflash_persist_trace(dflash_ctx* c, uint64_t* out, int64_t capacity, int32_t* nwg, int32_t* stride) {
  if (!c || !nwg || !stride) return fail(DFLASH_E_ARG, "NULL pointer");
  auto& P = c->pst;
  *nwg = P.trace.p ? P.trace_nwg : 0;
  *stride = P.trace.p ? P.trace_stride : 0;
  const int64_t n = (int64_t)*nwg * *stride;
  if (n == 0 || !out) return DFLASH_OK;   // size query
  if (capacity < n) return fail(DFLASH_E_ARG, "capacity %lld < %lld", (long long)capacity, (long long)n);
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(out, P.trace.p, (size_t)n * 8, hipMemcpyDeviceToHost));
  return DFLASH_OK;
}

dflash_status dflash_profile_enable(dflash_ctx* c, uint32_t phase_mask) {
  if (!c) return fail(DFLASH_E_ARG, "ctx is NULL");
  c->prof.mask = phase_mask & ((1u << DFLASH_NUM_PHASES) - 1u);
  return DFLASH_OK;
}

dflash_status dflash_profile_read(dflash_ctx* c, double* ms, int64_t* count) {
  if (!c || !ms || !count) return fail(DFLASH_E_ARG, "NULL pointer");
  for (int i = 0; i < DFLASH_NUM_PHASES; ++i) {
    ms[i] = 0.0;
    count[i] = 0;
  }
  Profiler& p = c->prof;
  if (!p.recs.empty()) HIP_TRY(hipEventSynchronize(p.pool[p.recs.back().second + 1]));
  for (auto& r : p.recs) {
    float t = 0.f;
    HIP_TRY(hipEventElapsedTime(&t, p.pool[r.second], p.pool[r.second + 1]));
    ms[r.first] += t;
    count[r.first] += 1;
  }
  p.recs.clear();
  p.used = 0;
  return DFLASH_OK;
}

const char* dflash_phase_name(int32_t phase) {
  if (phase < 0 || phase >= DFLASH_NUM_PHASES) return "";
  return kPhaseNames[phase];
}

dflash_status dflash_accept(const int32_t* draft_ids, const int32_t* target_ids, int32_t batch, int32_t K,
                            int32_t* accept_len, void* stream) {
  if (!draft_ids || !target_ids || !accept_len) return fail(DFLASH_E_ARG, "NULL pointer");
  if (batch < 1 || batch > (1 << 20)) return fail(DFLASH_E_ARG, "batch = %d out of range", batch);
  if (K < 1 || K > DFLASH_MAX_K) return fail(DFLASH_E_ARG, "K = %d out of [1, %d]", K, DFLASH_MAX_K);
  HIP_TRY(launch_accept(draft_ids, target_ids, batch, K, accept_len, (hipStream_t)stream));
  return DFLASH_OK;
}

dflash_status dflash_decay_ce(const void* logits, dflash_dtype dtype, const int32_t* targets, int32_t rows,
                              int32_t vocab, int32_t block, double gamma, float* loss, float* ce, void* grad,
                              void* workspace, void* stream) {
  if (!loss || !workspace) return fail(DFLASH_E_ARG, "NULL pointer");
  if (rows > 0 && (!logits || !targets || !ce)) return fail(DFLASH_E_ARG, "NULL pointer");
  if ((uintptr_t)workspace % 8) return fail(DFLASH_E_ARG, "workspace not 8-byte aligned");
  const int32_t dt = abi_int(dtype);
  if (dt != DFLASH_F32 && dt != DFLASH_BF16) return fail(DFLASH_E_ARG, "dtype = %d", dt);
  if (rows < 0) return fail(DFLASH_E_ARG, "rows = %d", rows);
  if (vocab < 1) return fail(DFLASH_E_ARG, "vocab = %d", vocab);
  if (block < 1) return fail(DFLASH_E_ARG, "block = %d", block);
  if (!(gamma > 0.0) || !std::isfinite(gamma)) return fail(DFLASH_E_ARG, "gamma = %g", gamma);
  HIP_TRY(launch_decay_ce(logits, dt, targets, rows, vocab, block, gamma, loss, ce, rows > 0 ? grad : nullptr,
                          (double*)workspace, (hipStream_t)stream));
  return DFLASH_OK;
}

}  // extern "C"
