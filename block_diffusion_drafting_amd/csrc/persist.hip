// Persistent single-launch draft block for small blocks (batch * K <= 16
// rows) of bf16 drafters on gfx950.
//
// The draft forward (kongchang.com "D-Flash", "System architecture" and
// "Innovation 1"; Google Developers Blog, "Dual cache for attention") is a
// chain of weight-streaming products in which every output row of one
// product needs every column of the one before.  Run as one kernel per
// product, each pays launch, ramp-up and drain, and HBM idles across the
// gaps and across the small kernels in between.  Here one cooperative
// launch of one eight-wave workgroup per compute unit runs the whole block:
//
//   embed | per layer: QKV + RoPE | attention over [context || block], the
//   last split of a head merging the head's splits | O + residual + norm
//   inputs | gate/up + SwiGLU | down split over k, the last split of a tile
//   adding the splits into the residual | LM head + argmax, the last
//   workgroup writing the draft ids
//
// with a flag barrier between phases.  Weights do not depend on
// activations, so at every barrier the waiting workgroup issues
// direct-to-LDS loads of the first fragments of its next product's weights
// (the data is discarded): they land in its XCD's L2, HBM keeps streaming
// through the barrier, and the product then starts from L2.
//
// Memory visibility across XCDs (each XCD has its own L2): every buffer
// that one workgroup writes and another reads within the launch is written
// with device-scope (write-through) stores, at most once per launch and at
// an address of its own (one copy per layer and phase), so no XCD can hold
// a stale line of it; a workgroup's stores complete (s_waitcnt) before its
// flag or counter update, and readers load only after observing it.
// Nothing here uses a memory fence: on this GPU an agent-scope release
// writes back and invalidates the whole L2, which would also drop the
// prefetched weights.
//
// Every wait is bounded (about 2 s of the constant 100 MHz clock); a wait
// that expires sets the error word and every workgroup leaves the kernel.
#include "kernels.h"

namespace dflash {

namespace {

constexpr int PW = 8;        // waves per workgroup
constexpr int PT = PW * 64;  // threads per workgroup
constexpr unsigned long long kTimeoutTicks = 200000000ull;

// Workgroup barrier for LDS data only: the compiler fence keeps memory
// operations on their side, lgkmcnt(0) completes this wave's LDS accesses.
// (__syncthreads would also wait for the outstanding weight prefetches.)
__device__ __forceinline__ void lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Completes every memory operation this wave has issued.
__device__ __forceinline__ void drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// device-scope (write-through) stores
__device__ __forceinline__ void wt16(void* p, uint16_t v) {
  __hip_atomic_store((uint16_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wt32(void* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wt64(void* p, uint64_t v) {
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wtf(float* p, float v) { wt32(p, __float_as_uint(v)); }
__device__ __forceinline__ void wtf4(void* p, f32x4 v) {
  wt64(p, (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32));
  wt64((uint8_t*)p + 8, (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32));
}
__device__ __forceinline__ uint16_t h16(float v) { return __builtin_bit_cast(uint16_t, f2h(v)); }

// N (2 or 4) consecutive values of row m from column k into a bf16 hi/lo
// frag matrix (one m-tile), write-through.
template <int N>
__device__ __forceinline__ void frag_store_wt(const Frag& f, int m, int k, const float* v) {
  int e;
  const size_t slot = frag_slot<bf16_t>(f, m, k, e);
  uint64_t hw = 0, lw = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bf16_t h = f2bf(v[i]);
    const bf16_t l = f2bf(v[i] - bf2f(h));
    hw |= (uint64_t)h << (16 * i);
    lw |= (uint64_t)l << (16 * i);
  }
  bf16_t* ph = (bf16_t*)(f.hi + slot) + e;
  bf16_t* pl = (bf16_t*)(f.lo + slot) + e;
  if constexpr (N == 4) {
    wt64(ph, hw);
    wt64(pl, lw);
  } else {
    wt32(ph, (uint32_t)hw);
    wt32(pl, (uint32_t)lw);
  }
}

__device__ __forceinline__ float silu_f(float t) { return t / (1.0f + expf(-t)); }

__device__ __forceinline__ void rope2(float x1, float x2, int pos, double inv, float& o1, float& o2) {
  double sn, cs;
  sincos((double)pos * inv, &sn, &cs);
  const float c = (float)cs, s = (float)sn;
  o1 = x1 * c - x2 * s;
  o2 = x2 * c + x1 * s;
}

// ---------------------------------------------------------------------------
// shared memory
// ---------------------------------------------------------------------------
constexpr int KROW128 = 128 * 2 + 16;   // padded K row (bytes), head_dim 128, fp16
constexpr int VROW = 64 * 2 + 16;       // padded V^T row (bytes), 64-key chunk

struct PShared {
  union {
    struct {
      uint8_t kl[2][64 * KROW128];
      uint8_t vl[2][128 * VROW];
    } att;
    f32x4 red[PW][8][64];
  } u;
  float npart[32][16];
  float rn[16];
  unsigned long long kmax[16];
  int bad;
  int last;
};

struct Wave {
  int w;      // workgroup
  int wave;   // wave in the workgroup (scalar)
  int lane;
  int tid;
  unsigned long long* tr;   // timeline slots of the current phase, or null
};
// timeline mark k of the current phase (thread 0 only)
__device__ __forceinline__ void mark(const Wave& wv, int k) {
  if (wv.tr && wv.tid == 0) wv.tr[k] = wall_clock64();
}

// ---------------------------------------------------------------------------
// work assignment (the same functions plan the products and their warm-up)
// ---------------------------------------------------------------------------
struct Work {
  const Packed* W;
  int tile0, nt;    // this workgroup's tiles
  int kbA, kbB;     // its range of k-blocks
};

__device__ __forceinline__ void even_range(int n, int parts, int i, int& a, int& cnt) {
  a = (int)((long)i * n / parts);
  cnt = (int)((long)(i + 1) * n / parts) - a;
}

__device__ __forceinline__ Work work_full(const Packed* W, int w) {
  Work k;
  k.W = W;
  even_range(W->n_tiles, (int)gridDim.x, w, k.tile0, k.nt);
  k.kbA = 0;
  k.kbB = W->nkb;
  return k;
}
// split over k: workgroup w takes split w % S of the tiles of group w / S
__device__ __forceinline__ Work work_split(const Packed* W, int S, int w) {
  Work k;
  k.W = W;
  const int groups = (int)gridDim.x / S;
  const int s = w % S, gi = w / S;
  if (gi >= groups) {
    k.tile0 = 0;
    k.nt = 0;
  } else {
    even_range(W->n_tiles, groups, gi, k.tile0, k.nt);
  }
  int c;
  even_range(W->nkb, S, s, k.kbA, c);
  k.kbB = k.kbA + c;
  return k;
}
// the k-blocks of wave v within [kbA, kbB)
__device__ __forceinline__ void wave_krange(int kbA, int kbB, int v, int& k0, int& k1) {
  const int per = (kbB - kbA + PW - 1) / PW;
  k0 = min(kbB, kbA + v * per);
  k1 = min(kbB, k0 + per);
}
// tiles of pass p of npass over nt tiles
__device__ __forceinline__ void pass_range(int tile0, int nt, int npass, int p, int& t0, int& n) {
  int a;
  even_range(nt, npass, p, a, n);
  t0 = tile0 + a;
}

// Warm-up: direct-to-LDS loads (data discarded into the wave's own slot)
// of the first `nfrag` weight fragments that wave `share` will read in the
// first pass of `k` (batch order: k-block major, then tile).
__device__ __forceinline__ void warm_share(const Work& k, int ntg, int share, int nfrag, int lane,
                                           lds_void_t* slot) {
  if (k.nt <= 0 || nfrag <= 0) return;
  const int npass = (k.nt + ntg - 1) / ntg;
  int t0, nt;
  pass_range(k.tile0, k.nt, npass, 0, t0, nt);
  int k0, k1;
  wave_krange(k.kbA, k.kbB, share, k0, k1);
  const uint8_t* base = k.W->w + (size_t)lane * FRAG_BYTES;
  int cnt = 0;
  for (int kb = k0; kb < k1 && cnt < nfrag; ++kb)
    for (int t = 0; t < nt && cnt < nfrag; ++t, ++cnt)
      __builtin_amdgcn_global_load_lds((const void*)(base + ((size_t)(t0 + t) * k.W->nkb + kb) * BLOCK_BYTES), slot,
                                       16, 0, 0);
}
// The shares of all eight waves are warmed by waves first..7 (round robin):
// wave 0 polls the flags and never warms, and waves that work in the next
// phase should not have loads queued ahead of that work.
__device__ __forceinline__ void warm_work(const Work& k, int ntg, int nfrag, const Wave& wv, lds_void_t* slot,
                                          int first = 1) {
  if (wv.wave < first) return;
  for (int s = wv.wave - first; s < PW; s += PW - first) warm_share(k, ntg, s, nfrag, wv.lane, slot);
}

// ---------------------------------------------------------------------------
// the flag barrier
// ---------------------------------------------------------------------------
// Every workgroup publishes base + step in its flag once its stores are
// complete (`stored`: this wave may have stores outstanding); wave 0 then
// reads all flags until each has reached the step.
// Returns false when the launch is abandoned.
template <class F>
__device__ __forceinline__ bool grid_barrier(const PArgs& a, PShared& sh, unsigned step, const Wave& wv,
                                             F&& warm, bool stored = true) {
  if (stored) drain();
  lds_sync();
  const unsigned target = a.base + step;
  mark(wv, 6);
  if (wv.tid == 0) wt32(a.flags + wv.w, target);
  warm();
  if (wv.wave == 0) {
    const int n = (int)gridDim.x;
    const unsigned long long t0 = wall_clock64();
    int bad = 0;
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = wv.lane * 4 + j;
        if (i < n) {
          const unsigned v = __hip_atomic_load(a.flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = ok && (int)(v - target) >= 0;
        }
      }
      const unsigned err = __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__all(ok)) break;
      if (__builtin_amdgcn_readfirstlane(err) != 0u) {
        bad = 1;
        break;
      }
      if (wall_clock64() - t0 > kTimeoutTicks) {
        if (wv.lane == 0) atomicOr(a.err, 1u);
        bad = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (wv.lane == 0) sh.bad = bad;
    mark(wv, 7);
  }
  lds_sync();
  return sh.bad == 0;
}

// ---------------------------------------------------------------------------
// weight products (one 16-row activation tile, bf16 hi/lo pair)
// ---------------------------------------------------------------------------
// acc[t] = sum over this wave's k-blocks [kw0, kw1) of W tile (tile0 + t)
// times the activation fragments (hi and lo).  nt, kw0, kw1 are uniform.
// A pointer that is the same on every lane, in scalar registers.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (P*)(((uint64_t)hi << 32) | lo);
}

// acc[t] = sum over this wave's k-blocks [kw0, kw1) of W tile (tile0 + t)
// times the activation fragments (hi and lo).  nt, kw0, kw1 are uniform;
// the tile and activation bases are scalar, the lane's 16 bytes an offset.
template <int NTG, int CHK>
__device__ __forceinline__ void gemm_core(const Packed& W, const u32x4* xh_, const u32x4* xl_, int tile0, int nt,
                                          int kw0, int kw1, int lane, f32x4 (&acc)[NTG]) {
  using E = Elem<bf16_t>;
  const uint8_t* w0 = uniform_ptr(W.w);
  const int nkb = __builtin_amdgcn_readfirstlane(W.nkb);
  const uint8_t* xh = (const uint8_t*)uniform_ptr(xh_);
  const uint8_t* xl = (const uint8_t*)uniform_ptr(xl_);
  const uint32_t lo = (uint32_t)lane * FRAG_BYTES;
  const uint8_t* wt[NTG];
#pragma unroll
  for (int t = 0; t < NTG; ++t) wt[t] = w0 + (size_t)(tile0 + min(t, nt - 1)) * nkb * BLOCK_BYTES;
#pragma unroll
  for (int t = 0; t < NTG; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  struct Batch {
    u32x4 wf[NTG][CHK];
    u32x4 xh[CHK], xl[CHK];
  };
  auto wload = [&](int t, int kb) {
    return __builtin_nontemporal_load((const u32x4*)(wt[t] + (size_t)kb * BLOCK_BYTES + lo));
  };
  auto xload = [&](const uint8_t* x, int kb) { return *(const u32x4*)(x + (size_t)kb * BLOCK_BYTES + lo); };
  auto load_full = [&](Batch& b, int kb) {
#pragma unroll
    for (int j = 0; j < CHK; ++j)
#pragma unroll
      for (int t = 0; t < NTG; ++t) b.wf[t][j] = wload(t, kb + j);
#pragma unroll
    for (int j = 0; j < CHK; ++j) {
      b.xh[j] = xload(xh, kb + j);
      b.xl[j] = xload(xl, kb + j);
    }
  };
  auto load_part = [&](Batch& b, int kb) {
#pragma unroll
    for (int j = 0; j < CHK; ++j) {
      const bool ok = kb + j < kw1;
#pragma unroll
      for (int t = 0; t < NTG; ++t) b.wf[t][j] = (ok && t < nt) ? wload(t, kb + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < CHK; ++j) {
      const bool ok = kb + j < kw1;
      b.xh[j] = ok ? xload(xh, kb + j) : u32x4{0u, 0u, 0u, 0u};
      b.xl[j] = ok ? xload(xl, kb + j) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto compute = [&](const Batch& b) {
#pragma unroll
    for (int j = 0; j < CHK; ++j)
#pragma unroll
      for (int t = 0; t < NTG; ++t) {
        if (t >= nt) continue;
        acc[t] = E::mma(b.wf[t][j], b.xh[j], acc[t]);
        acc[t] = E::mma(b.wf[t][j], b.xl[j], acc[t]);
      }
  };
  const int nfull = nt == NTG ? (kw1 - kw0) / CHK : 0;
  int kb = kw0;
  for (int i = 0; i < nfull; ++i, kb += CHK) {
    Batch b;
    load_full(b, kb);
    compute(b);
  }
  for (; kb < kw1; kb += CHK) {
    Batch b;
    load_part(b, kb);
    compute(b);
  }
}

// RMSNorm row scales, rn[m] = rsqrt(sum_g ssq[g][m] / H + eps) over the
// per-16-column sums of squares ssq[g][16] (g < H/16): thread t loads rows
// t % 16 of groups t / 16 + 32 j before the product's weights stream (the
// values are only needed by the epilogue), adds them after, and the 32
// partial sums of a row are added in order through LDS.
constexpr int NORM_MAX = 8;    // groups per thread: H <= 4096
struct NormLoad {
  float v[NORM_MAX];
};
__device__ __forceinline__ void norm_issue(const PArgs& a, const float* ssq, const Wave& wv, NormLoad& nl) {
  const int r = wv.tid & 15, part = wv.tid >> 4;
  const int groups = a.H / 16;
#pragma unroll
  for (int j = 0; j < NORM_MAX; ++j) {
    const int g = part + 32 * j;
    nl.v[j] = (g < groups && r < a.M) ? ssq[g * 16 + r] : 0.f;
  }
}
__device__ __forceinline__ void norm_part(PShared& sh, const NormLoad& nl, const Wave& wv) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NORM_MAX; ++j) s += nl.v[j];
  sh.npart[wv.tid >> 4][wv.tid & 15] = s;
}
// after an lds_sync that follows norm_part in every thread
__device__ __forceinline__ void norm_finish(const PArgs& a, PShared& sh, const Wave& wv) {
  if (wv.tid < 16) {
    float t = 0.f;
#pragma unroll
    for (int p = 0; p < 32; ++p) t += sh.npart[p][wv.tid];
    sh.rn[wv.tid] = wv.tid < a.M ? rsqrtf(t / (float)a.H + a.eps) : 0.f;
  }
}

// The waves' sums of each tile added in wave order through LDS, then
// epi(i, sum) for tile i of the pass on one wave.  With `nl`, the norm's
// partial sums go through LDS with the tile sums and rn is ready for epi.
template <int NTG, class F>
__device__ __forceinline__ void reduce_tiles(const PArgs& a, PShared& sh, const f32x4 (&acc)[NTG], int nt,
                                             const Wave& wv, const NormLoad* nl, F&& epi) {
#pragma unroll
  for (int i = 0; i < NTG; ++i)
    if (i < nt) sh.u.red[wv.wave][i][wv.lane] = acc[i];
  if (nl) norm_part(sh, *nl, wv);
  lds_sync();
  if (nl) {
    norm_finish(a, sh, wv);
    lds_sync();
  }
  for (int i = wv.wave; i < nt; i += PW) {
    f32x4 s = sh.u.red[0][i][wv.lane];
#pragma unroll
    for (int v = 1; v < PW; ++v) s += sh.u.red[v][i][wv.lane];
    epi(i, s);
  }
  lds_sync();
}

// One product phase: passes of up to NTG tiles; epi(tile, sum) per tile;
// after(t0, n) once per pass after its epilogues.  ssq (or null): the
// norm applied by the epilogue.
template <int NTG, int CHK, class F, class G>
__device__ __forceinline__ void product(const PArgs& a, PShared& sh, const Work& k, const Frag& X, const Wave& wv,
                                        const float* ssq, F&& epi, G&& after) {
  if (k.nt <= 0) return;
  NormLoad nl;
  if (ssq) norm_issue(a, ssq, wv, nl);
  const int npass = (k.nt + NTG - 1) / NTG;
  int kw0, kw1;
  wave_krange(k.kbA, k.kbB, wv.wave, kw0, kw1);
  kw0 = __builtin_amdgcn_readfirstlane(kw0);
  kw1 = __builtin_amdgcn_readfirstlane(kw1);
  for (int p = 0; p < npass; ++p) {
    int t0, nt;
    pass_range(k.tile0, k.nt, npass, p, t0, nt);
    t0 = __builtin_amdgcn_readfirstlane(t0);
    nt = __builtin_amdgcn_readfirstlane(nt);
    f32x4 acc[NTG];
    gemm_core<NTG, CHK>(*k.W, X.hi, X.lo, t0, nt, kw0, kw1, wv.lane, acc);
    if (p == 0) mark(wv, 2);
    reduce_tiles<NTG>(a, sh, acc, nt, wv, (ssq && p == 0) ? &nl : nullptr, [&](int i, f32x4 s) { epi(t0 + i, s); });
    if (p == 0) mark(wv, 3);
    after(t0, nt);
  }
  mark(wv, 4);
}

// ---------------------------------------------------------------------------
// per-launch buffers (one copy per layer and phase; see the file comment)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float* xs_v(const PArgs& a, int v) { return a.xs + (size_t)v * 16 * a.H; }
__device__ __forceinline__ float* ssq_v(const PArgs& a, int v) { return a.ssq + (size_t)v * a.H; }
__device__ __forceinline__ Frag frag_v(u32x4* base, int nkb, int v) {
  Frag f;
  f.hi = base + (size_t)v * 2 * nkb * WAVE;
  f.lo = f.hi + (size_t)nkb * WAVE;
  f.mtiles = 1;
  f.nkb = nkb;
  return f;
}
__device__ __forceinline__ Frag xg_v(const PArgs& a, int v) { return frag_v(a.xg, a.H / 32, v); }

// x_out = x_in + y (tile columns), x_out * gain -> frag, sums of squares of
// the tile's 16 columns.
__device__ __forceinline__ void resnorm_tile(const PArgs& a, int tile, f32x4 y, int lane, const float* x_in,
                                             float* x_out, const float* gain, const Frag& xg, float* ssq) {
  const int g4 = lane >> 4, m = lane & 15;
  const int n = tile * 16 + g4 * 4;
  const bool ok = m < a.M;
  float ss = 0.f;
  if (ok) {
    const f32x4 x = *(const f32x4*)(x_in + (size_t)m * a.H + n) + y;
    wtf4(x_out + (size_t)m * a.H + n, x);
    const f32x4 gn = *(const f32x4*)(gain + n);
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ss = fmaf(x[j], x[j], ss);
      v[j] = x[j] * gn[j];
    }
    frag_store_wt<4>(xg, m, n, v);
  }
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  if (ok && g4 == 0) wtf(ssq + tile * 16 + m, ss);
}

// ---------------------------------------------------------------------------
// phases
// ---------------------------------------------------------------------------
// (a4) block embedding: x0 = E[id], xg0 = x0 * attn gain of layer 0,
// ssq0 per 16 columns; argmax keys cleared.  Thread: row m, 4 columns.
__device__ __forceinline__ void phase_embed(const PArgs& a, const Wave& wv) {
  const int per_row = a.H / 4;
  const int total = a.M * per_row;
  const Frag xg = xg_v(a, 0);
  const float* gain = a.layers[0].attn_gain;
  for (int base = wv.w * PT; base < ((total + 63) / 64) * 64; base += (int)gridDim.x * PT) {
    const int idx = base + wv.tid;
    const bool ok = idx < total;
    const int m = ok ? idx / per_row : 0;
    const int n0 = ok ? (idx - m * per_row) * 4 : 0;
    float ss = 0.f;
    if (ok) {
      int id = a.ids[m];
      id = id < 0 ? 0 : (id >= a.V ? a.V - 1 : id);
      const uint2 raw = *(const uint2*)(a.embed + (size_t)id * a.H + n0);
      float v[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xFFFF0000u),
                    __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xFFFF0000u)};
      wtf4(xs_v(a, 0) + (size_t)m * a.H + n0, f32x4{v[0], v[1], v[2], v[3]});
      float g[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ss = fmaf(v[j], v[j], ss);
        g[j] = v[j] * gain[n0 + j];
      }
      frag_store_wt<4>(xg, m, n0, g);
    }
    // the four threads of a 16-column group are consecutive lanes
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    if (ok && (n0 & 15) == 0) wtf(ssq_v(a, 0) + (n0 / 16) * 16 + m, ss);
  }
  if (wv.w == 0 && wv.tid < 16) wt64(a.keys + wv.tid, 0ull);
}

__device__ __forceinline__ Work work_qkv(const PArgs& a, int l, int w) { return work_full(&a.layers[l].qkv, w); }
__device__ __forceinline__ Work work_o(const PArgs& a, int l, int w) { return work_full(&a.layers[l].o, w); }
__device__ __forceinline__ Work work_gu(const PArgs& a, int l, int w) { return work_full(&a.layers[l].gu, w); }
__device__ __forceinline__ Work work_down(const PArgs& a, int l, int w) {
  return work_split(&a.layers[l].down, a.down_splits, w);
}
__device__ __forceinline__ Work work_lm(const PArgs& a, int w) { return work_full(&a.lm, w); }

constexpr int NTG_QKV = 2, CHK_QKV = 10;
constexpr int NTG_O = 1, CHK_O = 10;
constexpr int NTG_GU = 5, CHK_GU = 4;
constexpr int NTG_DN = 5, CHK_DN = 4;
constexpr int NTG_LM = 8, CHK_LM = 2;

// (a5) RMSNorm + QKV + RoPE; q, block K, block V^T of layer l.
template <int D>
__device__ __forceinline__ void phase_qkv(const PArgs& a, PShared& sh, int l, const Wave& wv) {
  const int v_in = 2 * l;
  const int qd = a.nq * D, kvd = a.nkv * D, h2 = D / 2;
  f16_t* q = a.q + (size_t)l * 16 * qd;
  f16_t* bk = a.bk + (size_t)l * a.B * a.nkv * a.Kpad * D;
  f16_t* bvt = a.bvt + (size_t)l * a.B * a.nkv * D * a.Kpad;
  const Work k = work_qkv(a, l, wv.w);
  product<NTG_QKV, CHK_QKV>(
      a, sh, k, xg_v(a, v_in), wv, ssq_v(a, v_in),
      [&](int tile, f32x4 acc) {
        const int g4 = wv.lane >> 4, m = wv.lane & 15;
        if (m >= a.M) return;
        const float r = sh.rn[m];
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = acc[j] * r;
        const int b = m / a.K, i = m - b * a.K;
        const int pos = a.seqs[b].ctx_len + i;
        const int n = tile * 16;
        if (n < qd + kvd) {
          const bool isq = n < qd;
          const int nn = isq ? n : n - qd;
          const int head = nn / D, th = (nn % D) / 16;
          const int p0 = th * 8 + g4 * 2;
          float a1, a2, b1, b2;
          rope2(y[0], y[1], pos, a.inv_freq[p0], a1, a2);
          rope2(y[2], y[3], pos, a.inv_freq[p0 + 1], b1, b2);
          f16_t* dst = isq ? q + (size_t)m * qd + head * D : bk + (((size_t)b * a.nkv + head) * a.Kpad + i) * D;
          wt32(dst + p0, (uint32_t)h16(a1) | ((uint32_t)h16(b1) << 16));
          wt32(dst + p0 + h2, (uint32_t)h16(a2) | ((uint32_t)h16(b2) << 16));
        } else {
          const int nn = n - qd - kvd;
          const int head = nn / D, f0 = nn % D + g4 * 4;
          f16_t* dst = bvt + (((size_t)b * a.nkv + head) * D + f0) * a.Kpad + i;
#pragma unroll
          for (int j = 0; j < 4; ++j) wt16(dst + (size_t)j * a.Kpad, h16(y[j]));
        }
      },
      [](int, int) {});
}

// attention work units: (sequence, KV head, key split)
__device__ __forceinline__ int n_splits(const PArgs& a, int ctx_len) {
  return (ctx_len + a.chunk - 1) / a.chunk + (a.K + a.chunk - 1) / a.chunk;
}

// (a6) one unit on waves 0..3 (query tile = wave); waves 4..7 only take
// part in the workgroup barriers.  Writes the unit's partial (m, l, O^T).
template <int D>
__device__ __forceinline__ void attention_unit(const PArgs& a, PShared& sh, int l, int b, int g, int s, const Wave& wv) {
  using T = f16_t;
  using E = Elem<T>;
  constexpr int CK = 64;                        // keys per LDS chunk
  constexpr int ES = 2;
  constexpr int KROW = D * ES + 16;
  constexpr int NFD = D * ES / 64;
  constexpr int NDT = D / 16;
  constexpr int KP = 4 * E::KPL;                // keys per P.V step (32)
  constexpr int KP_ROW = D * ES / 16;
  constexpr int KPIECES = CK * KP_ROW;
  constexpr int VP_ROW = CK * ES / 16;
  constexpr int VPIECES = D * VP_ROW;
  constexpr int EPP = 16 / ES;
  constexpr int NTH = 256;
  constexpr int KPT = KPIECES / NTH, VPT = VPIECES / NTH;
  static_assert(KPIECES % NTH == 0 && VPIECES % NTH == 0, "chunk staging");
  const bool act = wv.wave < 4;
  const int lane = wv.lane, g4 = lane >> 4, col = lane & 15;
  const int t = wv.tid;   // staging thread (< 256 on active waves)

  const DevSeq sq = a.seqs[b];
  const int ctx_len = sq.ctx_len;
  const int n_cs = (ctx_len + a.chunk - 1) / a.chunk;
  const T* kbase;
  const T* vbase;
  int vstride, k0, k1;
  if (s < n_cs) {
    kbase = (const T*)sq.k + ((size_t)l * a.nkv + g) * sq.phys * D;
    vbase = (const T*)sq.vt + ((size_t)l * a.nkv + g) * D * sq.phys;
    vstride = sq.phys;
    k0 = s * a.chunk;
    k1 = min(ctx_len, k0 + a.chunk);
  } else {
    kbase = a.bk + (size_t)l * a.B * a.nkv * a.Kpad * D + ((size_t)b * a.nkv + g) * a.Kpad * D;
    vbase = a.bvt + (size_t)l * a.B * a.nkv * D * a.Kpad + ((size_t)b * a.nkv + g) * D * a.Kpad;
    vstride = a.Kpad;
    k0 = (s - n_cs) * a.chunk;
    k1 = min(a.K, k0 + a.chunk);
  }
  const int rep = a.nq / a.nkv;
  const int nrows = a.K * rep;
  const int r = wv.wave * 16 + col;
  const bool row_ok = act && r < nrows;
  const int h = g * rep + (row_ok ? r / a.K : 0);
  const int i = row_ok ? r % a.K : 0;
  u32x4 qf[NFD];
  {
    const T* qp = a.q + (size_t)l * 16 * a.nq * D + ((size_t)(b * a.K + i) * a.nq + h) * D;
#pragma unroll
    for (int f = 0; f < NFD; ++f) qf[f] = row_ok ? gld16(qp + f * E::KB + g4 * E::KPL) : u32x4{0u, 0u, 0u, 0u};
  }
  f32x4 o[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  u32x4 kr[KPT], vr[VPT];
  auto gload = [&](int c0, int cend) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int tt = t + j * NTH;
      const int row = tt / KP_ROW, pc = tt % KP_ROW;
      kr[j] = (c0 + row < cend) ? gld16((const uint8_t*)(kbase + (size_t)(c0 + row) * D) + pc * 16)
                                : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int tt = t + j * NTH;
      const int dr = tt / VP_ROW, pc = tt % VP_ROW;
      const int key = c0 + pc * EPP;
      const T* src = vbase + (size_t)dr * vstride + key;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (key + EPP <= cend) {
        v = gld16(src);
      } else if (key < cend) {
        T tmp[EPP];
#pragma unroll
        for (int e2 = 0; e2 < EPP; ++e2) tmp[e2] = (key + e2 < cend) ? gld(src + e2) : (T)0;
        v = *(const u32x4*)tmp;
      }
      vr[j] = v;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int tt = t + j * NTH;
      *(u32x4*)(sh.u.att.kl[buf] + (tt / KP_ROW) * KROW + (tt % KP_ROW) * 16) = kr[j];
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int tt = t + j * NTH;
      *(u32x4*)(sh.u.att.vl[buf] + (tt / VP_ROW) * VROW + (tt % VP_ROW) * 16) = vr[j];
    }
  };

  const int nchunks = (k1 - k0 + CK - 1) / CK;
  if (act) {
    gload(k0, min(k1, k0 + CK));
    lstore(0);
  }
  lds_sync();
  for (int c = 0; c < nchunks; ++c) {
    const int c0 = k0 + c * CK;
    const int cend = min(k1, c0 + CK);
    const int buf = c & 1;
    if (act) {
      if (c + 1 < nchunks) gload(c0 + CK, min(k1, c0 + 2 * CK));
      const uint8_t* klb = sh.u.att.kl[buf];
      const uint8_t* vlb = sh.u.att.vl[buf];
#pragma unroll
      for (int sub = 0; sub < CK / KP; ++sub) {
        const int kb = sub * KP;
        // two S^T tiles: tile A rows -> keys 8*(row/4) + row%4, tile B -> +4
        const int rowA = kb + ((col >> 2) << 3) + (col & 3);
        const int rowB = rowA + 4;
        f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < NFD; ++f) {
          const u32x4 ka = *(const u32x4*)(klb + rowA * KROW + f * 64 + g4 * 16);
          const u32x4 kb2 = *(const u32x4*)(klb + rowB * KROW + f * 64 + g4 * 16);
          sa = E::mma(ka, qf[f], sa);
          sb = E::mma(kb2, qf[f], sb);
        }
        float sv[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sv[j] = sa[j];
          sv[4 + j] = sb[j];
        }
        // lane holds keys c0 + kb + g4*8 + j for query column `col`
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = c0 + kb + g4 * 8 + j;
          sv[j] = (key < cend) ? sv[j] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sv[j]);
        }
        mx = wave_xor_max16_32(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_safe);
        float pv[8];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = exp2f(sv[j] - m_safe);
          psum += pv[j];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int d = 0; d < NDT; ++d) o[d] *= alpha;
        const u32x4 pf = f_to_frag<T>(pv);
#pragma unroll
        for (int d = 0; d < NDT; ++d) {
          const u32x4 vf = *(const u32x4*)(vlb + (d * 16 + col) * VROW + kb * ES + g4 * 16);
          o[d] = E::mma(vf, pf, o[d]);
        }
      }
      if (c + 1 < nchunks) lstore(buf ^ 1);
    }
    lds_sync();
  }
  if (!act) return;
  l_run = wave_xor_sum16_32(l_run);
  const size_t wstride = (size_t)D * 16 + 32;
  const size_t unit = ((size_t)b * a.nkv + g) * a.max_splits + s;
  float* pp = a.apart + ((size_t)l * a.B * a.nkv * a.max_splits + unit) * 4 * wstride + wv.wave * wstride;
#pragma unroll
  for (int d = 0; d < NDT; ++d) wtf4(pp + (d * 64 + lane) * 4, o[d]);
  if (g4 == 0) {
    wtf(pp + D * 16 + col, m_run);
    wtf(pp + D * 16 + 16 + col, l_run);
  }
}

// Merge of the splits of (sequence b, KV head g) in split order on all
// eight waves: wave w takes query tile w % 4 and half w / 4 of the d-tiles,
// with the loads of MB splits in flight at once.  Writes o (frag layout
// over nq * D) of layer l.
template <int D>
__device__ __forceinline__ void attention_merge(const PArgs& a, int l, int b, int g, int ns, const Wave& wv) {
  constexpr int NDT = D / 16, HD = NDT / 2, MB = 8;
  const int qt = wv.wave & 3, dh = wv.wave >> 2;
  const int lane = wv.lane, g4 = lane >> 4, col = lane & 15;
  const size_t wstride = (size_t)D * 16 + 32;
  const float* base = a.apart + ((size_t)l * a.B * a.nkv * a.max_splits + ((size_t)b * a.nkv + g) * a.max_splits) * 4 *
                                    wstride + qt * wstride;
  float M = -INFINITY, L = 0.f;
  f32x4 o[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += MB) {
    float ms[MB], ls[MB];
    f32x4 os[MB][HD];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const bool ok = s0 + j < ns;
      const float* pp = base + (size_t)(ok ? s0 + j : 0) * 4 * wstride;
      ms[j] = ok ? pp[D * 16 + col] : -INFINITY;
      ls[j] = ok ? pp[D * 16 + 16 + col] : 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d)
        os[j][d] = ok ? *(const f32x4*)(pp + ((dh * HD + d) * 64 + lane) * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      if (ms[j] == -INFINITY) continue;
      const float Mn = fmaxf(M, ms[j]);
      const float a0 = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
      const float a1 = exp2f(ms[j] - Mn);
      L = L * a0 + ls[j] * a1;
#pragma unroll
      for (int d = 0; d < HD; ++d) o[d] = o[d] * a0 + os[j][d] * a1;
      M = Mn;
    }
  }
  const int rep = a.nq / a.nkv;
  const int r = qt * 16 + col;
  if (r >= a.K * rep) return;
  const int h = g * rep + r / a.K, i = r % a.K;
  const float inv = 1.f / L;
  const Frag of = frag_v(a.of, a.nq * D / 32, l);
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    float v[4] = {o[d][0] * inv, o[d][1] * inv, o[d][2] * inv, o[d][3] * inv};
    frag_store_wt<4>(of, b * a.K + i, h * D + (dh * HD + d) * 16 + g4 * 4, v);
  }
}

template <int D>
__device__ __forceinline__ void phase_attention(const PArgs& a, PShared& sh, int l, const Wave& wv) {
  const int units = a.B * a.nkv * a.max_splits;
  for (int u = wv.w; u < units; u += (int)gridDim.x) {
    const int s = u % a.max_splits;
    const int g = (u / a.max_splits) % a.nkv;
    const int b = u / (a.max_splits * a.nkv);
    const int ns = n_splits(a, a.seqs[b].ctx_len);
    if (s >= ns) continue;
    attention_unit<D>(a, sh, l, b, g, s, wv);
    mark(wv, 1);
    // count the finished split; the last one merges (b, g)
    if (wv.wave < 4) drain();
    lds_sync();
    mark(wv, 2);
    if (wv.tid == 0) {
      unsigned* cnt = a.acnt + (size_t)l * a.B * a.nkv + b * a.nkv + g;
      const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = (int)old + 1 == ns;
      if (last) wt32(cnt, 0u);
      sh.last = last;
    }
    lds_sync();
    mark(wv, 3);
    if (sh.last) attention_merge<D>(a, l, b, g, ns, wv);
    lds_sync();
    if (sh.last) mark(wv, 4);
  }
}

// (a7) output projection + residual: x_{2l+1} = x_{2l} + o W_o^T, with the
// MLP norm's inputs.
__device__ __forceinline__ void phase_o(const PArgs& a, PShared& sh, int l, const Wave& wv) {
  const Work k = work_o(a, l, wv.w);
  const float* x_in = xs_v(a, 2 * l);
  float* x_out = xs_v(a, 2 * l + 1);
  const Frag xg = xg_v(a, 2 * l + 1);
  float* ssq = ssq_v(a, 2 * l + 1);
  const float* gain = a.layers[l].mlp_gain;
  product<NTG_O, CHK_O>(
      a, sh, k, frag_v(a.of, a.nq * a.d / 32, l), wv, nullptr,
      [&](int tile, f32x4 acc) { resnorm_tile(a, tile, acc, wv.lane, x_in, x_out, gain, xg, ssq); },
      [](int, int) {});
}

// (a8) RMSNorm + gate/up + SwiGLU -> act of layer l.
__device__ __forceinline__ void phase_gu(const PArgs& a, PShared& sh, int l, const Wave& wv) {
  const Frag act = frag_v(a.act, a.nkb_i, l);
  const Work k = work_gu(a, l, wv.w);
  product<NTG_GU, CHK_GU>(
      a, sh, k, xg_v(a, 2 * l + 1), wv, ssq_v(a, 2 * l + 1),
      [&](int tile, f32x4 acc) {
        const int g4 = wv.lane >> 4, m = wv.lane & 15;
        if (m >= a.M) return;
        const float r = sh.rn[m];
        // tile rows 4*g4 + j: gate f, up f, gate f+1, up f+1 with f = tile*8 + 2*g4
        float v[2] = {silu_f(acc[0] * r) * (acc[1] * r), silu_f(acc[2] * r) * (acc[3] * r)};
        frag_store_wt<2>(act, m, tile * 8 + g4 * 2, v);
      },
      [](int, int) {});
}

// (a8) down projection split over k; the last split of each tile adds the
// splits (in split order) into the residual: x_{2l+2} = x_{2l+1} + sum.
__device__ __forceinline__ void phase_down(const PArgs& a, PShared& sh, int l, const Wave& wv) {
  const Work k = work_down(a, l, wv.w);
  const int S = a.down_splits;
  const int T = a.H / 16;
  const int split = wv.w % S;
  float* part = a.dpart + (size_t)l * S * T * 256;
  const float* x_in = xs_v(a, 2 * l + 1);
  float* x_out = xs_v(a, 2 * l + 2);
  const Frag xg = xg_v(a, 2 * l + 2);
  float* ssq = ssq_v(a, 2 * l + 2);
  const float* gain = l + 1 < a.L ? a.layers[l + 1].attn_gain : a.final_gain;
  product<NTG_DN, CHK_DN>(
      a, sh, k, frag_v(a.act, a.nkb_i, l), wv, nullptr,
      [&](int tile, f32x4 acc) { wtf4(part + (((size_t)split * T + tile) * 64 + wv.lane) * 4, acc); },
      [&](int t0, int nt) {
        drain();
        lds_sync();
        if (wv.tid < nt) {
          unsigned* cnt = a.dcnt + (size_t)l * T + t0 + wv.tid;
          const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const bool last = (int)old + 1 == S;
          if (last) wt32(cnt, 0u);
          sh.u.red[0][0][wv.tid][0] = last ? 1.f : 0.f;   // flag of tile t0 + tid
        }
        lds_sync();
        for (int i = wv.wave; i < nt; i += PW) {
          if (sh.u.red[0][0][i][0] == 0.f) continue;
          const int tile = t0 + i;
          f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int s0 = 0; s0 < S; s0 += 8) {   // eight loads in flight, added in split order
            f32x4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
              v[j] = s0 + j < S ? *(const f32x4*)(part + (((size_t)(s0 + j) * T + tile) * 64 + wv.lane) * 4)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 8; ++j) sum += v[j];
          }
          resnorm_tile(a, tile, sum, wv.lane, x_in, x_out, gain, xg, ssq);
        }
        lds_sync();
      });
}

// (a9) final norm + LM head + argmax; the last workgroup to finish writes
// the draft ids and the final-normed hidden rows.
__device__ __forceinline__ void phase_lm(const PArgs& a, PShared& sh, const Wave& wv) {
  const int vL = 2 * a.L;
  if (wv.tid < 16) sh.kmax[wv.tid] = 0ull;
  lds_sync();
  const Work k = work_lm(a, wv.w);
  product<NTG_LM, CHK_LM>(
      a, sh, k, xg_v(a, vL), wv, ssq_v(a, vL),
      [&](int tile, f32x4 acc) {
        const int g4 = wv.lane >> 4, m = wv.lane & 15;
        if (m >= a.M) return;
        const float r = sh.rn[m];
        const int n = tile * 16 + g4 * 4;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = acc[j] * r;
        if (a.logits) {
          float* lp = a.logits + (size_t)m * a.V + n;
          if (n + 4 <= a.V && (a.V & 3) == 0) {
            *(f32x4*)lp = f32x4{y[0], y[1], y[2], y[3]};
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (n + j < a.V) lp[j] = y[j];
          }
        }
        unsigned long long best = 0ull;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (n + j < a.V) {
            const unsigned long long key = argmax_key(y[j], (uint32_t)(n + j));
            best = key > best ? key : best;
          }
        }
        atomicMax(sh.kmax + m, best);
      },
      [](int, int) {});
  lds_sync();
  if (wv.tid < a.M && sh.kmax[wv.tid] != 0ull) atomicMax(a.keys + wv.tid, sh.kmax[wv.tid]);
  drain();
  lds_sync();
  if (wv.tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(a.lmcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old + 1 == gridDim.x;
    if (last) wt32(a.lmcnt, 0u);
    sh.last = last;
  }
  lds_sync();
  if (!sh.last) return;
  // (a9) draft ids and the final-normed hidden rows
  if (wv.tid < a.M) {
    const unsigned long long key = __hip_atomic_load(a.keys + wv.tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.draft[wv.tid] = (int32_t)argmax_index(key);
  }
  if (a.hidden) {
    const float* x = xs_v(a, vL);
    bf16_t* hid = (bf16_t*)a.hidden;
    for (int idx = wv.tid; idx < a.M * a.H; idx += PT) {
      const int m = idx / a.H, c = idx - m * a.H;
      hid[idx] = f2bf(x[idx] * sh.rn[m] * a.final_gain[c]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(PT) void persist_draft_kernel(PArgs a) {
  __shared__ PShared sh;
  __shared__ __attribute__((aligned(1024))) uint8_t warm_slot[PW][BLOCK_BYTES];
  Wave wv;
  wv.w = blockIdx.x;
  wv.tid = threadIdx.x;
  wv.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  wv.lane = threadIdx.x & 63;
  lds_void_t* slot = (lds_void_t*)&warm_slot[wv.wave][0];
  if (wv.tid == 0) {
    sh.bad = 0;
    sh.last = 0;
  }
  const int pf = a.pf_frags;
  // timeline: 8 slots per phase (0 start, 1-5 inside, 6 barrier arrival, 7 release)
  unsigned long long* trw = a.trace ? a.trace + (size_t)wv.w * a.trace_stride : nullptr;
  wv.tr = trw;
  mark(wv, 0);
  phase_embed(a, wv);
  unsigned step = 1;
  // barrier `step`, then the timeline moves on to the next phase
  auto barrier = [&](auto&& warm, bool stored) -> bool {
    const bool ok = grid_barrier(a, sh, step, wv, warm, stored);
    ++step;
    if (trw) {
      wv.tr = trw + (size_t)(step - 1) * 8;
      mark(wv, 0);
    }
    return ok;
  };
  if (!barrier([&] { warm_work(work_qkv(a, 0, wv.w), NTG_QKV, pf, wv, slot); }, true)) return;
  for (int l = 0; l < a.L; ++l) {
    phase_qkv<D>(a, sh, l, wv);
    {
      // next weights: this workgroup's O tile, or its gate/up tiles, warmed
      // by waves 4..7, which are idle during attention
      const Work ko = work_o(a, l, wv.w);
      const bool has_o = ko.nt > 0;
      if (!barrier(
              [&] {
                if (has_o)
                  warm_work(ko, NTG_O, a.pf_att, wv, slot, 4);
                else
                  warm_work(work_gu(a, l, wv.w), NTG_GU, a.pf_att, wv, slot, 4);
              },
              true))
        return;
    }
    phase_attention<D>(a, sh, l, wv);
    // waves 4..7 stored nothing and may still have warm-up loads in flight
    if (!barrier([] {}, wv.wave < 4)) return;
    phase_o(a, sh, l, wv);
    if (!barrier(
            [&] {
              if (work_o(a, l, wv.w).nt > 0) warm_work(work_gu(a, l, wv.w), NTG_GU, pf, wv, slot);
            },
            true))
      return;
    phase_gu(a, sh, l, wv);
    if (!barrier([&] { warm_work(work_down(a, l, wv.w), NTG_DN, pf, wv, slot); }, true)) return;
    phase_down(a, sh, l, wv);
    if (!barrier(
            [&] {
              if (l + 1 < a.L)
                warm_work(work_qkv(a, l + 1, wv.w), NTG_QKV, pf, wv, slot);
              else
                warm_work(work_lm(a, wv.w), NTG_LM, pf, wv, slot);
            },
            true))
      return;
  }
  phase_lm(a, sh, wv);
  mark(wv, 6);
}

}  // namespace

unsigned persist_steps(int L) { return 1u + 5u * (unsigned)L; }

hipError_t persist_occupancy(int d, int* blocks_per_cu) {
  const void* f = d == 64 ? (const void*)persist_draft_kernel<64> : (const void*)persist_draft_kernel<128>;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, f, PT, 0);
}

hipError_t launch_persist_draft(const PArgs& a, int nwg, hipStream_t s) {
  void* args[] = {(void*)&a};
  const void* f = a.d == 64 ? (const void*)persist_draft_kernel<64> : (const void*)persist_draft_kernel<128>;
  if (a.d != 64 && a.d != 128) return hipErrorInvalidValue;
  return hipLaunchCooperativeKernel(f, dim3(nwg), dim3(PT), args, 0, s);
}

}  // namespace dflash
