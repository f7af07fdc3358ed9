// Single-launch draft block for small blocks (batch * K <= 16 rows) of bf16
// drafters on gfx950, with the weight stream decoupled from the phases.
//
// The draft forward (kongchang.com "D-Flash", "System architecture" and
// "Innovation 1"; Google Developers Blog, "Dual cache for attention") is a
// chain of weight-streaming products in which every output row of one
// product needs every column of the one before.  Run as one kernel per
// product, each pays launch, ramp-up and drain, and HBM idles across the
// gaps and across the small kernels in between (attention, split merges,
// residual passes).  Here one cooperative launch of one workgroup per
// compute unit runs the whole block, and the weights never wait for the
// activations:
//
//   * waves 4..7 are loaders: loader 4 + c streams, in order, every weight
//     fragment that compute wave c of this workgroup will multiply in the
//     whole block (its share of QKV, O, gate/up and down of every layer,
//     then of the LM head) into a ring of LDS slots owned by wave c,
//     RING_SLOTS deep, with LOAD_DEPTH fragments in flight in registers.
//     The schedule depends only on the shapes, so a loader runs ahead
//     through phase boundaries and attention, limited only by free slots;
//   * waves 0..3 compute: embed | per layer: QKV + RoPE | attention over
//     [context || block] split over keys | the merge of the splits, spread
//     over the grid | O + residual + norm inputs | gate/up + SwiGLU | down split
//     over k, the last split of a tile adding the splits into the residual
//     | LM head + argmax, the last workgroup writing the draft ids.  A
//     product takes its weight fragments from the ring and its activations
//     from memory; a flag barrier over the compute waves of all workgroups
//     separates the phases.
//
// The compute waves synchronise among themselves through an LDS counter
// (the loaders never reach a workgroup barrier, so s_barrier cannot be
// used after the start); a ring slot is published by its loader after the
// slot's LDS write has completed, and released by its compute wave after
// the slot's value has been used.
//
// Memory visibility across XCDs (each XCD has its own L2): every buffer that
// one workgroup writes and another reads within the launch is written with
// device-scope (write-through) stores, at most once per launch and at an
// address of its own (one copy per layer and phase), so no XCD can hold a
// stale line of it; a compute wave's stores complete (s_waitcnt) before its
// flag or counter update, and readers load only after observing it.  No
// memory fence is used (an agent-scope release writes back and invalidates
// the whole L2).
//
// Every wait is bounded (about 2 s of the constant 100 MHz clock) and also
// ends when another wave has recorded an error; a wait that expires sets
// the error word and its wave leaves the kernel, so every wave of the grid
// exits.
//
// Measured on a 5-layer Qwen3-4B-shaped drafter at K = 16 this launch is
// slower than the per-product kernels (0.74 against 0.48 ms): the LM head
// streams at 5.4 TB/s, but the layers' phases run at about 2.9 TB/s.  The
// loaders keep about 40 MB of weight reads in flight across the chip, and
// every load on the critical path (the activations after a barrier, the
// KV reads of attention, the barrier flags) queues behind them; with fewer
// reads in flight the stream itself slows.  The path is therefore off by
// default.
#include "kernels.h"

namespace dflash {

namespace {

constexpr int CW = 4;                  // compute waves per workgroup
constexpr int LW = 4;                  // loader waves (loader CW + c feeds compute wave c)
constexpr int PT = (CW + LW) * 64;     // threads per workgroup
constexpr int CT = CW * 64;            // compute threads
constexpr int RING_SLOTS = 28;         // 1 KiB weight fragments per compute wave in LDS
constexpr int LOAD_DEPTH = 40;         // fragments each loader keeps in flight (registers)
constexpr int PUB = 10;                // fragments a loader writes to its ring per publication
constexpr int MAX_PASSES = 40;         // passes of one loader's stream (checked before launch)
constexpr unsigned long long kTimeoutTicks = 200000000ull;   // 2 s of the 100 MHz clock

// Explicit address spaces: a generic (flat) access counts against both the
// vector-memory and the LDS counters, so every wait on one would also wait
// for the other; global and LDS accesses here are never flat.
typedef __attribute__((address_space(1))) uint16_t g_u16;
typedef __attribute__((address_space(1))) unsigned g_u32;
typedef __attribute__((address_space(1))) unsigned long long g_u64;
typedef __attribute__((address_space(1))) float g_f32;
typedef __attribute__((address_space(1))) f32x4 g_f32x4;
typedef __attribute__((address_space(3))) unsigned l_u32;
typedef __attribute__((address_space(3))) unsigned long long l_u64;
typedef __attribute__((address_space(3))) u32x4 l_u32x4;
template <typename T>
__device__ __forceinline__ T gload(const T* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}
// structures field by field (scalars only in an explicit address space)
__device__ __forceinline__ Packed gload_packed(const Packed* p) {
  Packed r;
  r.w = (const uint8_t*)gload((const uint64_t*)&p->w);
  r.n_rows = gload(&p->n_rows);
  r.n_tiles = gload(&p->n_tiles);
  r.kd = gload(&p->kd);
  r.nkb = gload(&p->nkb);
  return r;
}
__device__ __forceinline__ DevSeq gload_seq(const DevSeq* p) {
  DevSeq r;
  r.ctx_len = gload(&p->ctx_len);
  r.cap = gload(&p->cap);
  r.phys = gload(&p->phys);
  r.pad = 0;
  r.ctxbuf = (void*)gload((const uint64_t*)&p->ctxbuf);
  r.k = (void*)gload((const uint64_t*)&p->k);
  r.vt = (void*)gload((const uint64_t*)&p->vt);
  return r;
}

// Completes every memory operation this wave has issued.
__device__ __forceinline__ void drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Completes this wave's LDS operations (lgkmcnt = 0, other counters free).
__device__ __forceinline__ void lds_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// device-scope (write-through) stores
__device__ __forceinline__ void wt16(void* p, uint16_t v) {
  __hip_atomic_store((g_u16*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wt32(void* p, uint32_t v) {
  __hip_atomic_store((g_u32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wt64(void* p, uint64_t v) {
  __hip_atomic_store((g_u64*)p, (unsigned long long)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// agent-scope atomics on global words
__device__ __forceinline__ unsigned gatom_ld(const unsigned* p) {
  return __hip_atomic_load((g_u32*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned gatom_add(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add((g_u32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void gatom_or(unsigned* p, unsigned v) {
  __hip_atomic_fetch_or((g_u32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
constexpr int NTG_MAX = 8;

struct PShared {
  union {
    struct {
      uint8_t kl[64 * KROW128];
      uint8_t vl[128 * VROW];
    } att;
    f32x4 red[CW][NTG_MAX][64];
  } u;
  float npart[16][16];
  float rn[16];
  unsigned long long kmax[16];
  int bad;
  int last;
  unsigned cbar;              // compute-wave barrier counter
  unsigned filled[CW];        // fragments written to ring c (monotone)
  unsigned consumed[CW];      // fragments of ring c released by its compute wave
  unsigned abort;             // set by a compute wave that leaves early: loaders stop
  // the packed weights of every product, [layer][QKV, O, gate/up, down], then
  // the LM head at index 4 L: loaders read them from here, never from global
  // memory (a global load on a loader would make the compiler wait for the
  // weight loads in flight)
  struct {
    const uint8_t* w;
    int32_t n_tiles, nkb;
  } prod[4 * PERSIST_MAX_LAYERS + 1];
  // every loader's passes in stream order (built at the start of the launch)
  struct Pass {
    const uint8_t* base;   // the tile t0 row of k-block 0
    int32_t nkb, nt, kw0, kw1, kwp;
  } pass[LW][MAX_PASSES];
  int32_t npass[LW];
};

// LDS counters are read and written atomically (workgroup scope) so that a
// poll is never hoisted out of its loop.
__device__ __forceinline__ unsigned lds_ld(unsigned* p) {
  return __hip_atomic_load((l_u32*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(unsigned* p, unsigned v) {
  __hip_atomic_store((l_u32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

struct Wave {
  int w;      // workgroup
  int wave;   // wave in the workgroup (scalar)
  int lane;
  int tid;
  unsigned long long* tr;   // timeline slots of the current phase, or null
};
// timeline mark k of the current phase (thread 0 only)
__device__ __forceinline__ void mark(const Wave& wv, int k) {
  if (wv.tr && wv.tid == 0) *(g_u64*)(wv.tr + k) = wall_clock64();
}

// A bounded wait: true while the caller should keep polling.  Every 64
// polls it reads the clock and the grid's error word; on expiry it records
// the error.  `t0` is the start tick, `n` the poll count.
__device__ __forceinline__ bool keep_waiting(const PArgs& a, unsigned long long t0, unsigned& n, int lane) {
  if ((++n & 63u) != 0u) return true;
  const unsigned err = gatom_ld(a.err);
  if (__builtin_amdgcn_readfirstlane(err) != 0u) return false;
  if (wall_clock64() - t0 > kTimeoutTicks) {
    if (lane == 0) gatom_or(a.err, 1u);
    return false;
  }
  return true;
}

// The loaders' bounded wait: it reads the clock and the workgroup's abort
// flag (LDS), never global memory.
__device__ __forceinline__ bool loader_keep_waiting(const PArgs& a, PShared& sh, unsigned long long t0, unsigned& n,
                                                    int lane) {
  if ((++n & 63u) != 0u) return true;
  if (lds_ld(&sh.abort) != 0u) return false;
  if (wall_clock64() - t0 > kTimeoutTicks) {
    if (lane == 0) gatom_or(a.err, 1u);
    return false;
  }
  return true;
}

// Barrier of the CW compute waves of this workgroup (an LDS counter that
// every compute wave increments once per barrier; a wave cannot enter the
// next barrier before this one is complete, so its own increment tells it
// which multiple of CW to wait for).  Returns false when the wait was
// abandoned (error recorded).
__device__ __forceinline__ bool csync(const PArgs& a, PShared& sh, const Wave& wv) {
  lds_done();
  unsigned old = 0;
  if (wv.lane == 0) old = __hip_atomic_fetch_add((l_u32*)&sh.cbar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const unsigned target = ((unsigned)__builtin_amdgcn_readfirstlane((int)old) & ~(unsigned)(CW - 1)) + CW;
  if ((int)(lds_ld(&sh.cbar) - target) >= 0) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return true;
  }
  const unsigned long long t0 = wall_clock64();
  unsigned n = 0;
  while ((int)(lds_ld(&sh.cbar) - target) < 0) {
    if (!keep_waiting(a, t0, n, wv.lane)) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return true;
}

// A pointer that is the same on every lane, in scalar registers.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (P*)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// work assignment: the same functions give the loaders their schedule and
// the compute waves their products
// ---------------------------------------------------------------------------
struct Work {
  Packed W;
  int tile0, nt;    // this workgroup's tiles
  int kbA, kbB;     // its range of k-blocks
};

__device__ __forceinline__ void even_range(int n, int parts, int i, int& a, int& cnt) {
  a = (int)((long)i * n / parts);
  cnt = (int)((long)(i + 1) * n / parts) - a;
}

__device__ __forceinline__ Work work_full(const Packed& W, int w) {
  Work k;
  k.W = W;
  even_range(W.n_tiles, (int)gridDim.x, w, k.tile0, k.nt);
  k.kbA = 0;
  k.kbB = W.nkb;
  return k;
}
// split over k: workgroup w takes split w % S of the tiles of group w / S
__device__ __forceinline__ Work work_split(const Packed& W, int S, int w) {
  Work k;
  k.W = W;
  const int groups = (int)gridDim.x / S;
  const int s = w % S, gi = w / S;
  if (gi >= groups) {
    k.tile0 = 0;
    k.nt = 0;
  } else {
    even_range(W.n_tiles, groups, gi, k.tile0, k.nt);
  }
  int c;
  even_range(W.nkb, S, s, k.kbA, c);
  k.kbB = k.kbA + c;
  return k;
}
// the k-blocks of compute wave v within [kbA, kbB)
__device__ __forceinline__ void wave_krange(int kbA, int kbB, int v, int& k0, int& k1) {
  const int per = (kbB - kbA + CW - 1) / CW;
  k0 = min(kbB, kbA + v * per);
  k1 = min(kbB, k0 + per);
}
// tiles of pass p of npass over nt tiles
__device__ __forceinline__ void pass_range(int tile0, int nt, int npass, int p, int& t0, int& n) {
  int a;
  even_range(nt, npass, p, a, n);
  t0 = tile0 + a;
}

// products of the stream, in order: per layer QKV, O, gate/up, down; then
// the LM head (layer index L)
enum Prod { P_QKV = 0, P_O = 1, P_GU = 2, P_DN = 3, P_LM = 4 };
constexpr int NTG_QKV = 2, CHK_QKV = 20;
constexpr int NTG_O = 1, CHK_O = 16;
constexpr int NTG_GU = 5, CHK_GU = 20;
constexpr int NTG_DN = 5, CHK_DN = 10;
constexpr int NTG_LM = 4, CHK_LM = 20;
__device__ __forceinline__ int prod_ntg(int p) {
  return p == P_QKV ? NTG_QKV : p == P_O ? NTG_O : p == P_GU ? NTG_GU : p == P_DN ? NTG_DN : NTG_LM;
}
__device__ __forceinline__ int prod_chk(int p) {
  return p == P_QKV ? CHK_QKV : p == P_O ? CHK_O : p == P_GU ? CHK_GU : p == P_DN ? CHK_DN : CHK_LM;
}
// k-blocks a wave's stream holds for a range of n: whole batches of chk
// (the padding is zero fragments, multiplied by re-read activations)
__device__ __forceinline__ int padded_kb(int n, int chk) { return (n + chk - 1) / chk * chk; }
__device__ __forceinline__ Work prod_work(const PArgs& a, PShared& sh, int l, int p, int w) {
  const int i = p == P_LM ? 4 * a.L : 4 * l + p;
  Packed W;
  W.w = sh.prod[i].w;
  W.n_tiles = sh.prod[i].n_tiles;
  W.nkb = sh.prod[i].nkb;
  W.n_rows = 0;
  W.kd = 0;
  return p == P_DN ? work_split(W, a.down_splits, w) : work_full(W, w);
}

// ---------------------------------------------------------------------------
// the weight stream: loader waves
// ---------------------------------------------------------------------------
// The fragments compute wave c of workgroup w multiplies, in the order it
// multiplies them: product by product; per product, pass by pass (up to NTG
// tiles); per pass, the wave's k-blocks padded to whole batches of CHK and,
// per k-block, the pass's tiles in order.  A padding k-block's fragments are
// zero.  The passes are listed in LDS once per launch (build_passes).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ void build_passes(const PArgs& a, PShared& sh, int w, int c, int lane) {
  int n = 0;
  for (int l = 0; l <= a.L; ++l) {
    for (int p = 0; p < (l == a.L ? 1 : 4); ++p) {
      const int pp = l == a.L ? (int)P_LM : p;
      const Work k = prod_work(a, sh, l, pp, w);
      int k0, k1;
      wave_krange(k.kbA, k.kbB, c, k0, k1);
      if (k.nt <= 0 || k1 <= k0) continue;
      const int ntg = prod_ntg(pp);
      const int np = (k.nt + ntg - 1) / ntg;
      for (int q = 0; q < np; ++q) {
        int t0, nt;
        pass_range(k.tile0, k.nt, np, q, t0, nt);
        if (lane == 0 && n < MAX_PASSES) {
          PShared::Pass& e = sh.pass[c][n];
          e.base = k.W.w + (size_t)t0 * k.W.nkb * BLOCK_BYTES;
          e.nkb = k.W.nkb;
          e.nt = nt;
          e.kw0 = k0;
          e.kw1 = k1;
          e.kwp = k0 + padded_kb(k1 - k0, prod_chk(pp));
        }
        ++n;
      }
    }
  }
  if (lane == 0) sh.npass[c] = n;
}

struct PassRegs {
  const uint8_t* base;   // packed weights of the pass's first tile
  int nkb, nt, kw0, kw1, kwp;
};
// Pass i of loader c, read from LDS into scalar registers.
__device__ __forceinline__ PassRegs pass_regs(PShared& sh, int c, int i) {
  const PShared::Pass& e = sh.pass[c][i];
  PassRegs r;
  r.base = uniform_ptr(e.base);
  r.nkb = uni(e.nkb);
  r.nt = uni(e.nt);
  r.kw0 = uni(e.kw0);
  r.kw1 = uni(e.kw1);
  r.kwp = uni(e.kwp);
  return r;
}

// Loader wave c: streams wave c's fragments into its ring.  Register set j
// holds fragment j (mod LOAD_DEPTH) of the stream: it is written to LDS and
// then loaded again with the fragment LOAD_DEPTH later, so LOAD_DEPTH loads
// stay in flight.  Every load is issued unconditionally (padding fragments,
// and register sets past the end of the stream, load a zero fragment that
// stays in L2), and the loop holds no other memory access on a conditional
// path (the next pass's entry is read once per publication, a pass being
// longer than a publication), so that each write waits only for its own
// load.  Writes go in publications of PUB fragments, each waiting for PUB
// free slots.
static_assert(PUB + 8 <= RING_SLOTS + 1, "a publication and a k-block of the largest pass must fit the ring");
static_assert(LOAD_DEPTH % PUB == 0, "publications divide the loads in flight");
static_assert(PUB <= CHK_DN && PUB <= CHK_O && PUB <= CHK_QKV && PUB <= CHK_GU && PUB <= CHK_LM,
              "every pass is at least one publication long");
__device__ __forceinline__ void loader(const PArgs& a, PShared& sh, l_u32x4* ring, int c, int lane) {
  const int npass = uni(sh.npass[c]);
  if (npass > MAX_PASSES) {   // more passes than the list holds (excluded before launch)
    if (lane == 0) gatom_or(a.err, 2u);
    return;
  }
  if (npass == 0) return;
  PassRegs cur = pass_regs(sh, c, 0);
  PassRegs nxt = cur;
  int pass = 0, kb = cur.kw0, t = 0;
  bool done = false, live = true;
  const uint8_t* zero = uniform_ptr(a.zero_frag);
  const uint32_t lo = (uint32_t)lane * FRAG_BYTES;
  unsigned issued = 0, written = 0;
  unsigned free_upto = RING_SLOTS;   // slots below this index are free to write
  int slot = 0;
  u32x4 buf[LOAD_DEPTH];
  // the next fragment's address (or the zero fragment's), then advance
  auto next = [&]() -> const uint8_t* {
    const uint64_t real = (!done && kb < cur.kw1) ? ~0ull : 0ull;
    const uint64_t at = (uint64_t)(cur.base + ((size_t)t * cur.nkb + kb) * BLOCK_BYTES);
    if (!done) {   // (uniform; scalar work only)
      ++issued;
      if (++t == cur.nt) {
        t = 0;
        if (++kb == cur.kwp) {
          if (++pass < npass) {
            cur = nxt;
            kb = cur.kw0;
          } else {
            done = true;
          }
        }
      }
    }
    return (const uint8_t*)((at & real) | ((uint64_t)zero & ~real));
  };
  if (npass > 1) nxt = pass_regs(sh, c, 1);
#pragma unroll
  for (int j = 0; j < LOAD_DEPTH; ++j) {
    if (j % PUB == 0) nxt = pass_regs(sh, c, min(pass + 1, npass - 1));
    buf[j] = __builtin_nontemporal_load((const gu32x4*)(next() + lo));
  }
  while (written < issued) {
#pragma unroll
    for (int j = 0; j < LOAD_DEPTH; ++j) {
      if (j % PUB == 0) {
        nxt = pass_regs(sh, c, min(pass + 1, npass - 1));
        // room for this publication
        const unsigned n = min((unsigned)PUB, issued - written);
        if ((int)(written + n - free_upto) > 0) {
          const unsigned long long t0 = wall_clock64();
          unsigned cnt = 0;
          for (;;) {
            free_upto = lds_ld(&sh.consumed[c]) + RING_SLOTS;
            if ((int)(written + n - free_upto) <= 0) break;
            if (!loader_keep_waiting(a, sh, t0, cnt, lane)) {
              // abandoned: drop the rest of the stream and publish nothing
              // more; the loop ends after this pass over the register sets.
              // (Leaving the loop from here would add an edge into it that
              // shortens the waits of all its loads.)
              done = true;
              live = false;
              written = issued;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
      }
      if (written < issued) {   // (uniform)
        ring[slot * WAVE + lane] = buf[j];
        ++written;
        slot = slot + 1 == RING_SLOTS ? 0 : slot + 1;
      }
      buf[j] = __builtin_nontemporal_load((const gu32x4*)(next() + lo));
      if (j % PUB == PUB - 1 && live) {
        lds_done();
        lds_st(&sh.filled[c], written);
      }
    }
  }
}

// A compute wave's read side of its ring.
struct RingRd {
  l_u32x4* ring;
  unsigned* filled;
  unsigned* consumed;
  unsigned idx;       // fragments taken
  unsigned avail;     // fragments known to be written
  int slot;
};

// ---------------------------------------------------------------------------
// weight products (one 16-row activation tile, bf16 hi/lo pair)
// ---------------------------------------------------------------------------

// acc[t] = sum over this wave's k-blocks [kw0, kw1) of W tile (t0 + t) times
// the activation fragments (hi and lo), for NT tiles; the weight fragments
// come from the ring in stream order (CHK k-blocks per batch, the last
// batch padded with zero fragments).  Returns false when a wait was
// abandoned.
template <int NT, int CHK, int NTG>
__device__ __forceinline__ bool ring_gemm_nt(const PArgs& a, RingRd& rr, const uint8_t* xh, const uint8_t* xl,
                                             int kw0, int kw1, int lane, f32x4 (&acc)[NTG]) {
  using E = Elem<bf16_t>;
  const uint32_t lo = (uint32_t)lane * FRAG_BYTES;
  for (int kb0 = kw0; kb0 < kw1; kb0 += CHK) {
    const int last = kw1 - 1;
    u32x4 ah[CHK], al[CHK];
#pragma unroll
    for (int j = 0; j < CHK; ++j) {
      const int kb = min(kb0 + j, last);   // padding: re-read the last (its weights are zero)
      ah[j] = gld16(xh + (size_t)kb * BLOCK_BYTES + lo);
      al[j] = gld16(xl + (size_t)kb * BLOCK_BYTES + lo);
    }
#pragma unroll
    for (int j = 0; j < CHK; ++j) {
      const unsigned need = rr.idx + (unsigned)NT;
      if ((int)(need - rr.avail) > 0) {
        const unsigned long long t0 = wall_clock64();
        unsigned cnt = 0;
        for (;;) {
          rr.avail = lds_ld(rr.filled);
          if ((int)(need - rr.avail) <= 0) break;
          if (!keep_waiting(a, t0, cnt, lane)) return false;
          __builtin_amdgcn_s_sleep(0);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int sl = rr.slot + t >= RING_SLOTS ? rr.slot + t - RING_SLOTS : rr.slot + t;
        const u32x4 wf = rr.ring[sl * WAVE + lane];
        acc[t] = E::mma(wf, ah[j], acc[t]);
        acc[t] = E::mma(wf, al[j], acc[t]);
      }
      rr.slot = rr.slot + NT >= RING_SLOTS ? rr.slot + NT - RING_SLOTS : rr.slot + NT;
      rr.idx = need;
      // the slots of this k-block have been read: release them
      lds_done();
      lds_st(rr.consumed, rr.idx);
    }
  }
  return true;
}

template <int NTG, int CHK>
__device__ __forceinline__ bool ring_gemm(const PArgs& a, RingRd& rr, const u32x4* xh_, const u32x4* xl_, int nt,
                                          int kw0, int kw1, int lane, f32x4 (&acc)[NTG]) {
  const uint8_t* xh = (const uint8_t*)uniform_ptr(xh_);
  const uint8_t* xl = (const uint8_t*)uniform_ptr(xl_);
#pragma unroll
  for (int t = 0; t < NTG; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (kw1 <= kw0) return true;
  bool ok = true;
  switch (nt) {   // (uniform)
    case 1: ok = ring_gemm_nt<1, CHK, NTG>(a, rr, xh, xl, kw0, kw1, lane, acc); break;
    case 2: if constexpr (NTG >= 2) ok = ring_gemm_nt<2, CHK, NTG>(a, rr, xh, xl, kw0, kw1, lane, acc); break;
    case 3: if constexpr (NTG >= 3) ok = ring_gemm_nt<3, CHK, NTG>(a, rr, xh, xl, kw0, kw1, lane, acc); break;
    case 4: if constexpr (NTG >= 4) ok = ring_gemm_nt<4, CHK, NTG>(a, rr, xh, xl, kw0, kw1, lane, acc); break;
    case 5: if constexpr (NTG >= 5) ok = ring_gemm_nt<5, CHK, NTG>(a, rr, xh, xl, kw0, kw1, lane, acc); break;
    default: break;
  }
  return ok;
}

// RMSNorm row scales, rn[m] = rsqrt(sum_g ssq[g][m] / H + eps) over the
// per-16-column sums of squares ssq[g][16] (g < H/16): compute thread t
// loads rows t % 16 of groups t / 16 + 16 j before the product (the values
// are only needed by the epilogue), adds them after, and the 16 partial
// sums of a row are added in order through LDS.
constexpr int NORM_MAX = 16;   // groups per thread: H <= 4096
struct NormLoad {
  float v[NORM_MAX];
};
__device__ __forceinline__ void norm_issue(const PArgs& a, const float* ssq, const Wave& wv, NormLoad& nl) {
  const int r = wv.tid & 15, part = wv.tid >> 4;
  const int groups = a.H / 16;
#pragma unroll
  for (int j = 0; j < NORM_MAX; ++j) {
    const int g = part + 16 * j;
    nl.v[j] = (g < groups && r < a.M) ? gload(ssq + g * 16 + r) : 0.f;
  }
}
__device__ __forceinline__ void norm_part(PShared& sh, const NormLoad& nl, const Wave& wv) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NORM_MAX; ++j) s += nl.v[j];
  sh.npart[wv.tid >> 4][wv.tid & 15] = s;
}
// after a csync that follows norm_part in every compute thread
__device__ __forceinline__ void norm_finish(const PArgs& a, PShared& sh, const Wave& wv) {
  if (wv.tid < 16) {
    float t = 0.f;
#pragma unroll
    for (int p = 0; p < 16; ++p) t += sh.npart[p][wv.tid];
    sh.rn[wv.tid] = wv.tid < a.M ? rsqrtf(t / (float)a.H + a.eps) : 0.f;
  }
}

// The compute waves' sums of each tile added in wave order through LDS,
// then epi(i, sum) for tile i of the pass on one wave.  With `nl`, the
// norm's partial sums go through LDS with the tile sums and rn is ready for
// epi.
template <int NTG, class F>
__device__ __forceinline__ bool reduce_tiles(const PArgs& a, PShared& sh, const f32x4 (&acc)[NTG], int nt,
                                             const Wave& wv, const NormLoad* nl, F&& epi) {
#pragma unroll
  for (int i = 0; i < NTG; ++i)
    if (i < nt) sh.u.red[wv.wave][i][wv.lane] = acc[i];
  if (nl) norm_part(sh, *nl, wv);
  if (!csync(a, sh, wv)) return false;
  if (nl) {
    norm_finish(a, sh, wv);
    if (!csync(a, sh, wv)) return false;
  }
  for (int i = wv.wave; i < nt; i += CW) {
    f32x4 s = sh.u.red[0][i][wv.lane];
#pragma unroll
    for (int v = 1; v < CW; ++v) s += sh.u.red[v][i][wv.lane];
    epi(i, s);
  }
  return csync(a, sh, wv);
}

// One product phase: passes of up to NTG tiles; epi(tile, sum) per tile;
// after(t0, n) once per pass after its epilogues (returns false to abandon).
// ssq (or null): the norm applied by the epilogue.
template <int NTG, int CHK, class F, class G>
__device__ __forceinline__ bool product(const PArgs& a, PShared& sh, RingRd& rr, const Work& k, const Frag& X,
                                        const Wave& wv, const float* ssq, F&& epi, G&& after) {
  if (k.nt <= 0) return true;
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
    if (!ring_gemm<NTG, CHK>(a, rr, X.hi, X.lo, nt, kw0, kw1, wv.lane, acc)) return false;
    if (p == 0) mark(wv, 2);
    if (!reduce_tiles<NTG>(a, sh, acc, nt, wv, (ssq && p == 0) ? &nl : nullptr,
                           [&](int i, f32x4 s) { epi(t0 + i, s); }))
      return false;
    if (p == 0) mark(wv, 3);
    if (!after(t0, nt)) return false;
  }
  mark(wv, 4);
  return true;
}

// ---------------------------------------------------------------------------
// the flag barrier over the compute waves of every workgroup
// ---------------------------------------------------------------------------
// Every workgroup publishes base + step in its flag once its compute waves'
// stores are complete; compute wave 0 then reads all flags until each has
// reached the step.  Returns false when the launch is abandoned.
__device__ __forceinline__ bool grid_barrier(const PArgs& a, PShared& sh, unsigned step, const Wave& wv) {
  drain();
  if (!csync(a, sh, wv)) return false;
  const unsigned target = a.base + step;
  mark(wv, 6);
  if (wv.tid == 0) wt32(a.flags + wv.w, target);
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
          const unsigned v = gatom_ld(a.flags + i);
          ok = ok && (int)(v - target) >= 0;
        }
      }
      const unsigned err = gatom_ld(a.err);
      if (__all(ok)) break;
      if (__builtin_amdgcn_readfirstlane(err) != 0u) {
        bad = 1;
        break;
      }
      if (wall_clock64() - t0 > kTimeoutTicks) {
        if (wv.lane == 0) gatom_or(a.err, 1u);
        bad = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (wv.lane == 0) sh.bad = bad;
    mark(wv, 7);
  }
  if (!csync(a, sh, wv)) return false;
  return sh.bad == 0;
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
    const f32x4 x = gload((const f32x4*)(x_in + (size_t)m * a.H + n)) + y;
    wtf4(x_out + (size_t)m * a.H + n, x);
    const f32x4 gn = gload((const f32x4*)(gain + n));
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
// phases (compute waves)
// ---------------------------------------------------------------------------
// (a4) block embedding: x0 = E[id], xg0 = x0 * attn gain of layer 0,
// ssq0 per 16 columns; argmax keys cleared.  Thread: row m, 4 columns.
__device__ __forceinline__ void phase_embed(const PArgs& a, const Wave& wv) {
  const int per_row = a.H / 4;
  const int total = a.M * per_row;
  const Frag xg = xg_v(a, 0);
  const float* gain = gload(&a.layers[0].attn_gain);
  for (int base = wv.w * CT; base < ((total + 63) / 64) * 64; base += (int)gridDim.x * CT) {
    const int idx = base + wv.tid;
    const bool ok = idx < total;
    const int m = ok ? idx / per_row : 0;
    const int n0 = ok ? (idx - m * per_row) * 4 : 0;
    float ss = 0.f;
    if (ok) {
      int id = gload(a.ids + m);
      id = id < 0 ? 0 : (id >= a.V ? a.V - 1 : id);
      const u32x2 raw = gload((const u32x2*)(a.embed + (size_t)id * a.H + n0));
      float v[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xFFFF0000u),
                    __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xFFFF0000u)};
      wtf4(xs_v(a, 0) + (size_t)m * a.H + n0, f32x4{v[0], v[1], v[2], v[3]});
      float g[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ss = fmaf(v[j], v[j], ss);
        g[j] = v[j] * gload(gain + n0 + j);
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

struct NoAfter {
  __device__ bool operator()(int, int) const { return true; }
};

// (a5) RMSNorm + QKV + RoPE; q, block K, block V^T of layer l.
template <int D>
__device__ __forceinline__ bool phase_qkv(const PArgs& a, PShared& sh, RingRd& rr, int l, const Wave& wv) {
  const int v_in = 2 * l;
  const int qd = a.nq * D, kvd = a.nkv * D, h2 = D / 2;
  f16_t* q = a.q + (size_t)l * 16 * qd;
  f16_t* bk = a.bk + (size_t)l * a.B * a.nkv * a.Kpad * D;
  f16_t* bvt = a.bvt + (size_t)l * a.B * a.nkv * D * a.Kpad;
  const Work k = prod_work(a, sh, l, P_QKV, wv.w);
  return product<NTG_QKV, CHK_QKV>(
      a, sh, rr, k, xg_v(a, v_in), wv, ssq_v(a, v_in),
      [&](int tile, f32x4 acc) {
        const int g4 = wv.lane >> 4, m = wv.lane & 15;
        if (m >= a.M) return;
        const float r = sh.rn[m];
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = acc[j] * r;
        const int b = m / a.K, i = m - b * a.K;
        const int pos = gload(&a.seqs[b].ctx_len) + i;
        const int n = tile * 16;
        if (n < qd + kvd) {
          const bool isq = n < qd;
          const int nn = isq ? n : n - qd;
          const int head = nn / D, th = (nn % D) / 16;
          const int p0 = th * 8 + g4 * 2;
          float a1, a2, b1, b2;
          rope2(y[0], y[1], pos, gload(a.inv_freq + p0), a1, a2);
          rope2(y[2], y[3], pos, gload(a.inv_freq + p0 + 1), b1, b2);
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
      NoAfter{});
}

// attention work units: (sequence, KV head, key split)
__device__ __forceinline__ int n_splits(const PArgs& a, int ctx_len) {
  return (ctx_len + a.chunk - 1) / a.chunk + (a.K + a.chunk - 1) / a.chunk;
}

// (a6) one unit on the compute waves (query tile = wave).  Writes the
// unit's partial (m, l, O^T).  Returns false when a wait was abandoned.
template <int D>
__device__ __forceinline__ bool attention_unit(const PArgs& a, PShared& sh, int l, int b, int g, int s,
                                               const Wave& wv) {
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
  constexpr int NTH = CT;
  constexpr int KPT = KPIECES / NTH, VPT = VPIECES / NTH;
  static_assert(KPIECES % NTH == 0 && VPIECES % NTH == 0, "chunk staging");
  const int lane = wv.lane, g4 = lane >> 4, col = lane & 15;
  const int t = wv.tid;   // staging thread

  const DevSeq sq = gload_seq(a.seqs + b);
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
  const bool row_ok = r < nrows;
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
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int tt = t + j * NTH;
      *(u32x4*)(sh.u.att.kl + (tt / KP_ROW) * KROW + (tt % KP_ROW) * 16) = kr[j];
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int tt = t + j * NTH;
      *(u32x4*)(sh.u.att.vl + (tt / VP_ROW) * VROW + (tt % VP_ROW) * 16) = vr[j];
    }
  };

  // one LDS stage: chunk c + 1 is loaded into registers while chunk c is
  // computed from LDS, and stored after every wave is done with chunk c
  const int nchunks = (k1 - k0 + CK - 1) / CK;
  gload(k0, min(k1, k0 + CK));
  lstore();
  if (!csync(a, sh, wv)) return false;
  for (int c = 0; c < nchunks; ++c) {
    const int c0 = k0 + c * CK;
    const int cend = min(k1, c0 + CK);
    if (c + 1 < nchunks) gload(c0 + CK, min(k1, c0 + 2 * CK));
    const uint8_t* klb = sh.u.att.kl;
    const uint8_t* vlb = sh.u.att.vl;
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
    if (c + 1 < nchunks) {
      if (!csync(a, sh, wv)) return false;
      lstore();
    }
    if (!csync(a, sh, wv)) return false;
  }
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
  return true;
}

// Merge of the key splits, spread over every compute wave of the grid: a
// unit is (sequence b, KV head g, query tile qt, d-tile dt) of 16 query rows
// x 16 head dimensions; the wave adds its splits' partials in split order
// (loads of MB splits in flight at once) and writes its piece of o (frag
// layout over nq * D) of layer l.
template <int D>
__device__ __forceinline__ void merge_unit(const PArgs& a, int l, int b, int g, int qt, int dt, int ns,
                                           const Wave& wv) {
  constexpr int MB = 8;
  const int lane = wv.lane, g4 = lane >> 4, col = lane & 15;
  const size_t wstride = (size_t)D * 16 + 32;
  const float* base = a.apart + ((size_t)l * a.B * a.nkv * a.max_splits + ((size_t)b * a.nkv + g) * a.max_splits) * 4 *
                                    wstride + qt * wstride;
  const int rep = a.nq / a.nkv;
  const int r = qt * 16 + col;
  const bool row_ok = r < a.K * rep;
  const int h = g * rep + (row_ok ? r / a.K : 0), i = row_ok ? r % a.K : 0;
  float M = -INFINITY, L = 0.f;
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += MB) {
    float ms[MB], ls[MB];
    f32x4 os[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const bool ok = s0 + j < ns;
      const float* pp = base + (size_t)(ok ? s0 + j : 0) * 4 * wstride;
      ms[j] = ok ? gload(pp + D * 16 + col) : -INFINITY;
      ls[j] = ok ? gload(pp + D * 16 + 16 + col) : 0.f;
      os[j] = ok ? gload((const f32x4*)(pp + (dt * 64 + lane) * 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      if (ms[j] == -INFINITY) continue;
      const float Mn = fmaxf(M, ms[j]);
      const float a0 = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
      const float a1 = exp2f(ms[j] - Mn);
      L = L * a0 + ls[j] * a1;
      o = o * a0 + os[j] * a1;
      M = Mn;
    }
  }
  if (!row_ok) return;
  const float inv = 1.f / L;
  const Frag of = frag_v(a.of, a.nq * D / 32, l);
  float v[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
  frag_store_wt<4>(of, b * a.K + i, h * D + dt * 16 + g4 * 4, v);
}

template <int D>
__device__ __forceinline__ bool phase_attention(const PArgs& a, PShared& sh, int l, const Wave& wv) {
  const int units = a.B * a.nkv * a.max_splits;
  for (int u = wv.w; u < units; u += (int)gridDim.x) {
    const int s = u % a.max_splits;
    const int g = (u / a.max_splits) % a.nkv;
    const int b = u / (a.max_splits * a.nkv);
    const int ns = n_splits(a, gload(&a.seqs[b].ctx_len));
    if (s >= ns) continue;
    if (!attention_unit<D>(a, sh, l, b, g, s, wv)) return false;
    mark(wv, 1);
  }
  return true;
}

// (a6) the merge of every (sequence, KV head)'s splits; wave (w, v) takes
// units v * grid + w, v * grid + w + CW * grid, ... so that every workgroup
// has work before any has two.
template <int D>
__device__ __forceinline__ void phase_merge(const PArgs& a, int l, const Wave& wv) {
  constexpr int NDT = D / 16;
  const int units = a.B * a.nkv * 4 * NDT;
  for (int u = wv.wave * (int)gridDim.x + wv.w; u < units; u += CW * (int)gridDim.x) {
    const int dt = u % NDT;
    const int qt = (u / NDT) % 4;
    const int g = (u / (NDT * 4)) % a.nkv;
    const int b = u / (NDT * 4 * a.nkv);
    if (qt * 16 >= a.K * (a.nq / a.nkv)) continue;   // query tile past the rows
    merge_unit<D>(a, l, b, g, qt, dt, n_splits(a, gload(&a.seqs[b].ctx_len)), wv);
  }
}

// (a7) output projection + residual: x_{2l+1} = x_{2l} + o W_o^T, with the
// MLP norm's inputs.
__device__ __forceinline__ bool phase_o(const PArgs& a, PShared& sh, RingRd& rr, int l, const Wave& wv) {
  const Work k = prod_work(a, sh, l, P_O, wv.w);
  const float* x_in = xs_v(a, 2 * l);
  float* x_out = xs_v(a, 2 * l + 1);
  const Frag xg = xg_v(a, 2 * l + 1);
  float* ssq = ssq_v(a, 2 * l + 1);
  const float* gain = gload(&a.layers[l].mlp_gain);
  return product<NTG_O, CHK_O>(
      a, sh, rr, k, frag_v(a.of, a.nq * a.d / 32, l), wv, nullptr,
      [&](int tile, f32x4 acc) { resnorm_tile(a, tile, acc, wv.lane, x_in, x_out, gain, xg, ssq); }, NoAfter{});
}

// (a8) RMSNorm + gate/up + SwiGLU -> act of layer l.
__device__ __forceinline__ bool phase_gu(const PArgs& a, PShared& sh, RingRd& rr, int l, const Wave& wv) {
  const Frag act = frag_v(a.act, a.nkb_i, l);
  const Work k = prod_work(a, sh, l, P_GU, wv.w);
  return product<NTG_GU, CHK_GU>(
      a, sh, rr, k, xg_v(a, 2 * l + 1), wv, ssq_v(a, 2 * l + 1),
      [&](int tile, f32x4 acc) {
        const int g4 = wv.lane >> 4, m = wv.lane & 15;
        if (m >= a.M) return;
        const float r = sh.rn[m];
        // tile rows 4*g4 + j: gate f, up f, gate f+1, up f+1 with f = tile*8 + 2*g4
        float v[2] = {silu_f(acc[0] * r) * (acc[1] * r), silu_f(acc[2] * r) * (acc[3] * r)};
        frag_store_wt<2>(act, m, tile * 8 + g4 * 2, v);
      },
      NoAfter{});
}

// (a8) down projection split over k; the last split of each tile adds the
// splits (in split order) into the residual: x_{2l+2} = x_{2l+1} + sum.
__device__ __forceinline__ bool phase_down(const PArgs& a, PShared& sh, RingRd& rr, int l, const Wave& wv) {
  const Work k = prod_work(a, sh, l, P_DN, wv.w);
  const int S = a.down_splits;
  const int T = a.H / 16;
  const int split = wv.w % S;
  float* part = a.dpart + (size_t)l * S * T * 256;
  const float* x_in = xs_v(a, 2 * l + 1);
  float* x_out = xs_v(a, 2 * l + 2);
  const Frag xg = xg_v(a, 2 * l + 2);
  float* ssq = ssq_v(a, 2 * l + 2);
  const float* gain = l + 1 < a.L ? gload(&a.layers[l + 1].attn_gain) : a.final_gain;
  return product<NTG_DN, CHK_DN>(
      a, sh, rr, k, frag_v(a.act, a.nkb_i, l), wv, nullptr,
      [&](int tile, f32x4 acc) { wtf4(part + (((size_t)split * T + tile) * 64 + wv.lane) * 4, acc); },
      [&](int t0, int nt) {
        drain();
        if (!csync(a, sh, wv)) return false;
        if (wv.tid < nt) {
          unsigned* cnt = a.dcnt + (size_t)l * T + t0 + wv.tid;
          const unsigned old = gatom_add(cnt, 1u);
          const bool last = (int)old + 1 == S;
          if (last) wt32(cnt, 0u);
          sh.u.red[0][0][wv.tid][0] = last ? 1.f : 0.f;   // flag of tile t0 + tid
        }
        if (!csync(a, sh, wv)) return false;
        for (int i = wv.wave; i < nt; i += CW) {
          if (sh.u.red[0][0][i][0] == 0.f) continue;
          const int tile = t0 + i;
          f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int s0 = 0; s0 < S; s0 += 8) {   // eight loads in flight, added in split order
            f32x4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
              v[j] = s0 + j < S ? gload((const f32x4*)(part + (((size_t)(s0 + j) * T + tile) * 64 + wv.lane) * 4))
                                : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 8; ++j) sum += v[j];
          }
          resnorm_tile(a, tile, sum, wv.lane, x_in, x_out, gain, xg, ssq);
        }
        return csync(a, sh, wv);
      });
}

// (a9) final norm + LM head + argmax; the last workgroup to finish writes
// the draft ids and the final-normed hidden rows.
__device__ __forceinline__ bool phase_lm(const PArgs& a, PShared& sh, RingRd& rr, const Wave& wv) {
  const int vL = 2 * a.L;
  if (wv.tid < 16) sh.kmax[wv.tid] = 0ull;
  if (!csync(a, sh, wv)) return false;
  const Work k = prod_work(a, sh, a.L, P_LM, wv.w);
  if (!product<NTG_LM, CHK_LM>(
          a, sh, rr, k, xg_v(a, vL), wv, ssq_v(a, vL),
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
                *(g_f32x4*)lp = f32x4{y[0], y[1], y[2], y[3]};
              } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  if (n + j < a.V) ((g_f32*)lp)[j] = y[j];
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
            __hip_atomic_fetch_max((l_u64*)(sh.kmax + m), best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          },
          NoAfter{}))
    return false;
  if (!csync(a, sh, wv)) return false;
  if (wv.tid < a.M && sh.kmax[wv.tid] != 0ull)
    __hip_atomic_fetch_max((g_u64*)(a.keys + wv.tid), sh.kmax[wv.tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  drain();
  if (!csync(a, sh, wv)) return false;
  if (wv.tid == 0) {
    const unsigned old = gatom_add(a.lmcnt, 1u);
    const int last = old + 1 == gridDim.x;
    if (last) wt32(a.lmcnt, 0u);
    sh.last = last;
  }
  if (!csync(a, sh, wv)) return false;
  if (!sh.last) return true;
  // (a9) draft ids and the final-normed hidden rows
  if (wv.tid < a.M) {
    const unsigned long long key = __hip_atomic_load((g_u64*)(a.keys + wv.tid), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *(g_u32*)(a.draft + wv.tid) = argmax_index(key);
  }
  if (a.hidden) {
    const float* x = xs_v(a, vL);
    bf16_t* hid = (bf16_t*)a.hidden;
    for (int idx = wv.tid; idx < a.M * a.H; idx += CT) {
      const int m = idx / a.H, c = idx - m * a.H;
      *(g_u16*)(hid + idx) = f2bf(gload(x + idx) * sh.rn[m] * gload(a.final_gain + c));
    }
  }
  return true;
}

template <int D>
__global__ __launch_bounds__(PT) void persist_draft_kernel(PArgs a) {
  __shared__ PShared sh;
  __shared__ __attribute__((aligned(1024))) u32x4 ring[CW][RING_SLOTS][WAVE];
  l_u32x4* ring_l = (l_u32x4*)&ring[0][0][0];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  if (tid == 0) {
    sh.bad = 0;
    sh.last = 0;
    sh.cbar = 0;
  }
  if (tid < CW) {
    sh.filled[tid] = 0;
    sh.consumed[tid] = 0;
  }
  if (tid == 0) sh.abort = 0;
  if (tid <= 4 * a.L) {
    const PLayer* L = a.layers + tid / 4;
    const int q = tid % 4;
    const Packed P = tid == 4 * a.L ? a.lm
                     : gload_packed(q == 0 ? &L->qkv : q == 1 ? &L->o : q == 2 ? &L->gu : &L->down);
    sh.prod[tid].w = P.w;
    sh.prod[tid].n_tiles = P.n_tiles;
    sh.prod[tid].nkb = P.nkb;
  }
  __syncthreads();   // the only barrier of all eight waves: the loaders never reach another
  if (wave >= CW) {
    build_passes(a, sh, (int)blockIdx.x, wave - CW, lane);
    lds_done();
    loader(a, sh, ring_l + (size_t)(wave - CW) * RING_SLOTS * WAVE, wave - CW, lane);
    return;
  }
  Wave wv;
  wv.w = blockIdx.x;
  wv.tid = tid;
  wv.wave = wave;
  wv.lane = lane;
  RingRd rr;
  rr.ring = ring_l + (size_t)wave * RING_SLOTS * WAVE;
  rr.filled = &sh.filled[wave];
  rr.consumed = &sh.consumed[wave];
  rr.idx = 0;
  rr.avail = 0;
  rr.slot = 0;
  // timeline: 8 slots per phase (0 start, 1-5 inside, 6 barrier arrival, 7 release)
  unsigned long long* trw = a.trace ? a.trace + (size_t)wv.w * a.trace_stride : nullptr;
  wv.tr = trw;
  mark(wv, 0);
  phase_embed(a, wv);
  unsigned step = 1;
  // barrier `step`, then the timeline moves on to the next phase
  auto barrier = [&]() -> bool {
    const bool ok = grid_barrier(a, sh, step, wv);
    ++step;
    if (trw) {
      wv.tr = trw + (size_t)(step - 1) * 8;
      mark(wv, 0);
    }
    return ok;
  };
  // a compute wave that leaves early stops this workgroup's loaders
  auto bail = [&]() { lds_st(&sh.abort, 1u); };
  if (!barrier()) return bail();
  for (int l = 0; l < a.L; ++l) {
    if (!phase_qkv<D>(a, sh, rr, l, wv) || !barrier()) return bail();
    if (!phase_attention<D>(a, sh, l, wv) || !barrier()) return bail();
    phase_merge<D>(a, l, wv);
    if (!barrier()) return bail();
    if (!phase_o(a, sh, rr, l, wv) || !barrier()) return bail();
    if (!phase_gu(a, sh, rr, l, wv) || !barrier()) return bail();
    if (!phase_down(a, sh, rr, l, wv) || !barrier()) return bail();
  }
  if (!phase_lm(a, sh, rr, wv)) return bail();
  mark(wv, 6);
}

}  // namespace

unsigned persist_steps(int L) { return 1u + 6u * (unsigned)L; }

// An upper bound of the passes one loader streams (every workgroup's share
// of a product rounded up to whole tiles, then to passes of NTG tiles).
bool persist_passes_fit(int nwg, int down_splits, int L, int qkv_tiles, int o_tiles, int gu_tiles, int down_tiles,
                        int lm_tiles) {
  auto per = [](int tiles, int parts, int ntg) {
    const int t = (tiles + parts - 1) / parts;
    return (t + ntg - 1) / ntg;
  };
  const long n = (long)L * (per(qkv_tiles, nwg, NTG_QKV) + per(o_tiles, nwg, NTG_O) + per(gu_tiles, nwg, NTG_GU) +
                            per(down_tiles, nwg / down_splits, NTG_DN)) +
                 per(lm_tiles, nwg, NTG_LM);
  return n <= MAX_PASSES;
}

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
