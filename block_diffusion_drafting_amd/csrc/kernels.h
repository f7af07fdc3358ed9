// Internal launch interface between the C-ABI host code and the HIP kernels.
//
// Activation layout.  Every activation matrix X[M][Kd] that feeds a weight
// product is stored in MFMA fragment order ("frag layout"): m-tile mt,
// k-block kb, lane l hold 16 bytes = KPL consecutive reduction elements of
// row mt*16 + l%16 starting at kb*KB + (l/16)*KPL.  A wave loads one
// fragment with a single coalesced 1 KiB read.  For bf16 models a matrix is
// a pair of such arrays: `hi` (values rounded to bf16) and `lo` (the
// rounded remainder); products that use both see about 16 mantissa bits of
// the activation.  For fp32 models only `hi` (fp32 values) exists.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

#define DFLASH_ROWMAP_MAX 256

namespace dflash {

enum Epi : int {
  EPI_QKV = 0,     // norm scale, RoPE on q/k, scatter q / block k / block v^T
  EPI_SWIGLU = 1,  // norm scale, silu(gate) * up -> act (frag layout)
  EPI_PART = 2,    // write split-K partial tiles (combined by a later kernel)
  EPI_ARGMAX = 3,  // norm scale, optional logits, per-row argmax keys
  EPI_FC = 4,      // full context projection rows -> context buffer + staging
  EPI_KV = 5,      // K (RoPE) / V^T rows -> every layer's cache
  EPI_RESNORM = 6, // full-K product added into the residual x; the next
                   // RMSNorm's inputs (x * gain -> frag, sums of squares per
                   // 16 columns) written alongside
  EPI_PARTRES = 7, // split-K partial tiles; the last split of a tile group
                   // to finish adds the group's partials in split order and
                   // runs the EPI_RESNORM epilogue on the sums
};
constexpr bool is_part(int epi) { return epi == EPI_PART || epi == EPI_PARTRES; }
constexpr int MAX_SPLITS = 8;   // k-splits of a split product (plan_gemm)

// A weight matrix repacked into 16-row x 64-byte blocks (see common.h):
// tile t (rows 16t..16t+15) holds nkb consecutive 1 KiB blocks.
struct Packed {
  const uint8_t* w = nullptr;
  int32_t n_rows = 0;   // logical rows (before padding to 16)
  int32_t n_tiles = 0;
  int32_t kd = 0;       // logical reduction length
  int32_t nkb = 0;      // 64-byte blocks per row (padded)
};

// An activation matrix in frag layout.
struct Frag {
  u32x4* hi = nullptr;
  u32x4* lo = nullptr;   // bf16 models only
  int32_t mtiles = 0;    // allocated m-tiles
  int32_t nkb = 0;       // k-blocks per m-tile
};

struct EpiArgs {
  int32_t M;                // activation rows of the call
  // RMSNorm scale applied after the product:
  //   r[m] = rsqrt(sum_g ssq[g*M + m] / norm_dim + eps)
  const float* ssq;
  int32_t ssq_groups;
  int32_t norm_dim;
  float eps;
  // geometry
  int32_t Kblk, Kpad, nq, nkv, d, H, I, V, L;
  const DevSeq* seqs;
  const double* inv_freq;   // [d/2] theta^(-2m/d)
  // outputs
  void* q;                  // [M][nq*d]          attention type
  void* bk;                 // [B][nkv][Kpad][d]  attention type
  void* bvt;                // [B][nkv][d][Kpad]  attention type
  Frag act;                 // SwiGLU output, frag layout over I
  float* part;              // split-K partials [nsplit][n_tiles][mtiles][64] f32x4
  int32_t part_ntiles;
  int32_t part_mtiles;
  float* logits;            // [M][V] or null
  unsigned long long* keys; // [M] argmax keys
  Frag cbuf;                // context features, frag layout over hidden
  const RowMap* rowmap;     // [M] (EPI_FC, EPI_KV) or [n_ctx] (fused QKV)
  // fused step: context rows appended to the QKV activations from m-tile
  // ctx_mt0 on; their K/V go to layer `layer` of the caches
  int32_t ctx_mt0, n_ctx, layer;
  // block verification (EPI_QKV): the block rows' K/V go to layer `layer`
  // of the caches at slot = position = ctx_len + i instead of bk / bvt
  int32_t kv_cache;
  // EPI_RESNORM: residual x [M][H] (fp32), gain of the next norm, its frag
  // output and sums of squares [H/16][M]
  float* xres;
  const float* gain;
  Frag xout;
  float* ssq_out;
  // EPI_PARTRES: arrival counters, one per (tile group, m-group) of the
  // launch, zero before it and left zero by it
  unsigned* fix_cnt;
};

struct GemmArgs {
  Packed W;
  // activations: frag layout, or row-major model type (context projection)
  Frag X;
  const void* Xrow;
  int32_t ldx;
  int32_t M;
  int32_t kbu;            // k-blocks per unit (split)
  int32_t nsplit;
  int32_t n_groups;       // groups of NTG tiles
  int32_t m_groups;       // groups of MTT m-tiles
};

struct GemmPlan {
  int mtt;     // m-tiles per group (1, 2, 4, 8)
  int ntg;     // tiles per group (wide_kernel: per wave slot, two slots per group)
  int kbu, nsplit, n_groups, m_groups;
  bool split;  // use hi + lo fragments
  bool rowmajor;
  bool fixed;  // fixed tile groups (the context path at prefill sizes)
  bool wide;   // wide_kernel (128-row m-groups, activations and weights staged in LDS)
  size_t part_floats;
};

GemmPlan plan_gemm(int epi, const Packed& W, int M, bool split_ok, bool rowmajor);

// head_kernel: HEAD_WAVES waves per workgroup, each over up to HEAD_NTW
// weight tiles with the whole reduction, sharing the activations via LDS.
constexpr int HEAD_WAVES = 8;
constexpr int HEAD_NTW = 3;

// Tile groups per m-group of head_kernel: about two rounds of 256
// workgroups over all m-groups, at most HEAD_WAVES * HEAD_NTW tiles each.
inline int head_groups(int n_tiles, int m_groups) {
  const int cap = HEAD_WAVES * HEAD_NTW;
  const int want = (512 + m_groups - 1) / m_groups;
  int G = n_tiles < want ? n_tiles : want;
  if ((n_tiles + G - 1) / G > cap) G = (n_tiles + cap - 1) / cap;
  return G;
}

// Products of a bf16 model that run head_kernel instead of gemm_kernel:
// the LM head over m-groups of 8 or 4 m-tiles (hi part of the
// activations), and gate/up over m-groups of 8 m-tiles (hi/lo pair) when
// there are enough of them to give each wave two tiles or more.  With fewer tiles per wave its
// waves keep too few loads in flight (measured on MI355X: at two m-groups
// of the Qwen3-4B gate/up it takes 1.8x the time of gemm_kernel, at eight
// m-groups 0.68x).
inline bool uses_head_kernel(int epi, const GemmPlan& p, int n_tiles, int elem_bytes) {
  if (elem_bytes != 2 || p.rowmajor || p.fixed) return false;
  if (epi == EPI_ARGMAX) return !p.split && (p.mtt == 8 || p.mtt == 4);
  if (epi != EPI_SWIGLU || !p.split || p.mtt != 8) return false;
  const int G = head_groups(n_tiles, p.m_groups);
  return (n_tiles + G - 1) / G >= 2 * HEAD_WAVES;
}

template <typename T>
hipError_t launch_gemm(int epi, const GemmPlan& p, const GemmArgs& g, const EpiArgs& e,
                       hipStream_t s);
// One epilogue's compiled variants (defined in gemm_kernel.h).
template <typename T, int EPI>
hipError_t launch_gemm_epi(const GemmPlan& p, GemmArgs g, const EpiArgs& e, hipStream_t s);

// L2 warm-up of a later product's weights by extra workgroups appended to
// a latency-bound kernel's grid.  Workgroups are dealt to the eight XCDs
// round robin by block index, so warm-up workgroup k (block first + k,
// first a multiple of 8) sits on the XCD of the product's workgroup k and
// loads, into that XCD's L2, the first `frags` weight fragments each of
// its waves will read (k-block major, then tile; data discarded).
struct Warm {
  const uint8_t* w;            // packed weights; null = no warm-up
  int32_t nkb, n_tiles;
  int32_t n_groups, nsplit, kbu;
  int32_t waves;               // waves per product workgroup
  int32_t frags;               // fragments per product wave
  int32_t consumers;           // product workgroups to warm for (m-group 0)
  int32_t first;               // block index of the first warm-up workgroup
};

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with only the vector-memory count set (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14; expcnt and lgkmcnt at their maxima = no wait).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte-per-lane direct load to LDS (global_load_lds_dwordx4): lane
// l's 16 bytes at base + off go to LDS address lds + 16 l; lds must be the
// same in every lane.  A load decrements the vector-memory count once its
// bytes are in LDS, so an explicit vmcnt wait taken before a barrier
// (lds_barrier, which leaves later stages' loads in flight) makes a stage
// visible to every wave.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((const void*)(base + off), (lds_void_t*)lds, 16, 0, 0);
}

// Workgroup barrier that leaves vector-memory loads in flight.
// __syncthreads() also fences at workgroup scope, and its release completes
// every outstanding vector-memory load, the prefetches of later stages
// included, which shortens a multi-stage pipeline to one stage in flight
// across each barrier.  The staged pipelines only need their LDS traffic
// ordered: this wave's LDS reads and writes are completed (lgkmcnt(0)), the
// stage to be read after the barrier is covered by the explicit vmcnt wait
// (direct loads) or the compiler's wait before the LDS store (register
// staging) that precede the call, and the compiler-only fences keep memory
// accesses on their side of the barrier.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Warm-up workgroup k with nw waves (this is wave `wave`): product
// workgroup k's waves cw = wave, wave + nw, ... ; `slot` is this wave's own
// 1 KiB of LDS.  Waits for its loads before returning.
__device__ __forceinline__ void warm_consumer(const Warm& m, int k, int nw, int wave, int lane, lds_void_t* slot) {
  if (k >= m.consumers) return;
  const int s = k % m.nsplit;
  const int ng = (k / m.nsplit) % m.n_groups;
  const int tile0 = (int)((long)ng * m.n_tiles / m.n_groups);
  const int nt = (int)((long)(ng + 1) * m.n_tiles / m.n_groups) - tile0;
  const int kbA = s * m.kbu, kbB = min(m.nkb, kbA + m.kbu);
  const int per = (kbB - kbA + m.waves - 1) / m.waves;
  const uint8_t* base = m.w + (size_t)lane * FRAG_BYTES;
  for (int cw = wave; cw < m.waves; cw += nw) {
    const int k0 = kbA + cw * per, k1 = min(kbB, k0 + per);
    int cnt = 0;
    for (int kb = k0; kb < k1 && cnt < m.frags; ++kb)
      for (int t = 0; t < nt && cnt < m.frags; ++t, ++cnt)
        __builtin_amdgcn_global_load_lds((const void*)(base + ((size_t)(tile0 + t) * m.nkb + kb) * BLOCK_BYTES), slot,
                                         16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

struct AttnArgs {
  Warm warm;              // weights of the output projection that follows
  const void* q;
  const void* bk;
  const void* bvt;
  const DevSeq* seqs;
  float* part;            // [B][nkv][qgroups][max_splits][4 waves][O / l, m, l] (attn_part_floats)
  int32_t B, K, Kpad, nq, nkv, d, layer;
  int32_t qgroups, chunk, max_splits;
  float scale_log2;
  // block verification: every key comes from the cache (the block's were
  // stored there by the QKV product), block row i sees keys 0..ctx_len+i
  int32_t causal;
  // the context K/V read per block is too large to stay cached between
  // blocks: the register-staged kernel loads it nontemporally
  int32_t stream;
};
// Splits of one (sequence, KV head): context keys, then block keys (or, in
// the causal form, ctx_len + K cache keys).
__host__ __device__ inline void attn_split_counts(const AttnArgs& a, int ctx_len, int& n_cs, int& n_s) {
  if (a.causal) {
    n_cs = (ctx_len + a.K + a.chunk - 1) / a.chunk;
    n_s = n_cs;
  } else {
    n_cs = (ctx_len + a.chunk - 1) / a.chunk;
    n_s = n_cs + (a.K + a.chunk - 1) / a.chunk;
  }
}
// Query groups (64 query rows each) per attention workgroup: one (four
// waves), two (eight waves), or, for 2-byte operands and at least four
// groups, four (eight waves of two query tiles each).
inline int attn_groups_per_wg(int elem_bytes, int qgroups) {
  return qgroups >= 4 && elem_bytes == 2 ? 4 : qgroups > 1 ? 2 : 1;
}
// Bytes per element of O / l in the split partials: 2 (fp16) from the
// four-query-group kernel (2-byte operands, head_dim 128), else 4 (fp32).
inline int attn_part_o_bytes(int elem_bytes, int qgroups, int d) {
  return elem_bytes == 2 && d == 128 && attn_groups_per_wg(elem_bytes, qgroups) == 4 ? 2 : 4;
}
size_t attn_part_floats(int B, int nkv, int qgroups, int max_splits, int d, int part_o_bytes);
template <typename T>
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// Merge attention splits in index order; write o (frag layout over nq*d).
template <typename CT, typename T>
hipError_t launch_attn_combine(const AttnArgs& a, Frag o, hipStream_t s);

// x[m] = E[id], xg = x * gain -> frag, ssq per 64-column group; keys = 0.
template <typename T>
hipError_t launch_embed(const int32_t* ids, const void* embed, const float* gain, int M, int H,
                        int V, float* x, Frag xg, float* ssq, unsigned long long* keys,
                        hipStream_t s);
// Rows of one context append: rows [start[b], start[b+1]) belong to
// sequence b and go to slots ctx0[b] + (row - start[b]) (host values).
struct RowInfo {
  int32_t start[DFLASH_ROWMAP_MAX + 1];
  int32_t ctx0[DFLASH_ROWMAP_MAX];
};
// c = sum of split-K partials -> context buffer rows + staging frag (rows
// from row0 on); also writes the row map and advances the device context
// lengths.
template <typename T>
hipError_t launch_fc_finalize(const float* part, int nsplit, int mtiles, int M, int H, const RowInfo& ri, int B,
                              const int32_t* positions, RowMap* rowmap, DevSeq* seqs, Frag cbuf,
                              int row0, hipStream_t s);
// launch_fc_finalize (without positions) and launch_embed as one launch
// (the fused step: the appended context rows and the block rows of the
// first QKV product's activations are independent)
template <typename T>
hipError_t launch_fc_finalize_embed(const float* part, int nsplit, int mtiles, int M, int H, const RowInfo& ri,
                                    int B, RowMap* rowmap, DevSeq* seqs, Frag cbuf, int row0,
                                    const int32_t* ids, const void* embed, const float* gain, int Mb, int V,
                                    float* x, Frag xg, float* ssq, unsigned long long* keys, hipStream_t s);
// x += sum of split-K partials (fixed order); xg = x * gain -> frag; ssq
// per 64-column group.
template <typename T>
hipError_t launch_resid_norm(const float* part, int nsplit, int mtiles, int M, int H, float* x,
                             const float* gain, Frag xg, float* ssq, hipStream_t s);
// out[m][tap*H + h] = x[m][h] in the model type (a tapped hidden state;
// out rows are n_taps*H long).
template <typename T>
hipError_t launch_tap(const float* x, int M, int H, int tap, int n_taps, void* out, hipStream_t s);
// draft ids from argmax keys; optional final-normed hidden rows.
template <typename T>
hipError_t launch_finalize(const unsigned long long* keys, int M, int32_t* draft, const float* x,
                           const float* ssq, int groups, const float* gain, int H, float eps,
                           void* hidden, hipStream_t s);
hipError_t launch_accept(const int32_t* draft, const int32_t* target, int B, int K,
                         int32_t* out, hipStream_t s);
// Loss-decay weighted cross-entropy (loss.hip); wsum is one device double.
hipError_t launch_decay_ce(const void* logits, int dtype, const int32_t* targets, int R, int V, int block,
                           double gamma, float* loss, float* ce, void* grad, double* wsum, hipStream_t s);
int decay_ce_resident_max(int elem_bytes);
template <typename T>
hipError_t launch_pack(const uint64_t* row_src, int n_rows_padded, int kd, int nkb, uint8_t* dst,
                       hipStream_t s);
template <typename T>
hipError_t launch_to_f32(const void* src, float* dst, int n, hipStream_t s);
hipError_t launch_rowmap(const RowInfo& ri, int B, int total, const int32_t* positions, DevSeq* seqs,
                         RowMap* out, hipStream_t s);
hipError_t launch_set_seq(DevSeq* seqs, int b, DevSeq v, hipStream_t s);
template <typename T>
hipError_t launch_grow_copy(DevSeq oldv, DevSeq newv, int L, int nkv, int d, int H,
                            hipStream_t s);
hipError_t launch_fill_u32(unsigned* p, size_t n, unsigned v, hipStream_t s);

// ---------------------------------------------------------------------------
// persistent single-launch draft block (bf16 drafters, batch * K <= 16)
// ---------------------------------------------------------------------------
constexpr int PERSIST_MAX_LAYERS = 16;   // layers of a drafter the single launch takes

struct PLayer {
  Packed qkv, o, gu, down;
  const float* attn_gain;
  const float* mlp_gain;
};

struct PArgs {
  const PLayer* layers;      // device [L]
  Packed lm;
  const bf16_t* embed;       // [V][H]
  const float* final_gain;
  const double* inv_freq;    // [d/2]
  const DevSeq* seqs;
  const int32_t* ids;        // [M]
  int32_t* draft;            // [M]
  float* logits;             // [M][V] or null
  void* hidden;              // [M][H] bf16 or null
  int32_t B, K, M, H, nq, nkv, d, I, V, L, Kpad, nkb_i;
  float eps, scale_log2;
  int32_t chunk, max_splits; // attention: keys per split, splits per (sequence, head)
  int32_t down_splits;       // k-splits of the down projection (divides the grid)
  // per-launch buffers, one copy per layer / phase (16 activation rows)
  float* xs;                 // [2L+1][16][H]          residual versions
  u32x4* xg;                 // [2L+1][hi, lo][H/32][64] normed-input frags
  float* ssq;                // [2L+1][H/16][16]       sums of squares
  f16_t* q;                  // [L][16][nq*d]
  f16_t* bk;                 // [L][B][nkv][Kpad][d]
  f16_t* bvt;                // [L][B][nkv][d][Kpad]
  float* apart;              // [L][B*nkv*max_splits][4][d*16 + 32]
  u32x4* of;                 // [L][hi, lo][nq*d/32][64]
  u32x4* act;                // [L][hi, lo][nkb_i][64]
  float* dpart;              // [L][down_splits][H/16][64][4]
  unsigned long long* keys;  // [16]
  unsigned* acnt;            // [L][B*nkv]  split counters (self-resetting)
  unsigned* dcnt;            // [L][H/16]   down split counters (self-resetting)
  unsigned* lmcnt;           // [1]
  unsigned* flags;           // [grid]      barrier flags (monotone)
  unsigned* err;             // nonzero: a wait expired
  const uint8_t* zero_frag;  // one fragment (1 KiB) of zeros, never written
  unsigned base;             // flag value before this launch's first step
  // optional timeline (null = off): per workgroup, 8 slots per phase
  // (embed, 5 per layer, LM head) of the constant 100 MHz clock: [0] start,
  // [1]-[5] marks inside the phase, [6] arrival at the barrier that ends it
  // (the LM head: end of work), [7] that barrier's release
  unsigned long long* trace;
  int32_t trace_stride;
};
// barrier steps of one launch with L layers
unsigned persist_steps(int L);
bool persist_passes_fit(int nwg, int down_splits, int L, int qkv_tiles, int o_tiles, int gu_tiles, int down_tiles,
                        int lm_tiles);
hipError_t persist_occupancy(int d, int* blocks_per_cu);
hipError_t launch_persist_draft(const PArgs& a, int nwg, hipStream_t s);

// Frag-layout slot (16-byte unit index) of element (m, k) and its position
// `e` inside the fragment.
template <typename T>
__device__ __forceinline__ size_t frag_slot(const Frag& f, int m, int k, int& e) {
  const int kb = k / Elem<T>::KB;
  const int r = k - kb * Elem<T>::KB;
  const int lane = (r / Elem<T>::KPL) * 16 + (m & 15);
  e = r % Elem<T>::KPL;
  return ((size_t)(m >> 4) * f.nkb + kb) * WAVE + lane;
}

// Store N consecutive fp32 values of row m from column k (k % N == 0, N
// divides KPL) into a frag matrix: hi = round(v), lo = round(v - hi).
template <typename T, int N>
__device__ __forceinline__ void frag_store(const Frag& f, int m, int k, const float* v) {
  int e;
  const size_t slot = frag_slot<T>(f, m, k, e);
  if constexpr (sizeof(T) == 2) {
    bf16_t h[N], l[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      h[i] = f2bf(v[i]);
      l[i] = f2bf(v[i] - bf2f(h[i]));
    }
    auto ph = gp((bf16_t*)(f.hi + slot) + e);
    auto pl = gp((bf16_t*)(f.lo + slot) + e);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      ph[i] = h[i];
      pl[i] = l[i];
    }
  } else {
    auto ph = gp((float*)(f.hi + slot) + e);
#pragma unroll
    for (int i = 0; i < N; ++i) ph[i] = v[i];
  }
}

}  // namespace dflash
