// Weight-streaming products of the draft block (kernel and launch templates), Y^T = W X^T, with W
// repacked into MFMA fragments and the fused epilogue of each projection.
//
// At K*batch <= 128 activation rows every weight byte feeds at most 128
// multiply-adds, so these products are bound by streaming W from HBM.  The
// kernel is built so that a launch is one uninterrupted stream:
//   * a workgroup owns NTG 16-row tiles of W and a range of k-blocks; its
//     four waves split that range, each loading CHK weight fragments per
//     tile (1 KiB coalesced reads) and the matching activation fragments
//     (frag layout, from L2), then issuing the MFMAs;
//   * the four partial sums are added through LDS in wave order and the
//     epilogue runs on complete sums inside the workgroup;
//   * nothing in a launch waits for another workgroup: products split over
//     k across workgroups write their partial tiles, and either the next
//     kernel (EPI_PART) or the last split of each tile group to finish
//     (EPI_PARTRES, counted by an agent-scope atomic) adds them in split
//     order.  Results are therefore deterministic, and no device-scope
//     fence (an L2 writeback + invalidate on this GPU) is ever executed.
// Rows of the activation matrix beyond M are computed but never stored.
#pragma once

#include "kernels.h"

namespace dflash {

// ---------------------------------------------------------------------------
// epilogue helpers
// ---------------------------------------------------------------------------
constexpr bool needs_norm(int epi) { return epi == EPI_QKV || epi == EPI_SWIGLU || epi == EPI_ARGMAX; }

__device__ __forceinline__ void rope_pair(float x1, float x2, int pos, double inv, float& o1,
                                          float& o2) {
  double sn, cs;
  sincos((double)pos * inv, &sn, &cs);
  const float c = (float)cs, s = (float)sn;
  o1 = x1 * c - x2 * s;
  o2 = x2 * c + x1 * s;
}

__device__ __forceinline__ float silu(float t) { return t / (1.0f + expf(-t)); }

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m);
  hi = __shfl_xor(hi, m);
  return ((unsigned long long)hi << 32) | lo;
}

// Device-scope (write-through) store and load of four floats: data passed
// between workgroups of one launch, which may sit on different XCDs (each
// with its own L2).
__device__ __forceinline__ void store_agent_f32x4(float* p, f32x4 v) {
  typedef __attribute__((address_space(1))) unsigned long long g_u64;
  __hip_atomic_store((g_u64*)p, (unsigned long long)__float_as_uint(v[0]) | ((unsigned long long)__float_as_uint(v[1]) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store((g_u64*)(p + 2), (unsigned long long)__float_as_uint(v[2]) | ((unsigned long long)__float_as_uint(v[3]) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 load_agent_f32x4(const float* p) {
  typedef __attribute__((address_space(1))) unsigned long long g_u64;
  const unsigned long long a = __hip_atomic_load((g_u64*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long b = __hip_atomic_load((g_u64*)(p + 2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x4{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)), __uint_as_float((uint32_t)b),
               __uint_as_float((uint32_t)(b >> 32))};
}

// Context K/V rows: nn = offset inside one layer's [K rows | V rows] block
// (K rows in RoPE pair order), row map rm of the context row, values acc.
template <typename CT>
__device__ __forceinline__ void store_ctx_kv(const EpiArgs& e, int l, int nn, const RowMap& rm, f32x4 acc,
                                             int g4) {
  const int kvd = e.nkv * e.d;
  const DevSeq sq = e.seqs[rm.b];
  if (nn < kvd) {
    const int head = nn / e.d, th = (nn % e.d) / 16;
    const int p0 = th * 8 + g4 * 2;
    float a1, a2, b1, b2;
    rope_pair(acc[0], acc[1], rm.pos, e.inv_freq[p0], a1, a2);
    rope_pair(acc[2], acc[3], rm.pos, e.inv_freq[p0 + 1], b1, b2);
    auto dst = gp((CT*)sq.k + (((size_t)l * e.nkv + head) * sq.phys + rm.slot) * e.d);
    const int h2 = e.d / 2;
    dst[p0] = Elem<CT>::from_f(a1);
    dst[p0 + 1] = Elem<CT>::from_f(b1);
    dst[p0 + h2] = Elem<CT>::from_f(a2);
    dst[p0 + 1 + h2] = Elem<CT>::from_f(b2);
  } else {
    const int v = nn - kvd;
    const int head = v / e.d, f0 = v % e.d + g4 * 4;
    auto dst = gp((CT*)sq.vt + (((size_t)l * e.nkv + head) * e.d + f0) * sq.phys + rm.slot);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[(size_t)j * sq.phys] = Elem<CT>::from_f(acc[j]);
  }
}

// Residual epilogue of one output tile (EPI_RESNORM, EPI_PARTRES): lane
// (g4, r) owns x[m][n..n+3] with m = mt*16 + r, n = tile*16 + 4*g4.  Its
// inputs (the residual quad and the next norm's gain) are loaded apart, so
// that they can be in flight with the loads of the sums.
struct ResIn {
  f32x4 x, gn;
};
__device__ __forceinline__ ResIn resnorm_load(const EpiArgs& e, int tile, int mt, int lane) {
  const int m = mt * 16 + (lane & 15), n = tile * 16 + (lane >> 4) * 4;
  ResIn r{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  if (m < e.M) {
    r.x = *gp((const f32x4*)(e.xres + (size_t)m * e.H + n));
    r.gn = gld((const f32x4*)(e.gain + n));
  }
  return r;
}
// x += y; x * gain -> frag; sum of squares of the tile's 16 columns of row
// m (all lanes take part in the reduction)
template <typename T>
__device__ __forceinline__ void resnorm_tile(const EpiArgs& e, int tile, int mt, f32x4 acc, int lane,
                                             const ResIn& in) {
  const int g4 = lane >> 4;
  const int m = mt * 16 + (lane & 15), n = tile * 16 + g4 * 4;
  const bool ok = m < e.M;
  float ss = 0.f;
  if (ok) {
    const f32x4 x = in.x + acc;
    *gp((f32x4*)(e.xres + (size_t)m * e.H + n)) = x;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ss = fmaf(x[j], x[j], ss);
      v[j] = x[j] * in.gn[j];
    }
    frag_store<T, 4>(e.xout, m, n, v);
  }
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  if (ok && g4 == 0) e.ssq_out[(size_t)tile * e.M + m] = ss;
}

// One complete 16x16 output tile: acc[j] is output row n = tile*16 +
// 4*(lane/16) + j of activation row m = mt*16 + lane%16.  Runs on one wave.
template <typename T, int EPI>
__device__ void epilogue_tile(const EpiArgs& e, int s, int tile, int mt, f32x4 acc, int lane,
                              float r, unsigned long long* kmax) {
  using CT = typename CacheOf<T>::type;
  const int g4 = lane >> 4;
  const int m = mt * 16 + (lane & 15);
  if constexpr (EPI == EPI_RESNORM) {
    resnorm_tile<T>(e, tile, mt, acc, lane, resnorm_load(e, tile, mt, lane));
    return;
  }
  if constexpr (EPI == EPI_PART) {
    if (mt >= e.part_mtiles) return;   // m-tile past the rows of the call: no slot
    *gp((f32x4*)(e.part + ((((size_t)s * e.part_ntiles + tile) * e.part_mtiles + mt) * 64 + lane) * 4)) = acc;
    return;
  }
  if constexpr (EPI == EPI_PARTRES) {
    // write-through: another XCD's workgroup adds the partials in this launch
    if (mt >= e.part_mtiles) return;
    float* p = e.part + ((((size_t)s * e.part_ntiles + tile) * e.part_mtiles + mt) * 64 + lane) * 4;
    store_agent_f32x4(p, acc);
    return;
  }
  if constexpr (EPI == EPI_QKV) {
    // context rows appended below the block (fused step): their K and V
    // (no norm, no gain) go to this layer's caches; their Q is not needed
    if (e.n_ctx > 0 && mt >= e.ctx_mt0) {
      const int j = (mt - e.ctx_mt0) * 16 + (lane & 15);
      const int qd = e.nq * e.d;
      const int n = tile * 16;
      if (j < e.n_ctx && n >= qd) store_ctx_kv<CT>(e, e.layer, n - qd, e.rowmap[j], acc, g4);
      return;
    }
  }
  if (m >= e.M) return;
  if constexpr (EPI == EPI_QKV) {
    const int qd = e.nq * e.d, kvd = e.nkv * e.d;
    const int n = tile * 16;
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = acc[j] * r;
    const int b = m / e.Kblk, i = m - b * e.Kblk;
    const int pos = e.seqs[b].ctx_len + i;
    if (e.kv_cache && n >= qd) {
      // verified block: K/V straight into the cache at slot = position
      const RowMap rm{b, pos, pos, 0};
      store_ctx_kv<CT>(e, e.layer, n - qd, rm, f32x4{y[0], y[1], y[2], y[3]}, g4);
      return;
    }
    if (n < qd + kvd) {
      const bool isq = n < qd;
      const int nn = isq ? n : n - qd;
      const int head = nn / e.d, th = (nn % e.d) / 16;
      const int p0 = th * 8 + g4 * 2;
      float a1, a2, b1, b2;
      rope_pair(y[0], y[1], pos, e.inv_freq[p0], a1, a2);
      rope_pair(y[2], y[3], pos, e.inv_freq[p0 + 1], b1, b2);
      auto dst = gp(isq ? (CT*)e.q + (size_t)m * qd + head * e.d
                        : (CT*)e.bk + (((size_t)b * e.nkv + head) * e.Kpad + i) * e.d);
      const int h2 = e.d / 2;
      dst[p0] = Elem<CT>::from_f(a1);
      dst[p0 + 1] = Elem<CT>::from_f(b1);
      dst[p0 + h2] = Elem<CT>::from_f(a2);
      dst[p0 + 1 + h2] = Elem<CT>::from_f(b2);
    } else {
      const int nn = n - qd - kvd;
      const int head = nn / e.d, f0 = nn % e.d + g4 * 4;
      auto dst = gp((CT*)e.bvt + (((size_t)b * e.nkv + head) * e.d + f0) * e.Kpad + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[(size_t)j * e.Kpad] = Elem<CT>::from_f(y[j]);
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // tile rows 4*g4 + j: gate f, up f, gate f+1, up f+1 with f = tile*8 + 2*g4
    float v[2] = {silu(acc[0] * r) * (acc[1] * r), silu(acc[2] * r) * (acc[3] * r)};
    frag_store<T, 2>(e.act, m, tile * 8 + g4 * 2, v);
  } else if constexpr (EPI == EPI_ARGMAX) {
    const int n = tile * 16 + g4 * 4;
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = acc[j] * r;
    if (e.logits) {
      auto lp = gp(e.logits + (size_t)m * e.V + n);
      if (n + 4 <= e.V && (e.V & 3) == 0) {
        *gp((f32x4*)(e.logits + (size_t)m * e.V + n)) = f32x4{y[0], y[1], y[2], y[3]};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n + j < e.V) lp[j] = y[j];
      }
    }
    unsigned long long best = 0ull;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (n + j < e.V) {
        const unsigned long long k = argmax_key(y[j], (uint32_t)(n + j));
        best = k > best ? k : best;
      }
    }
    atomicMax(kmax + (lane & 15), best);   // LDS, per column of this m-tile
  } else if constexpr (EPI == EPI_FC) {
    const int n = tile * 16 + g4 * 4;
    const RowMap rm = e.rowmap[m];
    *gp((f32x4*)((float*)e.seqs[rm.b].ctxbuf + (size_t)rm.slot * e.H + n)) = acc;
    float v[4] = {acc[0], acc[1], acc[2], acc[3]};
    frag_store<T, 4>(e.cbuf, m, n, v);
  } else if constexpr (EPI == EPI_KV) {
    const int n = tile * 16;
    const int l = n / (2 * e.nkv * e.d);
    store_ctx_kv<CT>(e, l, n - l * 2 * e.nkv * e.d, e.rowmap[m], acc, g4);
  }
}

// ---------------------------------------------------------------------------
// the product kernel
// ---------------------------------------------------------------------------
// Activation fragment(s) of m-tile mt, k-block kb; zero when !ok or outside
// the matrix.  `ok` and the m-tile test are wave-uniform (scalar branches);
// the row test of the row-major form is per lane and uses a select.
template <typename T, bool ROW, bool SPLIT>
__device__ __forceinline__ void load_x(const GemmArgs& g, int mt, int kb, bool ok, int lane, u32x4& hi,
                                       u32x4& lo) {
  using E = Elem<T>;
  hi = u32x4{0u, 0u, 0u, 0u};
  lo = u32x4{0u, 0u, 0u, 0u};
  if (!ok) return;
  if constexpr (ROW) {
    const int row0 = mt * 16 + (lane & 15);
    const int row = min(row0, g.M - 1);
    const int k = kb * E::KB + (lane >> 4) * E::KPL;
    const u32x4 v = gld16((const T*)g.Xrow + (size_t)row * g.ldx + k);
    const uint32_t keep = row0 < g.M ? 0xFFFFFFFFu : 0u;
    hi = v & keep;
  } else {
    if (mt < g.X.mtiles) {
      const size_t slot = ((size_t)mt * g.X.nkb + kb) * WAVE + lane;
      hi = g.X.hi[slot];
      if constexpr (SPLIT) lo = g.X.lo[slot];
    }
  }
}

// Default k-blocks per load batch: up to 16 weight and 16 activation
// fragments per wave in flight.
template <int MTT, int NTG, bool SPLIT>
struct DefaultChk {
  static constexpr int XF = MTT * (SPLIT ? 2 : 1);
  static constexpr int C0 = (16 / NTG) < (16 / XF) ? (16 / NTG) : (16 / XF);
  static constexpr int value = C0 < 1 ? 1 : C0;
};

template <typename T, int MTT, int NTG, int EPI, bool ROW, bool SPLIT, int WAVES = 4,
          int CHK = DefaultChk<MTT, NTG, SPLIT>::value, bool PIPE = false>
__global__ __launch_bounds__(WAVES * 64) void gemm_kernel(GemmArgs g, EpiArgs e) {
  using E = Elem<T>;
  constexpr int ITEMS = NTG * MTT;
  // the waves' sums are added through LDS in rounds of RB output tiles
  constexpr int RB = ITEMS < 64 / WAVES ? ITEMS : 64 / WAVES;
  __shared__ f32x4 red[WAVES][RB][WAVE];
  __shared__ unsigned long long kmax[MTT][16];
  __shared__ float rnorm[MTT * 16];

  const int lane = threadIdx.x & 63;
  // wave-uniform values held in scalar registers, so that the batch loop's
  // branches are scalar and the loads are never under an exec mask
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Work unit (tile group ng, split s) and m-group mg of this workgroup.
  // With several m-groups, the m-groups of one unit share blockIdx % 8 (one
  // XCD, as workgroups are dealt to the eight XCDs round robin) and sit
  // within 8 * m_groups consecutive blocks, so they run together and all
  // but one read the unit's weights from that XCD's L2: the weights stream
  // from HBM about once rather than once per m-group.  Blocks past the
  // last unit (the grid is padded to a multiple of 8 units) do nothing.
  int s, ng, mg;
  if (g.m_groups > 1) {
    const int q = (int)(blockIdx.x >> 3);
    const int unit = (q / g.m_groups) * 8 + (int)(blockIdx.x & 7);
    if (unit >= g.n_groups * g.nsplit) return;
    mg = q % g.m_groups;
    s = unit % g.nsplit;
    ng = unit / g.nsplit;
  } else {
    int u = blockIdx.x;
    s = u % g.nsplit;
    u /= g.nsplit;
    ng = u % g.n_groups;
    mg = u / g.n_groups;
  }
  // balanced tile ranges: group ng owns tiles [tile0, tile0 + nt), nt <= NTG
  const int tile0 = (int)((long)ng * g.W.n_tiles / g.n_groups);
  const int nt = __builtin_amdgcn_readfirstlane((int)((long)(ng + 1) * g.W.n_tiles / g.n_groups) - tile0);
  const int mt0 = mg * MTT;
  const int kbA = s * g.kbu;
  const int kbB = min(g.W.nkb, kbA + g.kbu);
  const int per = (kbB - kbA + WAVES - 1) / WAVES;
  const int kw0 = __builtin_amdgcn_readfirstlane(kbA + wave * per);
  const int kw1 = __builtin_amdgcn_readfirstlane(min(kbB, kw0 + per));

  const uint8_t* wb[NTG];
#pragma unroll
  for (int t = 0; t < NTG; ++t) {
    const int tile = tile0 + min(t, nt - 1);   // slots past the range re-read its last tile, never used
    wb[t] = g.W.w + (size_t)tile * g.W.nkb * BLOCK_BYTES + lane * FRAG_BYTES;
  }
  f32x4 acc[NTG][MTT];
#pragma unroll
  for (int t = 0; t < NTG; ++t)
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The norm scale of this workgroup's rows: thread (part p, row r) adds
  // groups p, p + P, ... of row r, then the P parts are added in order.
  // With one or two m-tiles the thread's first NPRE groups (all of them up
  // to 4096 columns) are loaded here, before the first weight batch, from
  // in-range addresses whatever the row (so no load waits on a branch),
  // and added after the main loop: the weights start streaming at once.
  // With more rows the sum is formed here, before the main loop.
  constexpr int NR = MTT * 16, NP = WAVES * 64 / NR;
  constexpr int NPRE = (needs_norm(EPI) && MTT <= 2) ? 256 / NP : 0;
  __shared__ float npart[NP][NR];
  float npre[NPRE > 0 ? NPRE : 1];
  const int nr = threadIdx.x % NR, npt = threadIdx.x / NR;
  const int nm = mt0 * 16 + nr;
  auto norm_finish = [&](float sum) {
    npart[npt][nr] = sum;
    __syncthreads();
    if (threadIdx.x < NR) {
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < NP; ++q) t += npart[q][threadIdx.x];
      rnorm[threadIdx.x] = nm < e.M ? rsqrtf(t / (float)e.norm_dim + e.eps) : 0.f;
    }
  };
  if constexpr (NPRE > 0) {
    const int mc = min(nm, e.M - 1);
#pragma unroll
    for (int j = 0; j < NPRE; ++j) {
      const int gi = npt + j * NP;
      npre[j] = e.ssq[(size_t)min(gi, e.ssq_groups - 1) * e.M + mc];
    }
  } else if constexpr (needs_norm(EPI)) {
    float sum = 0.f;
    if (nm < e.M) {
#pragma unroll 4
      for (int g = npt; g < e.ssq_groups; g += NP) sum += e.ssq[(size_t)g * e.M + nm];
    }
    norm_finish(sum);
  }

  // One batch: CHK k-blocks of weight fragments (HBM) and the matching
  // activation fragments (L2), then the MFMAs.
  struct Batch {
    u32x4 wf[NTG][CHK];
    u32x4 xh[MTT][CHK], xl[MTT][CHK];
  };
  // Full batches (every tile of the group, every k-block in the wave's range,
  // every m-tile present) load unconditionally, so the waits before the
  // MFMAs count exactly the loads they need; the other batches test each
  // fragment (uniform conditions: scalar branches).
  auto load_full = [&](Batch& b, int kb) {
#pragma unroll
    for (int j = 0; j < CHK; ++j)
#pragma unroll
      for (int t = 0; t < NTG; ++t)
        b.wf[t][j] = __builtin_nontemporal_load((const u32x4*)(wb[t] + (size_t)(kb + j) * BLOCK_BYTES));
#pragma unroll
    for (int j = 0; j < CHK; ++j)
#pragma unroll
      for (int mt = 0; mt < MTT; ++mt) {
        if constexpr (ROW) {
          load_x<T, ROW, SPLIT>(g, mt0 + mt, kb + j, true, lane, b.xh[mt][j], b.xl[mt][j]);
        } else {
          const size_t slot = ((size_t)(mt0 + mt) * g.X.nkb + kb + j) * WAVE + lane;
          b.xh[mt][j] = g.X.hi[slot];
          if constexpr (SPLIT) b.xl[mt][j] = g.X.lo[slot];
        }
      }
  };
  auto load_part = [&](Batch& b, int kb) {
#pragma unroll
    for (int j = 0; j < CHK; ++j) {
      const bool ok = kb + j < kw1;
#pragma unroll
      for (int t = 0; t < NTG; ++t)
        b.wf[t][j] = (ok && t < nt)
                         ? __builtin_nontemporal_load((const u32x4*)(wb[t] + (size_t)(kb + j) * BLOCK_BYTES))
                         : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < CHK; ++j) {
      const bool ok = kb + j < kw1;
#pragma unroll
      for (int mt = 0; mt < MTT; ++mt) load_x<T, ROW, SPLIT>(g, mt0 + mt, kb + j, ok, lane, b.xh[mt][j], b.xl[mt][j]);
    }
  };
  auto compute = [&](const Batch& b) {
#pragma unroll
    for (int j = 0; j < CHK; ++j)
#pragma unroll
      for (int t = 0; t < NTG; ++t) {
        if (t >= nt) continue;   // uniform over the workgroup
#pragma unroll
        for (int mt = 0; mt < MTT; ++mt) {
          acc[t][mt] = E::mma(b.wf[t][j], b.xh[mt][j], acc[t][mt]);
          if constexpr (SPLIT) acc[t][mt] = E::mma(b.wf[t][j], b.xl[mt][j], acc[t][mt]);
        }
      }
  };
  const bool full_group = nt == NTG && (ROW || mt0 + MTT <= g.X.mtiles);
  const int nfull = full_group ? (kw1 - kw0) / CHK : 0;
  int kb = kw0;
  if constexpr (PIPE) {
    // two batches in flight: batch i+1 loads while batch i computes (the
    // last iteration re-loads a batch it does not use, so that every load
    // stays unconditional)
    if (nfull > 0) {
      Batch b0, b1;
      load_full(b0, kb);
      int i = 0;
      for (; i + 2 <= nfull; i += 2) {
        load_full(b1, kb + CHK);
        compute(b0);
        load_full(b0, kb + (i + 2 < nfull ? 2 * CHK : CHK));
        compute(b1);
        kb += 2 * CHK;
      }
      if (i < nfull) {
        compute(b0);
        kb += CHK;
      }
    }
  } else {
    for (int i = 0; i < nfull; ++i, kb += CHK) {
      Batch b;
      load_full(b, kb);
      compute(b);
    }
  }
  for (; kb < kw1; kb += CHK) {
    Batch b;
    load_part(b, kb);
    compute(b);
  }

  if constexpr (NPRE > 0) {
    // the norm sums loaded before the main loop, added in group order (the
    // groups past NPRE * NP, above 4096 columns, loaded now)
    float sum = 0.f;
    if (nm < e.M) {
#pragma unroll
      for (int j = 0; j < NPRE; ++j)
        if (npt + j * NP < e.ssq_groups) sum += npre[j];
      for (int g = npt + NPRE * NP; g < e.ssq_groups; g += NP) sum += e.ssq[(size_t)g * e.M + nm];
    }
    norm_finish(sum);   // rnorm is read after the next barrier
  }

  // add the waves' sums in wave order, RB tiles per round
  if constexpr (EPI == EPI_ARGMAX) {
    if (threadIdx.x < MTT * 16) (&kmax[0][0])[threadIdx.x] = 0ull;
  }
#pragma unroll
  for (int r0 = 0; r0 < ITEMS; r0 += RB) {
    if (r0 >= nt * MTT) break;   // uniform over the workgroup
    if (r0 > 0) __syncthreads();
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int it = r0 + i;
      if (it < ITEMS) red[wave][i][lane] = acc[it / MTT][it % MTT];
    }
    __syncthreads();
    for (int i = wave; i < RB && r0 + i < nt * MTT; i += WAVES) {
      const int it = r0 + i;
      const int t = it / MTT, mt = it % MTT;
      f32x4 sum = red[0][i][lane];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][i][lane];
      epilogue_tile<T, EPI>(e, s, tile0 + t, mt0 + mt, sum, lane, rnorm[mt * 16 + (lane & 15)], kmax[mt]);
    }
  }
  if constexpr (EPI == EPI_ARGMAX) {
    __syncthreads();
    if (threadIdx.x < MTT * 16) {
      const int m = (mt0 + threadIdx.x / 16) * 16 + (threadIdx.x & 15);
      const unsigned long long k = (&kmax[0][0])[threadIdx.x];
      if (m < e.M && k) atomicMax(e.keys + m, k);
    }
  }
  if constexpr (EPI == EPI_PARTRES) {
    // Arrival of this split of the tile group (ng, mg): every wave's partial
    // stores have completed (waited for, write-through) before one atomic
    // increment at agent scope.  The split that brings the count to nsplit
    // resets it (for the next launch) and adds the group's partials, split 0
    // first, then runs the residual epilogue on the sums.  No workgroup
    // waits for another.
    __shared__ unsigned is_last;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (threadIdx.x == 0) {
      typedef __attribute__((address_space(1))) unsigned g_u32;
      g_u32* cnt = (g_u32*)(e.fix_cnt + (size_t)ng * g.m_groups + mg);
      const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned last = old + 1u == (unsigned)g.nsplit ? 1u : 0u;
      if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      is_last = last;
    }
    __syncthreads();
    if (!is_last) return;
    // every load of a tile (the partials of all splits, the residual quad
    // and the gain) is issued before the first is used: a split past
    // nsplit re-reads the last one, which is not added
    const size_t sstride = (size_t)e.part_ntiles * e.part_mtiles * 64 * 4;   // floats between splits
    for (int it = wave; it < nt * MTT; it += WAVES) {
      const int tile = tile0 + it / MTT, mt = mt0 + it % MTT;
      if (mt >= e.part_mtiles) continue;   // uniform over the wave
      const float* p = e.part + (((size_t)tile * e.part_mtiles + mt) * 64 + lane) * 4;
      f32x4 pv[MAX_SPLITS];
#pragma unroll
      for (int sp = 0; sp < MAX_SPLITS; ++sp) pv[sp] = load_agent_f32x4(p + min(sp, g.nsplit - 1) * sstride);
      const ResIn in = resnorm_load(e, tile, mt, lane);
      f32x4 sum = pv[0];
#pragma unroll
      for (int sp = 1; sp < MAX_SPLITS; ++sp)
        if (sp < g.nsplit) sum += pv[sp];
      resnorm_tile<T>(e, tile, mt, sum, lane, in);
    }
  }
}

// ---------------------------------------------------------------------------
// launch of one compiled variant (instantiated per epilogue in gemm_<epi>.hip)
// ---------------------------------------------------------------------------
// k-blocks per load batch: about 20 weight fragments per wave in flight for
// one m-tile, fewer activation fragments for more m-tiles
template <int MTT, int NTG, bool SPLIT>
struct HotChk {
  static constexpr int W = NTG <= 2 ? 10 : 20 / NTG;       // weight-fragment bound
  static constexpr int X = 16 / (MTT * (SPLIT ? 2 : 1));   // activation-fragment bound
  static constexpr int C = MTT == 1 ? W : (W < X ? W : X);
  static constexpr int value = C < 1 ? 1 : C;
};

template <typename T, int MTT, int NTG, int EPI, bool ROW, bool SPLIT, int WAVES, int CHK,
          bool PIPE = false>
inline hipError_t launch_v(const GemmPlan& p, const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  // several m-groups: units padded to a multiple of 8 (see the kernel)
  const unsigned units = (unsigned)p.n_groups * p.nsplit;
  dim3 grid(p.m_groups > 1 ? (units + 7u) / 8u * 8u * (unsigned)p.m_groups : units);
  hipLaunchKernelGGL((gemm_kernel<T, MTT, NTG, EPI, ROW, SPLIT, WAVES, CHK, PIPE>), grid, dim3(WAVES * 64), 0,
                     s, g, e);
  return hipGetLastError();
}

template <typename T, int MTT, int NTG, int EPI, bool ROW, bool SPLIT>
inline hipError_t launch_h(const GemmPlan& p, const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  // Measured on the Qwen3-4B shapes: eight waves for one, two and eight
  // m-tiles; the pipelined form (the next load batch in flight during the
  // MFMAs of the current one; two batches in registers, so half the batch
  // size) for four m-tiles and for two m-tiles over at most two tiles per
  // workgroup.
  constexpr int WAVES = MTT == 4 ? 4 : 8;
  constexpr bool PIPE = MTT == 4 || (MTT == 2 && NTG <= 2);
  constexpr int CHK = MTT > 1 ? (HotChk<MTT, NTG, SPLIT>::value + 1) / 2 : HotChk<MTT, NTG, SPLIT>::value;
  return launch_v<T, MTT, NTG, EPI, ROW, SPLIT, WAVES, CHK, PIPE>(p, g, e, s);
}

// Compiled combinations: bf16 products take the hi/lo activation pair at
// every m-tile count, the LM head up to two m-tiles (above that it runs
// head_kernel on the hi part); the per-step context products (row-major
// features, K/V injection) have at most two m-tiles.
template <typename T, int MTT, int EPI, bool ROW, bool SPLIT>
constexpr bool compiled() {
  if constexpr (ROW) return !SPLIT && MTT <= 2;
  if constexpr (EPI == EPI_KV) return MTT <= 2 && SPLIT == (sizeof(T) == 2);
  if constexpr (EPI == EPI_ARGMAX && sizeof(T) == 2) return SPLIT == (MTT <= 2);
  return SPLIT == (sizeof(T) == 2);
}

template <typename T, int MTT, int EPI, bool ROW, bool SPLIT>
inline hipError_t launch_mtt(const GemmPlan& p, const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  if constexpr (!compiled<T, MTT, EPI, ROW, SPLIT>()) {
    return hipErrorInvalidValue;
  } else {
    switch (p.ntg) {
      case 1: return launch_h<T, MTT, 1, EPI, ROW, SPLIT>(p, g, e, s);
      case 2: return launch_h<T, MTT, 2, EPI, ROW, SPLIT>(p, g, e, s);
      case 4: return launch_h<T, MTT, 4, EPI, ROW, SPLIT>(p, g, e, s);
    }
    if constexpr (MTT <= 4 || is_part(EPI)) {
      if (p.ntg == 5) return launch_h<T, MTT, 5, EPI, ROW, SPLIT>(p, g, e, s);
    }
    if constexpr (MTT <= 2 || (MTT == 4 && EPI == EPI_QKV)) {
      if (p.ntg == 8) return launch_h<T, MTT, 8, EPI, ROW, SPLIT>(p, g, e, s);
    }
    if constexpr (MTT == 1) {
      if (p.ntg == 6) return launch_h<T, MTT, 6, EPI, ROW, SPLIT>(p, g, e, s);
    }
    return hipErrorInvalidValue;
  }
}

template <typename T, int EPI, bool ROW, bool SPLIT>
inline hipError_t launch_hot(const GemmPlan& p, const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  switch (p.mtt) {
    case 1: return launch_mtt<T, 1, EPI, ROW, SPLIT>(p, g, e, s);
    case 2: return launch_mtt<T, 2, EPI, ROW, SPLIT>(p, g, e, s);
    case 4: return launch_mtt<T, 4, EPI, ROW, SPLIT>(p, g, e, s);
    default: return launch_mtt<T, 8, EPI, ROW, SPLIT>(p, g, e, s);
  }
}

template <typename T, int EPI, bool ROW, bool SPLIT>
inline hipError_t launch_fixed(const GemmPlan& p, const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  constexpr int NTG = EPI == EPI_FC ? 4 : 2;
  if (p.ntg != NTG) return hipErrorInvalidValue;
  switch (p.mtt) {
    case 1: return launch_v<T, 1, NTG, EPI, ROW, SPLIT, 4, 4>(p, g, e, s);
    case 2: return launch_v<T, 2, NTG, EPI, ROW, SPLIT, 4, DefaultChk<2, NTG, SPLIT>::value>(p, g, e, s);
    case 4: return launch_v<T, 4, NTG, EPI, ROW, SPLIT, 4, DefaultChk<4, NTG, SPLIT>::value>(p, g, e, s);
    default: return launch_v<T, 8, NTG, EPI, ROW, SPLIT, 4, DefaultChk<8, NTG, SPLIT>::value>(p, g, e, s);
  }
}

// ---------------------------------------------------------------------------
// Products over m-groups of MTT = 8 or 4 m-tiles (128 or 64 rows; bf16
// model; the LM head on the hi part of the activations, and gate/up on the
// hi/lo pair when there are enough m-groups): the waves of a workgroup
// split its tiles (up to NTW each, the whole reduction each), so one copy
// of each activation fragment, staged in LDS, feeds every wave; in the form
// above, every workgroup of four or five tiles re-reads the whole
// activation from L2 and each wave keeps one load batch in flight.  Stages
// of KC k-blocks x MTT m-tiles are double buffered; the next stage's
// activation and weight loads are in flight
// while the current one is computed, and the last stage is peeled so that
// every load in the loop is unconditional (a weight tile past the wave's
// range re-reads its last tile, never used; activation k-blocks past the
// end are zero).  The epilogue is that of gemm_kernel, per tile, on
// complete sums.
// ---------------------------------------------------------------------------
constexpr int HEAD_KC = 2;    // k-blocks per stage

template <typename T, int MTT, int EPI, bool SPLIT>
__global__ __launch_bounds__(HEAD_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2))) void head_kernel(GemmArgs g,
                                                                                                  EpiArgs e) {
  using E = Elem<T>;
  constexpr int NTW = HEAD_NTW, KC = HEAD_KC, NTH = HEAD_WAVES * 64;
  constexpr int XPT = KC * MTT * WAVE / NTH;   // activation fragments staged per thread
  constexpr int NX = SPLIT ? 2 : 1;            // hi (and lo) parts
  static_assert(XPT * NTH == KC * MTT * WAVE, "stage");
  __shared__ u32x4 xs[NX][2][KC][MTT][WAVE];
  __shared__ unsigned long long kmax[MTT][16];
  __shared__ float rnorm[MTT * 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // unit (tile group) and m-group, numbered as in gemm_kernel
  int ng, mg;
  if (g.m_groups > 1) {
    const int q = (int)(blockIdx.x >> 3);
    ng = (q / g.m_groups) * 8 + (int)(blockIdx.x & 7);
    if (ng >= g.n_groups) return;
    mg = q % g.m_groups;
  } else {
    ng = blockIdx.x;
    mg = 0;
  }
  const int tile0 = (int)((long)ng * g.W.n_tiles / g.n_groups);
  const int nt = (int)((long)(ng + 1) * g.W.n_tiles / g.n_groups) - tile0;
  const int ntw = (nt + HEAD_WAVES - 1) / HEAD_WAVES;              // <= NTW (checked at launch)
  const int wt0 = tile0 + wave * ntw;
  const int wnt = __builtin_amdgcn_readfirstlane(max(0, min(ntw, tile0 + nt - wt0)));
  const int mt0 = mg * MTT;
  const int nkb = g.W.nkb;

  const uint8_t* wb[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int tile = wnt > 0 ? wt0 + min(t, wnt - 1) : tile0;
    wb[t] = g.W.w + (size_t)tile * nkb * BLOCK_BYTES + lane * FRAG_BYTES;
  }
  f32x4 acc[NTW][MTT];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // norm scale of the rows: thread (part p, row r) adds groups p, p + P, ...
  if constexpr (needs_norm(EPI)) {
    constexpr int R = MTT * 16, P = NTH / R;
    __shared__ float npart[P][R];
    const int r = threadIdx.x % R, part = threadIdx.x / R;
    const int m = mt0 * 16 + r;
    float sum = 0.f;
    if (m < e.M)
      for (int q = part; q < e.ssq_groups; q += P) sum += e.ssq[(size_t)q * e.M + m];
    npart[part][r] = sum;
    __syncthreads();
    if (threadIdx.x < R) {
      float tt = 0.f;
#pragma unroll
      for (int q = 0; q < P; ++q) tt += npart[q][threadIdx.x];
      rnorm[threadIdx.x] = m < e.M ? rsqrtf(tt / (float)e.norm_dim + e.eps) : 0.f;
    }
  }

  struct Stage {
    u32x4 x[NX][XPT];
    u32x4 w[NTW][KC];
  };
  // stage s: k-blocks s*KC .. s*KC+KC-1 (past nkb: activation zero, weight
  // address clamped to the last k-block)
  auto load = [&](Stage& st, int s) {
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = threadIdx.x + j * NTH;
      const int kbi = i / (MTT * WAVE), mt = (i / WAVE) % MTT, ln = i % WAVE;
      const int kb = s * KC + kbi;
      const bool ok = kb < nkb && mt0 + mt < g.X.mtiles;
      const size_t slot = ((size_t)min(mt0 + mt, g.X.mtiles - 1) * g.X.nkb + min(kb, nkb - 1)) * WAVE + ln;
      const u32x4 v = g.X.hi[slot];
      st.x[0][j] = ok ? v : u32x4{0u, 0u, 0u, 0u};
      if constexpr (SPLIT) {
        const u32x4 vl = g.X.lo[slot];
        st.x[1][j] = ok ? vl : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int kb = min(s * KC + k, nkb - 1);
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        st.w[t][k] = __builtin_nontemporal_load((const u32x4*)(wb[t] + (size_t)kb * BLOCK_BYTES));
    }
  };
  auto stash = [&](const Stage& st, int buf) {
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = threadIdx.x + j * NTH;
#pragma unroll
      for (int h = 0; h < NX; ++h) (&xs[h][buf][0][0][0])[i] = st.x[h][j];
    }
  };
  auto compute = [&](const Stage& st, int buf) {
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      u32x4 xf[NX][MTT];
#pragma unroll
      for (int h = 0; h < NX; ++h)
#pragma unroll
        for (int mt = 0; mt < MTT; ++mt) xf[h][mt] = xs[h][buf][k][mt][lane];
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        if (t >= wnt) continue;   // uniform over the wave
#pragma unroll
        for (int mt = 0; mt < MTT; ++mt) {
          acc[t][mt] = E::mma(st.w[t][k], xf[0][mt], acc[t][mt]);
          if constexpr (SPLIT) acc[t][mt] = E::mma(st.w[t][k], xf[1][mt], acc[t][mt]);
        }
      }
    }
  };

  if constexpr (EPI == EPI_ARGMAX) {
    if (threadIdx.x < MTT * 16) (&kmax[0][0])[threadIdx.x] = 0ull;   // visible after the first barrier
  }
  const int nst = (nkb + KC - 1) / KC;
  Stage a, b;
  load(a, 0);
  stash(a, 0);
  __syncthreads();
  int s = 0;
  for (; s + 1 < nst; ++s) {
    load(b, s + 1);
    compute(a, s & 1);
    stash(b, (s + 1) & 1);
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int k = 0; k < KC; ++k) a.w[t][k] = b.w[t][k];
    __syncthreads();
  }
  compute(a, s & 1);

#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    if (t >= wnt) continue;
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt)
      epilogue_tile<T, EPI>(e, 0, wt0 + t, mt0 + mt, acc[t][mt], lane,
                            needs_norm(EPI) ? rnorm[mt * 16 + (lane & 15)] : 1.f, kmax[mt]);
  }
  if constexpr (EPI == EPI_ARGMAX) {
    __syncthreads();
    if (threadIdx.x < MTT * 16) {
      const int m = (mt0 + threadIdx.x / 16) * 16 + (threadIdx.x & 15);
      const unsigned long long k = (&kmax[0][0])[threadIdx.x];
      if (m < e.M && k) atomicMax(e.keys + m, k);
    }
  }
}

template <typename T, int EPI>
inline hipError_t launch_head(const GemmPlan& p, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  g.n_groups = head_groups(g.W.n_tiles, p.m_groups);
  g.m_groups = p.m_groups;
  g.nsplit = 1;
  g.kbu = g.W.nkb;
  if ((g.W.n_tiles + g.n_groups - 1) / g.n_groups > HEAD_WAVES * HEAD_NTW || g.X.nkb < g.W.nkb ||
      g.X.mtiles < 1)
    return hipErrorInvalidValue;
  const unsigned units = (unsigned)g.n_groups;
  dim3 grid(p.m_groups > 1 ? (units + 7u) / 8u * 8u * (unsigned)p.m_groups : units);
  constexpr bool SPLIT = EPI != EPI_ARGMAX;   // the LM head reads the hi part alone
  if (p.split != SPLIT || (SPLIT && !g.X.lo)) return hipErrorInvalidValue;
  if (p.mtt == 8) hipLaunchKernelGGL((head_kernel<T, 8, EPI, SPLIT>), grid, dim3(HEAD_WAVES * 64), 0, s, g, e);
  else if (p.mtt == 4) hipLaunchKernelGGL((head_kernel<T, 4, EPI, SPLIT>), grid, dim3(HEAD_WAVES * 64), 0, s, g, e);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K products over m-groups of 128 rows with the hi/lo pair (bf16
// model): the output and down projections above four m-tiles.  Four waves,
// one workgroup per CU: wave w covers tile slot w % 2 (up to NTW tiles of
// the workgroup's range) and m-half w / 2 (4 m-tiles), over the
// workgroup's k-range.  Each k-block's activation fragments (8 m-tiles x
// hi/lo) and weight fragments (the workgroup's tiles) are staged once per
// workgroup in a ring of WIDE_STAGES LDS stages by direct loads, issued
// WIDE_STAGES - 1 k-blocks ahead; each wave reads the next k-block's
// fragments from LDS into its second register set while the MFMAs of the
// current one run.  In gemm_kernel's form every wave loads its own 16
// activation fragments per k-block through the vector-memory path with one
// load batch in flight, which bounds the 128-row split products (measured
// at the Qwen3-4B shape, 128 rows, per launch: o + down average 21.1 ->
// 16.2 us).  Per k-block a CU reads 48 KiB from LDS and writes 24 KiB into
// it beside 128 MFMAs per SIMD; a barrier and the direct loads add about
// 170 and 180 cycles to the 740 of the LDS reads and MFMAs alone
// (measured), which bounds this form near 1000 cycles per k-block.  The
// epilogue is gemm_kernel's split-K store, per tile.
// ---------------------------------------------------------------------------
constexpr int WIDE_STAGES = 4;

template <typename T, int NTW>
__global__ __launch_bounds__(256, 1) void wide_kernel(GemmArgs g, EpiArgs e) {
  static_assert(sizeof(T) == 2, "bf16 models (hi/lo pair)");
  using E = Elem<T>;
  constexpr int MT = 8, MPW = 4, XF = 2 * MT, FR = XF + 2 * NTW;
  constexpr int DPW = (FR + 3) / 4;            // direct loads per wave per stage
  constexpr int NF = 2 * MPW + NTW;            // fragments a wave reads per k-block
  constexpr int NS = WIDE_STAGES;
  constexpr int NW0 = DPW * (NS - 2), NW1 = DPW * (NS - 3);   // loads issued after the awaited stage
  static_assert(NS >= 3 && NW0 < 64, "stages");
  // One LDS object.  (With several, the compiler tells them apart and
  // completes every outstanding direct load before each read of the ring;
  // the explicit waits below are what order those reads.)
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS][4 * DPW][BLOCK_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ts = wave & 1, mp = wave >> 1;
  // unit (tile group ng, split s) and m-group mg, numbered as in
  // gemm_kernel: the m-groups of one unit share an XCD and run together, so
  // the unit's weights stream from HBM about once for all of them
  int s, ng, mg;
  if (g.m_groups > 1) {
    const int q = (int)(blockIdx.x >> 3);
    const int unit = (q / g.m_groups) * 8 + (int)(blockIdx.x & 7);
    if (unit >= g.n_groups * g.nsplit) return;   // the whole workgroup, before any barrier
    mg = q % g.m_groups;
    s = unit % g.nsplit;
    ng = unit / g.nsplit;
  } else {
    s = (int)blockIdx.x % g.nsplit;
    ng = (int)blockIdx.x / g.nsplit;
    mg = 0;
  }
  const int mt0 = mg * 8;
  const int tile0 = (int)((long)ng * g.W.n_tiles / g.n_groups);
  const int nt = (int)((long)(ng + 1) * g.W.n_tiles / g.n_groups) - tile0;
  const int wt0 = tile0 + (ts * nt) / 2;   // this wave's tiles: [wt0, wt0 + wnt), wnt <= NTW
  const int wnt = __builtin_amdgcn_readfirstlane(tile0 + ((ts + 1) * nt) / 2 - wt0);
  const int kbA = s * g.kbu;
  const int nk = min(g.W.nkb, kbA + g.kbu) - kbA;   // >= 1: the plan leaves no split empty

  // Direct load d of this wave fills stage fragment f = wave * DPW + d:
  //   f < XF        activation part f / MT (hi, lo) of m-tile f % MT (an
  //                 m-tile past the activation repeats its last one: those
  //                 rows are never stored)
  //   f < FR        weight tile (f - XF) % NTW of slot (f - XF) / NTW (a slot
  //                 past its range repeats its last tile, never used)
  //   otherwise     a repeat of fragment 0 into a spare slot, never read
  // Offsets are 32-bit from the matrix base (checked at launch).
  const uint8_t* dsrc[DPW];
  uint32_t doff[DPW];
#pragma unroll
  for (int d = 0; d < DPW; ++d) {
    const int f = wave * DPW + d;
    if (f < XF || f >= FR) {
      const int fx = f < XF ? f : 0;
      const int mt = min(mt0 + fx % MT, g.X.mtiles - 1);
      dsrc[d] = (const uint8_t*)(fx / MT ? g.X.lo : g.X.hi);
      doff[d] = (uint32_t)(((size_t)mt * g.X.nkb + kbA) * BLOCK_BYTES + lane * FRAG_BYTES);
    } else {
      const int slot = (f - XF) / NTW, t = (f - XF) % NTW;
      const int st0 = tile0 + (slot * nt) / 2, sn = tile0 + ((slot + 1) * nt) / 2 - st0;
      const int tile = min(st0 + min(t, max(sn, 1) - 1), g.W.n_tiles - 1);
      dsrc[d] = g.W.w;
      doff[d] = (uint32_t)(((size_t)tile * g.W.nkb + kbA) * BLOCK_BYTES + lane * FRAG_BYTES);
    }
  }
  // stage of k-block i of the range (past the end: its last k-block again)
  auto issue = [&](int i) {
    const uint32_t kb = (uint32_t)min(i, nk - 1) * BLOCK_BYTES;
    uint8_t* st = &ring[i % NS][0][0];
#pragma unroll
    for (int d = 0; d < DPW; ++d) dma16(dsrc[d], doff[d] + kb, st + (wave * DPW + d) * BLOCK_BYTES);
  };
  u32x4 fr[2][NF];
  auto read = [&](u32x4 (&dst)[NF], int i) {
    const uint8_t* st = &ring[i % NS][0][0] + lane * FRAG_BYTES;
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      dst[2 * m] = *(const u32x4*)(st + (mp * MPW + m) * BLOCK_BYTES);
      dst[2 * m + 1] = *(const u32x4*)(st + (MT + mp * MPW + m) * BLOCK_BYTES);
    }
#pragma unroll
    for (int t = 0; t < NTW; ++t) dst[2 * MPW + t] = *(const u32x4*)(st + (XF + ts * NTW + t) * BLOCK_BYTES);
  };
  f32x4 acc[NTW][MPW];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int m = 0; m < MPW; ++m) acc[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  // hi then lo per k-block, k-blocks in order: the summation order of gemm_kernel's waves
  auto compute = [&](const u32x4 (&f)[NF]) {
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        acc[t][m] = E::mma(f[2 * MPW + t], f[2 * m], acc[t][m]);
        acc[t][m] = E::mma(f[2 * MPW + t], f[2 * m + 1], acc[t][m]);
      }
  };

#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue(p);
  wait_vm<NW0>();
  lds_barrier();
  read(fr[0], 0);
  // k-block i: wait for stage i + 1 and make it visible, refill the stage of
  // k-block i - 1 (its reads completed before this barrier) with k-block
  // i + NS - 1, read stage i + 1 into the other register set, and run k-block
  // i's MFMAs on the set read one step earlier
  auto step = [&](int i, int par, bool guard) {
    wait_vm<NW1>();
    lds_barrier();
    issue(i + NS - 1);
    read(fr[par ^ 1], i + 1);
    if (!guard || i < nk) compute(fr[par]);
  };
  int i = 0;
  for (; i + 2 <= nk; i += 2) {
    step(i, 0, false);
    step(i + 1, 1, false);
  }
  if (i < nk) step(i, 0, true);
  wait_vm<0>();   // the stages issued past the end

#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    if (t >= wnt) continue;   // uniform over the wave
#pragma unroll
    for (int m = 0; m < MPW; ++m)
      epilogue_tile<T, EPI_PART>(e, s, wt0 + t, mt0 + mp * MPW + m, acc[t][m], lane, 1.f, nullptr);
  }
}

template <typename T, int EPI>
inline hipError_t launch_wide(const GemmPlan& p, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  if constexpr (sizeof(T) != 2 || EPI != EPI_PART) {
    return hipErrorInvalidValue;
  } else {
    g.kbu = p.kbu;
    g.nsplit = p.nsplit;
    g.n_groups = p.n_groups;
    g.m_groups = p.m_groups;
    // every tile in a range of at most 2 * ntg tiles (ntg per wave slot);
    // direct-load offsets within 32 bits; every split non-empty
    const size_t wbytes = (size_t)g.W.n_tiles * g.W.nkb * BLOCK_BYTES;
    const size_t xbytes = (size_t)g.X.mtiles * g.X.nkb * BLOCK_BYTES;
    if (!p.split || !g.X.lo || p.m_groups < 1 || g.X.mtiles < 1 || g.X.nkb < g.W.nkb || p.n_groups < 1 ||
        (g.W.n_tiles + p.n_groups - 1) / p.n_groups > 2 * p.ntg || wbytes >= (1ull << 32) ||
        xbytes >= (1ull << 32) || (size_t)(p.nsplit - 1) * p.kbu >= (size_t)g.W.nkb)
      return hipErrorInvalidValue;
    // several m-groups: units padded to a multiple of 8 (see the kernel)
    const unsigned units = (unsigned)p.n_groups * p.nsplit;
    const dim3 grid(p.m_groups > 1 ? (units + 7u) / 8u * 8u * (unsigned)p.m_groups : units);
    switch (p.ntg) {
      case 2: hipLaunchKernelGGL((wide_kernel<T, 2>), grid, dim3(256), 0, s, g, e); break;
      case 3: hipLaunchKernelGGL((wide_kernel<T, 3>), grid, dim3(256), 0, s, g, e); break;
      case 4: hipLaunchKernelGGL((wide_kernel<T, 4>), grid, dim3(256), 0, s, g, e); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
}

template <typename T, int EPI>
hipError_t launch_gemm_epi(const GemmPlan& p, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  if constexpr ((EPI == EPI_ARGMAX || EPI == EPI_SWIGLU) && sizeof(T) == 2) {
    if (uses_head_kernel(EPI, p, g.W.n_tiles, (int)sizeof(T))) return launch_head<T, EPI>(p, g, e, s);
  }
  if (p.wide) return launch_wide<T, EPI>(p, g, e, s);
  g.kbu = p.kbu;
  g.nsplit = p.nsplit;
  g.n_groups = p.n_groups;
  g.m_groups = p.m_groups;
  // every tile must fall in a range of at most NTG tiles
  if (p.n_groups < 1 || (g.W.n_tiles + p.n_groups - 1) / p.n_groups > p.ntg) return hipErrorInvalidValue;
  if (p.rowmajor) {
    if constexpr (EPI == EPI_FC || EPI == EPI_KV || EPI == EPI_PART) {
      if (p.fixed) return launch_fixed<T, EPI, true, false>(p, g, e, s);
      if constexpr (EPI == EPI_PART) return launch_hot<T, EPI, true, false>(p, g, e, s);
    }
    return hipErrorInvalidValue;
  }
  if constexpr (EPI == EPI_FC || EPI == EPI_KV) {
    if (p.fixed) {
      if constexpr (sizeof(T) == 2) {
        if (p.split) return launch_fixed<T, EPI, false, true>(p, g, e, s);
      }
      return launch_fixed<T, EPI, false, false>(p, g, e, s);
    }
  }
  if constexpr (EPI != EPI_FC) {
    if constexpr (sizeof(T) == 2) {
      if (p.split) return launch_hot<T, EPI, false, true>(p, g, e, s);
    }
    return launch_hot<T, EPI, false, false>(p, g, e, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dflash
