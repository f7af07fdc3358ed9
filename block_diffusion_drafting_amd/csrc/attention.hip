// Bidirectional GQA attention of the draft block over [context KV || block KV]
// (and, in its causal form, the target's attention for block verification).
//
// The block is denoised in one non-causal forward (kongchang.com "D-Flash",
// "System architecture"; Google Developers Blog, "Dual cache for
// attention"): every block row attends to every committed context position
// of its sequence and to every block row, with no mask.  Context K/V come
// from the sequence's static cache, block K/V from this layer's QKV
// epilogue.
//
// Work unit (one 256-thread workgroup): sequence b, KV head g, a group of up
// to four 16-row query tiles (rows = block position x query head sharing g),
// and one split of the key range (its partial result goes to a buffer that
// attn_combine merges in split order).  A split is a run of 64-key chunks;
// each chunk is staged in LDS once (K row-major, V transposed, padded rows
// against bank conflicts) and read by all four waves, and the global loads
// of the next chunk are in flight while the current one is computed.  S^T = K Q^T and O^T += V^T P^T run on MFMA; the
// softmax is online per wave in fp32 (exp2 with the log2(e) folded into
// the scale).  For bf16 the two 16-key S^T tiles of a 32-key step hold keys
// in the order that makes each lane's probabilities the B-fragment of the
// P.V product directly.
//
// Causal form (block verification, Google Developers Blog "Overcoming the
// autoregressive bottleneck"): the QKV product has already stored the block
// rows' K/V in the cache at slots ctx_len + i, so every split reads the
// cache, over ctx_len + K keys, and block row i masks keys past ctx_len + i.
//
// T is the attention operand type: fp16 for bf16 models (queries, keys,
// values and probabilities), fp32 for fp32 models.  The output is fp32.
#include "kernels.h"

namespace dflash {

// Keys per LDS chunk (two chunks are resident): 64, or 32 for fp32 operands
// with head_dim 128.
template <typename T, int D>
constexpr int chunk_keys() { return (sizeof(T) == 4 && D == 128) ? 32 : 64; }

size_t attn_part_floats(int B, int nkv, int qgroups, int max_splits, int d) {
  // per wave: O^T [d][16] + m[16] + l[16]
  return (size_t)B * nkv * qgroups * max_splits * 4 * (d * 16 + 32);
}

// Two waves per SIMD (two 4-wave or one 8-wave workgroup per compute unit,
// as the grid is planned): at most 256 registers per wave.
template <typename T, int D, int QG>
__global__ __launch_bounds__(256 * QG) __attribute__((amdgpu_waves_per_eu(2))) void attention_kernel(AttnArgs a) {
  using E = Elem<T>;
  constexpr int CHUNK_KEYS = chunk_keys<T, D>();
  constexpr int ES = sizeof(T);
  constexpr int KROW = D * ES + 16;           // padded LDS row of K (bytes)
  constexpr int VROW = CHUNK_KEYS * ES + 16;  // padded LDS row of V^T (bytes)
  constexpr int NFD = D * ES / 64;            // 16-byte fragments along d per lane
  constexpr int NDT = D / 16;                 // 16-row tiles of d
  constexpr int KP = 4 * E::KPL;              // keys per P.V step (32 bf16, 16 fp32)
  constexpr int KP_ROW = D * ES / 16;                   // 16-byte pieces per K row
  constexpr int KPIECES = CHUNK_KEYS * KP_ROW;
  constexpr int VP_ROW = CHUNK_KEYS * ES / 16;          // 16-byte pieces per V^T row
  constexpr int VPIECES = D * VP_ROW;
  constexpr int EPP = 16 / ES;                          // keys per V^T piece
  constexpr int NTH = 256 * QG;   // threads of the workgroup
  constexpr int KPT = KPIECES / NTH, VPT = VPIECES / NTH;
  static_assert(KPIECES % NTH == 0 && VPIECES % NTH == 0, "chunk staging");
  __shared__ __attribute__((aligned(16))) uint8_t kl[2][CHUNK_KEYS * KROW];
  __shared__ __attribute__((aligned(16))) uint8_t vl[2][D * VROW];

  // appended workgroups warm the output projection's weights instead
  if (a.warm.w && (int)blockIdx.x >= a.warm.first) {
    warm_consumer(a.warm, (int)blockIdx.x - a.warm.first, 4 * QG, (int)(threadIdx.x >> 6), (int)(threadIdx.x & 63),
                  (lds_void_t*)(kl[0] + (threadIdx.x >> 6) * 1024));
    return;
  }
  // QG query groups share each staged chunk: wave w is query tile w % 4 of
  // query group qgp * QG + w / 4
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & 3;
  const int g4 = lane >> 4, col = lane & 15;
  // Workgroups of the same (sequence, KV head, split) and different query
  // groups read the same keys; blocks are dealt to the 8 XCDs round-robin,
  // so they are numbered to share blockIdx % 8 (one L2) -- see attn_grid.
  const int nqgp = (a.qgroups + QG - 1) / QG;
  const int lo = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int qg = (rest % nqgp) * QG + (int)(threadIdx.x >> 8);
  int u = (rest / nqgp) * 8 + lo;
  if (u >= a.B * a.nkv * a.max_splits) return;
  const int s = u % a.max_splits;
  u /= a.max_splits;
  const int g = u % a.nkv;
  const int b = u / a.nkv;

  const DevSeq sq = a.seqs[b];
  const int ctx_len = sq.ctx_len;
  int n_cs, n_s;
  attn_split_counts(a, ctx_len, n_cs, n_s);
  if (s >= n_s) return;

  const T* kbase;
  const T* vbase;
  int vstride, k0, k1;
  if (s < n_cs) {
    kbase = (const T*)sq.k + ((size_t)a.layer * a.nkv + g) * sq.phys * D;
    vbase = (const T*)sq.vt + ((size_t)a.layer * a.nkv + g) * D * sq.phys;
    vstride = sq.phys;
    k0 = s * a.chunk;
    k1 = min(a.causal ? ctx_len + a.K : ctx_len, k0 + a.chunk);
  } else {
    kbase = (const T*)a.bk + ((size_t)b * a.nkv + g) * a.Kpad * D;
    vbase = (const T*)a.bvt + ((size_t)b * a.nkv + g) * D * a.Kpad;
    vstride = a.Kpad;
    k0 = (s - n_cs) * a.chunk;
    k1 = min(a.K, k0 + a.chunk);
  }

  // query rows of this wave: r = qtile*16 + col -> head h, block row i
  const int rep = a.nq / a.nkv;
  const int nrows = a.K * rep;
  const int qt = qg * 4 + wave;
  const int r = qt * 16 + col;
  const bool row_ok = qg < a.qgroups && r < nrows;
  const int h = g * rep + (row_ok ? r / a.K : 0);
  const int i = row_ok ? r % a.K : 0;
  // causal form: this lane's query (block row i) sees cache keys 0..ctx_len+i
  const int key_lim = a.causal ? ctx_len + i : 0x7FFFFFFF;
  u32x4 qf[NFD];
  {
    const T* qp = (const T*)a.q + ((size_t)(b * a.K + i) * a.nq + h) * D;
#pragma unroll
    for (int f = 0; f < NFD; ++f)
      qf[f] = row_ok ? gld16(qp + f * E::KB + g4 * E::KPL) : u32x4{0u, 0u, 0u, 0u};
  }

  f32x4 o[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Chunk staging through registers, two chunks in flight: while chunk c
  // is computed from LDS, the loads of chunks c+1 and c+2 are outstanding
  // in two register sets; chunk c+1 is stored to the other LDS buffer once
  // c is done.  Every lane issues the same loads on every path, so the wait
  // before a store covers only the older set: a chunk starts at a multiple
  // of 64 keys below the row length, and both the cache rows (a power of two
  // >= 64) and the block rows (padded to 64) are multiples of 64, so the
  // whole chunk is in bounds.  Keys at or past the split end are zeroed
  // when the chunk is stored to LDS (K rows and V^T columns).  Offsets are
  // 32-bit from the (uniform) slab base: a slab of one layer and KV head
  // holds under 2^31 bytes (checked where the caches are allocated).
  struct Regs {
    u32x4 kr[KPT], vr[VPT];
  };
  auto gload = [&](Regs& rg, int c0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int t = threadIdx.x + j * NTH;
      const int row = t / KP_ROW, pc = t % KP_ROW;
      rg.kr[j] = gld16((const uint8_t*)kbase + ((uint32_t)(c0 + row) * (D * ES) + pc * 16));
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int t = threadIdx.x + j * NTH;
      const int dr = t / VP_ROW, pc = t % VP_ROW;
      rg.vr[j] = gld16((const uint8_t*)vbase + ((uint32_t)(dr * vstride + c0 + pc * EPP) * ES));
    }
  };
  auto lstore = [&](Regs& rg, int buf, int c0, int cend) {
    if (cend - c0 < CHUNK_KEYS) {   // last chunk of the split (uniform)
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int t = threadIdx.x + j * NTH;
        if (c0 + t / KP_ROW >= cend) rg.kr[j] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int t = threadIdx.x + j * NTH;
        const int key = c0 + (t % VP_ROW) * EPP;
        if (key + EPP > cend) {
          T tmp[EPP];
          __builtin_memcpy(tmp, &rg.vr[j], 16);
#pragma unroll
          for (int e2 = 0; e2 < EPP; ++e2)
            if (key + e2 >= cend) tmp[e2] = (T)0;
          __builtin_memcpy(&rg.vr[j], tmp, 16);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int t = threadIdx.x + j * NTH;
      *(u32x4*)(kl[buf] + (t / KP_ROW) * KROW + (t % KP_ROW) * 16) = rg.kr[j];
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int t = threadIdx.x + j * NTH;
      *(u32x4*)(vl[buf] + (t / VP_ROW) * VROW + (t % VP_ROW) * 16) = rg.vr[j];
    }
  };
  // online softmax and P.V over chunk [c0, cend) held in LDS buffer buf
  auto compute = [&](int c0, int cend, int buf) {
    const uint8_t* klb = kl[buf];
    const uint8_t* vlb = vl[buf];
#pragma unroll
    for (int sub = 0; sub < CHUNK_KEYS / KP; ++sub) {
      const int kb = sub * KP;  // key offset of this P.V step within the chunk
      float sv[8];
      int nv;
      if constexpr (ES == 2) {
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
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sv[j] = sa[j];
          sv[4 + j] = sb[j];
        }
        nv = 8;
      } else {
        const int row = kb + col;
        f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < NFD; ++f) {
          const u32x4 ka = *(const u32x4*)(klb + row * KROW + f * 64 + g4 * 16);
          sa = E::mma(ka, qf[f], sa);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[j] = sa[j];
        nv = 4;
      }
      // lane holds keys c0 + kb + g4*nv + j for query column `col`
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < nv) {
          const int key = c0 + kb + g4 * nv + j;
          sv[j] = (key < cend && key <= key_lim) ? sv[j] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sv[j]);
        }
      }
      mx = wave_xor_max16_32(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_safe);
      float pv[8];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < nv) {
          pv[j] = exp2f(sv[j] - m_safe);
          psum += pv[j];
        }
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < NDT; ++t) o[t] *= alpha;
      const u32x4 pf = f_to_frag<T>(pv);
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        const u32x4 vf = *(const u32x4*)(vlb + (t * 16 + col) * VROW + kb * ES + g4 * 16);
        o[t] = E::mma(vf, pf, o[t]);
      }
    }
  };

  const int nchunks = (k1 - k0 + CHUNK_KEYS - 1) / CHUNK_KEYS;   // >= 1
  auto cbeg = [&](int c) { return k0 + c * CHUNK_KEYS; };
  auto cfin = [&](int c) { return min(k1, k0 + (c + 1) * CHUNK_KEYS); };
  Regs r0, r1;
  gload(r0, cbeg(0));
  gload(r1, cbeg(nchunks > 1 ? 1 : 0));   // a one-chunk split loads it twice
  lstore(r0, 0, cbeg(0), cfin(0));
  __syncthreads();
  // Steady state, loads unconditional: chunk c in LDS buffer 0, chunk c+1
  // in flight in r1, and chunks c+2 and c+3 exist.
  int c = 0;
  for (; c + 3 < nchunks; c += 2) {
    gload(r0, cbeg(c + 2));
    compute(cbeg(c), cfin(c), 0);
    lstore(r1, 1, cbeg(c + 1), cfin(c + 1));
    __syncthreads();
    gload(r1, cbeg(c + 3));
    compute(cbeg(c + 1), cfin(c + 1), 1);
    lstore(r0, 0, cbeg(c + 2), cfin(c + 2));
    __syncthreads();
  }
  // The last one to three chunks: c in buffer 0, c+1 (if any) in r1.
  if (c + 2 < nchunks) gload(r0, cbeg(c + 2));
  compute(cbeg(c), cfin(c), 0);
  if (c + 1 < nchunks) {
    lstore(r1, 1, cbeg(c + 1), cfin(c + 1));
    __syncthreads();
    compute(cbeg(c + 1), cfin(c + 1), 1);
    if (c + 2 < nchunks) {
      lstore(r0, 0, cbeg(c + 2), cfin(c + 2));
      __syncthreads();
      compute(cbeg(c + 2), cfin(c + 2), 0);
    }
  }
  l_run = wave_xor_sum16_32(l_run);

  // o[t][j] = O^T[d = 16t + 4*g4 + j][query column col]; every split writes
  // its partial (m, l, O); attn_combine merges them in split order.
  if (qg >= a.qgroups) return;   // padding query group of an odd count
  const size_t unit = ((size_t)b * a.nkv + g) * a.qgroups + qg;
  const size_t wstride = (size_t)D * 16 + 32;
  float* pp = a.part + ((unit * a.max_splits + s) * 4 + wave) * wstride;
#pragma unroll
  for (int t = 0; t < NDT; ++t) *(f32x4*)(pp + (t * 64 + lane) * 4) = o[t];
  if (g4 == 0) {
    pp[D * 16 + col] = m_run;
    pp[D * 16 + 16 + col] = l_run;
  }
}

// One workgroup per (sequence, KV head, query group, 16-row d-tile), 16
// waves: wave w handles query tile 4*qg + w%4 over the quarter w/4 of the
// splits (its loads all issued at once), then the quarters are merged in
// order through LDS.  Writes its part of o (frag layout of the model type T
// over nq*d, input of the output projection).
template <typename T, int D>
__global__ __launch_bounds__(1024) void attn_combine_kernel(AttnArgs a, Frag out) {
  constexpr int NDT = D / 16;
  constexpr int BATCH = 8;
  __shared__ float sm[4][4][64], sl[4][4][64];
  __shared__ f32x4 so[4][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qt = wave & 3, quarter = wave >> 2;
  const int g4 = lane >> 4, col = lane & 15;
  int u = blockIdx.x;
  const int t = u % NDT;
  u /= NDT;
  const int qg = u % a.qgroups;
  u /= a.qgroups;
  const int g = u % a.nkv;
  const int b = u / a.nkv;
  const int ctx_len = a.seqs[b].ctx_len;
  int n_cs, n_s;
  attn_split_counts(a, ctx_len, n_cs, n_s);
  const int per = (n_s + 3) / 4;
  const int s_begin = min(n_s, quarter * per), s_end = min(n_s, s_begin + per);
  const size_t unit = ((size_t)b * a.nkv + g) * a.qgroups + qg;
  const size_t wstride = (size_t)D * 16 + 32;
  const float* base = a.part + (unit * a.max_splits * 4 + qt) * wstride;
  const size_t sstride = 4 * wstride;   // next split, same query tile
  float M = -INFINITY, L = 0.f;
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = s_begin; s0 < s_end; s0 += BATCH) {
    float ms[BATCH], ls[BATCH];
    f32x4 os[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      if (s0 + k < s_end) {
        const float* pp = base + (s0 + k) * sstride;
        ms[k] = gld(pp + D * 16 + col);
        ls[k] = gld(pp + D * 16 + 16 + col);
        os[k] = gld((const f32x4*)(pp + (t * 64 + lane) * 4));
      } else {
        ms[k] = -INFINITY;
        ls[k] = 0.f;
        os[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      if (ms[k] == -INFINITY) continue;
      const float Mn = fmaxf(M, ms[k]);
      const float a0 = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
      const float a1 = exp2f(ms[k] - Mn);
      L = L * a0 + ls[k] * a1;
      o = o * a0 + os[k] * a1;
      M = Mn;
    }
  }
  sm[quarter][qt][lane] = M;
  sl[quarter][qt][lane] = L;
  so[quarter][qt][lane] = o;
  __syncthreads();
  if (quarter != 0) return;
  M = -INFINITY;
  L = 0.f;
  o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float mk = sm[k][qt][lane];
    if (mk == -INFINITY) continue;
    const float Mn = fmaxf(M, mk);
    const float a0 = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
    const float a1 = exp2f(mk - Mn);
    L = L * a0 + sl[k][qt][lane] * a1;
    o = o * a0 + so[k][qt][lane] * a1;
    M = Mn;
  }
  const int rep = a.nq / a.nkv;
  const int r = (qg * 4 + qt) * 16 + col;
  if (r >= a.K * rep) return;
  const int h = g * rep + r / a.K, i = r % a.K;
  const float inv = 1.f / L;
  float v[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
  frag_store<T, 4>(out, b * a.K + i, h * D + t * 16 + g4 * 4, v);
}

// (sequence, KV head, split) units padded to a multiple of 8, times the
// workgroups of query groups (QG per workgroup)
static unsigned attn_grid(const AttnArgs& a, int qg_per_wg) {
  const unsigned units = (unsigned)a.B * a.nkv * a.max_splits;
  return (units + 7u) / 8u * 8u * (unsigned)((a.qgroups + qg_per_wg - 1) / qg_per_wg);
}

template <typename T>
hipError_t launch_attention(const AttnArgs& a_in, hipStream_t s) {
  AttnArgs a = a_in;
  // two query groups per workgroup (eight waves) whenever there are several:
  // each staged K/V chunk then serves 128 query rows
  const int QG = a_in.qgroups > 1 ? 2 : 1;
  unsigned nblk = attn_grid(a, QG);   // a multiple of 8
  if (a.warm.w) {
    a.warm.first = (int)nblk;
    nblk += (unsigned)a.warm.consumers;
  }
  dim3 grid(nblk);
  switch (a.d * 4 + QG) {
    case 64 * 4 + 1: hipLaunchKernelGGL((attention_kernel<T, 64, 1>), grid, dim3(256), 0, s, a); break;
    case 64 * 4 + 2: hipLaunchKernelGGL((attention_kernel<T, 64, 2>), grid, dim3(512), 0, s, a); break;
    case 128 * 4 + 1: hipLaunchKernelGGL((attention_kernel<T, 128, 1>), grid, dim3(256), 0, s, a); break;
    case 128 * 4 + 2: hipLaunchKernelGGL((attention_kernel<T, 128, 2>), grid, dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_attention<f16_t>(const AttnArgs&, hipStream_t);
template hipError_t launch_attention<float>(const AttnArgs&, hipStream_t);

template <typename CT, typename T>
hipError_t launch_attn_combine(const AttnArgs& a, Frag o, hipStream_t s) {
  dim3 grid((unsigned)a.B * a.nkv * a.qgroups * (a.d / 16));
  switch (a.d) {
    case 64: hipLaunchKernelGGL((attn_combine_kernel<T, 64>), grid, dim3(1024), 0, s, a, o); break;
    case 128: hipLaunchKernelGGL((attn_combine_kernel<T, 128>), grid, dim3(1024), 0, s, a, o); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template hipError_t launch_attn_combine<f16_t, bf16_t>(const AttnArgs&, Frag, hipStream_t);
template hipError_t launch_attn_combine<float, float>(const AttnArgs&, Frag, hipStream_t);

}  // namespace dflash
