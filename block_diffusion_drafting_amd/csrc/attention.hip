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
// Work unit: sequence b, KV head g, one to four query groups of up to four
// 16-row query tiles (rows = block position x query head sharing g), and
// one split of the key range (its partial result goes to a buffer that
// attn_combine merges in split order).  A split is a run of 64-key chunks;
// each chunk is staged in LDS once and read by every wave of the workgroup,
// and the loads of the next chunks are in flight while the current one is
// computed.  attention_kernel stages chunks through two register sets into
// padded LDS rows (one 4-wave query group, two groups on 8 waves, or four
// groups on 8 waves of two query tiles each at head_dim 64);
// attention_mq_kernel (fp16, head_dim 128, at least four query groups)
// loads them straight into four LDS stages, its waves carrying two query
// tiles each.  S^T = K Q^T and O^T += V^T P^T run on MFMA; the softmax is
// online per query column in fp32, with the scale and log2(e) folded into
// the exponent of the hardware 2^x and the rescaling of O done lazily.  For
// 2-byte operands the two 16-key S^T tiles of a 32-key step hold keys in
// the order that makes each lane's probabilities the B-fragment of the P.V
// product directly.
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

// Split partials, per (sequence, KV head, query group, split, wave): O^T / l
// of the wave's 16 query columns (d x 16, in the MFMA accumulator layout:
// lane l, d tile t holds four values at element (t * 64 + l) * 4), then
// m[16] and l[16] in fp32.  O / l is a convex combination of V rows, so
// |O / l| is at most the largest |V|.  The four-query-group kernel keeps it
// in fp16 (its V is fp16; 11 significant bits against the 8 of the bf16
// output the merge writes), halving the traffic of its large partials; the
// register-staged kernel, whose few partials are merged at the latency of a
// round trip either way, keeps fp32 (PB: bytes per element of O / l).
template <int PB, int D>
constexpr int part_wave_floats() { return D * 16 * PB / 4 + 32; }

size_t attn_part_floats(int B, int nkv, int qgroups, int max_splits, int d, int part_o_bytes) {
  const size_t wave = (size_t)d * 16 * part_o_bytes / 4 + 32;
  return (size_t)B * nkv * qgroups * max_splits * 4 * wave;
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// d tile t of a wave's partial: this lane's four values of O^T, times inv
// (1 / l of the lane's query column)
template <int PB>
__device__ __forceinline__ void store_part_o(float* pp, int t, int lane, f32x4 o, float inv) {
  if constexpr (PB == 2) {
    const f16x4 h = {(_Float16)(o[0] * inv), (_Float16)(o[1] * inv), (_Float16)(o[2] * inv), (_Float16)(o[3] * inv)};
    *(u32x2*)((uint8_t*)pp + (size_t)(t * 64 + lane) * 8) = __builtin_bit_cast(u32x2, h);
  } else {
    *(f32x4*)(pp + (t * 64 + lane) * 4) = o * inv;
  }
}
template <int PB>
__device__ __forceinline__ f32x4 load_part_o(const float* pp, int t, int lane) {
  if constexpr (PB == 2) {
    const f16x4 h = __builtin_bit_cast(f16x4, gld((const u32x2*)((const uint8_t*)pp + (size_t)(t * 64 + lane) * 8)));
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  } else {
    return gld((const f32x4*)(pp + (t * 64 + lane) * 4));
  }
}

// 16-byte nontemporal (streaming) global load.
__device__ __forceinline__ u32x4 gld16_nt(const void* p) { return __builtin_nontemporal_load((gu32x4*)p); }

// Two waves per SIMD (two 4-wave or one 8-wave workgroup per compute unit,
// as the grid is planned): at most 256 registers per wave.  QG: 4-wave
// groups of the workgroup (1 or 2); QT: query tiles per wave (1 or 2).  A
// workgroup serves QG * QT query groups of 64 rows, and with QT = 2 every K
// or V^T fragment read from LDS feeds two MFMAs.  NT: K/V chunks are loaded
// nontemporally (the context K/V of a block too large to stay in the caches
// between blocks; otherwise the default policy lets it stay there, as the
// weights stream nontemporally).
template <typename T, int D, int QG, int QT, bool NT>
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
  // QG * QT query groups share each staged chunk: tile j of wave w is query
  // tile w % 4 of query group qgp * QG * QT + j * QG + w / 4
  constexpr int GPW = QG * QT;
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & 3;
  const int g4 = lane >> 4, col = lane & 15;
  // Workgroups of the same (sequence, KV head, split) and different query
  // groups read the same keys; blocks are dealt to the 8 XCDs round-robin,
  // so they are numbered to share blockIdx % 8 (one L2) -- see attn_grid.
  const int nqgp = (a.qgroups + GPW - 1) / GPW;
  const int lo = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  int qg[QT];
#pragma unroll
  for (int j = 0; j < QT; ++j) qg[j] = (rest % nqgp) * GPW + j * QG + (int)(threadIdx.x >> 8);
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

  // query rows of tile j: r = qtile*16 + col -> head h, block row i
  const int rep = a.nq / a.nkv;
  const int nrows = a.K * rep;
  u32x4 qf[QT][NFD];
  int key_lim[QT];
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    const int r = (qg[j] * 4 + wave) * 16 + col;
    const bool row_ok = qg[j] < a.qgroups && r < nrows;
    const int h = g * rep + (row_ok ? r / a.K : 0);
    const int i = row_ok ? r % a.K : 0;
    // causal form: this lane's query (block row i) sees cache keys 0..ctx_len+i
    key_lim[j] = a.causal ? ctx_len + i : 0x7FFFFFFF;
    const T* qp = (const T*)a.q + ((size_t)(b * a.K + i) * a.nq + h) * D;
#pragma unroll
    for (int f = 0; f < NFD; ++f)
      qf[j][f] = row_ok ? gld16(qp + f * E::KB + g4 * E::KPL) : u32x4{0u, 0u, 0u, 0u};
  }

  f32x4 o[QT][NDT];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int j = 0; j < QT; ++j) {
#pragma unroll
    for (int t = 0; t < NDT; ++t) o[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
  }

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
      const uint8_t* src = (const uint8_t*)kbase + ((uint32_t)(c0 + row) * (D * ES) + pc * 16);
      rg.kr[j] = NT ? gld16_nt(src) : gld16(src);
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int t = threadIdx.x + j * NTH;
      const int dr = t / VP_ROW, pc = t % VP_ROW;
      const uint8_t* src = (const uint8_t*)vbase + ((uint32_t)(dr * vstride + c0 + pc * EPP) * ES);
      rg.vr[j] = NT ? gld16_nt(src) : gld16(src);
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
  // online softmax and P.V over chunk [c0, cend) held in LDS buffer buf;
  // each K and V^T fragment read from LDS serves the wave's QT tiles
  auto compute = [&](int c0, int cend, int buf) {
    const uint8_t* klb = kl[buf];
    const uint8_t* vlb = vl[buf];
#pragma unroll
    for (int sub = 0; sub < CHUNK_KEYS / KP; ++sub) {
      const int kb = sub * KP;  // key offset of this P.V step within the chunk
      constexpr int NV = ES == 2 ? 8 : 4;   // keys per lane of this step
      float sv[QT][NV];
      if constexpr (ES == 2) {
        // two S^T tiles: tile A rows -> keys 8*(row/4) + row%4, tile B -> +4
        const int rowA = kb + ((col >> 2) << 3) + (col & 3);
        const int rowB = rowA + 4;
        f32x4 sa[QT], sb[QT];
#pragma unroll
        for (int j = 0; j < QT; ++j) sa[j] = sb[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < NFD; ++f) {
          const u32x4 ka = *(const u32x4*)(klb + rowA * KROW + f * 64 + g4 * 16);
          const u32x4 kb2 = *(const u32x4*)(klb + rowB * KROW + f * 64 + g4 * 16);
#pragma unroll
          for (int j = 0; j < QT; ++j) {
            sa[j] = E::mma(ka, qf[j][f], sa[j]);
            sb[j] = E::mma(kb2, qf[j][f], sb[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < QT; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sv[j][e] = sa[j][e];
            sv[j][4 + e] = sb[j][e];
          }
      } else {
        const int row = kb + col;
        f32x4 sa[QT];
#pragma unroll
        for (int j = 0; j < QT; ++j) sa[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < NFD; ++f) {
          const u32x4 ka = *(const u32x4*)(klb + row * KROW + f * 64 + g4 * 16);
#pragma unroll
          for (int j = 0; j < QT; ++j) sa[j] = E::mma(ka, qf[j][f], sa[j]);
        }
#pragma unroll
        for (int j = 0; j < QT; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[j][e] = sa[j][e];
      }
      // lane holds keys c0 + kb + g4*NV + e for query column `col`; maxima
      // on the raw scores, the scale folded into the exponent (as in
      // attention_mq_kernel)
      const float sc = a.scale_log2;
      u32x4 pf[QT];
#pragma unroll
      for (int j = 0; j < QT; ++j) {
        // every key of the chunk valid and visible to every query of the
        // wave (wave-uniform): no per-element mask
        if (!(cend - c0 == CHUNK_KEYS && __ballot(c0 + CHUNK_KEYS - 1 > key_lim[j]) == 0ull)) {
#pragma unroll
          for (int e = 0; e < NV; ++e) {
            const int key = c0 + kb + g4 * NV + e;
            sv[j][e] = (key < cend && key <= key_lim[j]) ? sv[j][e] : -INFINITY;
          }
        }
        float mx = sv[j][0];
#pragma unroll
        for (int e = 1; e < NV; ++e) mx = fmax_ieee(mx, sv[j][e]);
        mx = wave_xor_max16_32(mx) * sc;
        // lazy rescaling and the hardware 2^x (as in attention_mq_kernel):
        // the reference moves only when a column's maximum exceeds it by
        // more than 8 (log2 units)
        if (__ballot(mx > m_run[j] + 8.f) != 0ull) {   // wave-uniform
          const float m_new = fmax_ieee(m_run[j], mx);
          const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[j] - m_new);
          l_run[j] *= alpha;
#pragma unroll
          for (int t = 0; t < NDT; ++t) o[j][t] *= alpha;
          m_run[j] = m_new;
        }
        const float m_safe = (m_run[j] == -INFINITY) ? 0.f : m_run[j];
        float pv[8];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (e < NV) {
            pv[e] = __builtin_amdgcn_exp2f(fmaf(sv[j][e], sc, -m_safe));
            psum += pv[e];
          }
        }
        l_run[j] += psum;
        if constexpr (ES == 2) {
          // probabilities lie in [0, 2^8]: round to fp16 without the clamp
          const f16x8 ph = {(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3],
                            (_Float16)pv[4], (_Float16)pv[5], (_Float16)pv[6], (_Float16)pv[7]};
          pf[j] = __builtin_bit_cast(u32x4, ph);
        } else {
          pf[j] = f_to_frag<T>(pv);
        }
      }
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        const u32x4 vf = *(const u32x4*)(vlb + (t * 16 + col) * VROW + kb * ES + g4 * 16);
#pragma unroll
        for (int j = 0; j < QT; ++j) o[j][t] = E::mma(vf, pf[j], o[j][t]);
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
    lds_barrier();
    gload(r1, cbeg(c + 3));
    compute(cbeg(c + 1), cfin(c + 1), 1);
    lstore(r0, 0, cbeg(c + 2), cfin(c + 2));
    lds_barrier();
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
  // o[j][t][e] = O^T[d = 16t + 4*g4 + e][query column col] of tile j; every
  // split writes its partial (m, l, O / l); attn_combine merges them in
  // split order.  Padding query groups (past the count) write nothing.
  constexpr int PB = 4, WF = part_wave_floats<PB, D>(), MO = WF - 32;
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    const float l_sum = wave_xor_sum16_32(l_run[j]);
    if (qg[j] >= a.qgroups) continue;
    const size_t unit = ((size_t)b * a.nkv + g) * a.qgroups + qg[j];
    float* pp = a.part + ((unit * a.max_splits + s) * 4 + wave) * (size_t)WF;
    const float inv = l_sum > 0.f ? 1.f / l_sum : 0.f;   // (no key seen: l = 0, m = -inf)
#pragma unroll
    for (int t = 0; t < NDT; ++t) store_part_o<PB>(pp, t, lane, o[j][t], inv);
    if (g4 == 0) {
      pp[MO + col] = m_run[j];
      pp[MO + 16 + col] = l_sum;
    }
  }
}

// Attention for many query rows (at least four query groups of 64 rows)
// with fp16 operands and head_dim 128.  The work is bound by the MFMA
// chains and the softmax between them, so each wave carries two 16-row
// query tiles (every K or V^T fragment read from LDS feeds two MFMAs and
// the two tiles' chains interleave) and a workgroup of 8 waves serves four
// query groups.  Two tiles' accumulators leave no registers for data in
// transit, so chunks (64 keys: K rows 16 KiB, V^T columns 16 KiB) are loaded
// straight into one of MQ_STAGES LDS stages by 16-byte-per-lane direct
// loads, MQ_STAGES - 1 chunks in flight while one is computed.  A direct
// load writes 1 KiB of consecutive LDS per wave instruction, so rows are not
// padded; the 16-byte pieces of a row are XOR-permuted instead (the lane's
// global address picks the piece), so that the fragment reads of 16 rows
// hit 16 different bank groups:
//   K stage: row r (key), piece p (16 bytes of d) at r * 256 + 16 * (p ^ kswz(r));
//   V stage: row t (d), piece p (8 keys) at t * 128 + 16 * (p ^ vswz(t)).
// Tile j of wave w is query tile w % 4 of query group 4 * qgp + 2 j + w / 4;
// the split partials have the layout of the register-staged kernel.
constexpr int MQ_STAGES = 4;

__device__ __forceinline__ int kswz(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }
__device__ __forceinline__ int vswz(int t) { return (t >> 1) & 7; }

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void attention_mq_kernel(AttnArgs a) {
  using T = f16_t;
  using E = Elem<T>;
  constexpr int D = 128, QT = 2, NS = MQ_STAGES;
  constexpr int CK = 64;                 // keys per chunk
  constexpr int KBYTES = CK * D * 2;     // 16 KiB of K rows
  constexpr int SBYTES = 2 * KBYTES;     // one stage: K rows and V^T columns
  constexpr int NFD = D * 2 / 64;        // 32-element d steps of S^T = K Q^T
  constexpr int NDT = D / 16;            // 16-row d tiles of O^T
  constexpr int LPW = KBYTES / 1024 / 8; // direct loads per wave per half-stage (2)
  static_assert(NS >= 2 && NS * SBYTES <= 160 * 1024, "stages");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * SBYTES];

  const int w = (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (a.warm.w && (int)blockIdx.x >= a.warm.first) {
    warm_consumer(a.warm, (int)blockIdx.x - a.warm.first, 8, w, lane, (lds_void_t*)(lds + w * 1024));
    return;
  }
  const int g4 = lane >> 4, col = lane & 15;
  const int wave = w & 3;                       // query tile within its group
  const int nqgp = (a.qgroups + 3) / 4;
  const int lo = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  int qg[QT];
#pragma unroll
  for (int j = 0; j < QT; ++j) qg[j] = (rest % nqgp) * 4 + 2 * j + (w >> 2);
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

  const int rep = a.nq / a.nkv;
  const int nrows = a.K * rep;
  u32x4 qf[QT][NFD];
  int key_lim[QT];
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    const int r = (qg[j] * 4 + wave) * 16 + col;
    const bool row_ok = qg[j] < a.qgroups && r < nrows;
    const int h = g * rep + (row_ok ? r / a.K : 0);
    const int i = row_ok ? r % a.K : 0;
    key_lim[j] = a.causal ? ctx_len + i : 0x7FFFFFFF;
    const T* qp = (const T*)a.q + ((size_t)(b * a.K + i) * a.nq + h) * D;
#pragma unroll
    for (int f = 0; f < NFD; ++f)
      qf[j][f] = row_ok ? gld16(qp + f * E::KB + g4 * E::KPL) : u32x4{0u, 0u, 0u, 0u};
  }
  wait_vm<0>();   // the queries, before any direct load is outstanding

  // Direct loads of chunk c into stage c % NS: wave w fills K blocks 2w,
  // 2w+1 (four key rows each) and V^T blocks 2w, 2w+1 (eight d rows each).
  // A chunk starts at a multiple of 64 keys below the row length, which is
  // a multiple of 64 for both the caches (a power of two >= 64) and the
  // block buffers (padded to 64), so every load is in bounds; keys past the
  // split end are masked when computed.  Offsets are 32-bit from the
  // uniform slab base (a slab is under 2^31 bytes, checked where the caches
  // are allocated).
  const uint8_t* kb8 = (const uint8_t*)kbase;
  const uint8_t* vb8 = (const uint8_t*)vbase;
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int blk = w * LPW + j;
    const int kr = blk * 4 + (lane >> 4), kp = (lane & 15) ^ kswz(kr);
    koff[j] = (uint32_t)(kr * D * 2 + kp * 16);
    const int vr = blk * 8 + (lane >> 3), vp = (lane & 7) ^ vswz(vr);
    voff[j] = (uint32_t)(vr * vstride * 2 + vp * 16);
  }
  auto issue = [&](int c) {
    const uint32_t c0 = (uint32_t)(k0 + c * CK);
    uint8_t* st = lds + (c % NS) * SBYTES;
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma16(kb8, c0 * (D * 2) + koff[j], st + (w * LPW + j) * 1024);
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma16(vb8, c0 * 2 + voff[j], st + KBYTES + (w * LPW + j) * 1024);
  };

  f32x4 o[QT][NDT];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int j = 0; j < QT; ++j) {
#pragma unroll
    for (int t = 0; t < NDT; ++t) o[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
  }

  auto compute = [&](int c) {
    const int c0 = k0 + c * CK;
    const int lim = min(k1, c0 + CK) - c0;   // valid keys of the chunk
    const uint8_t* ks = lds + (c % NS) * SBYTES;
    const uint8_t* vs = ks + KBYTES;
#pragma unroll
    for (int kb = 0; kb < CK; kb += 32) {   // one P.V step of 32 keys
      // two S^T tiles: tile A rows -> keys kb + 8*(row/4) + row%4, tile B -> +4
      const int rowA = kb + ((col >> 2) << 3) + (col & 3);
      const int rowB = rowA + 4;
      f32x4 sa[QT], sb[QT];
#pragma unroll
      for (int j = 0; j < QT; ++j) sa[j] = sb[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < NFD; ++f) {
        const int p = f * 4 + g4;
        const u32x4 ka = *(const u32x4*)(ks + rowA * (D * 2) + ((p ^ kswz(rowA)) << 4));
        const u32x4 kb2 = *(const u32x4*)(ks + rowB * (D * 2) + ((p ^ kswz(rowB)) << 4));
#pragma unroll
        for (int j = 0; j < QT; ++j) {
          sa[j] = E::mma(ka, qf[j][f], sa[j]);
          sb[j] = E::mma(kb2, qf[j][f], sb[j]);
        }
      }
      // lane holds keys c0 + kb + 8*g4 + e (e < 8) for query column `col`.
      // Maxima are taken on the raw scores (the scale is positive) and the
      // scale is folded into the exponent: p = 2^(s * scale - m).
      const float sc = a.scale_log2;
      u32x4 pf[QT];
#pragma unroll
      for (int j = 0; j < QT; ++j) {
        float sv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[e] = sa[j][e];
          sv[4 + e] = sb[j][e];
        }
        // every key of the chunk valid and visible to every query of the
        // wave (wave-uniform): no per-element mask
        if (!(lim == CK && __ballot(c0 + CK - 1 > key_lim[j]) == 0ull)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int kk = kb + 8 * g4 + e;
            sv[e] = (kk < lim && c0 + kk <= key_lim[j]) ? sv[e] : -INFINITY;
          }
        }
        float mx = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmax_ieee(mx, sv[e]);
        mx = wave_xor_max16_32(mx) * sc;
        // Lazy rescaling: the reference m_run moves (and O and l are
        // rescaled) only when some column's maximum exceeds it by more than
        // 8 (log2 units), so exponentials stay below 2^8 (safe in fp32 and
        // as fp16 probabilities) and the rescaling, which costs more VALU
        // work than the rest of the step, is skipped once the maxima settle.
        // O / l is the same for any reference; the merge of the splits
        // takes (m, l, O / l) with any reference.
        if (__ballot(mx > m_run[j] + 8.f) != 0ull) {   // wave-uniform
          const float m_new = fmax_ieee(m_run[j], mx);
          const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[j] - m_new);
          l_run[j] *= alpha;
#pragma unroll
          for (int t = 0; t < NDT; ++t) o[j][t] *= alpha;
          m_run[j] = m_new;
        }
        // (the hardware 2^x: arguments lie in [-inf, 8], and a result it
        // flushes below 2^-126 is negligible beside the column's largest
        // probability, which is at least 1)
        const float m_safe = (m_run[j] == -INFINITY) ? 0.f : m_run[j];
        float pv[8];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], sc, -m_safe));
          psum += pv[e];
        }
        l_run[j] += psum;
        // probabilities lie in [0, 2^8]: round to fp16 without the clamp
        const f16x8 ph = {(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3],
                          (_Float16)pv[4], (_Float16)pv[5], (_Float16)pv[6], (_Float16)pv[7]};
        pf[j] = __builtin_bit_cast(u32x4, ph);
      }
      const int p = (kb >> 3) + g4;
      if (lim == CK) {   // (uniform)
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          const int dr = t * 16 + col;
          const u32x4 vf = *(const u32x4*)(vs + dr * (CK * 2) + ((p ^ vswz(dr)) << 4));
#pragma unroll
          for (int j = 0; j < QT; ++j) o[j][t] = E::mma(vf, pf[j], o[j][t]);
        }
      } else {
        // V^T columns past the split end hold whatever the cache holds
        // there: zero them so that 0 * V stays 0
        const int vlim = lim - (kb + 8 * g4);   // valid keys of this lane's eight
        uint32_t keep[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          keep[e2] = (2 * e2 + 1 < vlim) ? 0xFFFFFFFFu : (2 * e2 < vlim) ? 0x0000FFFFu : 0u;
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          const int dr = t * 16 + col;
          u32x4 vf = *(const u32x4*)(vs + dr * (CK * 2) + ((p ^ vswz(dr)) << 4));
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) vf[e2] &= keep[e2];
#pragma unroll
          for (int j = 0; j < QT; ++j) o[j][t] = E::mma(vf, pf[j], o[j][t]);
        }
      }
    }
  };

  // Pipeline: chunks 0 .. NS-2 in flight; at chunk c wait for it (the loads
  // of later chunks may stay outstanding), barrier (it is visible to every
  // wave, and every wave is done with chunk c - 1), issue chunk c + NS - 1
  // into the stage chunk c - 1 used, compute chunk c.
  const int nchunks = (k1 - k0 + CK - 1) / CK;   // >= 1
#pragma unroll
  for (int c = 0; c < NS - 1; ++c)
    if (c < nchunks) issue(c);
  for (int c = 0; c < nchunks; ++c) {
    const int later = min(NS - 2, nchunks - 1 - c);   // chunks issued after c
    static_assert(NS - 2 <= 3, "wait ladder");
    if (later == 3) wait_vm<2 * LPW * 3>();
    else if (later == 2) wait_vm<2 * LPW * 2>();
    else if (later == 1) wait_vm<2 * LPW>();
    else wait_vm<0>();
    lds_barrier();
    if (c + NS - 1 < nchunks) issue(c + NS - 1);
    compute(c);
  }
  wait_vm<0>();   // (none outstanding: the last chunk waited for all)

  constexpr int PB = 2, WF = part_wave_floats<PB, D>(), MO = WF - 32;
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    const float l_sum = wave_xor_sum16_32(l_run[j]);
    if (qg[j] >= a.qgroups) continue;   // padding query group
    const size_t unit = ((size_t)b * a.nkv + g) * a.qgroups + qg[j];
    float* pp = a.part + ((unit * a.max_splits + s) * 4 + wave) * (size_t)WF;
    const float inv = l_sum > 0.f ? 1.f / l_sum : 0.f;   // (no key seen: l = 0, m = -inf)
#pragma unroll
    for (int t = 0; t < NDT; ++t) store_part_o<PB>(pp, t, lane, o[j][t], inv);
    if (g4 == 0) {
      pp[MO + col] = m_run[j];
      pp[MO + 16 + col] = l_sum;
    }
  }
}

// One workgroup per (sequence, KV head, query group, DT 16-row d tiles)
// with 4 Q waves: wave w handles query tile 4*qg + w%4 over the part w/4 of
// Q of the splits (the running max and sum of a query column are shared by
// its d tiles), then the parts are merged in order through LDS.  Q = 4 when
// there are many splits, 1 (four waves, no LDS merge) when there are at most
// eight.  Writes its part of o (frag layout of the model type T over nq*d,
// input of the output projection).
template <typename T, int D, int Q, int PB, int DT>
__global__ __launch_bounds__(256 * Q) void attn_combine_kernel(AttnArgs a, Frag out) {
  constexpr int NDT = D / 16, NG = NDT / DT;
  static_assert(NDT % DT == 0, "d tiles per workgroup");
  constexpr int BATCH = 8;
  __shared__ float sm[Q][4][64], sl[Q][4][64];
  __shared__ f32x4 so[Q][4][DT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qt = wave & 3, quarter = wave >> 2;
  const int g4 = lane >> 4, col = lane & 15;
  int u = blockIdx.x;
  const int t0 = (u % NG) * DT;
  u /= NG;
  const int qg = u % a.qgroups;
  u /= a.qgroups;
  const int g = u % a.nkv;
  const int b = u / a.nkv;
  const int ctx_len = a.seqs[b].ctx_len;
  int n_cs, n_s;
  attn_split_counts(a, ctx_len, n_cs, n_s);
  const int per = (n_s + Q - 1) / Q;
  const int s_begin = min(n_s, quarter * per), s_end = min(n_s, s_begin + per);
  const size_t unit = ((size_t)b * a.nkv + g) * a.qgroups + qg;
  constexpr int WF = part_wave_floats<PB, D>(), MO = WF - 32;
  const float* base = a.part + (unit * a.max_splits * 4 + qt) * (size_t)WF;
  const size_t sstride = 4 * (size_t)WF;   // next split, same query tile
  float M = -INFINITY, L = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = s_begin; s0 < s_end; s0 += BATCH) {
    // (loads under a branch: the compiler waits for each split's before the
    // next split's, and yet measured faster than a batch of unconditional
    // loads that re-read the last split for the indices past the end)
    float ms[BATCH], ls[BATCH];
    f32x4 os[BATCH][DT];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      if (s0 + k < s_end) {
        const float* pp = base + (s0 + k) * sstride;
        ms[k] = gld(pp + MO + col);
        ls[k] = gld(pp + MO + 16 + col);
#pragma unroll
        for (int d = 0; d < DT; ++d) os[k][d] = load_part_o<PB>(pp, t0 + d, lane);   // O / l of split s0 + k
      } else {
        ms[k] = -INFINITY;
        ls[k] = 0.f;
#pragma unroll
        for (int d = 0; d < DT; ++d) os[k][d] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      // a split that saw no key of this column has m = -inf, l = 0, O / l = 0
      if (ms[k] == -INFINITY) continue;
      const float Mn = fmaxf(M, ms[k]);
      const float a0 = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
      const float a1 = exp2f(ms[k] - Mn);
      const float w = ls[k] * a1;
      L = L * a0 + w;
#pragma unroll
      for (int d = 0; d < DT; ++d) o[d] = o[d] * a0 + os[k][d] * w;
      M = Mn;
    }
  }
  if constexpr (Q > 1) {
    sm[quarter][qt][lane] = M;
    sl[quarter][qt][lane] = L;
#pragma unroll
    for (int d = 0; d < DT; ++d) so[quarter][qt][d][lane] = o[d];
    __syncthreads();
    if (quarter != 0) return;
    M = -INFINITY;
    L = 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < Q; ++k) {
      const float mk = sm[k][qt][lane];
      if (mk == -INFINITY) continue;
      const float Mn = fmaxf(M, mk);
      const float a0 = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
      const float a1 = exp2f(mk - Mn);
      L = L * a0 + sl[k][qt][lane] * a1;
#pragma unroll
      for (int d = 0; d < DT; ++d) o[d] = o[d] * a0 + so[k][qt][d][lane] * a1;
      M = Mn;
    }
  }
  const int rep = a.nq / a.nkv;
  const int r = (qg * 4 + qt) * 16 + col;
  if (r >= a.K * rep) return;
  const int h = g * rep + r / a.K, i = r % a.K;
  const float inv = 1.f / L;
#pragma unroll
  for (int d = 0; d < DT; ++d) {
    float v[4] = {o[d][0] * inv, o[d][1] * inv, o[d][2] * inv, o[d][3] * inv};
    frag_store<T, 4>(out, b * a.K + i, h * D + (t0 + d) * 16 + g4 * 4, v);
  }
}

// (sequence, KV head, split) units padded to a multiple of 8, times the
// workgroups of query groups (QG per workgroup)
static unsigned attn_grid(const AttnArgs& a, int qg_per_wg) {
  const unsigned units = (unsigned)a.B * a.nkv * a.max_splits;
  return (units + 7u) / 8u * 8u * (unsigned)((a.qgroups + qg_per_wg - 1) / qg_per_wg);
}

template <typename T, int D, int QG, int QT>
static void launch_ak(bool nt, dim3 grid, hipStream_t s, const AttnArgs& a) {
  if (nt) hipLaunchKernelGGL((attention_kernel<T, D, QG, QT, true>), grid, dim3(256 * QG), 0, s, a);
  else hipLaunchKernelGGL((attention_kernel<T, D, QG, QT, false>), grid, dim3(256 * QG), 0, s, a);
}

template <typename T>
hipError_t launch_attention(const AttnArgs& a_in, hipStream_t s) {
  AttnArgs a = a_in;
  // query groups per workgroup (see attn_groups_per_wg): one 4-wave group,
  // two (eight waves), or four (eight waves of two query tiles each)
  const int GPW = attn_groups_per_wg((int)sizeof(T), a_in.qgroups);
  unsigned nblk = attn_grid(a, GPW);   // a multiple of 8
  if (a.warm.w) {
    a.warm.first = (int)nblk;
    nblk += (unsigned)a.warm.consumers;
  }
  dim3 grid(nblk);
  const bool nt = a.stream != 0;
  switch (a.d * 8 + GPW) {
    case 64 * 8 + 1: launch_ak<T, 64, 1, 1>(nt, grid, s, a); break;
    case 64 * 8 + 2: launch_ak<T, 64, 2, 1>(nt, grid, s, a); break;
    case 128 * 8 + 1: launch_ak<T, 128, 1, 1>(nt, grid, s, a); break;
    case 128 * 8 + 2: launch_ak<T, 128, 2, 1>(nt, grid, s, a); break;
    case 64 * 8 + 4:
      if constexpr (sizeof(T) == 2) launch_ak<T, 64, 2, 2>(nt, grid, s, a);
      else return hipErrorInvalidValue;
      break;
    case 128 * 8 + 4:
      if constexpr (sizeof(T) == 2) hipLaunchKernelGGL(attention_mq_kernel, grid, dim3(512), 0, s, a);
      else return hipErrorInvalidValue;
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_attention<f16_t>(const AttnArgs&, hipStream_t);
template hipError_t launch_attention<float>(const AttnArgs&, hipStream_t);

template <typename T, int D, int Q, int PB>
static void launch_comb(int dt, unsigned units, hipStream_t s, const AttnArgs& a, Frag o) {
  constexpr int NDT = D / 16;
  if (dt == 2) hipLaunchKernelGGL((attn_combine_kernel<T, D, Q, PB, 2>), dim3(units * (NDT / 2)), dim3(256 * Q), 0, s, a, o);
  else hipLaunchKernelGGL((attn_combine_kernel<T, D, Q, PB, 1>), dim3(units * NDT), dim3(256 * Q), 0, s, a, o);
}

template <typename CT, typename T>
hipError_t launch_attn_combine(const AttnArgs& a, Frag o, hipStream_t s) {
  const unsigned units = (unsigned)a.B * a.nkv * a.qgroups;
  const bool few = a.max_splits <= 8;   // one part: four waves per workgroup
  const int pb = attn_part_o_bytes((int)sizeof(CT), a.qgroups, a.d);
  // Two d tiles per 16-wave workgroup when one per workgroup would give more
  // workgroups than CUs: their dispatch spread over 4.3 us at K = 128 (512
  // workgroups; merge 62 -> 52 us per block with two tiles), while a grid
  // under one workgroup per CU is faster with one tile each (K = 16: 41
  // against 46 us per block with two).  Four tiles spill registers.
  const int dt = !few && units * (unsigned)(a.d / 16) > 256u ? 2 : 1;
  switch (a.d * 4 + (few ? 1 : 0) + (pb == 2 ? 2 : 0)) {
    case 64 * 4: launch_comb<T, 64, 4, 4>(dt, units, s, a, o); break;
    case 64 * 4 + 1: launch_comb<T, 64, 1, 4>(1, units, s, a, o); break;
    case 128 * 4: launch_comb<T, 128, 4, 4>(dt, units, s, a, o); break;
    case 128 * 4 + 1: launch_comb<T, 128, 1, 4>(1, units, s, a, o); break;
    case 128 * 4 + 2: launch_comb<T, 128, 4, 2>(dt, units, s, a, o); break;
    case 128 * 4 + 3: launch_comb<T, 128, 1, 2>(1, units, s, a, o); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template hipError_t launch_attn_combine<f16_t, bf16_t>(const AttnArgs&, Frag, hipStream_t);
template hipError_t launch_attn_combine<float, float>(const AttnArgs&, Frag, hipStream_t);

}  // namespace dflash
