// Small kernels of the draft-block path: block embedding, greedy acceptance,
// weight repacking, projection row mapping and buffer growth.
#include "kernels.h"

namespace dflash {

// ---------------------------------------------------------------------------
// (a4) block embedding.  One workgroup per 16 block rows and 64 columns:
// x = E[id] (the fp32 residual stream), xg = x * gain (frag layout, input
// of the first normed product), ssq[c][m] = sum of x^2 over columns
// 64c..64c+63, keys[m] = 0 (argmax of this block).
// Thread t: row (t / 16) of the tile, columns 4*(t % 16) .. +3 of the slab.
// ---------------------------------------------------------------------------
struct EmbedArgs {
  const int32_t* ids;
  const void* embed;
  const float* gain;
  int M, H, V;
  float* x;
  Frag xg;
  float* ssq;
  unsigned long long* keys;
};

// Block (bx, by) of the embedding: rows 16 bx.., columns 64 by..
template <typename T>
__device__ __forceinline__ void embed_block(const EmbedArgs& a, int bx, int by) {
  const int32_t* ids = a.ids;
  const T* embed = (const T*)a.embed;
  const float* gain = a.gain;
  const int M = a.M, H = a.H, V = a.V;
  float* x = a.x;
  const Frag& xg = a.xg;
  const int m = bx * 16 + (threadIdx.x >> 4);
  const int n0 = by * 64 + (threadIdx.x & 15) * 4;
  float ss = 0.f;
  if (m < M) {
    int id = ids[m];
    id = id < 0 ? 0 : (id >= V ? V - 1 : id);
    const T* row = embed + (size_t)id * H + n0;
    float v[4], w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = Elem<T>::to_f(row[j]);
      w[j] = v[j] * gain[n0 + j];
      ss += v[j] * v[j];
    }
    *(f32x4*)(x + (size_t)m * H + n0) = f32x4{v[0], v[1], v[2], v[3]};
    frag_store<T, 4>(xg, m, n0, w);
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if (m < M && (threadIdx.x & 15) == 0) {
    a.ssq[(size_t)by * M + m] = ss;
    if (by == 0) a.keys[m] = 0ull;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
  embed_block<T>(a, blockIdx.x, blockIdx.y);
}

template <typename T>
hipError_t launch_embed(const int32_t* ids, const void* embed, const float* gain, int M, int H,
                        int V, float* x, Frag xg, float* ssq, unsigned long long* keys,
                        hipStream_t s) {
  dim3 grid((M + 15) / 16, H / 64);
  const EmbedArgs a{ids, embed, gain, M, H, V, x, xg, ssq, keys};
  hipLaunchKernelGGL((embed_kernel<T>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
template hipError_t launch_embed<bf16_t>(const int32_t*, const void*, const float*, int, int, int,
                                         float*, Frag, float*, unsigned long long*, hipStream_t);
template hipError_t launch_embed<float>(const int32_t*, const void*, const float*, int, int, int,
                                        float*, Frag, float*, unsigned long long*, hipStream_t);

// Sum over splits of a partial output tile element quad: rows of m-tile mt,
// output columns n0..n0+3 (n0 % 4 == 0), in split order.
__device__ __forceinline__ f32x4 sum_parts(const float* part, int nsplit, int ntiles, int mtiles,
                                           int m, int n0) {
  const int tile = n0 >> 4;
  const int lane = ((n0 & 15) >> 2) * 16 + (m & 15);
  const size_t stride = (size_t)ntiles * mtiles * 64 * 4;   // floats between splits
  const float* p = part + (((size_t)tile * mtiles + (m >> 4)) * 64 + lane) * 4;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 4 <= nsplit; s += 4) {   // independent loads, added in split order
    const f32x4 a0 = *(const f32x4*)(p + (s + 0) * stride);
    const f32x4 a1 = *(const f32x4*)(p + (s + 1) * stride);
    const f32x4 a2 = *(const f32x4*)(p + (s + 2) * stride);
    const f32x4 a3 = *(const f32x4*)(p + (s + 3) * stride);
    acc += a0;
    acc += a1;
    acc += a2;
    acc += a3;
  }
  for (; s < nsplit; ++s) acc += *(const f32x4*)(p + s * stride);
  return acc;
}

// ---------------------------------------------------------------------------
// Residual add of a product split over k, and the next RMSNorm's inputs:
// x += sum_s part_s (split order); xg = x * gain (frag layout); ssq per 64
// columns.  Grid (m-tiles, H/64), thread layout as in embed_kernel.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void resid_norm_kernel(const float* part, int nsplit, int mtiles,
                                                         int M, int H, float* x,
                                                         const float* gain, Frag xg, float* ssq) {
  // block b: m-tile b % mtiles, 64-column group b / mtiles
  const int mtile = (int)blockIdx.x % mtiles, cgrp = (int)blockIdx.x / mtiles;
  const int m = mtile * 16 + (threadIdx.x >> 4);
  const int n0 = cgrp * 64 + (threadIdx.x & 15) * 4;
  float ss = 0.f;
  if (m < M) {
    const f32x4 add = sum_parts(part, nsplit, H / 16, mtiles, m, n0);
    f32x4* xp = (f32x4*)(x + (size_t)m * H + n0);
    const f32x4 v = *xp + add;
    *xp = v;
    float w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = v[j] * gain[n0 + j];
      ss += v[j] * v[j];
    }
    frag_store<T, 4>(xg, m, n0, w);
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if (m < M && (threadIdx.x & 15) == 0) ssq[(size_t)cgrp * M + m] = ss;
}

template <typename T>
hipError_t launch_resid_norm(const float* part, int nsplit, int mtiles, int M, int H, float* x,
                             const float* gain, Frag xg, float* ssq, hipStream_t s) {
  const unsigned nblk = (unsigned)(mtiles * (H / 64));
  hipLaunchKernelGGL((resid_norm_kernel<T>), dim3(nblk), dim3(256), 0, s, part, nsplit, mtiles, M, H, x,
                     gain, xg, ssq);
  return hipGetLastError();
}
template hipError_t launch_resid_norm<bf16_t>(const float*, int, int, int, int, float*, const float*,
                                              Frag, float*, hipStream_t);
template hipError_t launch_resid_norm<float>(const float*, int, int, int, int, float*, const float*,
                                             Frag, float*, hipStream_t);

// ---------------------------------------------------------------------------
// (a1)-(a2) context projection split over k: c = sum_s part_s, written to
// the sequence's context buffer row (fp32) and to the frag staging that
// feeds the KV injection product.  The row -> (sequence, slot, position) map
// is computed here from the host's row starts and context lengths (passed
// by value) and stored for the KV injection; block (0, 0) then advances the
// device copy of every context length (nothing in this launch reads it).
// ---------------------------------------------------------------------------
__device__ __forceinline__ RowMap map_row(const RowInfo& ri, int B, int j, const int32_t* positions) {
  int lo = 0, hi = B;  // b with start[b] <= j < start[b + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ri.start[mid] <= j) lo = mid; else hi = mid;
  }
  RowMap r;
  r.b = lo;
  r.slot = ri.ctx0[lo] + (j - ri.start[lo]);
  r.pos = positions ? positions[j] : r.slot;
  r.pad = 0;
  return r;
}

struct FcFinArgs {
  const float* part;
  int nsplit, mtiles, M, H;
  RowInfo ri;
  int B;
  const int32_t* positions;
  RowMap* rowmap;
  DevSeq* seqs;
  Frag cbuf;
  int row0;
};

// Block (bx, by): rows 16 bx.., columns 64 by..
template <typename T>
__device__ __forceinline__ void fc_finalize_block(const FcFinArgs& a, int bx, int by) {
  const int B = a.B, M = a.M, H = a.H;
  if (bx == 0 && by == 0)
    for (int b = threadIdx.x; b < B; b += blockDim.x) a.seqs[b].ctx_len = a.ri.ctx0[b] + a.ri.start[b + 1] - a.ri.start[b];
  const int m = bx * 16 + (threadIdx.x >> 4);
  const int n0 = by * 64 + (threadIdx.x & 15) * 4;
  if (m >= M) return;
  const RowMap rm = map_row(a.ri, B, m, a.positions);
  if (by == 0 && (threadIdx.x & 15) == 0) a.rowmap[m] = rm;
  const f32x4 c = sum_parts(a.part, a.nsplit, H / 16, a.mtiles, m, n0);
  *gp((f32x4*)((float*)a.seqs[rm.b].ctxbuf + (size_t)rm.slot * H + n0)) = c;
  float v[4] = {c[0], c[1], c[2], c[3]};
  frag_store<T, 4>(a.cbuf, a.row0 + m, n0, v);
}

template <typename T>
__global__ __launch_bounds__(256) void fc_finalize_kernel(FcFinArgs a) {
  fc_finalize_block<T>(a, blockIdx.x, blockIdx.y);
}

template <typename T>
hipError_t launch_fc_finalize(const float* part, int nsplit, int mtiles, int M, int H, const RowInfo& ri, int B,
                              const int32_t* positions, RowMap* rowmap, DevSeq* seqs, Frag cbuf,
                              int row0, hipStream_t s) {
  if (B > DFLASH_ROWMAP_MAX) return hipErrorInvalidValue;
  dim3 grid((M + 15) / 16, H / 64);
  const FcFinArgs a{part, nsplit, mtiles, M, H, ri, B, positions, rowmap, seqs, cbuf, row0};
  hipLaunchKernelGGL((fc_finalize_kernel<T>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Blocks [0, nf): the context rows (fc_finalize_block), then the block
// rows' embedding (embed_block); both grids are m-tile major.
template <typename T>
__global__ __launch_bounds__(256) void fc_finalize_embed_kernel(FcFinArgs f, EmbedArgs e) {
  const int fx = (f.M + 15) / 16, nf = fx * (f.H / 64);
  const int b = blockIdx.x;
  if (b < nf) {
    fc_finalize_block<T>(f, b % fx, b / fx);
  } else {
    const int ex = (e.M + 15) / 16, k = b - nf;
    embed_block<T>(e, k % ex, k / ex);
  }
}

template <typename T>
hipError_t launch_fc_finalize_embed(const float* part, int nsplit, int mtiles, int M, int H, const RowInfo& ri,
                                    int B, RowMap* rowmap, DevSeq* seqs, Frag cbuf, int row0,
                                    const int32_t* ids, const void* embed, const float* gain, int Mb, int V,
                                    float* x, Frag xg, float* ssq, unsigned long long* keys, hipStream_t s) {
  if (B > DFLASH_ROWMAP_MAX || M < 1 || Mb < 1) return hipErrorInvalidValue;
  const FcFinArgs f{part, nsplit, mtiles, M, H, ri, B, nullptr, rowmap, seqs, cbuf, row0};
  const EmbedArgs e{ids, embed, gain, Mb, H, V, x, xg, ssq, keys};
  const unsigned nblk = (unsigned)(((M + 15) / 16) * (H / 64) + ((Mb + 15) / 16) * (H / 64));
  hipLaunchKernelGGL((fc_finalize_embed_kernel<T>), dim3(nblk), dim3(256), 0, s, f, e);
  return hipGetLastError();
}
template hipError_t launch_fc_finalize_embed<bf16_t>(const float*, int, int, int, int, const RowInfo&, int, RowMap*,
                                                     DevSeq*, Frag, int, const int32_t*, const void*, const float*,
                                                     int, int, float*, Frag, float*, unsigned long long*, hipStream_t);
template hipError_t launch_fc_finalize_embed<float>(const float*, int, int, int, int, const RowInfo&, int, RowMap*,
                                                    DevSeq*, Frag, int, const int32_t*, const void*, const float*,
                                                    int, int, float*, Frag, float*, unsigned long long*, hipStream_t);
template hipError_t launch_fc_finalize<bf16_t>(const float*, int, int, int, int, const RowInfo&, int,
                                               const int32_t*, RowMap*, DevSeq*, Frag, int, hipStream_t);
template hipError_t launch_fc_finalize<float>(const float*, int, int, int, int, const RowInfo&, int,
                                              const int32_t*, RowMap*, DevSeq*, Frag, int, hipStream_t);

// ---------------------------------------------------------------------------
// (a9) end of the block: draft ids from the argmax keys; optionally the
// final-normed hidden rows z = x * rsqrt(mean(x^2) + eps) * g.
// One workgroup per block row.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void finalize_kernel(const unsigned long long* keys, int M,
                                                       int32_t* draft, const float* x,
                                                       const float* ssq, int groups,
                                                       const float* gain, int H, float eps,
                                                       T* hidden) {
  const int m = blockIdx.x;
  if (threadIdx.x == 0) draft[m] = (int32_t)argmax_index(keys[m]);
  if (!hidden) return;
  float s = 0.f;
  for (int g = 0; g < groups; ++g) s += ssq[(size_t)g * M + m];
  const float r = rsqrtf(s / (float)H + eps);
  for (int c = threadIdx.x; c < H; c += blockDim.x)
    hidden[(size_t)m * H + c] = Elem<T>::from_f(x[(size_t)m * H + c] * r * gain[c]);
}

template <typename T>
hipError_t launch_finalize(const unsigned long long* keys, int M, int32_t* draft, const float* x,
                           const float* ssq, int groups, const float* gain, int H, float eps,
                           void* hidden, hipStream_t s) {
  hipLaunchKernelGGL((finalize_kernel<T>), dim3(M), dim3(256), 0, s, keys, M, draft, x, ssq, groups,
                     gain, H, eps, (T*)hidden);
  return hipGetLastError();
}
template hipError_t launch_finalize<bf16_t>(const unsigned long long*, int, int32_t*, const float*,
                                            const float*, int, const float*, int, float, void*,
                                            hipStream_t);
template hipError_t launch_finalize<float>(const unsigned long long*, int, int32_t*, const float*,
                                           const float*, int, const float*, int, float, void*,
                                           hipStream_t);

// ---------------------------------------------------------------------------
// (a10) greedy acceptance: one wave per sequence; a ballot of mismatches
// over 64 positions at a time gives the first disagreement.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void accept_kernel(const int32_t* draft, const int32_t* target,
                                                    int K, int32_t* out) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  int first = K;
  for (int i0 = 0; i0 < K; i0 += 64) {
    const int i = i0 + lane;
    const bool miss = i < K && draft[(size_t)b * K + i] != target[(size_t)b * K + i];
    const unsigned long long bal = __ballot(miss);
    if (bal) {
      first = i0 + __ffsll((long long)bal) - 1;
      break;
    }
  }
  if (lane == 0) out[b] = 1 + first;
}

hipError_t launch_accept(const int32_t* draft, const int32_t* target, int B, int K, int32_t* out,
                         hipStream_t s) {
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(64), 0, s, draft, target, K, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// weight repacking: packed row r comes from the source row at address
// row_src[r] (0 = zero row).  Output: tile r/16, block kb, lane
// (quarter*16 + r%16), 16 bytes holding KPL consecutive reduction elements.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void pack_kernel(const uint64_t* row_src, int n_rows, int kd, int nkb, uint8_t* dst) {
  using E = Elem<T>;
  const size_t pieces_per_row = (size_t)nkb * 4;
  const size_t total = (size_t)n_rows * pieces_per_row;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(t / pieces_per_row);
    const int pc = (int)(t % pieces_per_row);
    const int kb = pc >> 2, quarter = pc & 3;
    const T* src = (const T*)row_src[r];
    T vals[E::KPL];
#pragma unroll
    for (int e = 0; e < E::KPL; ++e) {
      const int k = kb * E::KB + quarter * E::KPL + e;
      vals[e] = (src && k < kd) ? src[k] : (T)0;
    }
    const int tile = r >> 4, rr = r & 15;
    uint8_t* out = dst + (((size_t)tile * nkb + kb) * WAVE + quarter * 16 + rr) * FRAG_BYTES;
    *(u32x4*)out = *(const u32x4*)vals;
  }
}

template <typename T>
hipError_t launch_pack(const uint64_t* row_src, int n_rows_padded, int kd, int nkb, uint8_t* dst,
                       hipStream_t s) {
  hipLaunchKernelGGL((pack_kernel<T>), dim3(2048), dim3(256), 0, s, row_src, n_rows_padded, kd,
                     nkb, dst);
  return hipGetLastError();
}
template hipError_t launch_pack<bf16_t>(const uint64_t*, int, int, int, uint8_t*, hipStream_t);
template hipError_t launch_pack<float>(const uint64_t*, int, int, int, uint8_t*, hipStream_t);

template <typename T>
__global__ void to_f32_kernel(const T* src, float* dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = Elem<T>::to_f(src[i]);
}
template <typename T>
hipError_t launch_to_f32(const void* src, float* dst, int n, hipStream_t s) {
  hipLaunchKernelGGL((to_f32_kernel<T>), dim3((n + 255) / 256), dim3(256), 0, s, (const T*)src,
                     dst, n);
  return hipGetLastError();
}
template hipError_t launch_to_f32<bf16_t>(const void*, float*, int, hipStream_t);
template hipError_t launch_to_f32<float>(const void*, float*, int, hipStream_t);

// ---------------------------------------------------------------------------
// (a2) projection rows: row j of a call goes to sequence b (from the prefix
// sums of n_new) at buffer row ctx_len[b] + (j - start[b]); its RoPE
// position is positions[j] or that row.  Then ctx_len[b] += n_new[b].
// One workgroup, so the reads of ctx_len precede the update.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rowmap_kernel(RowInfo ri, int B, int total,
                                                     const int32_t* positions, DevSeq* seqs,
                                                     RowMap* out) {
  for (int j = threadIdx.x; j < total; j += blockDim.x) out[j] = map_row(ri, B, j, positions);
  for (int b = threadIdx.x; b < B; b += blockDim.x) seqs[b].ctx_len = ri.ctx0[b] + ri.start[b + 1] - ri.start[b];
}

hipError_t launch_rowmap(const RowInfo& ri, int B, int total, const int32_t* positions, DevSeq* seqs,
                         RowMap* out, hipStream_t s) {
  if (B > DFLASH_ROWMAP_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rowmap_kernel, dim3(1), dim3(256), 0, s, ri, B, total, positions, seqs, out);
  return hipGetLastError();
}

__global__ void set_seq_kernel(DevSeq* seqs, int b, DevSeq v) { seqs[b] = v; }
hipError_t launch_set_seq(DevSeq* seqs, int b, DevSeq v, hipStream_t s) {
  hipLaunchKernelGGL(set_seq_kernel, dim3(1), dim3(1), 0, s, seqs, b, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// growth: copy the held rows [0, ctx_len) of the context buffer (fp32) and
// of every layer's K and V^T (attention type T) into larger buffers.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void grow_copy_kernel(DevSeq o, DevSeq n, int L, int nkv, int d, int H) {
  const int len = o.ctx_len;
  const size_t n_ctx = o.ctxbuf ? (size_t)len * H : 0;   // a target's sequences have no feature buffer
  const size_t n_k = (size_t)L * nkv * len * d;
  const size_t n_v = (size_t)L * nkv * d * len;
  const size_t total = n_ctx + n_k + n_v;
  const float* oc = (const float*)o.ctxbuf;
  const T* ok = (const T*)o.k;
  const T* ov = (const T*)o.vt;
  float* nc = (float*)n.ctxbuf;
  T* nk = (T*)n.k;
  T* nv = (T*)n.vt;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (size_t)gridDim.x * blockDim.x) {
    if (t < n_ctx) {
      nc[t] = oc[t];
    } else if (t < n_ctx + n_k) {
      const size_t u = t - n_ctx;
      const size_t row = u / d, e = u % d;           // row over (l, g, pos)
      const size_t lg = row / len, pos = row % len;
      nk[(lg * n.phys + pos) * d + e] = ok[(lg * o.phys + pos) * d + e];
    } else {
      const size_t u = t - n_ctx - n_k;
      const size_t row = u / len, pos = u % len;     // row over (l, g, d)
      nv[row * n.phys + pos] = ov[row * o.phys + pos];
    }
  }
}

template <typename T>
hipError_t launch_grow_copy(DevSeq oldv, DevSeq newv, int L, int nkv, int d, int H,
                            hipStream_t s) {
  if (oldv.ctx_len == 0) return hipSuccess;
  hipLaunchKernelGGL((grow_copy_kernel<T>), dim3(1024), dim3(256), 0, s, oldv, newv, L, nkv, d, H);
  return hipGetLastError();
}
template hipError_t launch_grow_copy<f16_t>(DevSeq, DevSeq, int, int, int, int, hipStream_t);
template hipError_t launch_grow_copy<float>(DevSeq, DevSeq, int, int, int, int, hipStream_t);

template <typename T>
__global__ void tap_kernel(const float* x, int M, int H, int tap, int n_taps, T* out) {
  const size_t n = (size_t)M * H;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (size_t)gridDim.x * blockDim.x) {
    const size_t m = t / H, h = t % H;
    out[(m * n_taps + tap) * H + h] = Elem<T>::from_f(x[t]);
  }
}

template <typename T>
hipError_t launch_tap(const float* x, int M, int H, int tap, int n_taps, void* out, hipStream_t s) {
  const size_t n = (size_t)M * H;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
  hipLaunchKernelGGL((tap_kernel<T>), dim3(blocks), dim3(256), 0, s, x, M, H, tap, n_taps, (T*)out);
  return hipGetLastError();
}
template hipError_t launch_tap<bf16_t>(const float*, int, int, int, int, void*, hipStream_t);
template hipError_t launch_tap<float>(const float*, int, int, int, int, void*, hipStream_t);

__global__ void fill_u32_kernel(unsigned* p, size_t n, unsigned v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}
hipError_t launch_fill_u32(unsigned* p, size_t n, unsigned v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace dflash
