// Loss-decay weighted cross-entropy of block-drafter logits (training side).
//
// kongchang.com "D-Flash", "Innovation 4: loss-decay weighted training":
// the cross-entropy of the token at in-block position k is weighted by
// gamma^k, so that early positions (whose errors void the rest of the
// block) weigh more; "Innovation 3: random anchor sampling": each block
// starts at a clean anchor and its rows predict the following tokens.
//
// Rows [R][V] are blocks of `block` rows (row r at in-block position
// r % block).  Targets outside [0, V) mark rows without a token.
//   w_r  = gamma^(r % block) for rows with a token, else 0
//   CE_r = logsumexp(l_r) - l_r[t_r]
//   loss = sum_r w_r CE_r / sum_r w_r        (0 when no row has a token)
//   grad = w_r / sum w * (softmax(l_r) - onehot(t_r))
//
// The weights depend on the targets only, so sum w is known before any
// logit is read, and each row's gradient needs nothing but its own
// log-sum-exp.  Three launches:
//   ce_scale  one workgroup: sum w in a fixed order (fp64) and each row's
//             gradient scale w_r / sum w;
//   ce_row    one 1024-thread workgroup per row, one row per compute unit
//             at a time: the row is loaded once into registers (16-byte
//             nontemporal loads, all in flight together), the sum of
//             exponentials runs as the loads land, then the gradient is
//             written from the registers, so HBM sees one read of the
//             logits and one write of the gradient.  Rows too long for the register file, or not
//             16-byte aligned, take a variant that reads the row twice
//             (the second time mostly from cache);
//   ce_loss   one workgroup: sum w CE / sum w in a fixed order (fp64), so
//             the loss is bitwise reproducible.
#include <limits.h>
#include <math.h>

#include <cmath>
#include <mutex>

#include "../../include/dflash.h"
#include "common.h"

namespace dflash {
namespace {

constexpr int RT = 1024;  // threads of a row workgroup
constexpr int RW = RT / WAVE;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;

template <typename T> __device__ __forceinline__ float ld1(const T* p) { return Elem<T>::to_f(*p); }

__device__ __forceinline__ bool has_token(int t, int V) { return t >= 0 && t < V; }

// A pointer that is the same in every lane, in scalar registers.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (P*)(((uint64_t)hi << 32) | lo);
}

// 2^y by the hardware instruction (about 1 ulp; results below the normal
// range may flush to zero, which neither the sums nor the gradient notice).
__device__ __forceinline__ float fexp2(float y) { return __builtin_amdgcn_exp2f(y); }

// gamma^k by binary powering (at most 2 log2 k + 1 roundings).
__device__ __forceinline__ double powi(double g, int k) {
  double r = 1.0;
  for (; k; k >>= 1) {
    if (k & 1) r *= g;
    g *= g;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Sums over rows in a fixed order: thread k takes the contiguous rows
// [k R / RT, (k+1) R / RT) in order (the weight by binary powering at the
// start of the range, then by the recurrence w <- w * gamma, reset to 1 at
// block starts), then an xor butterfly per wave and the 16 wave sums in
// order.  The result (thread 0's) depends on the inputs only, never on
// timing.  term(r, w) is added for rows with a token.
template <class F>
__device__ __forceinline__ double ordered_sum(const int32_t* targets, int R, int V, int block, double gamma,
                                              double* sh, F&& term) {
  const int a = (int)((long long)threadIdx.x * R / RT), b = (int)((long long)(threadIdx.x + 1) * R / RT);
  double acc = 0.0;
  if (a < b) {
    int k = a % block;
    double w = powi(gamma, k);
    for (int r = a; r < b; ++r) {
      if (has_token(targets[r], V)) acc += term(r, w);
      if (++k == block) {
        k = 0;
        w = 1.0;
      } else {
        w *= gamma;
      }
    }
  }
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & (WAVE - 1)) == 0) sh[threadIdx.x / WAVE] = acc;
  __syncthreads();
  double tot = 0.0;
  if (threadIdx.x == 0)
    for (int w = 0; w < RW; ++w) tot += sh[w];
  return tot;
}

// sum w, and every row's gradient scale c_r = w_r / sum w (0 for rows
// without a token) into ce[r], where the row kernel picks it up before it
// writes the row's cross-entropy there.
__global__ __launch_bounds__(RT) void ce_scale_kernel(const int32_t* targets, int R, int V, int block, double gamma,
                                                      double* wsum, float* ce) {
  __shared__ double sh[RW];
  __shared__ double W_sh;
  const double W = ordered_sum(targets, R, V, block, gamma, sh, [](int, double w) { return w; });
  if (threadIdx.x == 0) {
    *wsum = W;
    W_sh = W;
  }
  __syncthreads();
  const double Wb = W_sh;
  const int a = (int)((long long)threadIdx.x * R / RT), b = (int)((long long)(threadIdx.x + 1) * R / RT);
  if (a < b) {
    int k = a % block;
    double w = powi(gamma, k);
    for (int r = a; r < b; ++r) {
      ce[r] = (has_token(targets[r], V) && Wb > 0.0) ? (float)(w / Wb) : 0.f;
      if (++k == block) {
        k = 0;
        w = 1.0;
      } else {
        w *= gamma;
      }
    }
  }
}

__global__ __launch_bounds__(RT) void ce_loss_kernel(const int32_t* targets, const float* ce, int R, int V, int block,
                                                     double gamma, const double* wsum, float* loss) {
  __shared__ double sh[RW];
  const double S =
      ordered_sum(targets, R, V, block, gamma, sh, [ce](int r, double w) { return w * (double)ce[r]; });
  if (threadIdx.x == 0) {
    const double W = *wsum;
    *loss = W > 0.0 ? (float)(S / W) : 0.f;
  }
}

// ---------------------------------------------------------------------------
// (shift, sum of 2^(y - shift)) pairs in base-2 units (y = x log2 e); a pair
// with shift -inf is empty.
struct MS {
  float m, s;
};
__device__ __forceinline__ MS ms_merge(MS a, MS b) {
  if (a.m == -INFINITY) return b;
  if (b.m == -INFINITY) return a;
  const float mm = fmaxf(a.m, b.m);
  return {mm, a.s * fexp2(a.m - mm) + b.s * fexp2(b.m - mm)};
}
// Workgroup-wide merge; every thread gets the result.
__device__ __forceinline__ MS block_ms(MS v, MS* sh) {
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) v = ms_merge(v, {__shfl_xor(v.m, o), __shfl_xor(v.s, o)});
  if ((threadIdx.x & (WAVE - 1)) == 0) sh[threadIdx.x / WAVE] = v;
  __syncthreads();
  MS t = sh[0];
#pragma unroll
  for (int w = 1; w < RW; ++w) t = ms_merge(t, sh[w]);
  return t;
}

// 16-byte vectors of the row.  For bf16, word w of a vector holds elements
// 2w (low half) and 2w + 1 (high half).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <typename T> struct RowVec;
template <> struct RowVec<bf16_t> {
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
  static __device__ __forceinline__ float vmax(u32x4 v) {
    float m = fmaxf(lo(v[0]), hi(v[0]));
#pragma unroll
    for (int i = 1; i < 4; ++i) m = fmaxf(m, fmaxf(lo(v[i]), hi(v[i])));
    return m;
  }
  template <class F>
  static __device__ __forceinline__ float sum(u32x4 v, F&& f) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += f(lo(v[i])) + f(hi(v[i]));
    return s;
  }
  static __device__ __forceinline__ void unpack(u32x4 v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = lo(v[i]);
      o[2 * i + 1] = hi(v[i]);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float* f) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){f[2 * i], f[2 * i + 1]}, bf16x2_t));
    return r;
  }
};
template <> struct RowVec<float> {
  static __device__ __forceinline__ float vmax(u32x4 v) {
    return fmaxf(fmaxf(__uint_as_float(v[0]), __uint_as_float(v[1])),
                 fmaxf(__uint_as_float(v[2]), __uint_as_float(v[3])));
  }
  template <class F>
  static __device__ __forceinline__ float sum(u32x4 v, F&& f) {
    return (f(__uint_as_float(v[0])) + f(__uint_as_float(v[1]))) + (f(__uint_as_float(v[2])) + f(__uint_as_float(v[3])));
  }
  static __device__ __forceinline__ void unpack(u32x4 v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
  }
  static __device__ __forceinline__ u32x4 pack(const float* f) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
    return r;
  }
};

// Hides the row registers' contents from the optimiser, so that each pass
// unpacks the packed values again instead of keeping the unpacked copies
// (twice the registers for bf16) alive from the previous pass.
template <int NV>
__device__ __forceinline__ void opaque(u32x4 (&x)[NV]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(x[i]));
}

// Register-resident row: one 1024-thread workgroup per row; the row lives
// in NV 16-byte vectors per thread (vector j of the row in thread j % RT,
// slot j / RT), with NV = ceil(nvec / RT) so that only the last slot is
// partly empty (its loads are clamped into the row and its surplus lanes
// masked).  Requires V * sizeof(T) % 16 == 0 and 16-byte aligned bases, so
// every row is aligned.  All NV loads are issued at once.
//
// Each thread shifts its exponentials by the largest value of its first
// slot, so that its sum proceeds as the slots land, and the per-thread
// (shift, sum) pairs are merged exactly; then the gradient is written from
// the registers.  A thread whose sum could overflow in the merge, or whose
// first slot holds no finite value, redoes its sum from memory with its
// true maximum.
template <typename T, int NV, bool GRAD>
__global__ __launch_bounds__(RT) void ce_row_kernel(const T* logits, const int32_t* targets, int V, float* ce,
                                                    T* grad) {
  constexpr int N = Elem<T>::KPL;
  typedef RowVec<T> RV;
  __shared__ MS sh[RW];
  __shared__ float c_sh;  // the row's gradient scale
  const int r = blockIdx.x;
  const int nvec = V / N;
  const int jl = threadIdx.x + (NV - 1) * RT;  // this thread's vector in the last slot
  const bool last_ok = jl < nvec;
  const int jlc = last_ok ? jl : nvec - 1;
  // Vector of slot i: a uniform base (scalar registers) plus this thread's
  // 32-bit offset, shared by all full slots.
  const uint32_t off_full = threadIdx.x * 16u, off_last = (uint32_t)(jlc - (NV - 1) * RT) * 16u;
  const uint8_t* lrow = (const uint8_t*)uniform_ptr(logits + (size_t)r * V);
  auto vec = [&](int i) { return (const u32x4*)(lrow + (size_t)i * RT * 16 + (i < NV - 1 ? off_full : off_last)); };

  u32x4 x[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) x[i] = __builtin_nontemporal_load(vec(i));
  // After the row's loads: the target, the gradient scale (thread 0's copy
  // is used; thread 0 overwrites ce[r] below) and the target's logit, loaded
  // without branches so that waiting for them never holds up the row.
  const int t = targets[r];
  const float c0 = ce[r];
  const bool has_t = has_token(t, V);
  const float xt_any = ld1(logits + (size_t)r * V + (has_t ? t : 0));
  const float xt = has_t ? xt_any : 0.f;

  float mt = (NV > 1 || last_ok) ? RV::vmax(x[0]) * LOG2E : -INFINITY;
  float st = 0.f;
  if (mt != -INFINITY) {
    const float m = mt;
    auto ex = [m](float y) { return fexp2(fmaf(y, LOG2E, -m)); };
#pragma unroll
    for (int i = 0; i < NV - 1; ++i) st += RV::sum(x[i], ex);
    if (last_ok) st += RV::sum(x[NV - 1], ex);
  }
  // Sums up to 1e30 cannot overflow in the merges below (they only scale
  // down).  Rare: a larger or non-finite sum, or a first slot without a
  // finite value, is redone from memory with the thread's true maximum (a
  // rolled loop keeps the registers of the resident row).
  if (!(st <= 1.0e30f) || mt == -INFINITY) {
    const u32x4* row = (const u32x4*)lrow;
    float m = -INFINITY;
#pragma nounroll
    for (int j = threadIdx.x; j < nvec; j += RT) m = fmaxf(m, RV::vmax(row[j]));
    mt = m * LOG2E;
    st = 0.f;
    if (mt != -INFINITY) {
      const float mm = mt;
#pragma nounroll
      for (int j = threadIdx.x; j < nvec; j += RT)
        st += RV::sum(row[j], [mm](float y) { return fexp2(fmaf(y, LOG2E, -mm)); });
    }
  }
  if (threadIdx.x == 0) c_sh = c0;
  const MS tot = block_ms({mt, st}, sh);  // its barrier also publishes c_sh
  const float lse2 = tot.m + log2f(tot.s);  // log-sum-exp in base 2
  if (threadIdx.x == 0) ce[r] = has_t ? lse2 * LN2 - xt : 0.f;
  if constexpr (GRAD) {
    // c * 2^(y - lse2) as one exponential: 2^(y - (lse2 - log2 c)); c = 0
    // gives a shift of +inf and zeros.  At the target: c * (p_t - 1).
    const float c = c_sh;
    const float shift = c > 0.f ? lse2 - log2f(c) : INFINITY;
    const float gt = c * (fexp2(fmaf(xt, LOG2E, -lse2)) - 1.f);
    const int jt = has_t ? t / N : -1;  // vector holding the target
    const int it = has_t ? jt / RT : -1;  // its slot (the same for every thread)
    uint8_t* grow = (uint8_t*)uniform_ptr(grad + (size_t)r * V);
    opaque(x);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float f[N];
      RV::unpack(x[i], f);
#pragma unroll
      for (int e = 0; e < N; ++e) f[e] = fexp2(fmaf(f[e], LOG2E, -shift));
      if (i == it && (int)threadIdx.x + i * RT == jt) {
#pragma unroll
        for (int e = 0; e < N; ++e)
          if (e == t - jt * N) f[e] = gt;
      }
      if (i < NV - 1 || last_ok)
        __builtin_nontemporal_store(RV::pack(f),
                                    (u32x4*)(grow + (size_t)i * RT * 16 + (i < NV - 1 ? off_full : off_last)));
    }
  }
}

// Any V and alignment: the row is read twice, 16 bytes at a time between
// an unaligned head and tail.  The first read keeps a running (shift, sum)
// per thread, rescaled when a larger value appears; the second writes the
// gradient (16-byte stores when the gradient row has the logits row's
// alignment, else element stores).
template <typename T>
__global__ __launch_bounds__(RT) void ce_row2_kernel(const T* logits, const int32_t* targets, int V, float* ce,
                                                     T* grad) {
  constexpr int N = Elem<T>::KPL;
  typedef RowVec<T> RV;
  __shared__ MS sh[RW];
  __shared__ float c_sh;
  const int r = blockIdx.x;
  const T* row = logits + (size_t)r * V;
  const int head = min(V, (int)(((16 - ((uintptr_t)row & 15)) & 15) / sizeof(T)));
  const int nvec = (V - head) / N;
  const int tail0 = head + nvec * N;
  const u32x4* vrow = (const u32x4*)(row + head);
  const int t = targets[r];
  const bool has_t = has_token(t, V);
  if (threadIdx.x == 0) c_sh = ce[r];  // the gradient scale; thread 0 overwrites it below
  MS acc = {-INFINITY, 0.f};
  auto add1 = [&](float x) {
    const float y = x * LOG2E;
    if (y > acc.m) {
      acc.s = acc.m == -INFINITY ? 0.f : acc.s * fexp2(acc.m - y);
      acc.m = y;
    }
    if (acc.m != -INFINITY) acc.s += fexp2(fmaf(x, LOG2E, -acc.m));
  };
  for (int v = threadIdx.x; v < head; v += RT) add1(ld1(row + v));
  for (int v = tail0 + threadIdx.x; v < V; v += RT) add1(ld1(row + v));
  for (int j = threadIdx.x; j < nvec; j += RT) {
    const u32x4 x = __builtin_nontemporal_load(vrow + j);
    const float ym = RV::vmax(x) * LOG2E;
    if (ym > acc.m) {
      acc.s = acc.m == -INFINITY ? 0.f : acc.s * fexp2(acc.m - ym);
      acc.m = ym;
    }
    const float m = acc.m;
    if (m != -INFINITY) acc.s += RV::sum(x, [m](float v) { return fexp2(fmaf(v, LOG2E, -m)); });
  }
  const MS tot = block_ms(acc, sh);  // its barrier also publishes c_sh
  const float lse2 = tot.m + log2f(tot.s);
  if (threadIdx.x == 0) ce[r] = has_t ? lse2 * LN2 - ld1(row + t) : 0.f;
  if (!grad) return;
  const float c = c_sh;
  const float shift = c > 0.f ? lse2 - log2f(c) : INFINITY;
  const float gt = has_t ? c * (fexp2(fmaf(ld1(row + t), LOG2E, -lse2)) - 1.f) : 0.f;
  T* g = grad + (size_t)r * V;
  auto gval = [&](int v, float x) { return v == t ? gt : fexp2(fmaf(x, LOG2E, -shift)); };
  for (int v = threadIdx.x; v < head; v += RT) g[v] = Elem<T>::from_f(gval(v, ld1(row + v)));
  for (int v = tail0 + threadIdx.x; v < V; v += RT) g[v] = Elem<T>::from_f(gval(v, ld1(row + v)));
  const bool co_aligned = (((uintptr_t)(g + head)) & 15) == 0;
  for (int j = threadIdx.x; j < nvec; j += RT) {
    const u32x4 x = __builtin_nontemporal_load(vrow + j);
    float f[N];
    RV::unpack(x, f);
    const int v0 = head + j * N;
#pragma unroll
    for (int e = 0; e < N; ++e) f[e] = gval(v0 + e, f[e]);
    if (co_aligned) {
      __builtin_nontemporal_store(RV::pack(f), (u32x4*)(g + v0));
    } else {
#pragma unroll
      for (int e = 0; e < N; ++e) g[v0 + e] = Elem<T>::from_f(f[e]);
    }
  }
}

constexpr int NV_MAX = 20;  // 80 registers of row data per thread

template <typename T, int NV>
hipError_t row_launch(int need, const void* logits, const int32_t* targets, int R, int V, float* ce, void* grad,
                      hipStream_t s) {
  if constexpr (NV > NV_MAX) {
    return hipErrorInvalidValue;
  } else {
    if (need > NV) return row_launch<T, NV + 1>(need, logits, targets, R, V, ce, grad, s);
    if (grad)
      hipLaunchKernelGGL((ce_row_kernel<T, NV, true>), dim3(R), dim3(RT), 0, s, (const T*)logits, targets, V, ce,
                         (T*)grad);
    else
      hipLaunchKernelGGL((ce_row_kernel<T, NV, false>), dim3(R), dim3(RT), 0, s, (const T*)logits, targets, V, ce,
                         (T*)grad);
    return hipGetLastError();
  }
}

template <typename T>
hipError_t rows(const void* logits, const int32_t* targets, int R, int V, float* ce, void* grad, hipStream_t s) {
  constexpr int N = Elem<T>::KPL;
  const bool aligned = ((uintptr_t)logits % 16 == 0) && ((size_t)V * sizeof(T) % 16 == 0) &&
                       (!grad || (uintptr_t)grad % 16 == 0);
  const int nvec = V / N;
  const int need = (nvec + RT - 1) / RT;
  if (aligned && need >= 1 && need <= NV_MAX) return row_launch<T, 1>(need, logits, targets, R, V, ce, grad, s);
  hipLaunchKernelGGL((ce_row2_kernel<T>), dim3(R), dim3(RT), 0, s, (const T*)logits, targets, V, ce, (T*)grad);
  return hipGetLastError();
}

}  // namespace

int decay_ce_resident_max(int elem_bytes) { return NV_MAX * RT * (16 / elem_bytes); }

hipError_t launch_decay_ce(const void* logits, int dtype, const int32_t* targets, int R, int V, int block,
                           double gamma, float* loss, float* ce, void* grad, double* wsum, hipStream_t s) {
  hipLaunchKernelGGL(ce_scale_kernel, dim3(1), dim3(RT), 0, s, targets, R, V, block, gamma, wsum, ce);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (R > 0) {
    e = dtype == DFLASH_BF16 ? rows<bf16_t>(logits, targets, R, V, ce, grad, s)
                             : rows<float>(logits, targets, R, V, ce, grad, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(ce_loss_kernel, dim3(1), dim3(RT), 0, s, targets, ce, R, V, block, gamma, wsum, loss);
  return hipGetLastError();
}

}  // namespace dflash

// ---------------------------------------------------------------------------
// The same call for callers that cannot allocate (code under stream capture,
// serving loops that forbid allocation): the weight sum lives in a
// file-scope device array instead of a caller workspace.
// ---------------------------------------------------------------------------
// One copy per GPU, held until the process ends.  The kernels use one
// double of it (the weight sum W, written by ce_scale_kernel before
// ce_loss_kernel reads it on the same stream), whatever the rows and the
// vocabulary, so no input size can exceed it.  Calls that overlap on one
// GPU (different streams) race on it.
static __device__ __align__(256) unsigned char scratch[DFLASH_DECAY_CE_WORKSPACE];
static_assert(sizeof(double) <= DFLASH_DECAY_CE_WORKSPACE, "the weight sum must fit the scratch array");

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];   // device address of `scratch` per GPU (null until looked up)
}  // namespace

dflash_status dflash_set_error(dflash_status st, const char* msg);

extern "C" dflash_status dflash_decay_ce_noalloc(const void* logits, dflash_dtype dtype, const int32_t* targets,
                                                 int32_t rows, int32_t vocab, int32_t block, double gamma, float* loss,
                                                 float* ce, void* grad, void* stream) {
  using namespace dflash;
  if (!loss) return dflash_set_error(DFLASH_E_ARG, "NULL pointer");
  if (rows > 0 && (!logits || !targets || !ce)) return dflash_set_error(DFLASH_E_ARG, "NULL pointer");
  const int32_t dt = abi_int(dtype);
  if (dt != DFLASH_F32 && dt != DFLASH_BF16) return dflash_set_error(DFLASH_E_ARG, "bad dtype");
  if (rows < 0) return dflash_set_error(DFLASH_E_ARG, "rows < 0");
  if (vocab < 1) return dflash_set_error(DFLASH_E_ARG, "vocab < 1");
  if (block < 1) return dflash_set_error(DFLASH_E_ARG, "block < 1");
  if (!(gamma > 0.0) || !std::isfinite(gamma)) return dflash_set_error(DFLASH_E_ARG, "gamma must be finite and > 0");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return dflash_set_error(DFLASH_E_HIP, "no current HIP device (or more than 64 devices)");
  void* ptr = nullptr;
  {
    // once per GPU, with that GPU current: the array's device address (the
    // array's name in host code is a host-side stand-in, never passed on)
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return dflash_set_error(DFLASH_E_HIP, "hipGetSymbolAddress of the decay-CE scratch array failed");
      }
      g_scratch_dev[dev] = p;
    }
    ptr = g_scratch_dev[dev];
  }
  const hipError_t e = launch_decay_ce(logits, dt, targets, rows, vocab, block, gamma, loss, ce,
                                       rows > 0 ? grad : nullptr, (double*)ptr, (hipStream_t)stream);
  if (e != hipSuccess) return dflash_set_error(DFLASH_E_HIP, hipGetErrorString(e));
  return DFLASH_OK;
}
