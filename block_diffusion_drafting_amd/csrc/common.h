// Device-side helpers shared by the DFlash HIP kernels (gfx950 / CDNA4).
//
// Fragment convention used by every MFMA in this library.  A "fragment" is
// 16 bytes per lane of a 64-lane wave: lane l holds row (l % 16) and the
// (l / 16)-th quarter of a 64-byte run along the reduction axis.  For bf16
// that is 8 elements (one v_mfma_f32_16x16x32_bf16), for fp32 4 elements
// (four v_mfma_f32_16x16x4_f32, element j of every lane in the j-th).  The
// A and B operands use the same per-lane reduction indices, so any fixed
// permutation of the reduction axis inside a fragment is harmless.
// Accumulator: lane l holds rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef uint16_t bf16_t;
typedef _Float16 f16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The int32 a caller stored in an enum field or parameter of the C ABI.  C
// lets such an enum hold any int, while loading a value outside its
// enumerators through the C++ enum type is undefined, so the bytes are read.
template <typename E>
inline int32_t abi_int(const E& v) {
  static_assert(sizeof(E) == sizeof(int32_t), "C ABI enums are 32-bit");
  int32_t i;
  __builtin_memcpy(&i, &v, sizeof i);
  return i;
}

constexpr int WAVE = 64;
constexpr int FRAG_BYTES = 16;
constexpr int BLOCK_BYTES = WAVE * FRAG_BYTES;  // one 16-row x 64-byte tile block

__device__ __forceinline__ float bf2f(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int KB = 32;   // reduction elements per 64-byte block row
  static constexpr int KPL = 8;   // elements per lane fragment
  __device__ static __forceinline__ float to_f(bf16_t v) { return bf2f(v); }
  __device__ static __forceinline__ bf16_t from_f(float v) { return f2bf(v); }
  __device__ static __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
// fp16 is the storage type of attention operands (KV caches, queries,
// probabilities) of bf16 models: the same bytes and MFMA rate as bf16 with
// three more mantissa bits.  Stores saturate to the finite fp16 range.
__device__ __forceinline__ f16_t f2h(float f) {
  f = fminf(fmaxf(f, -65504.f), 65504.f);
  return (f16_t)f;
}
template <> struct Elem<f16_t> {
  static constexpr int KB = 32;
  static constexpr int KPL = 8;
  __device__ static __forceinline__ float to_f(f16_t v) { return (float)v; }
  __device__ static __forceinline__ f16_t from_f(float v) { return f2h(v); }
  __device__ static __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <> struct Elem<float> {
  static constexpr int KB = 16;
  static constexpr int KPL = 4;
  __device__ static __forceinline__ float to_f(float v) { return v; }
  __device__ static __forceinline__ float from_f(float v) { return v; }
  __device__ static __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};

// Unpack a 16-byte fragment into KPL floats.
template <typename T>
__device__ __forceinline__ void frag_to_f(u32x4 v, float* out);
template <>
__device__ __forceinline__ void frag_to_f<bf16_t>(u32x4 v, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = v[i];
    o[2 * i] = __uint_as_float(w << 16);
    o[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void frag_to_f<f16_t>(u32x4 v, float* o) {
  const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)h[i];
}
template <>
__device__ __forceinline__ void frag_to_f<float>(u32x4 v, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
}
template <typename T>
__device__ __forceinline__ u32x4 f_to_frag(const float* f);
template <>
__device__ __forceinline__ u32x4 f_to_frag<bf16_t>(const float* f) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = (uint32_t)f2bf(f[2 * i]) | ((uint32_t)f2bf(f[2 * i + 1]) << 16);
  return r;
}
template <>
__device__ __forceinline__ u32x4 f_to_frag<f16_t>(const float* f) {
  f16x8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = f2h(f[i]);
  return __builtin_bit_cast(u32x4, h);
}
template <>
__device__ __forceinline__ u32x4 f_to_frag<float>(const float* f) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
  return r;
}

// Attention operand type of a model element type.
template <typename T> struct CacheOf { typedef T type; };
template <> struct CacheOf<bf16_t> { typedef f16_t type; };

// One fragment of fp32 activations as MFMA operands: `hi` rounds the values
// to T; `lo` rounds the remainder, so hi + lo carries about twice T's
// mantissa (used where activation rounding would dominate the error).
template <typename T, bool SPLIT>
__device__ __forceinline__ void split_frag(const float* v, u32x4& hi, u32x4& lo) {
  hi = f_to_frag<T>(v);
  if constexpr (SPLIT) {
    float h[Elem<T>::KPL], r[Elem<T>::KPL];
    frag_to_f<T>(hi, h);
#pragma unroll
    for (int i = 0; i < Elem<T>::KPL; ++i) r[i] = v[i] - h[i];
    lo = f_to_frag<T>(r);
  }
}

// Loads through pointers the compiler cannot prove global (fields of device
// structs) would otherwise become flat operations, which wait on both the
// memory and the LDS counters; these force global-memory instructions.
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
__device__ __forceinline__ u32x4 gld16(const void* p) { return *(gu32x4*)p; }
template <typename T>
__device__ __forceinline__ T gld(const T* p) {
  return *(__attribute__((address_space(1))) const T*)p;
}
// The same pointer as a global-memory pointer (for stores).
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gp(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// Monotone 32-bit key of a float (NaN maps below every number).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// 64-bit argmax key: larger value wins, then lower index.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  return ((unsigned long long)order_key(v) << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t argmax_index(unsigned long long key) {
  return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull);
}

// IEEE 754-2019 maximum (a NaN operand gives NaN): one v_maximum3_f32 for
// up to three operands.  fmaxf (maxNum) needs its operands quieted first in
// the default IEEE mode, one more VALU instruction per operand that is not
// the result of arithmetic (an MFMA result, a lane exchange).
__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Reductions over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes of one
// MFMA output column).  v_permlane16_swap / v_permlane32_swap applied to two
// copies of v leave, in every lane, v and the value of lane l ^ 16 (l ^ 32)
// as the pair: VALU instructions, where a shuffle (ds_bpermute) runs in the
// LDS pipeline and its wait also waits for every LDS read issued before it.
// Same results as the shuffles, bit for bit (maxima, and sums of two terms).
__device__ __forceinline__ float xor16_max(float v) {
  const unsigned u = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmax_ieee(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const unsigned u = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmax_ieee(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const unsigned u = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const unsigned u = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float wave_xor_max16_32(float v) { return xor32_max(xor16_max(v)); }
__device__ __forceinline__ float wave_xor_sum16_32(float v) { return xor32_sum(xor16_sum(v)); }

// Per-sequence device descriptor of the proposer state.
struct DevSeq {
  int32_t ctx_len;     // committed positions held
  int32_t cap;         // logical capacity (power of two, or 0)
  int32_t phys;        // allocated rows per buffer (>= cap, >= 64)
  int32_t pad;
  void* ctxbuf;        // [phys][hidden]
  void* k;             // [L][nkv][phys][d]
  void* vt;            // [L][nkv][d][phys]
};

// Row of a projection call: target sequence, buffer row, RoPE position.
struct RowMap {
  int32_t b, slot, pos, pad;
};

}  // namespace dflash
