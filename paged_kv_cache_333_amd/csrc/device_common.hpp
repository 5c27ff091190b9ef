// Device helpers shared by the gfx950 kernels: element types, 16-byte
// chunks, conversions, matrix-core products on chunks, and lane moves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element types.  Every K/V/q row is moved in 16-byte chunks (one
// global_load_dwordx4 per lane); EPL elements per chunk.
struct TF32 {
  static constexpr int kBytes = 4;
  static constexpr int kEPL = 4;
};
struct TF16 {
  static constexpr int kBytes = 2;
  static constexpr int kEPL = 8;
};
struct TBF16 {
  static constexpr int kBytes = 2;
  static constexpr int kEPL = 8;
};

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming load: the non-temporal hint keeps data that is read once from
// displacing reusable lines in the caches (the KV pool is read once per step).
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Word i of a chunk as a scalar.  (Bit-casting a vector element in place is
// not reliable: the element must be copied out first.)
__device__ __forceinline__ uint32_t word(u32x4 w, int i) {
  const uint32_t x = w[i];
  return x;
}

// fp32 -> storage type, round to nearest even.
__device__ __forceinline__ uint32_t from_float_bits(TF32, float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ uint16_t from_float_bits(TF16, float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
__device__ __forceinline__ uint16_t from_float_bits(TBF16, float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ void store_elem(T, void* base, int64_t idx, float x) {
  if constexpr (T::kBytes == 4)
    reinterpret_cast<uint32_t*>(base)[idx] = from_float_bits(T{}, x);
  else
    reinterpret_cast<uint16_t*>(base)[idx] = from_float_bits(T{}, x);
}

// ---------------------------------------------------------------------------
// Matrix-core products on 16-byte chunks.  For a 16x16 output tile C, lane
// l = 16 q + r supplies chunk a of row r of A and chunk b of column r of B;
// mma() adds, for every (m, n), the dot product of the chunks held by lanes
// {16 q + m} of A and {16 q + n} of B over all four q (4 x EPL elements).
// Lane 16 q + r receives C[4 q + j][r] in element j.  fp16/bf16 use one
// v_mfma_f32_16x16x32; fp32 uses four v_mfma_f32_16x16x4 (one per element).

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma(TF16, u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}
__device__ __forceinline__ f32x4 mma(TBF16, u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(TF32, u32x4 a, u32x4 b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, word(a, e)),
                                             __builtin_bit_cast(float, word(b, e)), c, 0, 0, 0);
  return c;
}

// EPL fp32 softmax weights -> one chunk of T, rounded to nearest even.  For
// bf16, `lo` receives the rounded residual p - hi, so hi + lo carries about
// 16 significant bits; the other types leave it untouched.
__device__ __forceinline__ void pack_p(TF32, const float* p, u32x4& hi, u32x4&) {
  hi = u32x4{__builtin_bit_cast(uint32_t, p[0]), __builtin_bit_cast(uint32_t, p[1]),
             __builtin_bit_cast(uint32_t, p[2]), __builtin_bit_cast(uint32_t, p[3])};
}
__device__ __forceinline__ void pack_p(TF16, const float* p, u32x4& hi, u32x4&) {
  f16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(p[e]);
  hi = __builtin_bit_cast(u32x4, h);
}
__device__ __forceinline__ void pack_p(TBF16, const float* p, u32x4& hi, u32x4& lo) {
  bf16x8 h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = static_cast<__bf16>(p[e]);
    l[e] = static_cast<__bf16>(p[e] - static_cast<float>(h[e]));
  }
  hi = __builtin_bit_cast(u32x4, h);
  lo = __builtin_bit_cast(u32x4, l);
}

// Bit mask keeping the first `keep` elements of a chunk (keep may be < 0 or > EPL).
__device__ __forceinline__ u32x4 keep_mask(TF32, int keep) {
  return u32x4{0 < keep ? ~0u : 0u, 1 < keep ? ~0u : 0u, 2 < keep ? ~0u : 0u, 3 < keep ? ~0u : 0u};
}
__device__ __forceinline__ u32x4 keep_mask_16(int keep) {
  u32x4 m;
#pragma unroll
  for (int w = 0; w < 4; ++w) m[w] = (2 * w < keep ? 0x0000ffffu : 0u) | (2 * w + 1 < keep ? 0xffff0000u : 0u);
  return m;
}
__device__ __forceinline__ u32x4 keep_mask(TF16, int keep) { return keep_mask_16(keep); }
__device__ __forceinline__ u32x4 keep_mask(TBF16, int keep) { return keep_mask_16(keep); }

// Value of lane J of this lane's quad (DPP quad_perm [J, J, J, J]).
template <int J>
__device__ __forceinline__ float quad_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               J | (J << 2) | (J << 4) | (J << 6), 0xf, 0xf,
                                                               false));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
