// Device helpers shared by the gfx950 kernels: element types, 16-byte row
// chunks, fp32 conversions, and cross-lane sums inside a row of lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// Unpack a 16-byte chunk into EPL floats (exact conversions).
__device__ __forceinline__ void to_float(TF32, u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __builtin_bit_cast(float, word(w, i));
}
__device__ __forceinline__ void to_float(TF16, u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = __builtin_bit_cast(f16x2, word(w, i));
    f[2 * i] = static_cast<float>(h[0]);
    f[2 * i + 1] = static_cast<float>(h[1]);
  }
}
__device__ __forceinline__ void to_float(TBF16, u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = word(w, i);
    f[2 * i] = __builtin_bit_cast(float, x << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, x & 0xffff0000u);
  }
}

// Dot product of two 16-byte chunks with fp32 accumulation.  fp16 and bf16
// use the packed two-element dot instructions (products are exact in fp32).
__device__ __forceinline__ float dot16(TF32, u32x4 a, u32x4 b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s = __builtin_fmaf(__builtin_bit_cast(float, word(a, i)), __builtin_bit_cast(float, word(b, i)), s);
  return s;
}
__device__ __forceinline__ float dot16(TF16, u32x4 a, u32x4 b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, word(a, i)), __builtin_bit_cast(f16x2, word(b, i)),
                               s, false);
  return s;
}
__device__ __forceinline__ float dot16(TBF16, u32x4 a, u32x4 b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, word(a, i)),
                                        __builtin_bit_cast(bf16x2, word(b, i)), s, false);
  return s;
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

// DPP lane moves inside a 16-lane row.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xb1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4e;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over each aligned group of LPR lanes; every lane of the group gets the sum.
// After the two quad steps all four lanes of a quad hold the quad's sum, so the
// mirror steps (lane i <-> 7-i, then i <-> 15-i) pair each lane with a lane of
// the other quad / half-row.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row width");
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp<kRowMirror>(x);
  if constexpr (LPR == 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
