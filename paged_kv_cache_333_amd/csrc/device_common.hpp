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
// 8-bit KV codes (the quantised cache): OCP FP8 E4M3 and two's-complement
// int8, 16 codes per chunk.  They are storage types only: decode widens them
// exactly to fp16/bf16 in registers.
struct TE4M3 {
  static constexpr int kBytes = 1;
  static constexpr int kEPL = 16;
};
struct TI8 {
  static constexpr int kBytes = 1;
  static constexpr int kEPL = 16;
};
// int8 codes with one fp32 scale per (token, KV head): each (block, KV head)
// tile holds its bs * D codes, then a scale area of whole 128-byte lines (so
// every tile's code rows stay line-aligned).  When the key and value scales of
// a block fit in one such area together (16-token blocks: 2 x 64 bytes in one
// line), the key tile's area holds the key scales, then the value scales, and
// the value tile's area is unused: a reader fetches one scale line per block
// instead of two half-used ones.  Otherwise each tile's area holds the scales
// of its own rows.
struct TI8T {
  static constexpr int kBytes = 1;
  static constexpr int kEPL = 16;
};
__host__ __device__ constexpr int64_t token_scale_area(int bs) { return (static_cast<int64_t>(bs) * 4 + 127) / 128 * 128; }
__host__ __device__ constexpr bool token_scales_paired(int bs) { return 8 * static_cast<int64_t>(bs) <= token_scale_area(bs); }
template <typename S>
struct row_scaled {
  static constexpr bool value = false;
};
template <>
struct row_scaled<TI8T> {
  static constexpr bool value = true;
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
// fp16 high part and fp16 residual of 8 weights (about 22 significant bits between them).
__device__ __forceinline__ void pack_p_split(TF16, const float* p, u32x4& hi, u32x4& lo) {
  f16x8 h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = static_cast<_Float16>(p[e]);
    l[e] = static_cast<_Float16>(p[e] - static_cast<float>(h[e]));
  }
  hi = __builtin_bit_cast(u32x4, h);
  lo = __builtin_bit_cast(u32x4, l);
}
__device__ __forceinline__ void pack_p_split(TBF16, const float* p, u32x4& hi, u32x4& lo) { pack_p(TBF16{}, p, hi, lo); }

// Low k bits set (k clamped to [0, 32]).
__device__ __forceinline__ uint32_t low_bits(int k) { return k <= 0 ? 0u : k >= 32 ? ~0u : (1u << k) - 1u; }

// Element mask of a chunk from a bit set: element e is kept iff bit e is set.
__device__ __forceinline__ u32x4 bits_mask(TF32, uint32_t bits) {
  return u32x4{bits & 1u ? ~0u : 0u, bits & 2u ? ~0u : 0u, bits & 4u ? ~0u : 0u, bits & 8u ? ~0u : 0u};
}
__device__ __forceinline__ u32x4 bits_mask_16(uint32_t bits) {
  u32x4 m;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    m[w] = ((bits >> (2 * w)) & 1u ? 0x0000ffffu : 0u) | ((bits >> (2 * w + 1)) & 1u ? 0xffff0000u : 0u);
  return m;
}
__device__ __forceinline__ u32x4 bits_mask(TF16, uint32_t bits) { return bits_mask_16(bits); }
__device__ __forceinline__ u32x4 bits_mask(TBF16, uint32_t bits) { return bits_mask_16(bits); }
__device__ __forceinline__ u32x4 bits_mask_8(uint32_t bits) {
  u32x4 m;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) x |= (bits >> (4 * w + i)) & 1u ? 0xffu << (8 * i) : 0u;
    m[w] = x;
  }
  return m;
}
__device__ __forceinline__ u32x4 bits_mask(TE4M3, uint32_t bits) { return bits_mask_8(bits); }
__device__ __forceinline__ u32x4 bits_mask(TI8, uint32_t bits) { return bits_mask_8(bits); }
__device__ __forceinline__ u32x4 bits_mask(TI8T, uint32_t bits) { return bits_mask_8(bits); }

// ---------------------------------------------------------------------------
// 8-bit codes -> fp16/bf16, exactly.  widen() turns one chunk of 16 codes into
// two chunks of the compute type: lo holds codes 0..7, hi codes 8..15, in
// order.  Every E4M3 value (subnormals and NaN included) and every int8 value
// is exact in both fp16 and bf16.

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Codes 2*HI and 2*HI + 1 of word w.  The gfx950 conversion scales by the
// power of two of its scale operand; 1.0 leaves the value as it is.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(TF16, uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(TBF16, uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// int8: for fp16, byte b is biased to u = b + 128 and placed in the mantissa
// of 1024 (f16 bits 0x6400 | u), then 1152 is subtracted: u - 128 = b, exact.
template <bool HI>
__device__ __forceinline__ uint32_t i8_pair(TF16, uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  // bytes (u0, 0x64, u1, 0x64) for HI = false, (u2, 0x64, u3, 0x64) for HI = true
  const uint32_t t = __builtin_amdgcn_perm(0x64646464u, u, HI ? 0x04030402u : 0x04010400u);
  const f16x2 v = __builtin_bit_cast(f16x2, t) - f16x2{static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  return __builtin_bit_cast(uint32_t, v);
}
template <bool HI>
__device__ __forceinline__ uint32_t i8_pair(TBF16, uint32_t w) {
  const float a = static_cast<float>(static_cast<int32_t>(w << (HI ? 8 : 24)) >> 24);  // byte 2 HI, signed
  const float b = static_cast<float>(static_cast<int32_t>(w << (HI ? 0 : 16)) >> 24);  // byte 2 HI + 1
  const bf16x2 v{static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T>
__device__ __forceinline__ void widen(TE4M3, T, u32x4 raw, u32x4& lo, u32x4& hi) {
  lo = u32x4{e4m3_pair<false>(T{}, raw[0]), e4m3_pair<true>(T{}, raw[0]), e4m3_pair<false>(T{}, raw[1]),
             e4m3_pair<true>(T{}, raw[1])};
  hi = u32x4{e4m3_pair<false>(T{}, raw[2]), e4m3_pair<true>(T{}, raw[2]), e4m3_pair<false>(T{}, raw[3]),
             e4m3_pair<true>(T{}, raw[3])};
}
template <typename T>
__device__ __forceinline__ void widen(TI8, T, u32x4 raw, u32x4& lo, u32x4& hi) {
  lo = u32x4{i8_pair<false>(T{}, raw[0]), i8_pair<true>(T{}, raw[0]), i8_pair<false>(T{}, raw[1]),
             i8_pair<true>(T{}, raw[1])};
  hi = u32x4{i8_pair<false>(T{}, raw[2]), i8_pair<true>(T{}, raw[2]), i8_pair<false>(T{}, raw[3]),
             i8_pair<true>(T{}, raw[3])};
}

template <typename T>
__device__ __forceinline__ void widen(TI8T, T, u32x4 raw, u32x4& lo, u32x4& hi) {
  widen(TI8{}, T{}, raw, lo, hi);
}

// ---------------------------------------------------------------------------
// fp32 -> 8-bit code, round to nearest even (the quantising write).

// E4M3: NaN -> 0x7F; |y| >= 448 (inf included) saturates to 448 (0x7E); the
// sign bit is kept, zeros included.  Below 2^-6 the codes are multiples of
// 2^-9 (subnormals; 8 * 2^-9 is the smallest normal, code 0x08, so the two
// ranges join).  Above, the fp32 mantissa is rounded to 3 bits on its bit
// pattern and the exponent rebiased from 127 to 7.
__device__ __forceinline__ uint32_t to_code(TE4M3, float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t ua = u & 0x7fffffffu;
  if (ua > 0x7f800000u) return 0x7fu;
  const float a = __builtin_bit_cast(float, ua);
  if (a >= 448.0f) return sign | 0x7eu;
  uint32_t mag;
  if (a < 0x1p-6f) {
    mag = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    const uint32_t r = ua + 0x7ffffu + ((ua >> 20) & 1u);
    mag = (r >> 20) - ((127u - 7u) << 3);
  }
  return sign | mag;
}
// int8: saturate to [-127, 127]; NaN -> 0.
__device__ __forceinline__ uint32_t to_code(TI8, float y) {
  if (y != y) return 0u;
  const float r = fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xffu;
}

// Storage element i of a chunk of a model type, as fp32 (exact).
__device__ __forceinline__ float elem_to_float(TF32, u32x4 c, int i) { return __builtin_bit_cast(float, word(c, i)); }
__device__ __forceinline__ float elem_to_float(TF16, u32x4 c, int i) {
  const uint32_t w = word(c, i >> 1);
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(i & 1 ? w >> 16 : w)));
}
__device__ __forceinline__ float elem_to_float(TBF16, u32x4 c, int i) {
  const uint32_t w = word(c, i >> 1);
  return __builtin_bit_cast(float, i & 1 ? w & 0xffff0000u : w << 16);
}

// Value of lane J of this lane's quad (DPP quad_perm [J, J, J, J]).
template <int J>
__device__ __forceinline__ float quad_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               J | (J << 2) | (J << 4) | (J << 6), 0xf, 0xf,
                                                               false));
}

// Value of lane J of this lane's row of 16 (DPP row_newbcast:J).
template <int J>
__device__ __forceinline__ float row_bcast_lane(float x) {
  static_assert(J >= 0 && J < 16, "a lane of the row");
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + J, 0xf, 0xf,
                                                               false));
}
// The same with the lane given by an expression that unrolling makes constant.
__device__ __forceinline__ float row_bcast(float x, int j) {
  switch (j) {
    case 0: return row_bcast_lane<0>(x);
    case 1: return row_bcast_lane<1>(x);
    case 2: return row_bcast_lane<2>(x);
    case 3: return row_bcast_lane<3>(x);
    case 4: return row_bcast_lane<4>(x);
    case 5: return row_bcast_lane<5>(x);
    case 6: return row_bcast_lane<6>(x);
    case 7: return row_bcast_lane<7>(x);
    case 8: return row_bcast_lane<8>(x);
    case 9: return row_bcast_lane<9>(x);
    case 10: return row_bcast_lane<10>(x);
    case 11: return row_bcast_lane<11>(x);
    case 12: return row_bcast_lane<12>(x);
    case 13: return row_bcast_lane<13>(x);
    case 14: return row_bcast_lane<14>(x);
    default: return row_bcast_lane<15>(x);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
